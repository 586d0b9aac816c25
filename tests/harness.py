"""Test-side glue between the oracle, the workload generator and the HIP path.

Nothing here computes the method: it lays out pools (from the documented
format), moves bytes between host and device, decodes packed rows with an
independent numpy unpacker, and states the parity criteria.
"""
from __future__ import annotations

import numpy as np

import oracle as O
import workload as W

# ----------------------------------------------------------------- format
def record_bytes(bits: int, d: int) -> int:
    if bits == 16:  # FP16 pivot record: the state as binary16, no scales
        return 2 * d * d
    return d * d * bits // 8 + 8 * d


def record_bytes_rows(row_bits, d: int) -> int:
    """A head with per-key-row widths: the rows' streams, r and c, padded to 256 B."""
    raw = sum(d * int(b) // 8 for b in row_bits) + 8 * d
    return (raw + 255) // 256 * 256


def head_record_bytes(bits: int, d: int, row_bits=None) -> int:
    return record_bytes_rows(row_bits, d) if bits == 0 else record_bytes(bits, d)


def layout(head_bits, d, row_bits=None):
    """slot_stride and per-head record offsets of the documented pool layout."""
    offs, pos = [], 0
    for h, b in enumerate(head_bits):
        offs.append(pos)
        pos += head_record_bytes(int(b), d, None if row_bits is None else row_bits[h])
    return pos, np.array(offs, np.int64)


def _unpack_rows(bits: int, raw: np.ndarray, d: int) -> np.ndarray:
    """raw: [n, d * bits / 8] packed rows -> codes [n, d]."""
    n = raw.shape[0]
    if bits == 8:
        return raw.view(np.int8).astype(np.int32)
    if bits == 4:
        lo = (raw & 0xF).astype(np.int32)
        hi = (raw >> 4).astype(np.int32)
        codes = np.stack([lo, hi], axis=-1).reshape(n, d)
        return np.where(codes >= 8, codes - 16, codes)
    g = raw.reshape(n, d // 4, 3).astype(np.uint32)
    word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    codes = np.stack([(word >> (6 * m)) & 63 for m in range(4)], axis=-1).reshape(n, d)
    codes = codes.astype(np.int32)
    return np.where(codes >= 32, codes - 64, codes)


def unpack_codes(bits: int, d: int, rec: np.ndarray, row_bits=None) -> np.ndarray:
    """Codes [d, d] of one record, decoded with numpy bit arithmetic (for an
    FP16 pivot record: the binary16 bit patterns; bits 0: per-row widths)."""
    if bits == 16:
        return rec[: 2 * d * d].view(np.uint16).reshape(d, d).astype(np.int32)
    if bits == 0:
        out, pos = [], 0
        for b in row_bits:
            n = d * int(b) // 8
            out.append(_unpack_rows(int(b), rec[pos:pos + n].reshape(1, n), d)[0])
            pos += n
        return np.stack(out)
    rb = d * bits // 8
    raw = rec[: d * rb].reshape(d, rb)
    if bits == 8:
        return raw.view(np.int8).astype(np.int32)
    if bits == 4:
        lo = (raw & 0xF).astype(np.int32)
        hi = (raw >> 4).astype(np.int32)
        codes = np.stack([lo, hi], axis=-1).reshape(d, d)
        return np.where(codes >= 8, codes - 16, codes)
    g = raw.reshape(d, d // 4, 3).astype(np.uint32)
    word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    codes = np.stack([(word >> (6 * m)) & 63 for m in range(4)], axis=-1).reshape(d, d)
    codes = codes.astype(np.int32)
    return np.where(codes >= 32, codes - 64, codes)


def record_scales(bits: int, d: int, rec: np.ndarray, row_bits=None):
    if bits == 16:
        return ()
    cb = sum(d * int(b) // 8 for b in row_bits) if bits == 0 else d * (d * bits // 8)
    sc = rec[cb: cb + 8 * d].view(np.float32)
    return sc[:d].copy(), sc[d:].copy()


# ----------------------------------------------------------------- pools
class HostPool:
    """Host image of a pool in the documented layout (oracle side)."""

    def __init__(self, n_slots, head_bits, d, row_bits=None):
        self.d = d
        self.head_bits = np.asarray(head_bits, np.uint8)
        self.row_bits = row_bits
        self.H = len(head_bits)
        self.stride, self.head_off = layout(head_bits, d, row_bits)
        self.bytes = np.zeros(n_slots * self.stride, np.uint8)

    def offsets(self, slots, heads):
        slots = np.asarray(slots, np.int64)
        heads = np.asarray(heads, np.int64)
        return slots * self.stride + self.head_off[heads]

    def record(self, slot, h):
        o = slot * self.stride + self.head_off[h]
        rb = None if self.row_bits is None else self.row_bits[h]
        return self.bytes[o: o + head_record_bytes(int(self.head_bits[h]), self.d, rb)]


def rows_all(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def inputs_f32(x: dict) -> dict:
    return {k: W.to_f32(v) for k, v in x.items()}


def oracle_warmup(wl: W.Workload, layer: W.Layer, rows, steps: int = W.WARMUP_STEPS):
    """Unquantized FP64 warm-up from S = 0 over steps t = -steps .. -1 for the
    given (b, h) rows; returns fp32 states [len(rows), d, d]."""
    d = wl.d
    S = np.zeros((len(rows), d, d), np.float64)
    for t in range(-steps, 0):
        x = inputs_f32(wl.step_inputs(layer, t, rows))
        O.f64_step(layer.gate == "kda", S, x["q"], x["k"], x["v"], x["beta"], x["g"])
    return S.astype(np.float32)


# ----------------------------------------------------------------- criteria
def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def to_bf16_f32(x) -> np.ndarray:
    """Round to bf16 (via fp32, nearest even) and widen back."""
    return W.bf16_to_f32(W.f32_to_bf16(np.asarray(x, np.float64).astype(np.float32)))


def compare_codes(q_gpu: np.ndarray, q_ref: np.ndarray):
    """Returns (max |dQ|, fraction of entries with dQ != 0)."""
    d = np.abs(q_gpu.astype(np.int64) - q_ref.astype(np.int64))
    return int(d.max()) if d.size else 0, float((d != 0).mean()) if d.size else 0.0


CODE_FLIP_FRACTION = 1e-4   # at most 1e-4 of the codes may differ, each by 1 LSB
SCALE_RTOL = 1e-5           # row / column scales
Y_REL_L2 = 1e-3             # per-step output
STATE_REL_L2 = 1e-3         # dequantized state after a trajectory
