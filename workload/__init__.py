"""Seeded synthetic workloads for the quantized gated Delta-rule decode step.

Holds no arithmetic of the method: it describes the five workload shapes and
draws their inputs through ``sqgen.c`` (counter-based SplitMix64, Box-Muller),
so that the CPU oracle and the HIP path always see the same bytes.

Workloads (the decode shapes the hybrid GDN / KDA serving case uses):

====  ====  ====  ====  ===  =====================  =====  =======  ======
name  gate  B     H     d    bits per head          dtype  slots    steps
====  ====  ====  ====  ===  =====================  =====  =======  ======
c0    GDN   1     1     64   6                      f32    1        64
c1    GDN   64    32    128  6                      bf16   64       256
c2    KDA   128   32    128  4/6/8 = 8/16/8 heads   bf16   128      256
c3a   GDN   512   48    128  6                      bf16   640      20
c3b   GDN   512   48    128  8 if half-life > 64    bf16   640      20
c4    GDN   1024  32    128  4/6/8 = 8/16/8 heads   bf16   1024     1024
      +KDA  (second layer, same shape)
====  ====  ====  ====  ===  =====================  =====  =======  ======

The half-life of a head with log-gate -a is ln 2 / a steps; "half-life > 64"
therefore means a < ln 2 / 64.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sqgen.c")
_LIB_PATH = os.path.join(_HERE, "libsqgen.so")
_lib = None

WARMUP_STEPS = 128


_SAN_PATH = os.path.join(_HERE, "libsqgen_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def build_lib(sanitize: bool = False) -> str:
    """Compile ``sqgen.c`` into ``libsqgen.so`` beside it (always recompiles).
    sanitize: AddressSanitizer + UndefinedBehaviorSanitizer build, written to
    libsqgen_san.so and loaded instead when SQ_SANITIZE=1."""
    out = _SAN_PATH if sanitize else _LIB_PATH
    tmp = out + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread"] +
        (SANITIZE_FLAGS if sanitize else []) + [_SRC, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        san = os.environ.get("SQ_SANITIZE") == "1"
        path = _SAN_PATH if san else _LIB_PATH
        if not os.path.exists(path):
            build_lib(sanitize=san)
        L = ctypes.CDLL(path)
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        L.sqg_key.restype = u64
        L.sqg_key.argtypes = [u64, u64, i64, i64, i64, i64]
        L.sqg_draw.restype = u64
        L.sqg_draw.argtypes = [u64, u64]
        L.sqg_uniform.restype = ctypes.c_double
        L.sqg_uniform.argtypes = [u64, u64]
        L.sqg_normal.restype = ctypes.c_double
        L.sqg_normal.argtypes = [u64, u64]
        L.sqg_gate_rates.restype = None
        L.sqg_gate_rates.argtypes = [u64, i64, i32, i32, i32, vp]
        L.sqg_shuffle.restype = None
        L.sqg_shuffle.argtypes = [u64, u64, i64, i32, vp]
        L.sqg_step_inputs.restype = i32
        L.sqg_step_inputs.argtypes = [u64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp,
                                      vp, vp, vp, vp, vp, i32]
        L.sqg_normals.restype = None
        L.sqg_normals.argtypes = [u64, i64, i64, i64, i64, i64, vp]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


ST_BITS, ST_SLOTS = 6, 7
LN2 = math.log(2.0)


def n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> raw bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


@dataclasses.dataclass
class Layer:
    """One gated Delta-rule layer of a workload."""
    gate: str                 # "gdn" (scalar gate per head) or "kda" (per key channel)
    head_bits: np.ndarray     # uint8 [H]
    gate_rates: np.ndarray    # float64 [H] (GDN) or [H, d] (KDA): log-gate = -rate
    slot_of: np.ndarray       # int32 [B]: request b lives in pool slot slot_of[b]
    index: int                # layer index in the seed key
    row_bits: Optional[np.ndarray] = None  # uint8 [H, d]: key-row widths of heads with bits 0


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    d: int
    dtype: str                # "f32" or "bf16"
    n_slots: int
    steps: int
    seed: int
    layers: list

    @property
    def in_dtype_code(self) -> int:
        return 0 if self.dtype == "f32" else 1

    def step_inputs(self, layer: Layer, t: int, rows: Optional[Sequence] = None) -> dict:
        """Inputs of step t for all B*H rows (or the given (b, h) rows).

        Returns raw arrays in the storage dtype (float32, or uint16 bf16 bits):
        q, k, v: [n, d]; beta: [n]; g: [n] (GDN) or [n, d] (KDA)."""
        return step_inputs(self.seed, layer, t, self.B, self.H, self.d, self.dtype, rows)


def step_inputs(seed, layer: Layer, t, B, H, d, dtype, rows=None) -> dict:
    L = lib()
    kda = layer.gate == "kda"
    if rows is None:
        n = B * H
        bl = hl = None
    else:
        rows = np.asarray(rows, dtype=np.int32).reshape(-1, 2)
        n = rows.shape[0]
        bl = np.ascontiguousarray(rows[:, 0])
        hl = np.ascontiguousarray(rows[:, 1])
    npdt = np.float32 if dtype == "f32" else np.uint16
    q = np.empty((n, d), npdt)
    k = np.empty((n, d), npdt)
    v = np.empty((n, d), npdt)
    beta = np.empty((n,), npdt)
    g = np.empty((n, d) if kda else (n,), npdt)
    rates = np.ascontiguousarray(layer.gate_rates, dtype=np.float64)
    rc = L.sqg_step_inputs(seed, layer.index, t, H, d, int(kda), 0 if dtype == "f32" else 1,
                           n, _ptr(bl), _ptr(hl), _ptr(rates), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(beta), _ptr(g), n_threads())
    if rc != 0:
        raise ValueError("sqg_step_inputs rejected its arguments")
    return {"q": q, "k": k, "v": v, "beta": beta, "g": g}


def to_f32(a: np.ndarray) -> np.ndarray:
    """Storage dtype -> float32 (exact)."""
    return a if a.dtype == np.float32 else bf16_to_f32(a)


def gate_rates(seed: int, layer: int, H: int, d: int, per_channel: bool) -> np.ndarray:
    out = np.empty((H, d) if per_channel else (H,), np.float64)
    lib().sqg_gate_rates(seed, layer, H, d, int(per_channel), _ptr(out))
    return out


def shuffled(seed: int, stream: int, layer: int, values: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(values, dtype=np.int32).copy()
    lib().sqg_shuffle(seed, stream, layer, a.size, _ptr(a))
    return a


def mixed_bits(seed: int, layer: int, H: int) -> np.ndarray:
    """Bits 4/6/8 at exactly 25/50/25 % of the heads, placed by a seeded shuffle."""
    n4 = H // 4
    n8 = H // 4
    base = np.array([4] * n4 + [6] * (H - n4 - n8) + [8] * n8, np.int32)
    return shuffled(seed, ST_BITS, layer, base).astype(np.uint8)


def rounded_rates(rates: np.ndarray, dtype: str) -> np.ndarray:
    """The rate a the kernels actually see: -(log-gate rounded to the dtype)."""
    g = (-rates).astype(np.float32)
    if dtype == "bf16":
        g = bf16_to_f32(f32_to_bf16(g))
    return -g.astype(np.float64)


def halflife_bits(rates_seen: np.ndarray, horizon: float = 64.0) -> np.ndarray:
    """8 bits for heads whose half-life ln2 / a exceeds `horizon` steps, else 4."""
    return np.where(LN2 / rates_seen > horizon, 8, 4).astype(np.uint8)


def slot_permutation(seed: int, layer: int, B: int, n_slots: int) -> np.ndarray:
    perm = shuffled(seed, ST_SLOTS, layer, np.arange(n_slots, dtype=np.int32))
    return np.ascontiguousarray(perm[:B])


def make(name: str, seed: int = 0, steps: Optional[int] = None) -> Workload:
    """Build one of the named workloads (see the module docstring)."""
    def layer(gate, idx, H, d, bits, n_slots, B, permute, dtype):
        rates = gate_rates(seed, idx, H, d, gate == "kda")
        if isinstance(bits, str) and bits == "mixed":
            hb = mixed_bits(seed, idx, H)
        elif isinstance(bits, str) and bits == "halflife":
            hb = halflife_bits(rounded_rates(rates, dtype))
        else:
            hb = np.full(H, bits, np.uint8)
        slots = (slot_permutation(seed, idx, B, n_slots) if permute
                 else np.arange(B, dtype=np.int32))
        return Layer(gate, hb, rates, slots, idx)

    if name == "c0":
        B, H, d, dt, ns, st = 1, 1, 64, "f32", 1, 64
        layers = [layer("gdn", 0, H, d, 6, ns, B, False, dt)]
    elif name == "c1":
        B, H, d, dt, ns, st = 64, 32, 128, "bf16", 64, 256
        layers = [layer("gdn", 0, H, d, 6, ns, B, False, dt)]
    elif name == "c2":
        B, H, d, dt, ns, st = 128, 32, 128, "bf16", 128, 256
        layers = [layer("kda", 0, H, d, "mixed", ns, B, False, dt)]
    elif name in ("c3a", "c3b"):
        B, H, d, dt, ns, st = 512, 48, 128, "bf16", 640, 20
        if name == "c3b":
            # first seed at or above the requested one with at least one 8-bit head
            s = seed
            while True:
                r = rounded_rates(gate_rates(s, 0, H, d, False), dt)
                if (halflife_bits(r) == 8).any():
                    break
                s += 1
            seed = s
        layers = [layer("gdn", 0, H, d, 6 if name == "c3a" else "halflife", ns, B, True, dt)]
    elif name == "c4":
        B, H, d, dt, ns, st = 1024, 32, 128, "bf16", 1024, 1024
        layers = [layer("gdn", 0, H, d, "mixed", ns, B, False, dt),
                  layer("kda", 1, H, d, "mixed", ns, B, False, dt)]
    else:
        raise KeyError(name)
    return Workload(name, B, H, d, dt, ns, st if steps is None else steps, seed, layers)


def custom(gate: str, B: int, H: int, d: int, head_bits, dtype: str = "bf16",
           n_slots: Optional[int] = None, permute: bool = False, seed: int = 0,
           steps: int = 1, name: str = "custom", row_bits=None) -> Workload:
    """A workload of any shape with the same value recipe (used for edge cases).
    row_bits [H, d]: key-row widths of the heads whose head_bits is 0."""
    n_slots = B if n_slots is None else n_slots
    hb = np.asarray(head_bits, np.uint8)
    if hb.size == 1:
        hb = np.full(H, int(hb.reshape(-1)[0]), np.uint8)
    rates = gate_rates(seed, 0, H, d, gate == "kda")
    slots = slot_permutation(seed, 0, B, n_slots) if permute else np.arange(B, dtype=np.int32)
    rb = None if row_bits is None else np.ascontiguousarray(row_bits, np.uint8)
    return Workload(name, B, H, d, dtype, n_slots, steps, seed,
                    [Layer(gate, hb, rates, slots, 0, rb)])


def row_widths_by_lifetime(rates: np.ndarray, fractions=(0.25, 0.5, 0.25), grain: int = 8):
    """Key-row widths per head for a KDA layer whose key channels are stored
    in order of decreasing gate rate (increasing lifetime), i.e. after the
    offline channel permutation: the fastest-decaying rows 4-bit, the middle
    6-bit, the longest-lived 8-bit, in the given fractions rounded to the
    grain the pool layout needs.  Returns (row_bits [H, d], the channel
    permutation perm [H, d] with physical row p = channel perm[h, p])."""
    H, d = rates.shape
    perm = np.argsort(-rates, axis=1, kind="stable").astype(np.int64)
    n4 = int(round(fractions[0] * d / grain)) * grain
    n8 = int(round(fractions[2] * d / grain)) * grain
    w = np.array([4] * n4 + [6] * (d - n4 - n8) + [8] * n8, np.uint8)
    return np.tile(w, (H, 1)), perm


def normals(seed: int, layer: int, t: int, b: int, h: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().sqg_normals(seed, layer, t, b, h, n, _ptr(out))
    return out
