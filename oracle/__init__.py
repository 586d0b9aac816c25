"""CPU oracle for the quantized gated Delta-rule decode step (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.  It shares no code
with the HIP library; the arithmetic lives in ``sq_oracle.c`` (plain C).
Two step definitions live there: the textbook one (``gated_delta_f64``,
``f64_step``: the whole step in FP64 on the exact reconstruction, for S'
rounded once to fp32 and then the pinned fp32 quantizer), and the trajectory
contract (``step_update``, ``records_step``: the look-up in FP64 with u
rounded once to fp32, the rank-1 write element-wise in fp32, then the same
quantizer), which fixes every rounding the stored codes depend on.

Pins: every function here is checked, in the CPU tests, against closed
forms, identities, brute force on tiny inputs or an unquantized FP64
recurrence.  There is no worked numeric example on the pages to compare with.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsq_oracle.so")
_lib = None


_SAN_PATH = os.path.join(_HERE, "libsq_oracle_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def build_lib(sanitize: bool = False) -> str:
    """Compile the oracle (always recompiles).  No fast-math, no contraction.
    sanitize: AddressSanitizer + UndefinedBehaviorSanitizer build, written to
    libsq_oracle_san.so and loaded instead when SQ_SANITIZE=1 (the process
    must then have the ASan runtime preloaded)."""
    out = _SAN_PATH if sanitize else _LIB_PATH
    tmp = out + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
         "-fno-fast-math", "-pthread"] + (SANITIZE_FLAGS if sanitize else []) +
        [_SRC, "-o", tmp, "-lm"])
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
        i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.sqo_qmax.restype = i32
        L.sqo_qmax.argtypes = [i32]
        L.sqo_row_bytes.restype = i64
        L.sqo_row_bytes.argtypes = [i32, i32]
        L.sqo_f16_to_f32.restype = ctypes.c_float
        L.sqo_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.sqo_f32_to_f16.restype = ctypes.c_uint16
        L.sqo_f32_to_f16.argtypes = [ctypes.c_float]
        L.sqo_record_bytes.restype = i64
        L.sqo_record_bytes.argtypes = [i32, i32, i32]
        L.sqo_pack_row.restype = i32
        L.sqo_pack_row.argtypes = [i32, i32, vp, vp]
        L.sqo_unpack_row.restype = None
        L.sqo_unpack_row.argtypes = [i32, i32, vp, vp]
        L.sqo_quantize.restype = None
        L.sqo_quantize.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.sqo_quantize_rows.restype = None
        L.sqo_quantize_rows.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.sqo_record_bytes_rows.restype = ctypes.c_int64
        L.sqo_record_bytes_rows.argtypes = [vp, i32, i32]
        L.sqo_record_pack_rows.restype = i32
        L.sqo_record_pack_rows.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.sqo_record_unpack_rows.restype = i32
        L.sqo_record_unpack_rows.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.sqo_quant_step_codes_rows.restype = None
        L.sqo_quant_step_codes_rows.argtypes = [i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, f32,
                                                vp, vp, vp]
        L.sqo_quantize_kra.restype = None
        L.sqo_quantize_kra.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.sqo_quantize_kra_rows.restype = None
        L.sqo_quantize_kra_rows.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
        L.sqo_reconstruct_f64.restype = None
        L.sqo_reconstruct_f64.argtypes = [i32, i32, vp, vp, vp, vp]
        L.sqo_dequantize.restype = None
        L.sqo_dequantize.argtypes = [i32, i32, vp, vp, vp, vp]
        L.sqo_gated_delta_f64.restype = None
        L.sqo_gated_delta_f64.argtypes = [i32, i32, vp, vp, vp, vp, vp, ctypes.c_double, vp]
        L.sqo_step_update.restype = None
        L.sqo_step_update.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp]
        L.sqo_quant_step_codes.restype = None
        L.sqo_quant_step_codes.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, f32,
                                           vp, vp, vp]
        L.sqo_record_unpack.restype = i32
        L.sqo_record_unpack.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.sqo_record_pack.restype = i32
        L.sqo_record_pack.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.sqo_records_quantize.restype = i32
        L.sqo_records_quantize.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, i32]
        L.sqo_records_dequantize.restype = i32
        L.sqo_records_dequantize.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i32]
        L.sqo_records_step.restype = i32
        L.sqo_records_step.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, i32]
        L.sqo_f64_step.restype = i32
        L.sqo_f64_step.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32]
        L.sqo_f32_step.restype = i32
        L.sqo_f32_step.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def n_threads() -> int:
    """Host threads the drivers use: SQO_THREADS if set, else the usable
    cores (at most 16)."""
    if os.environ.get("SQO_THREADS"):
        return max(1, min(64, int(os.environ["SQO_THREADS"])))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- format
def qmax(bits: int) -> int:
    return lib().sqo_qmax(bits)


def row_bytes(bits: int, dv: int) -> int:
    return lib().sqo_row_bytes(bits, dv)


def record_bytes(bits: int, dk: int, dv: int) -> int:
    return lib().sqo_record_bytes(bits, dk, dv)


def f32_to_f16(x: float) -> int:
    """Nearest binary16 (ties to even), as raw bits."""
    return lib().sqo_f32_to_f16(float(x))


def f16_to_f32(h: int) -> float:
    return lib().sqo_f16_to_f32(int(h))


def pack_row(bits: int, codes) -> np.ndarray:
    codes = _c(codes, np.int32)
    out = np.zeros(row_bytes(bits, codes.size), np.uint8)
    if lib().sqo_pack_row(bits, codes.size, _p(codes), _p(out)) != 0:
        raise ValueError("code out of range for %d bits" % bits)
    return out


def unpack_row(bits: int, data, n: int) -> np.ndarray:
    data = _c(data, np.uint8)
    out = np.empty(n, np.int32)
    lib().sqo_unpack_row(bits, n, _p(data), _p(out))
    return out


# ---------------------------------------------------------------- quantizer
def quantize(bits: int, S) -> tuple:
    """Pinned fp32 dual-axis quantizer: returns (Q int32, r f32 [dk], c f32 [dv])."""
    S = _c(S, np.float32)
    dk, dv = S.shape
    Q = np.empty((dk, dv), np.int32)
    r = np.empty(dk, np.float32)
    c = np.empty(dv, np.float32)
    lib().sqo_quantize(bits, dk, dv, _p(S), _p(Q), _p(r), _p(c))
    return Q, r, c


def quantize_rows(row_bits, S) -> tuple:
    """The closed rule with a width per key row (row_bits [dk] in {4, 6, 8})."""
    S = _c(S, np.float32)
    rb = _c(row_bits, np.uint8)
    dk, dv = S.shape
    assert rb.shape == (dk,)
    Q = np.empty((dk, dv), np.int32)
    r = np.empty(dk, np.float32)
    c = np.empty(dv, np.float32)
    lib().sqo_quantize_rows(_p(rb), dk, dv, _p(S), _p(Q), _p(r), _p(c))
    return Q, r, c


def record_bytes_rows(row_bits, dv: int) -> int:
    rb = _c(row_bits, np.uint8)
    return int(lib().sqo_record_bytes_rows(_p(rb), rb.size, dv))


def record_pack_rows(row_bits, Q, r, c) -> np.ndarray:
    rb = _c(row_bits, np.uint8)
    Q = _c(Q, np.int32)
    dk, dv = Q.shape
    rec = np.zeros(record_bytes_rows(rb, dv), np.uint8)
    r = _c(r, np.float32)
    c = _c(c, np.float32)
    if lib().sqo_record_pack_rows(_p(rb), dk, dv, _p(Q), _p(r), _p(c), _p(rec)) != 0:
        raise ValueError("code out of range")
    return rec


def record_unpack_rows(row_bits, dv, rec) -> tuple:
    rb = _c(row_bits, np.uint8)
    rec = _c(rec, np.uint8)
    dk = rb.size
    Q = np.empty((dk, dv), np.int32)
    r = np.empty(dk, np.float32)
    c = np.empty(dv, np.float32)
    lib().sqo_record_unpack_rows(_p(rb), dk, dv, _p(rec), _p(Q), _p(r), _p(c))
    return Q, r, c


def quantize_kra(bits: int, S, imp) -> tuple:
    """Key-row-aware dual-axis fit with row-impact scores imp [dk] (> 0):
    returns (Q int32, r f32 [dk], c f32 [dv])."""
    S = _c(S, np.float32)
    imp = _c(imp, np.float32)
    dk, dv = S.shape
    assert imp.shape == (dk,)
    Q = np.empty((dk, dv), np.int32)
    r = np.empty(dk, np.float32)
    c = np.empty(dv, np.float32)
    lib().sqo_quantize_kra(bits, dk, dv, _p(S), _p(imp), _p(Q), _p(r), _p(c))
    return Q, r, c


def quantize_kra_rows(row_bits, S, imp) -> tuple:
    """The key-row-aware fit with each key row at its own width row_bits [dk]
    (4, 6 or 8): returns (Q int32, r f32 [dk], c f32 [dv])."""
    rb = _c(row_bits, np.uint8)
    S = _c(S, np.float32)
    imp = _c(imp, np.float32)
    dk, dv = S.shape
    assert imp.shape == (dk,) and rb.shape == (dk,)
    Q = np.empty((dk, dv), np.int32)
    r = np.empty(dk, np.float32)
    c = np.empty(dv, np.float32)
    lib().sqo_quantize_kra_rows(_p(rb), dk, dv, _p(S), _p(imp), _p(Q), _p(r), _p(c))
    return Q, r, c


def reconstruct_f64(Q, r, c) -> np.ndarray:
    """FP64 reconstruction ((double)Q * r) * c used inside the decode step."""
    Q = _c(Q, np.int32)
    r = _c(r, np.float32)
    c = _c(c, np.float32)
    dk, dv = Q.shape
    S = np.empty((dk, dv), np.float64)
    lib().sqo_reconstruct_f64(dk, dv, _p(Q), _p(r), _p(c), _p(S))
    return S


def dequantize(Q, r, c) -> np.ndarray:
    """fp32 export of the reconstruction: (float)(((double)Q * r) * c)."""
    Q = _c(Q, np.int32)
    r = _c(r, np.float32)
    c = _c(c, np.float32)
    dk, dv = Q.shape
    S = np.empty((dk, dv), np.float32)
    lib().sqo_dequantize(dk, dv, _p(Q), _p(r), _p(c), _p(S))
    return S


# ---------------------------------------------------------------- recurrence
def gated_delta_f64(S, alpha, q, k, v, beta) -> tuple:
    """One FP64 gated Delta-rule step on a copy of S: returns (S', y)."""
    S = np.array(S, dtype=np.float64, order="C")
    dk, dv = S.shape
    y = np.empty(dv, np.float64)
    a, q, k, v = (_c(x, np.float64) for x in (alpha, q, k, v))
    lib().sqo_gated_delta_f64(dk, dv, _p(S), _p(a), _p(q), _p(k), _p(v), float(beta), _p(y))
    return S, y


def step_update(Z, R, C, alpha, q, k, v, beta) -> tuple:
    """The update of one step on stored values Z [dk, dv] with row scales R,
    column scales C and retention alpha (all fp32): returns (S' fp32, y FP64)."""
    Z = _c(Z, np.float32)
    dk, dv = Z.shape
    R, C, alpha = _c(R, np.float32), _c(C, np.float32), _c(alpha, np.float32)
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    assert R.shape == (dk,) and C.shape == (dv,) and alpha.shape == (dk,)
    assert q.shape == (dk,) and k.shape == (dk,) and v.shape == (dv,)
    S = np.empty((dk, dv), np.float32)
    y = np.empty(dv, np.float64)
    lib().sqo_step_update(dk, dv, _p(Z), _p(R), _p(C), _p(alpha), _p(q), _p(k), _p(v),
                          float(np.float32(beta)), _p(S), _p(y))
    return S, y


def quant_step_codes(kda: bool, bits: int, Q, r, c, q, k, v, beta, g, imp=None) -> np.ndarray:
    """Quantized step on unpacked codes (any bits 2..24); Q, r, c updated in place.
    imp [dk]: requantize with the key-row-aware fit instead of the closed rule."""
    assert Q.dtype == np.int32 and r.dtype == np.float32 and c.dtype == np.float32
    assert Q.flags.c_contiguous
    dk, dv = Q.shape
    y = np.empty(dv, np.float64)
    g = np.atleast_1d(_c(g, np.float32))
    q, k, v = (_c(x, np.float32) for x in (q, k, v))
    imp = None if imp is None else _c(imp, np.float32)
    lib().sqo_quant_step_codes(int(kda), bits, dk, dv, _p(Q), _p(r), _p(c), _p(q), _p(k),
                               _p(v), float(beta), _p(g), _p(imp), _p(y))
    return y


def record_pack(bits, Q, r, c) -> np.ndarray:
    Q = _c(Q, np.int32)
    dk, dv = Q.shape
    rec = np.zeros(record_bytes(bits, dk, dv), np.uint8)
    r = _c(r, np.float32)
    c = _c(c, np.float32)
    if lib().sqo_record_pack(bits, dk, dv, _p(Q), _p(r), _p(c), _p(rec)) != 0:
        raise ValueError("code out of range")
    return rec


def record_unpack(bits, dk, dv, rec) -> tuple:
    rec = _c(rec, np.uint8)
    Q = np.empty((dk, dv), np.int32)
    r = np.empty(dk, np.float32)
    c = np.empty(dv, np.float32)
    if lib().sqo_record_unpack(bits, dk, dv, _p(rec), _p(Q), _p(r), _p(c)) != 0:
        raise ValueError("bad record shape")
    return Q, r, c


# ---------------------------------------------------------------- batches
def _rows(row_bits, n, dk):
    if row_bits is None:
        return None
    rb = _c(row_bits, np.uint8)
    assert rb.size == n * dk
    return rb


def _imp(imp, n, dk):
    if imp is None:
        return None
    imp = _c(imp, np.float32)
    assert imp.size == n * dk
    return imp


def records_quantize(base: np.ndarray, offs, bits, S, dk, dv, imp=None, row_bits=None):
    """imp [n, dk]: row-impact scores per record (key-row-aware fit), or None;
    row_bits [n, dk]: key-row widths of the records whose bits are 0."""
    offs = _c(offs, np.int64)
    bits = _c(bits, np.uint8)
    S = _c(S, np.float32)
    imp = _imp(imp, offs.size, dk)
    rb = _rows(row_bits, offs.size, dk)
    assert base.dtype == np.uint8 and base.flags.c_contiguous
    assert S.size == offs.size * dk * dv
    if lib().sqo_records_quantize(offs.size, dk, dv, _p(bits), _p(offs), _p(base), _p(S),
                                  _p(imp), _p(rb), n_threads()) != 0:
        raise ValueError("bad arguments")


def records_dequantize(base: np.ndarray, offs, bits, dk, dv, row_bits=None) -> np.ndarray:
    offs = _c(offs, np.int64)
    bits = _c(bits, np.uint8)
    S = np.empty((offs.size, dk, dv), np.float32)
    base = _c(base, np.uint8)
    rb = _rows(row_bits, offs.size, dk)
    if lib().sqo_records_dequantize(offs.size, dk, dv, _p(bits), _p(offs), _p(base),
                                    _p(S), _p(rb), n_threads()) != 0:
        raise ValueError("bad arguments")
    return S


def records_step(kda: bool, base: np.ndarray, offs, bits, dk, dv, q, k, v, beta, g,
                 imp=None, row_bits=None) -> np.ndarray:
    """Quantized decode step, in place on the records at base + offs[row]; returns y (f64).
    imp [n, dk]: requantize with the key-row-aware fit; row_bits as for records_quantize."""
    offs = _c(offs, np.int64)
    bits = _c(bits, np.uint8)
    n = offs.size
    imp = _imp(imp, n, dk)
    rb = _rows(row_bits, n, dk)
    assert base.dtype == np.uint8 and base.flags.c_contiguous
    y = np.empty((n, dv), np.float64)
    q, k, v, beta, g = (_c(x, np.float32) for x in (q, k, v, beta, g))
    if lib().sqo_records_step(int(kda), n, dk, dv, _p(bits), _p(offs), _p(base), _p(q), _p(k),
                              _p(v), _p(beta), _p(g), _p(imp), _p(rb), _p(y), n_threads()) != 0:
        raise ValueError("bad arguments")
    return y


def f64_step(kda: bool, S: np.ndarray, q, k, v, beta, g) -> np.ndarray:
    """Unquantized FP64 step on states S[n, dk, dv] (in place); returns y."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    n, dk, dv = S.shape
    y = np.empty((n, dv), np.float64)
    q, k, v, beta, g = (_c(x, np.float32) for x in (q, k, v, beta, g))
    if lib().sqo_f64_step(int(kda), n, dk, dv, _p(S), _p(q), _p(k), _p(v), _p(beta), _p(g), _p(y),
                          n_threads()) != 0:
        raise ValueError("bad arguments")
    return y


def f32_step(kda: bool, S: np.ndarray, q, k, v, beta, g) -> np.ndarray:
    """Step on fp32-stored states S[n, dk, dv] (widen, FP64 step, round back)."""
    assert S.dtype == np.float32 and S.flags.c_contiguous
    n, dk, dv = S.shape
    y = np.empty((n, dv), np.float64)
    q, k, v, beta, g = (_c(x, np.float32) for x in (q, k, v, beta, g))
    if lib().sqo_f32_step(int(kda), n, dk, dv, _p(S), _p(q), _p(k), _p(v), _p(beta), _p(g), _p(y),
                          n_threads()) != 0:
        raise ValueError("bad arguments")
    return y
