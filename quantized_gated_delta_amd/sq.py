"""Thin ctypes binding of the C ABI in include/sq.h.

Argument marshalling only: every step of the decode path runs in the HIP
library ``libsq.so``.  There is no CPU fallback; if the library is missing
or fails to load, every entry point raises.

Tensors are torch tensors (device memory and streams only); raw integer
device pointers are accepted too.  Functions keep the ABI's names.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; SQ_LIBRARY may name another build of the same sources
# (the instrumented timeline build, libsq_timeline.so)
LIB_PATH = os.environ.get("SQ_LIBRARY") or os.path.join(HERE, "libsq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "sq.h")

SQ_OK, SQ_EINVAL, SQ_EUNSUPPORTED, SQ_ENOMEM, SQ_EHIP = 0, 1, 2, 3, 4
SQ_GATE_GDN, SQ_GATE_KDA = 0, 1
SQ_F32, SQ_BF16 = 0, 1
STATUS_NAMES = {0: "SQ_OK", 1: "SQ_EINVAL", 2: "SQ_EUNSUPPORTED", 3: "SQ_ENOMEM", 4: "SQ_EHIP"}

_lib = None


class SQError(RuntimeError):
    def __init__(self, status: int, func: str, text: str):
        super().__init__("%s -> %s: %s" % (func, STATUS_NAMES.get(status, status), text))
        self.status = status
        self.func = func
        self.text = text


class _Desc(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("head_bits", ctypes.POINTER(ctypes.c_uint8)), ("gate", ctypes.c_int)]


def lib():
    """Load libsq.so (built in-tree).  Raises if it is missing: no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("library not built at %s: run __graft_entry__.build() or "
                              "python quantized_gated_delta_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        st = ctypes.c_int
        pdesc = ctypes.POINTER(_Desc)
        L.sq_pool_bytes.restype = st
        L.sq_pool_bytes.argtypes = [pdesc, ctypes.POINTER(ctypes.c_size_t)]
        L.sq_pool_create.restype = st
        L.sq_pool_create.argtypes = [pdesc, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        L.sq_pool_bytes_rows.restype = st
        L.sq_pool_bytes_rows.argtypes = [pdesc, vp, ctypes.POINTER(ctypes.c_size_t)]
        L.sq_pool_create_rows.restype = st
        L.sq_pool_create_rows.argtypes = [pdesc, vp, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        L.sq_pool_destroy.restype = st
        L.sq_pool_destroy.argtypes = [vp]
        L.sq_pool_layout.restype = st
        L.sq_pool_layout.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]
        L.sq_pool_set_row_impact.restype = st
        L.sq_pool_set_row_impact.argtypes = [vp, vp]
        L.sq_quant_state.restype = st
        L.sq_quant_state.argtypes = [vp, vp, i32, vp, vp]
        L.sq_dequant_state.restype = st
        L.sq_dequant_state.argtypes = [vp, vp, i32, vp, vp]
        L.sq_decode_step.restype = st
        L.sq_decode_step.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                     ctypes.c_int, vp]
        L.sq_decode_update.restype = st
        L.sq_decode_update.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                       ctypes.c_int, vp, vp]
        L.sq_split_step_noalloc.restype = st
        L.sq_split_step_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                            ctypes.c_int, vp]
        L.sq_f32_decode_step.restype = st
        L.sq_f32_decode_step.argtypes = [vp, i32, i32, i32, i32, ctypes.c_int, vp, i32, vp, vp,
                                         vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp]
        L.sq_check_slots.restype = st
        L.sq_check_slots.argtypes = [vp, vp, i32, vp]
        L.sq_arith_selfcheck.restype = st
        L.sq_arith_selfcheck.argtypes = [vp, vp]
        L.sq_device_copy.restype = st
        L.sq_device_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.sq_issue_probe.restype = st
        L.sq_issue_probe.argtypes = [ctypes.c_int, vp, vp]
        L.sq_last_error.restype = ctypes.c_char_p
        L.sq_last_error.argtypes = []
        L.sq_version.restype = ctypes.c_char_p
        L.sq_version.argtypes = []
        _lib = L
    return _lib


def header_symbols() -> list:
    """Names of the functions include/sq.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z0-9_]+)\s*\(", text)))


def _check(status: int, func: str):
    if status != SQ_OK:
        raise SQError(status, func, lib().sq_last_error().decode(errors="replace"))


def _ptr(x) -> Optional[int]:
    """Raw pointer of an int, a ctypes array or a torch tensor.  Tensors must
    be contiguous: the library reads them as dense row-major arrays."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "is_contiguous") and not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr()


def _need(t, name, numel, dtypes):
    """Shape / dtype / device check of one tensor argument (marshalling only)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SQ_F32
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    raise TypeError("tensor dtype must be float32 or bfloat16, got %s" % t.dtype)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _desc(n_slots, n_heads, d_k, d_v, head_bits: Sequence[int], gate):
    hb = (ctypes.c_uint8 * max(1, len(head_bits)))(*[int(b) for b in head_bits])
    d = _Desc(int(n_slots), int(n_heads), int(d_k), int(d_v),
              ctypes.cast(hb, ctypes.POINTER(ctypes.c_uint8)), int(gate))
    return d, hb


def version() -> str:
    return lib().sq_version().decode()


def sq_last_error() -> str:
    return lib().sq_last_error().decode(errors="replace")


def _row_bits(row_bits):
    if row_bits is None:
        return None
    flat = [int(b) for row in row_bits for b in row]
    return (ctypes.c_uint8 * max(1, len(flat)))(*flat)


def sq_pool_bytes(n_slots, n_heads, d_k, d_v, head_bits, gate, row_bits=None) -> int:
    """row_bits: [n_heads][d_k] key-row widths for heads with head_bits 0 (else None)."""
    d, keep = _desc(n_slots, n_heads, d_k, d_v, head_bits, gate)
    rb = _row_bits(row_bits)
    out = ctypes.c_size_t(0)
    if rb is None:
        _check(lib().sq_pool_bytes(ctypes.byref(d), ctypes.byref(out)), "sq_pool_bytes")
    else:
        _check(lib().sq_pool_bytes_rows(ctypes.byref(d), rb, ctypes.byref(out)),
               "sq_pool_bytes_rows")
    return out.value


def sq_pool_create(n_slots, n_heads, d_k, d_v, head_bits, gate, dev_buf, nbytes=None,
                   row_bits=None) -> int:
    """Wrap a caller-owned device buffer (tensor or pointer); returns the handle."""
    d, keep = _desc(n_slots, n_heads, d_k, d_v, head_bits, gate)
    rb = _row_bits(row_bits)
    if nbytes is None:
        nbytes = dev_buf.numel() * dev_buf.element_size()
    h = ctypes.c_void_p(0)
    if rb is None:
        _check(lib().sq_pool_create(ctypes.byref(d), _ptr(dev_buf), int(nbytes),
                                    ctypes.byref(h)), "sq_pool_create")
    else:
        _check(lib().sq_pool_create_rows(ctypes.byref(d), rb, _ptr(dev_buf), int(nbytes),
                                         ctypes.byref(h)), "sq_pool_create_rows")
    return h.value


def sq_pool_destroy(handle) -> None:
    _check(lib().sq_pool_destroy(handle), "sq_pool_destroy")


def sq_pool_layout(handle, n_heads: int):
    stride = ctypes.c_int64(0)
    off = (ctypes.c_int64 * n_heads)()
    rec = (ctypes.c_int64 * n_heads)()
    _check(lib().sq_pool_layout(handle, ctypes.byref(stride), off, rec), "sq_pool_layout")
    return stride.value, list(off), list(rec)


def sq_quant_state(handle, slot_idx, n: int, S, stream=None) -> None:
    _check(lib().sq_quant_state(handle, _ptr(slot_idx), int(n), _ptr(S), _stream(stream)),
           "sq_quant_state")


def sq_dequant_state(handle, slot_idx, n: int, S, stream=None) -> None:
    _check(lib().sq_dequant_state(handle, _ptr(slot_idx), int(n), _ptr(S), _stream(stream)),
           "sq_dequant_state")


def sq_decode_step(handle, slot_idx, n: int, q, k, v, beta, g, y, in_dtype=None, y_dtype=None,
                   stream=None) -> None:
    in_dtype = _dtype_code(q) if in_dtype is None else in_dtype
    y_dtype = _dtype_code(y) if y_dtype is None else y_dtype
    _check(lib().sq_decode_step(handle, _ptr(slot_idx), int(n), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(beta), _ptr(g), in_dtype, _ptr(y), y_dtype,
                                _stream(stream)), "sq_decode_step")


def sq_pool_set_row_impact(handle, impact) -> None:
    """impact: device tensor [n_heads, d_k] fp32 (kept alive by the caller), or None."""
    _check(lib().sq_pool_set_row_impact(handle, _ptr(impact)), "sq_pool_set_row_impact")


def sq_decode_update(handle, slot_idx, n: int, q, k, v, beta, g, y, S_out, in_dtype=None,
                     y_dtype=None, stream=None) -> None:
    in_dtype = _dtype_code(q) if in_dtype is None else in_dtype
    y_dtype = _dtype_code(y) if y_dtype is None else y_dtype
    _check(lib().sq_decode_update(handle, _ptr(slot_idx), int(n), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(beta), _ptr(g), in_dtype, _ptr(y), y_dtype, _ptr(S_out),
                                  _stream(stream)), "sq_decode_update")


def sq_split_step_noalloc(handle, slot_idx, n: int, q, k, v, beta, g, y, in_dtype=None,
                          y_dtype=None, stream=None) -> None:
    in_dtype = _dtype_code(q) if in_dtype is None else in_dtype
    y_dtype = _dtype_code(y) if y_dtype is None else y_dtype
    _check(lib().sq_split_step_noalloc(handle, _ptr(slot_idx), int(n), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(beta), _ptr(g), in_dtype, _ptr(y), y_dtype,
                                       _stream(stream)), "sq_split_step_noalloc")


def sq_f32_decode_step(state, n_slots, n_heads, d_k, d_v, gate, slot_idx, n, q, k, v, beta, g,
                       y, in_dtype=None, y_dtype=None, stream=None) -> None:
    in_dtype = _dtype_code(q) if in_dtype is None else in_dtype
    y_dtype = _dtype_code(y) if y_dtype is None else y_dtype
    _check(lib().sq_f32_decode_step(_ptr(state), int(n_slots), int(n_heads), int(d_k), int(d_v),
                                    int(gate), _ptr(slot_idx), int(n), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(beta), _ptr(g), in_dtype, _ptr(y), y_dtype,
                                    _stream(stream)), "sq_f32_decode_step")


def sq_check_slots(handle, slot_idx, n: int, stream=None) -> None:
    _check(lib().sq_check_slots(handle, _ptr(slot_idx), int(n), _stream(stream)),
           "sq_check_slots")


def sq_device_copy(src, dst, nbytes: int, stream=None) -> None:
    """Streaming copy of nbytes between two device buffers (measurement helper)."""
    _check(lib().sq_device_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)),
           "sq_device_copy")


# Opcode classes of sq_issue_probe and the operations one launch performs.
SQ_PROBE_FMA_F32, SQ_PROBE_MUL_F32, SQ_PROBE_MAX3_F32, SQ_PROBE_CVT_BYTE = 0, 1, 2, 3
SQ_PROBE_BFE, SQ_PROBE_ALIGNBIT, SQ_PROBE_FMA_F64, SQ_PROBE_FMA_CVT_PAIR = 4, 5, 6, 7
SQ_PROBE_COUNT = 8
SQ_PROBE_OPS_PER_LAUNCH = 17179869184
SQ_SPLIT_SCRATCH_BYTES = 64 << 20   # the static per-GPU buffer of sq_split_step_noalloc


def sq_issue_probe(op: int, sink, stream=None) -> None:
    """One launch of the issue-rate probe of opcode class op (measurement
    helper); sink: a device tensor of at least 4 bytes, never written in
    practice."""
    _check(lib().sq_issue_probe(int(op), _ptr(sink), _stream(stream)), "sq_issue_probe")


def sq_arith_selfcheck(counts, stream=None) -> None:
    """counts: a device tensor of 4 int64 that receives the mismatch counts."""
    _check(lib().sq_arith_selfcheck(_ptr(counts), _stream(stream)), "sq_arith_selfcheck")


class StatePool:
    """A packed state pool in a torch-owned device buffer.

    Convenience wrapper: allocates ``sq_pool_bytes`` bytes with torch on the
    given device, creates the pool handle and exposes the ABI calls."""

    def __init__(self, n_slots: int, n_heads: int, d: int, head_bits, gate: str = "gdn",
                 device="cuda", row_bits=None):
        """row_bits: [n_heads][d] key-row widths for the heads whose head_bits is 0."""
        import torch
        self.n_slots, self.n_heads, self.d = int(n_slots), int(n_heads), int(d)
        self.head_bits = [int(b) for b in head_bits]
        self.row_bits = None if row_bits is None else [[int(b) for b in r] for r in row_bits]
        self.gate = SQ_GATE_KDA if gate == "kda" else SQ_GATE_GDN
        nbytes = sq_pool_bytes(n_slots, n_heads, d, d, self.head_bits, self.gate, self.row_bits)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = sq_pool_create(n_slots, n_heads, d, d, self.head_bits, self.gate, self.buf,
                                     nbytes, self.row_bits)
        self.slot_stride, self.head_off, self.record_bytes = sq_pool_layout(self.handle, n_heads)

    def _step_args(self, slot_idx, q, k, v, beta, g, y):
        import torch
        n, H, d = slot_idx.numel(), self.n_heads, self.d
        _need(slot_idx, "slot_idx", n, (torch.int32,))
        dt = (q.dtype,)
        if q.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("q must be float32 or bfloat16")
        for name, t in (("q", q), ("k", k), ("v", v)):
            _need(t, name, n * H * d, dt)
        _need(beta, "beta", n * H, dt)
        _need(g, "g", n * H * (d if self.gate == SQ_GATE_KDA else 1), dt)
        _need(y, "y", n * H * d, (torch.float32, torch.bfloat16))

    def quant_state(self, slot_idx, S, stream=None):
        import torch
        n = slot_idx.numel()
        _need(slot_idx, "slot_idx", n, (torch.int32,))
        _need(S, "S", n * self.n_heads * self.d * self.d, (torch.float32,))
        sq_quant_state(self.handle, slot_idx, n, S, stream)

    def dequant_state(self, slot_idx, S=None, stream=None):
        import torch
        n = slot_idx.numel()
        if S is None:
            S = torch.empty((n, self.n_heads, self.d, self.d), dtype=torch.float32,
                            device=self.buf.device)
        _need(slot_idx, "slot_idx", n, (torch.int32,))
        _need(S, "S", n * self.n_heads * self.d * self.d, (torch.float32,))
        sq_dequant_state(self.handle, slot_idx, n, S, stream)
        return S

    def decode_step(self, slot_idx, q, k, v, beta, g, y, stream=None):
        self._step_args(slot_idx, q, k, v, beta, g, y)
        sq_decode_step(self.handle, slot_idx, slot_idx.numel(), q, k, v, beta, g, y,
                       stream=stream)

    def set_row_impact(self, impact):
        """Requantize with the key-row-aware fit from now on (impact: [H, d_k]
        fp32 device tensor, > 0), or with the closed rule (None)."""
        if impact is not None:
            impact = impact.contiguous()
            assert impact.shape == (self.n_heads, self.d) and impact.is_cuda
        self.impact = impact  # the library keeps only the pointer
        sq_pool_set_row_impact(self.handle, impact)

    def decode_update(self, slot_idx, q, k, v, beta, g, y, S_out, stream=None):
        """Split step, first half: y and S' (fp32) out, pool unchanged; store
        with quant_state(slot_idx, S_out) afterwards."""
        import torch
        self._step_args(slot_idx, q, k, v, beta, g, y)
        _need(S_out, "S_out", slot_idx.numel() * self.n_heads * self.d * self.d, (torch.float32,))
        sq_decode_update(self.handle, slot_idx, slot_idx.numel(), q, k, v, beta, g, y, S_out,
                         stream=stream)

    def split_step_noalloc(self, slot_idx, q, k, v, beta, g, y, stream=None):
        """Split step with S' in the library's static buffer: no allocation."""
        self._step_args(slot_idx, q, k, v, beta, g, y)
        sq_split_step_noalloc(self.handle, slot_idx, slot_idx.numel(), q, k, v, beta, g, y,
                              stream=stream)

    def check_slots(self, slot_idx, stream=None):
        sq_check_slots(self.handle, slot_idx, slot_idx.numel(), stream)

    def close(self):
        if getattr(self, "handle", None):
            sq_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
