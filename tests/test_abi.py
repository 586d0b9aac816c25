"""The C-ABI library on the host: symbols, layout and argument validation.

No test here launches work: every call either is host-only (pool descriptor,
layout) or is rejected by validation before any HIP call is made, so the
suite runs without a GPU.
"""
import ctypes
import functools
import os
import threading

import pytest

import bench
import quantized_gated_delta_amd as Q
from quantized_gated_delta_amd import sq as S

FAKE_DEV = 0x7F0000000000   # 256-byte aligned, never dereferenced on the host


def test_library_exports_every_declared_symbol():
    names = Q.header_symbols()
    for must in ("sq_pool_bytes", "sq_pool_create", "sq_pool_destroy", "sq_pool_layout",
                 "sq_quant_state", "sq_decode_step", "sq_decode_update", "sq_dequant_state",
                 "sq_f32_decode_step",
                 "sq_check_slots", "sq_last_error", "sq_version"):
        assert must in names
    lib = Q.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in Q.version()


PAGES = ("hyper.ai", "ta-paperlens", "blog.ontle.kr", "bayesiansapien", "thelatestinai")


def _declaration_comments():
    """Comment block right above each function declaration of include/sq.h."""
    import re
    text = open(S.HEADER).read()
    out = {}
    for m in re.finditer(r"/\*((?:[^*]|\*(?!/))*)\*/\s*\n(?:sq_status|const char \*)\s*(sq_\w+)\(",
                         text):
        out[m.group(2)] = m.group(1)
    return out


def test_boundary_calls_cite_their_passage():
    """Every call of the boundary says which passage of the pages defines what
    it computes, and states its errors; sq_last_error is this library's own
    error reporting."""
    com = _declaration_comments()
    for name in ("sq_pool_bytes", "sq_pool_create", "sq_pool_destroy", "sq_quant_state",
                 "sq_decode_step", "sq_dequant_state", "sq_f32_decode_step"):
        assert name in com, name
        assert any(p in com[name] for p in PAGES), "%s cites no page" % name
    for name in ("sq_pool_bytes", "sq_pool_create", "sq_quant_state", "sq_dequant_state",
                 "sq_f32_decode_step"):
        assert "SQ_EINVAL" in com[name] or "errors" in com[name].lower(), name
    assert "error" in com["sq_last_error"].lower()
    # the arithmetic the header states is the one the library and the oracle use
    assert "(float)(((double)code_ij * r_i) * c_j)" in com["sq_dequant_state"]
    assert "exact product s_ij * ir_i" in open(S.HEADER).read()


def _rec(b, d):
    # FP16 pivot records hold the binary16 state and no scales
    return 2 * d * d if b == 16 else d * d * b // 8 + 8 * d


def _layout(bits, d):
    offs, pos = [], 0
    for b in bits:
        offs.append(pos)
        pos += _rec(b, d)
    return pos, offs


@pytest.mark.parametrize("d,bits", [(128, [6] * 48), (128, [4, 6, 8, 6]), (64, [8, 4, 6]),
                                    (128, [16, 6, 4]), (64, [4, 16, 8, 16])])
def test_pool_bytes_and_layout(d, bits):
    stride, offs = _layout(bits, d)
    assert Q.sq_pool_bytes(640, len(bits), d, d, bits, Q.SQ_GATE_GDN) == 640 * stride
    h = Q.sq_pool_create(640, len(bits), d, d, bits, Q.SQ_GATE_KDA, FAKE_DEV, 640 * stride)
    try:
        st, ho, rb = Q.sq_pool_layout(h, len(bits))
        assert st == stride and ho == offs
        assert rb == [_rec(b, d) for b in bits]
        assert all(o % 256 == 0 for o in ho) and st % 256 == 0
    finally:
        Q.sq_pool_destroy(h)


def _expect(status, fn, *args, text=None):
    with pytest.raises(Q.SQError) as e:
        fn(*args)
    assert e.value.status == status, (e.value.status, e.value.text)
    if text:
        assert text in e.value.text, e.value.text
    return e.value


def test_descriptor_validation():
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 2, 128, 128, [6, 3], 0, text="head_bits[1]")
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 2, 128, 128, [16, 12], 0, text="head_bits[1]")
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 1, 128, 128, [32], 0, text="head_bits[0]")
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 1, 96, 96, [6], 0, text="64 or 128")
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 1, 128, 64, [6], 0, text="d_k must equal")
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 65, 128, 128, [6] * 65, 0, text="n_heads")
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 0, 128, 128, [6], 0, text="n_heads")
    _expect(Q.SQ_EINVAL, Q.sq_pool_bytes, 0, 1, 128, 128, [6], 0, text="n_slots")
    _expect(Q.SQ_EINVAL, Q.sq_pool_bytes, 4, 1, 128, 128, [6], 7, text="gate")
    L = Q.lib()
    assert L.sq_pool_bytes(None, ctypes.byref(ctypes.c_size_t())) == Q.SQ_EINVAL
    d = S._Desc(4, 1, 128, 128, None, 0)
    assert L.sq_pool_bytes(ctypes.byref(d), ctypes.byref(ctypes.c_size_t())) == Q.SQ_EINVAL
    assert "head_bits is NULL" in Q.sq_last_error()


def test_create_validation():
    need = Q.sq_pool_bytes(8, 2, 64, 64, [6, 6], 0)
    _expect(Q.SQ_ENOMEM, Q.sq_pool_create, 8, 2, 64, 64, [6, 6], 0, FAKE_DEV, need - 1)
    _expect(Q.SQ_EINVAL, Q.sq_pool_create, 8, 2, 64, 64, [6, 6], 0, FAKE_DEV + 64, need,
            text="256-byte")
    _expect(Q.SQ_EINVAL, Q.sq_pool_create, 8, 2, 64, 64, [6, 6], 0, 0, need, text="dev_buf")
    assert Q.lib().sq_pool_destroy(None) == Q.SQ_OK


@pytest.fixture
def pool():
    h = Q.sq_pool_create(8, 2, 128, 128, [6, 4], 0, FAKE_DEV,
                         Q.sq_pool_bytes(8, 2, 128, 128, [6, 4], 0))
    yield h
    Q.sq_pool_destroy(h)


def test_step_validation_without_launch(pool):
    P = FAKE_DEV + 4096
    ok = dict(q=P, k=P, v=P, beta=P, g=P, y=P)
    # n = 0 is a no-op: returns before any HIP call
    Q.sq_decode_step(pool, None, 0, in_dtype=1, y_dtype=1, stream=0, **ok)
    Q.sq_quant_state(pool, None, 0, None, stream=0)
    Q.sq_dequant_state(pool, None, 0, None, stream=0)
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P, -1, P, P, P, P, P, P, 1, 1, 0, text="n must")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P, 9, P, P, P, P, P, P, 1, 1, 0,
            text="exceeds n_slots")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, None, 2, P, P, P, P, P, P, 1, 1, 0,
            text="slot_idx is NULL")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P, 2, None, P, P, P, P, P, 1, 1, 0,
            text="q is NULL")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P, 2, P, P + 2, P, P, P, P, 1, 1, 0,
            text="k is not 16-byte")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P, 2, P, P, P, P, P, P, 5, 1, 0,
            text="in_dtype")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P, 2, P, P, P, P, P, P, 1, 9, 0,
            text="y_dtype")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, pool, P + 1, 2, P, P, P, P, P, P, 1, 1, 0,
            text="slot_idx is not 4-byte")
    _expect(Q.SQ_EINVAL, Q.sq_quant_state, pool, P, 2, None, 0, text="S is NULL")
    _expect(Q.SQ_EINVAL, Q.sq_dequant_state, pool, P, 2, P + 8, 0, text="S is not 16-byte")
    _expect(Q.SQ_EINVAL, Q.sq_decode_step, None, P, 2, P, P, P, P, P, P, 1, 1, 0,
            text="pool is NULL")


def test_arith_selfcheck_validation_without_launch():
    _expect(Q.SQ_EINVAL, Q.sq_arith_selfcheck, None, 0, text="counts is NULL")
    _expect(Q.SQ_EINVAL, Q.sq_arith_selfcheck, FAKE_DEV + 4, 0, text="counts is not 8-byte")


def test_split_update_validation_without_launch(pool):
    P = FAKE_DEV + 4096
    io = (P, P, P, P, P, P)
    Q.sq_decode_update(pool, None, 0, *io, None, in_dtype=1, y_dtype=1, stream=0)
    _expect(Q.SQ_EINVAL, Q.sq_decode_update, pool, P, 2, *io, None, 1, 1, 0, text="S_out is NULL")
    _expect(Q.SQ_EINVAL, Q.sq_decode_update, pool, P, 2, *io, P + 4, 1, 1, 0,
            text="S_out is not 16-byte")
    _expect(Q.SQ_EINVAL, Q.sq_decode_update, pool, P, 9, *io, P, 1, 1, 0, text="exceeds n_slots")
    _expect(Q.SQ_EINVAL, Q.sq_decode_update, pool, P, 2, P, P, P, P, P, None, P, 1, 1, 0,
            text="y is NULL")


def test_split_noalloc_validation_without_launch():
    """The no-allocation split step refuses a batch whose S' exceeds its
    static buffer before any HIP call; n = 0 is a no-op."""
    P = FAKE_DEV + 4096
    H, d = 64, 128
    fit = Q.SQ_SPLIT_SCRATCH_BYTES // (H * d * d * 4)      # 16 requests of 64 heads
    n_slots = fit + 1
    h = Q.sq_pool_create(n_slots, H, d, d, [6] * H, 0, FAKE_DEV,
                         Q.sq_pool_bytes(n_slots, H, d, d, [6] * H, 0))
    try:
        Q.sq_split_step_noalloc(h, None, 0, P, P, P, P, P, P, in_dtype=1, y_dtype=1, stream=0)
        e = _expect(Q.SQ_ENOMEM, Q.sq_split_step_noalloc, h, P, fit + 1, P, P, P, P, P, P, 1, 1,
                    0, text="static buffer")
        assert "at most %d requests" % fit in e.text
        _expect(Q.SQ_EINVAL, Q.sq_split_step_noalloc, h, P, 2, None, P, P, P, P, P, 1, 1, 0,
                text="q is NULL")
        _expect(Q.SQ_EINVAL, Q.sq_split_step_noalloc, None, P, 2, P, P, P, P, P, P, 1, 1, 0,
                text="pool is NULL")
    finally:
        Q.sq_pool_destroy(h)
    # the binding's constant is the header's
    assert "#define SQ_SPLIT_SCRATCH_BYTES ((size_t)64 << 20)" in open(S.HEADER).read()
    assert Q.SQ_SPLIT_SCRATCH_BYTES == 64 << 20


def test_f32_step_validation_without_launch():
    P = FAKE_DEV
    Q.sq_f32_decode_step(P, 4, 2, 128, 128, 0, None, 0, P, P, P, P, P, P, 1, 1, 0)
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_f32_decode_step, P, 4, 2, 96, 96, 0, P, 1,
            P, P, P, P, P, P, 1, 1, 0)
    _expect(Q.SQ_EINVAL, Q.sq_f32_decode_step, P, 4, 2, 128, 128, 3, P, 1,
            P, P, P, P, P, P, 1, 1, 0, text="gate")
    _expect(Q.SQ_EINVAL, Q.sq_f32_decode_step, P, 4, 2, 128, 128, 0, P, 5,
            P, P, P, P, P, P, 1, 1, 0, text="exceeds")
    _expect(Q.SQ_EINVAL, Q.sq_f32_decode_step, P, 4, 2, 128, 128, 0, None, 2,
            P, P, P, P, P, P, 1, 1, 0, text="slot_idx")
    _expect(Q.SQ_EINVAL, Q.sq_f32_decode_step, P + 4, 4, 2, 128, 128, 0, P, 2,
            P, P, P, P, P, P, 1, 1, 0, text="state_pool")


def test_device_copy_validation_without_launch():
    lib = Q.lib()
    assert lib.sq_device_copy(None, None, 0, None) == S.SQ_OK           # no-op
    assert lib.sq_device_copy(None, FAKE_DEV, 64, None) == S.SQ_EINVAL
    assert lib.sq_device_copy(FAKE_DEV, FAKE_DEV + 4, 64, None) == S.SQ_EINVAL   # misaligned
    assert lib.sq_device_copy(FAKE_DEV, FAKE_DEV + 4096, 24, None) == S.SQ_EINVAL  # not 16 x n
    assert "multiple of 16" in Q.sq_last_error()


def test_issue_probe_validation_without_launch():
    """The issue-rate probe rejects an unknown class and a missing or
    misaligned sink before launching anything; its per-launch operation count
    matches the header's."""
    lib = S.lib()
    assert lib.sq_issue_probe(-1, FAKE_DEV, None) == S.SQ_EINVAL
    assert lib.sq_issue_probe(Q.SQ_PROBE_COUNT, FAKE_DEV, None) == S.SQ_EINVAL
    assert "probe class" in Q.sq_last_error()
    assert lib.sq_issue_probe(Q.SQ_PROBE_FMA_F32, None, None) == S.SQ_EINVAL
    assert lib.sq_issue_probe(Q.SQ_PROBE_FMA_F32, FAKE_DEV + 2, None) == S.SQ_EINVAL
    text = open(S.HEADER).read()
    assert "#define SQ_PROBE_OPS_PER_LAUNCH %dLL" % Q.SQ_PROBE_OPS_PER_LAUNCH in text
    assert Q.SQ_PROBE_OPS_PER_LAUNCH == 8192 * 256 * 1024 * 8


def test_timeline_symbols_only_in_the_timeline_build():
    """The default library carries no timeline instrumentation; the
    instrumented build (libsq_timeline.so, behind bench.py --timeline)
    exports its two read-back calls next to the whole ABI."""
    import ctypes
    default = ctypes.CDLL(S.LIB_PATH)
    for name in ("sq_timeline_read", "sq_timeline_clear"):
        assert not hasattr(default, name), name
    tl_path = os.path.join(os.path.dirname(S.LIB_PATH), "libsq_timeline.so")
    if not os.path.exists(tl_path):
        pytest.skip("timeline build not present")
    tl = ctypes.CDLL(tl_path)
    for name in ("sq_timeline_read", "sq_timeline_clear") + tuple(Q.header_symbols()):
        assert hasattr(tl, name), name


def test_last_error_is_thread_local():
    _expect(Q.SQ_EUNSUPPORTED, Q.sq_pool_bytes, 4, 1, 96, 96, [6], 0)
    seen = []

    def other():
        Q.sq_pool_bytes(4, 1, 128, 128, [6], 0)
        seen.append(Q.sq_last_error())

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen == [""]
    assert "64 or 128" in Q.sq_last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(S, "_lib", None)
    monkeypatch.setattr(S, "LIB_PATH", str(tmp_path / "libsq.so"))
    with pytest.raises(ImportError):
        S.lib()


def test_bench_byte_model():
    # per (request, head) update at d = 128, bf16 I/O: codes and scales read
    # and written, q k v beta g read, y written; plus 4 B slot index per request
    assert bench.algo_bytes_per_step(1, 1, 128, [6], "gdn") == 27652 + 4
    assert bench.algo_bytes_per_step(1, 1, 128, [4], "gdn") == 19460 + 4
    assert bench.algo_bytes_per_step(1, 1, 128, [8], "gdn") == 35844 + 4
    assert bench.algo_bytes_per_step(1, 1, 128, [6], "kda") == 27652 + 254 + 4
    assert bench.algo_bytes_per_step(512, 48, 128, [6] * 48, "gdn") == 679577600
    assert bench.f32_bytes_per_step(1, 1, 128, "gdn") == 132100 + 4


def _rows_rec(w, d):
    raw = sum(d * int(b) // 8 for b in w) + 8 * d
    return (raw + 255) // 256 * 256


@pytest.mark.parametrize("d", [64, 128])
def test_per_row_width_layout(d):
    """Heads with head_bits 0 take key-row widths; their records are the rows'
    streams then the scales, padded to 256 bytes."""
    g = 8 if d == 128 else 16
    w0 = [4] * (2 * g) + [6] * (d - 3 * g) + [8] * g
    w2 = [6] * (d - g) + [8] * g
    rows = [w0, [6] * d, w2]
    bits = [0, 6, 0]
    want = [_rows_rec(w0, d), d * d * 6 // 8 + 8 * d, _rows_rec(w2, d)]
    assert Q.sq_pool_bytes(5, 3, d, d, bits, Q.SQ_GATE_KDA, row_bits=rows) == 5 * sum(want)
    h = Q.sq_pool_create(5, 3, d, d, bits, Q.SQ_GATE_KDA, FAKE_DEV, 5 * sum(want), row_bits=rows)
    try:
        st, ho, rb = Q.sq_pool_layout(h, 3)
        assert rb == want and ho == [0, want[0], want[0] + want[1]] and st == sum(want)
        # the key-row-aware fit also takes heads with per-key-row widths (no
        # compute call here: setting and clearing the scores only)
        Q.sq_pool_set_row_impact(h, FAKE_DEV)
        Q.sq_pool_set_row_impact(h, None)
    finally:
        Q.sq_pool_destroy(h)


def test_per_row_width_validation():
    d, g = 128, 8
    ok = [4] * 32 + [6] * 64 + [8] * 32
    _expect(Q.SQ_EINVAL, Q.sq_pool_bytes, 2, 1, d, d, [0], 1, text="needs per-row widths")
    bad = list(ok)
    bad[40] = 5
    _expect(Q.SQ_EUNSUPPORTED, functools.partial(Q.sq_pool_bytes, row_bits=[bad]),
            2, 1, d, d, [0], 1,
            text="must be 4, 6 or 8")
    dec = [6] * 64 + [4] * 64
    _expect(Q.SQ_EUNSUPPORTED, functools.partial(Q.sq_pool_bytes, row_bits=[dec]),
            2, 1, d, d, [0], 1,
            text="non-decreasing")
    off = [4] * 36 + [8] * 92
    _expect(Q.SQ_EUNSUPPORTED, functools.partial(Q.sq_pool_bytes, row_bits=[off]),
            2, 1, d, d, [0], 1,
            text="not a multiple of 8")
    off64 = [4] * 8 + [8] * 56
    _expect(Q.SQ_EUNSUPPORTED, functools.partial(Q.sq_pool_bytes, row_bits=[off64]),
            2, 1, 64, 64, [0], 1,
            text="not a multiple of 16")
    assert Q.sq_pool_bytes(2, 1, d, d, [0], 1, row_bits=[ok]) == 2 * _rows_rec(ok, d)
    # rows of uniform heads are not read
    assert Q.sq_pool_bytes(2, 2, d, d, [6, 0], 1, row_bits=[[0] * d, ok]) == \
        2 * (13312 + _rows_rec(ok, d))


def test_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4, 6)
    with pytest.raises(ValueError):
        S._ptr(t.t())                       # non-contiguous
    assert S._ptr(t) == t.data_ptr()
    with pytest.raises(ValueError):
        S._need(t, "q", 24, (torch.float32,))   # host tensor
    with pytest.raises(TypeError):
        S._need([1, 2], "q", 2, (torch.float32,))
