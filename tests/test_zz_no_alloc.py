"""sq_split_step_noalloc: the split step with S' in the library's static
per-GPU buffer (no allocation), checked against the existing split path
(sq_decode_update into a caller workspace, then sq_quant_state of it) and
against the fused sq_decode_step: records and y byte-identical, on two calls
in a row, the second with fewer requests than the first.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workload as W
import quantized_gated_delta_amd as Q

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_inputs(x: dict, n_req: int, H: int) -> dict:
    """Inputs of the first n_req requests on the device (bf16 kept as bf16)."""
    out = {}
    for k, v in x.items():
        v = np.ascontiguousarray(v[: n_req * H])
        if v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(v).to(DEV)
    return out


def warm_pool(wl, layer, pools):
    """Identical initial bytes in every pool: fp32 warm-up with the fp32-state
    step, then sq_quant_state into the first pool, copied to the others."""
    B, H, d = wl.B, wl.H, wl.d
    state = torch.zeros((B, H, d, d), dtype=torch.float32, device=DEV)
    ident = torch.arange(B, dtype=torch.int32, device=DEV)
    y = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    for t in range(-8, 0):
        x = dev_inputs(wl.step_inputs(layer, t), B, H)
        Q.sq_f32_decode_step(state, B, H, d, d, int(layer.gate == "kda"), ident, B, x["q"],
                             x["k"], x["v"], x["beta"], x["g"], y)
    slot = torch.from_numpy(layer.slot_of.astype(np.int32)).to(DEV)
    pools[0].buf.fill_(0x5A)
    pools[0].quant_state(slot, state)
    for p in pools[1:]:
        p.buf.copy_(pools[0].buf)
    torch.cuda.synchronize()


def row_widths(H, d, seed):
    """Per head a non-decreasing 4/6/8 width pattern on the layout's grain."""
    rng = np.random.default_rng(500 + seed)
    g = 8 if d == 128 else 16
    out = []
    for _ in range(H):
        cuts = np.sort(rng.integers(0, d // g + 1, 2)) * g
        out.append([4] * cuts[0] + [6] * (cuts[1] - cuts[0]) + [8] * (d - cuts[1]))
    return np.array(out, np.uint8)


CASES = [
    # gate, B, H, d, head bits (0: per-key-row widths), io dtype, key-row-aware fit
    ("gdn", 24, 8, 128, [6, 4, 8, 16, 6, 6, 4, 8], "bf16", False),   # 192 tiles, 12 MiB of S'
    ("kda", 40, 6, 64, [4, 6, 8, 16, 6, 4], "f32", False),           # 240 tiles at d = 64
    ("kda", 12, 3, 128, [0, 8, 0], "bf16", False),                   # per-key-row widths
    ("gdn", 10, 4, 128, [6, 16, 4, 8], "bf16", True),                # key-row-aware fit
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-d%d-%s%s" % (
    c[0], c[3], "rows" if 0 in c[4] else "heads", "-kra" if c[6] else ""))
def test_noalloc_matches_split_and_fused(case):
    gate, B, H, d, bits, dtype, kra = case
    log("noalloc %s" % (case,))
    rb = row_widths(H, d, B) if 0 in bits else None
    wl = W.custom(gate, B, H, d, bits, dtype=dtype, n_slots=B + 7, permute=True, seed=21,
                  row_bits=rb)
    layer = wl.layers[0]
    imp = None
    if kra:   # row-impact scores over about three decades, kept alive for every launch
        rng = np.random.default_rng(77)
        imp = torch.from_numpy(np.exp(rng.normal(0.0, 1.5, (H, d))).astype(np.float32)).to(DEV)

    def mk():
        p = Q.StatePool(wl.n_slots, H, d, bits, gate, row_bits=layer.row_bits)
        if imp is not None:
            p.set_row_impact(imp)
        return p
    na, sp, fu = mk(), mk(), mk()
    warm_pool(wl, layer, [na, sp, fu])
    ydt = torch.float32 if dtype == "f32" else torch.bfloat16
    # call 1: every request; call 2: the first n2 < B requests (other slots
    # and a smaller S' than the buffer holds from call 1)
    for t, n_req in ((0, B), (1, B // 3)):
        slot = torch.from_numpy(layer.slot_of[:n_req].astype(np.int32)).to(DEV)
        x = dev_inputs(wl.step_inputs(layer, t), n_req, H)
        args = (x["q"], x["k"], x["v"], x["beta"], x["g"])
        y_na = torch.full((n_req * H, d), float("nan"), dtype=ydt, device=DEV)
        y_sp = torch.full_like(y_na, float("nan"))
        y_fu = torch.full_like(y_na, float("nan"))
        na.split_step_noalloc(slot, *args, y_na)
        S_out = torch.full((n_req, H, d, d), float("nan"), dtype=torch.float32, device=DEV)
        sp.decode_update(slot, *args, y_sp, S_out)
        sp.quant_state(slot, S_out)
        fu.decode_step(slot, *args, y_fu)
        torch.cuda.synchronize()
        log("  call t=%d n=%d: records equal %s / %s" % (
            t, n_req, torch.equal(na.buf, sp.buf), torch.equal(na.buf, fu.buf)))
        assert torch.equal(na.buf, sp.buf), "call %d: records differ from the split path" % t
        assert torch.equal(na.buf, fu.buf), "call %d: records differ from the fused step" % t
        assert torch.equal(y_na.view(torch.int32 if dtype == "f32" else torch.int16),
                           y_sp.view(torch.int32 if dtype == "f32" else torch.int16)), t
        assert torch.equal(y_na.view(torch.int32 if dtype == "f32" else torch.int16),
                           y_fu.view(torch.int32 if dtype == "f32" else torch.int16)), t
    for p in (na, sp, fu):
        p.close()


def test_noalloc_rejects_more_than_the_buffer():
    """A call whose S' exceeds the static buffer is refused before any launch
    and leaves the pool untouched."""
    H, d = 64, 128
    per_req = H * d * d * 4
    n = Q.SQ_SPLIT_SCRATCH_BYTES // per_req + 1          # 17 requests: 68 MiB of S'
    log("noalloc limit: n=%d" % n)
    pool = Q.StatePool(n, H, d, [4] * H, "gdn")
    pool.buf.fill_(0x33)
    slot = torch.arange(n, dtype=torch.int32, device=DEV)
    x = torch.zeros((n * H, d), dtype=torch.bfloat16, device=DEV)
    s = torch.zeros((n * H,), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((n * H, d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(Q.SQError) as e:
        pool.split_step_noalloc(slot, x, x, x, s, s, y)
    assert e.value.status == Q.SQ_ENOMEM
    assert "static buffer" in e.value.text
    torch.cuda.synchronize()
    assert bool((pool.buf == 0x33).all())
    # one request fewer fits
    pool.split_step_noalloc(slot[: n - 1], x[: (n - 1) * H], x[: (n - 1) * H], x[: (n - 1) * H],
                            s[: (n - 1) * H], s[: (n - 1) * H], y[: (n - 1) * H])
    torch.cuda.synchronize()
    pool.close()


def test_noalloc_in_a_hip_graph():
    """What the entry point is for: it records into a HIP graph (it allocates
    nothing and enqueues no memset).  After one eager call (the first call on
    a device looks the buffer's address up), three replays, each with new
    inputs copied into the captured buffers and eager work in between, give
    records and y byte-identical to the same steps of the fused step run
    eagerly."""
    gate, B, H, d, bits = "kda", 6, 4, 128, [6, 4, 8, 16]
    log("noalloc hip graph")
    wl = W.custom(gate, B, H, d, bits, dtype="bf16", n_slots=8, permute=True, seed=23)
    layer = wl.layers[0]
    mk = lambda: Q.StatePool(wl.n_slots, H, d, bits, gate)
    gp, ep, warm = mk(), mk(), mk()
    warm_pool(wl, layer, [gp, ep, warm])
    slot = torch.from_numpy(layer.slot_of.astype(np.int32)).to(DEV)
    x0 = dev_inputs(wl.step_inputs(layer, 0), B, H)
    y_w = torch.empty((B * H, d), dtype=torch.bfloat16, device=DEV)
    warm.split_step_noalloc(slot, x0["q"], x0["k"], x0["v"], x0["beta"], x0["g"], y_w)
    torch.cuda.synchronize()
    static = {k: v.clone() for k, v in x0.items()}
    y_g = torch.empty((B * H, d), dtype=torch.bfloat16, device=DEV)
    saved = gp.buf.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gp.split_step_noalloc(slot, static["q"], static["k"], static["v"], static["beta"],
                              static["g"], y_g)
    torch.cuda.synchronize()
    gp.buf.copy_(saved)                               # capture does not run the kernels
    y_e = torch.empty_like(y_g)
    for t in range(3):
        x = dev_inputs(wl.step_inputs(layer, t), B, H)
        for k in static:
            static[k].copy_(x[k])
        g.replay()
        ep.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y_e)
        torch.cuda.synchronize()
        log("  replay %d: records equal %s" % (t, torch.equal(gp.buf, ep.buf)))
        assert torch.equal(gp.buf, ep.buf), t
        assert torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)), t
    for p in (gp, ep, warm):
        p.close()
