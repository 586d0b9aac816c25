"""The seeded input generator: determinism, recipe and workload shapes."""
import math

import numpy as np

import workload as W


def test_splitmix64_reference_values():
    """SplitMix64 finaliser chain, checked against an independent Python
    implementation of the published generator."""
    M = (1 << 64) - 1

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    G = 0x9E3779B97F4A7C15
    L = W.lib()
    key = mix((5 + G) & M)
    for part in (3, 1, 7, 2, 9):
        key = mix(key ^ part)
    assert L.sqg_key(5, 3, 1, 7, 2, 9) == key
    for i in (0, 1, 1000):
        assert L.sqg_draw(key, i) == mix((key + (i + 1) * G) & M)
    # the sequential SplitMix64 stream from state 0 starts with this value
    assert mix(G) == 0xE220A8397B1DCDAF


def test_inputs_deterministic_and_row_addressable():
    wl = W.make("c1")
    layer = wl.layers[0]
    a = wl.step_inputs(layer, 3)
    b = wl.step_inputs(layer, 3)
    for key in a:
        assert np.array_equal(a[key], b[key])
    rows = [(5, 7), (63, 31), (0, 0)]
    sub = wl.step_inputs(layer, 3, rows)
    for n, (bb, hh) in enumerate(rows):
        r = bb * wl.H + hh
        for key in ("q", "k", "v", "beta", "g"):
            assert np.array_equal(sub[key][n], a[key][r])
    c = wl.step_inputs(layer, 4)
    assert not np.array_equal(a["q"], c["q"])


def test_input_recipe_statistics():
    wl = W.make("c2")
    layer = wl.layers[0]
    x = {k: W.to_f32(v).astype(np.float64) for k, v in wl.step_inputs(layer, 0).items()}
    assert x["g"].shape == (wl.B * wl.H, wl.d)  # KDA: one gate per key channel
    nq = np.linalg.norm(x["q"], axis=1)
    nk = np.linalg.norm(x["k"], axis=1)
    assert np.abs(nq - 1).max() < 2e-2 and np.abs(nk - 1).max() < 2e-2  # bf16-rounded
    assert abs(x["v"].mean()) < 0.01 and abs(x["v"].var() - 1) < 0.02
    assert 0 < x["beta"].min() and x["beta"].max() < 1 and abs(x["beta"].mean() - 0.5) < 0.01
    a = -x["g"]
    assert a.min() >= 0.00099 and a.max() <= 0.502
    # the gate rates are fixed per (head, channel) across requests and steps
    g = x["g"].reshape(wl.B, wl.H, wl.d)
    assert np.array_equal(g[0], g[17])
    y = W.to_f32(wl.step_inputs(layer, 9)["g"]).reshape(wl.B, wl.H, wl.d)
    assert np.array_equal(g, y)


def test_normal_draws_are_standard():
    z = W.normals(1, 0, 0, 0, 0, 200000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs(((z > 1.96).mean()) - 0.025) < 0.002


def test_bit_mix_and_slots():
    wl = W.make("c2")
    hb = wl.layers[0].head_bits
    assert sorted(hb.tolist()) == [4] * 8 + [6] * 16 + [8] * 8
    wl4 = W.make("c4")
    assert len(wl4.layers) == 2 and wl4.layers[0].gate == "gdn" and wl4.layers[1].gate == "kda"
    assert not np.array_equal(wl4.layers[0].head_bits, wl4.layers[1].head_bits)
    w3 = W.make("c3a")
    s = w3.layers[0].slot_of
    assert s.size == 512 and len(set(s.tolist())) == 512 and s.min() >= 0 and s.max() < 640
    assert not np.array_equal(s, np.arange(512))
    assert (w3.layers[0].head_bits == 6).all()


def test_halflife_rule():
    w = W.make("c3b")
    layer = w.layers[0]
    a = W.rounded_rates(layer.gate_rates, w.dtype)
    want = np.where(math.log(2) / a > 64, 8, 4)
    assert np.array_equal(layer.head_bits, want)
    assert (layer.head_bits == 8).sum() >= 1
    assert set(layer.head_bits.tolist()) <= {4, 8}
    # the kernels see exactly these rates through the bf16 log-gate
    x = w.step_inputs(layer, 0, [(0, h) for h in range(w.H)])
    assert np.array_equal(-W.to_f32(x["g"]).astype(np.float64), a)


def test_bf16_conversion_round_trip():
    x = np.array([1.0, -2.5, 3.14159, 1e-30, 65504.0, 1.00390625, 1.01171875], np.float32)
    b = W.f32_to_bf16(x)
    back = W.bf16_to_f32(b)
    assert np.array_equal(back[:2], x[:2])
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert back[5] == 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: rounds to even (1 + 2^-6)
    assert back[6] == np.float32(1 + 2 ** -6)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -8)
