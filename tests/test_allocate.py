"""Lifetime-aware bit allocation with FP16 pivots (host logic, no GPU)."""
import itertools
import math

import numpy as np
import pytest

from quantized_gated_delta_amd import allocate as A


def test_lifetime_weights_closed_form():
    rho = np.array([0.5, 0.9, 0.99])
    w = A.lifetime_weights(np.log(rho))
    assert np.allclose(w, 1 / (1 - rho ** 2))
    assert np.all(np.diff(w) > 0)
    # a geometric series of squared retention: sum_j rho^(2j)
    assert math.isclose(w[1], sum(0.81 ** j for j in range(4000)), rel_tol=1e-9)


def test_mean_log_retention_axes():
    g = -np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4)
    assert np.allclose(A.mean_log_retention(g), g.mean(axis=(0, 2)))
    assert np.allclose(A.mean_log_retention(g[:, :, 0]), g[:, :, 0].mean(axis=0))


def test_head_lifetime_weights_gdn_and_kda():
    rng = np.random.default_rng(7)
    g = -rng.uniform(0.01, 1.0, (5, 3))                    # GDN [T, H]
    rho = np.exp(g.mean(axis=0))
    assert np.allclose(A.head_lifetime_weights(g), 1 / (1 - rho ** 2))
    # KDA: one slow row dominates a head whose mean log-gate is fast
    gk = np.full((4, 2, 8), -2.0)
    gk[:, 1, 0] = -0.01
    w = A.head_lifetime_weights(gk)
    slow = 1 / (1 - np.exp(-0.02))
    fast = 1 / (1 - np.exp(-4.0))
    assert np.isclose(w[0], fast) and np.isclose(w[1], (slow + 7 * fast) / 8)
    assert w[1] > A.lifetime_weights(A.mean_log_retention(gk))[1] * 5


def _objective(D, w, bits, cand):
    idx = [cand.index(b) for b in bits]
    return float(sum(w[h] * D[h, i] for h, i in enumerate(idx)))


@pytest.mark.parametrize("seed", range(12))
def test_greedy_matches_brute_force(seed):
    """With distortion falling geometrically in the width (convex), the
    greedy allocation equals the exhaustive optimum under the budget."""
    rng = np.random.default_rng(seed)
    H, cand = 6, [4, 6, 8]
    base = np.exp(rng.normal(0, 1, H))
    D = np.stack([base * 4.0 ** (-(b - 4) / 2 * rng.uniform(0.8, 1.2)) for b in cand], 1)
    w = A.lifetime_weights(-rng.uniform(0.001, 0.5, H))
    avg = rng.choice([4.0, 5.0, 6.0, 7.0, 8.0])
    bits = A.allocate_bits(D, w, avg, cand)
    assert bits.mean() <= avg + 1e-9
    best = min((_objective(D, w, c, cand), c) for c in itertools.product(cand, repeat=H)
               if np.mean(c) <= avg + 1e-9)
    assert math.isclose(_objective(D, w, bits.tolist(), cand), best[0], rel_tol=1e-12)


def test_longer_lifetime_gets_at_least_as_many_bits():
    D = np.tile([1.0, 0.25, 0.0625], (8, 1))
    w = A.lifetime_weights(-np.linspace(0.5, 0.002, 8))   # increasing lifetime
    bits = A.allocate_bits(D, w, 6.0)
    assert np.all(np.diff(bits.astype(int)) >= 0)
    assert bits.mean() <= 6.0


def test_pivots_are_the_highest_risk_heads():
    rng = np.random.default_rng(3)
    H = 10
    D = np.stack([np.exp(rng.normal(0, 1, H)) * s for s in (1, 0.25, 0.0625)], 1)
    w = A.lifetime_weights(-rng.uniform(0.001, 0.5, H))
    bits = A.allocate_bits(D, w, 6.0, n_pivots=2)
    risk = w * D[:, 0]
    assert set(np.nonzero(bits == 16)[0]) == set(np.argsort(-risk)[:2])
    assert bits[bits != 16].mean() <= 6.0


def test_pivots_inside_the_budget():
    D = np.tile([1.0, 0.25, 0.0625], (8, 1))
    w = np.arange(1.0, 9.0)
    bits = A.allocate_bits(D, w, 6.0, n_pivots=1, pivots_in_budget=True)
    assert bits[7] == 16
    assert bits.astype(int).sum() <= 6 * 8
    assert bits[:7].astype(int).sum() == 6 * 8 - 16


def test_budget_edges():
    D = np.tile([1.0, 0.5, 0.25], (4, 1))
    w = np.ones(4)
    assert (A.allocate_bits(D, w, 4.0) == 4).all()
    assert (A.allocate_bits(D, w, 8.0) == 8).all()
    with pytest.raises(ValueError):
        A.allocate_bits(D, w, 3.0)


def test_row_impact_closed_forms():
    rng = np.random.default_rng(11)
    T, H, d = 200, 3, 8
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    # beta = 0, gate 1: the weight is q itself -> imp ~ E[q_i^2], mean 1
    imp = A.row_impact(q, k, np.zeros((T, H)), np.zeros((T, H)))
    want = (q ** 2).mean(axis=0)
    assert np.allclose(imp, want / want.mean(axis=1, keepdims=True), rtol=1e-6)
    assert np.allclose(imp.mean(axis=1), 1.0, rtol=1e-6)
    # beta = 1, k = e_0: the write replaces row 0, so an error there never
    # reaches the read-out (w_0 = q_0 - q_0 = 0, floored); other rows keep q_i
    e0 = np.zeros_like(q)
    e0[..., 0] = 1.0
    imp0 = A.row_impact(q, e0, np.ones((T, H)), np.zeros((T, H)), floor=1e-6)
    assert (imp0[:, 0] == np.float32(1e-6)).all()
    w1 = want[:, 1:]
    assert np.allclose(imp0[:, 1:], w1 / (w1.sum(axis=1, keepdims=True) / d), rtol=1e-6)
    # KDA: a per-row gate scales row i's weight by a_i
    g = np.zeros((T, H, d))
    g[:, :, 2] = np.log(0.5)
    imp2 = A.row_impact(q, k, np.zeros((T, H)), g)
    ratio = imp2[:, 2] / imp2[:, 3]
    assert np.allclose(ratio, 0.25 * want[:, 2] / want[:, 3], rtol=1e-6)


def test_row_impact_floor_and_shapes():
    q = np.zeros((4, 2, 5))
    q[..., 0] = 1.0
    imp = A.row_impact(q, np.zeros_like(q), np.zeros((4, 2)), np.zeros((4, 2)), floor=1e-3)
    assert imp.dtype == np.float32 and imp.shape == (2, 5)
    assert (imp[:, 1:] == np.float32(1e-3)).all() and np.allclose(imp[:, 0], 5.0)
    with pytest.raises(ValueError):
        A.row_impact(q, q[:, :1], np.zeros((4, 2)), np.zeros((4, 2)))


def test_row_impact_streaming_equals_batch():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((30, 2, 6))
    k = rng.standard_normal((30, 2, 6))
    b = rng.uniform(0, 1, (30, 2))
    g = -rng.uniform(0, 0.5, (30, 2, 6))
    acc = A.RowImpact()
    for lo in range(0, 30, 7):
        acc.add(q[lo:lo + 7], k[lo:lo + 7], b[lo:lo + 7], g[lo:lo + 7])
    assert np.allclose(acc.scores(), A.row_impact(q, k, b, g), rtol=1e-6)


def test_row_lifetime_weights():
    g = np.zeros((5, 2, 4))
    g[:, 1, 3] = -0.1
    g[:, 0, 0] = -2.0
    w = A.row_lifetime_weights(g)
    assert w.shape == (2, 4)
    assert math.isclose(w[1, 3], 1 / (1 - math.exp(-0.2)), rel_tol=1e-12)
    assert math.isclose(w[0, 0], 1 / (1 - math.exp(-4.0)), rel_tol=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_row_bits_greedy_matches_brute_force(seed):
    """Small case: 2 heads x 2 groups of 2 rows.  With convex per-row
    distortion the greedy reaches the best assignment of widths to the
    risk-ordered groups (brute force); the returned widths are
    non-decreasing along the physical rows, grouped on the grain, within
    budget, and perm is a permutation that carries each row's terms."""
    rng = np.random.default_rng(40 + seed)
    H, d, grain, cand = 2, 4, 2, [4, 6, 8]
    base = np.exp(rng.normal(0, 1, (H, d)))
    D = np.stack([base * 4.0 ** (-(b - 4) / 2) for b in cand], axis=-1)
    w = A.lifetime_weights(-rng.uniform(0.001, 0.5, (H, d)))
    avg = float(rng.choice([5.0, 6.0, 7.0]))
    rb, perm = A.allocate_row_bits(D, w, avg, cand, grain)
    assert rb.shape == (H, d) and rb.mean() <= avg + 1e-9
    assert (np.diff(rb.astype(int), axis=1) >= 0).all()
    assert all(len(set(rb[h, g * grain:(g + 1) * grain])) == 1 for h in range(H) for g in range(2))
    assert all(sorted(perm[h]) == list(range(d)) for h in range(H))

    def objective(widths, pm):
        return sum(w[h, pm[h, p]] * D[h, pm[h, p], cand.index(widths[h, p])]
                   for h in range(H) for p in range(d))

    risk = np.argsort(w * D[:, :, 0], axis=1, kind="stable")
    best = None
    for combo in itertools.product(cand, repeat=H * 2):
        wd = np.repeat(np.array(combo).reshape(H, 2), grain, axis=1)
        if wd.mean() > avg + 1e-9:
            continue
        o = objective(wd, risk)
        best = o if best is None else min(best, o)
    assert math.isclose(objective(rb, perm), best, rel_tol=1e-9)
