"""Offline calibration: lifetime-aware bit allocation with FP16 pivots, and
the row-impact scores of the key-row-aware fit (once per model).

Source: hyper.ai summary of STEPQuant, "Method" paragraph 2, and blog.ontle.kr
(the lifetime-allocation paragraphs).  For each recurrent-state unit (here a
head) the method estimates the reconstruction distortion at each candidate
bit width and the mean log retention; the error retention after j updates is
approximated as exponential, which gives a lifetime weight; under an average
bit budget it picks widths that minimise the lifetime-weighted distortion,
and keeps the highest-risk units in FP16 as sparse pivots.  This runs
offline: the decode step only reads the resulting per-head bit table.

Readings (the pages give the recipe in words, no formulas):
  retention   rho = exp(mean log-gate over the calibration steps), per head
              for GDN and per key row (channel) of each head for KDA, whose
              decay acts row by row
  lifetime    w = sum_j rho^(2 j) = 1 / (1 - rho^2): squared error decays by
              rho^2 per step, so a unit of fresh squared error adds up to w
              over its life; a KDA head's weight is the mean of its rows'
              weights (its distortion is spread over the rows)
  distortion  D_h(b) = mean over calibration states of
              ||S - DQ_b(S)||^2 / ||S||^2 with the pool's own quantizer
              (measured with the GPU quant / dequant kernels)
  objective   minimise sum_h w_h D_h(b_h) subject to mean_h b_h <= budget over
              the non-pivot heads, b_h in the candidate widths (greedy on the
              largest objective decrease per extra bit)
  pivots      the n_pivots heads with the largest w_h D_h(b_min) are stored
              as FP16 (bits = 16) outside the nominal budget
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np


class RowImpact:
    """Running row-impact scores (hyper.ai summary, "Method", paragraph on
    the spatial distribution of errors: the expected squared weighting
    factor of a key row, from the transition matrix and the query).

    An error E in the stored state reaches the next read-out as E^T A^T q
    with A = (I - beta k k^T) diag(a) the next step's transition, so key row
    i enters with weight w_i = a_i (q_i - beta k_i (k . q)).  The score is
    the mean of w^2 over the calibration tokens, per head, scaled to mean 1
    over the key rows and floored (the fit needs scores > 0)."""

    def __init__(self):
        self.sum = None
        self.n = 0

    def add(self, q, k, beta, log_gates) -> None:
        """q, k: [T, H, d_k]; beta: [T, H]; log_gates: [T, H] (GDN) or
        [T, H, d_k] (KDA).  Tokens may be any samples (steps x requests)."""
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        beta = np.asarray(beta, np.float64)
        g = np.asarray(log_gates, np.float64)
        if q.ndim != 3 or k.shape != q.shape or beta.shape != q.shape[:2]:
            raise ValueError("q, k must be [T, H, d_k] and beta [T, H]")
        a = np.exp(g)[..., None] if g.ndim == 2 else np.exp(g)
        kq = (k * q).sum(axis=-1, keepdims=True)
        w = a * (q - beta[..., None] * k * kq)
        part = (w * w).sum(axis=0)
        self.sum = part if self.sum is None else self.sum + part
        self.n += q.shape[0]

    def scores(self, floor: float = 1e-6) -> np.ndarray:
        imp = self.sum / max(1, self.n)
        mean = imp.mean(axis=1, keepdims=True)
        imp = np.where(mean > 0, imp / np.where(mean > 0, mean, 1.0), 1.0)
        return np.maximum(imp, floor).astype(np.float32)


def row_impact(q, k, beta, log_gates, floor: float = 1e-6) -> np.ndarray:
    """Row-impact scores imp[h, i] of one batch of calibration tokens (see
    RowImpact)."""
    acc = RowImpact()
    acc.add(q, k, beta, log_gates)
    return acc.scores(floor)


def lifetime_weights(mean_log_retention) -> np.ndarray:
    """w = 1 / (1 - rho^2) with rho = exp(mean log retention) (< 1)."""
    mlr = np.minimum(np.asarray(mean_log_retention, np.float64), -1e-9)
    return 1.0 / -np.expm1(2.0 * mlr)


def head_lifetime_weights(log_gates) -> np.ndarray:
    """Per head lifetime weight from log-gates [T, H] (GDN) or [T, H, d_k]
    (KDA): the mean over key rows of each row's 1 / (1 - rho^2)."""
    g = np.asarray(log_gates, np.float64)
    w = lifetime_weights(g.mean(axis=0))
    return w if w.ndim == 1 else w.mean(axis=1)


def mean_log_retention(log_gates) -> np.ndarray:
    """Per head: mean of the log-gates over steps (and key channels for KDA).
    log_gates: [T, H] (GDN) or [T, H, d_k] (KDA), any float dtype."""
    g = np.asarray(log_gates, np.float64)
    axes = (0,) if g.ndim == 2 else (0, 2)
    return g.mean(axis=axes)


def allocate_bits(distortion: np.ndarray, weights: np.ndarray, avg_bits: float,
                  candidates: Sequence[int] = (4, 6, 8), n_pivots: int = 0,
                  pivot_bits: int = 16, pivots_in_budget: bool = False) -> np.ndarray:
    """distortion: [H, len(candidates)] (non-increasing in the width);
    weights: [H].  Returns the width per head (pivots get pivot_bits).
    The average is over the non-pivot heads, or over all heads with the
    pivots' bits counted when pivots_in_budget."""
    D = np.asarray(distortion, np.float64)
    w = np.asarray(weights, np.float64)
    cand = list(candidates)
    H = D.shape[0]
    if D.shape != (H, len(cand)) or w.shape != (H,):
        raise ValueError("distortion must be [H, n_candidates] and weights [H]")
    if sorted(cand) != cand:
        raise ValueError("candidates must be increasing")
    bits = np.full(H, cand[0], np.int64)
    risk = w * D[:, 0]
    pivots = np.argsort(-risk, kind="stable")[:n_pivots] if n_pivots > 0 else np.array([], int)
    free = np.setdiff1d(np.arange(H), pivots)
    level = np.zeros(H, np.int64)
    total = avg_bits * H - pivot_bits * len(pivots) if pivots_in_budget else avg_bits * len(free)
    budget = total - cand[0] * len(free)
    if budget < -1e-9:
        raise ValueError("budget below the smallest width")
    while True:
        best, best_gain = -1, 0.0
        for h in free:
            l = level[h]
            if l + 1 >= len(cand):
                continue
            extra = cand[l + 1] - cand[l]
            if extra > budget + 1e-9:
                continue
            gain = w[h] * (D[h, l] - D[h, l + 1]) / extra
            if gain > best_gain:
                best, best_gain = h, gain
        if best < 0:
            break
        budget -= cand[level[best] + 1] - cand[level[best]]
        level[best] += 1
    bits[free] = [cand[l] for l in level[free]]
    bits[pivots] = pivot_bits
    return bits.astype(np.uint8)


def measure_distortion(states, candidates: Sequence[int] = (4, 6, 8)) -> np.ndarray:
    """D[h, b]: mean over requests of ||S - DQ_b(S)||^2 / ||S||^2 for fp32
    device states [N, H, d, d], through the pool's quant / dequant kernels."""
    import torch

    from .sq import StatePool

    N, H, d, _ = states.shape
    slot = torch.arange(N, dtype=torch.int32, device=states.device)
    out = np.zeros((H, len(candidates)))
    energy = states.double().pow(2).sum(dim=(2, 3)).clamp_min(1e-300)
    for i, b in enumerate(candidates):
        pool = StatePool(N, H, d, [b] * H, "gdn", device=states.device)
        pool.quant_state(slot, states)
        back = pool.dequant_state(slot)
        err = (back.double() - states.double()).pow(2).sum(dim=(2, 3))
        out[:, i] = (err / energy).mean(dim=0).cpu().numpy()
        pool.close()
    return out


def row_lifetime_weights(log_gates) -> np.ndarray:
    """Per key row lifetime weights [H, d_k] from KDA log-gates [T, H, d_k]
    (the KDA unit of the allocation is the key row)."""
    g = np.asarray(log_gates, np.float64)
    if g.ndim != 3:
        raise ValueError("log_gates must be [T, H, d_k]")
    return lifetime_weights(g.mean(axis=0))


def allocate_row_bits(distortion: np.ndarray, weights: np.ndarray, avg_bits: float,
                      candidates: Sequence[int] = (4, 6, 8), grain: int = 8):
    """Key-row widths under an average budget over all rows of all heads.

    distortion: [H, d, len(candidates)] per-row distortion at each width
    (row i's codes depend only on its own width, so these come from uniform
    quantizations); weights: [H, d] per-row lifetime weights.

    The pool layout needs each head's widths grouped, non-decreasing, on a
    grain of `grain` rows; the key channels may be permuted offline to get
    there.  So each head's rows are ordered by risk (weight x distortion at
    the smallest width), cut into groups of `grain`, and the groups take
    widths greedily by the largest decrease of sum_i w_i D_i(b_i) per added
    bit.  Returns (row_bits [H, d] non-decreasing along the physical rows,
    perm [H, d]: physical row p of head h holds key channel perm[h, p])."""
    D = np.asarray(distortion, np.float64)
    w = np.asarray(weights, np.float64)
    cand = list(candidates)
    H, d, nc = D.shape
    if w.shape != (H, d) or nc != len(cand) or d % grain:
        raise ValueError("distortion [H, d, n_candidates], weights [H, d], d a multiple of grain")
    perm = np.argsort(w * D[:, :, 0], axis=1, kind="stable")
    Dp = np.take_along_axis(D, perm[:, :, None], axis=1)
    wp = np.take_along_axis(w, perm, axis=1)
    G = d // grain
    obj = (wp[:, :, None] * Dp).reshape(H, G, grain, nc).sum(axis=2)   # [H, G, nc]
    level = np.zeros((H, G), np.int64)
    budget = (avg_bits - cand[0]) * H * d
    if budget < -1e-9:
        raise ValueError("budget below the smallest width")
    while True:
        best, best_gain = None, 0.0
        for h in range(H):
            for g in range(G):
                l = level[h, g]
                if l + 1 >= nc:
                    continue
                extra = (cand[l + 1] - cand[l]) * grain
                if extra > budget + 1e-9:
                    continue
                gain = (obj[h, g, l] - obj[h, g, l + 1]) / extra
                if gain > best_gain:
                    best, best_gain = (h, g), gain
        if best is None:
            break
        h, g = best
        budget -= (cand[level[h, g] + 1] - cand[level[h, g]]) * grain
        level[h, g] += 1
    # groups in risk order normally come out non-decreasing; where they do
    # not, the group order is rearranged to match (rows move with their group)
    order = np.argsort(level, axis=1, kind="stable")
    level = np.take_along_axis(level, order, axis=1)
    perm = np.take_along_axis(perm.reshape(H, G, grain), order[:, :, None], axis=1).reshape(H, d)
    widths = np.asarray(cand)[level]
    return np.repeat(widths, grain, axis=1).astype(np.uint8), perm.astype(np.int64)


def measure_row_distortion(states, candidates: Sequence[int] = (4, 6, 8)) -> np.ndarray:
    """E[h, i, b]: mean over requests of ||S_i - DQ_b(S)_i||^2 / ||S||^2 for
    each key row i of fp32 device states [N, H, d, d], through the pool's
    quant / dequant kernels at uniform widths."""
    import torch

    from .sq import StatePool

    N, H, d, _ = states.shape
    slot = torch.arange(N, dtype=torch.int32, device=states.device)
    out = np.zeros((H, d, len(candidates)))
    energy = states.double().pow(2).sum(dim=(2, 3)).clamp_min(1e-300)     # [N, H]
    for i, b in enumerate(candidates):
        pool = StatePool(N, H, d, [b] * H, "kda", device=states.device)
        pool.quant_state(slot, states)
        back = pool.dequant_state(slot)
        err = (back.double() - states.double()).pow(2).sum(dim=3)          # [N, H, d]
        out[:, :, i] = (err / energy[:, :, None]).mean(dim=0).cpu().numpy()
        pool.close()
    return out


def calibrate(states, log_gates, avg_bits: float = 6.0, candidates=(4, 6, 8),
              n_pivots: int = 0) -> dict:
    """Bits per head from calibration states [N, H, d, d] (device, fp32) and
    the log-gates seen over the calibration steps."""
    D = measure_distortion(states, candidates)
    w = head_lifetime_weights(log_gates)
    bits = allocate_bits(D, w, avg_bits, candidates, n_pivots)
    return {"bits": bits, "distortion": D, "weights": w,
            "half_life_steps": math.log(2) / -np.log(np.sqrt(1 - 1 / w))}
