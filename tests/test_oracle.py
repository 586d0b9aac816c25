"""Pins of the CPU oracle against things other than itself.

Each check below is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign, a transposed operand, a wrong tie rule, a wrong scale
axis, a shifted bit field) fails at least one of them:

* encoding: hand-derived golden rows, an independent big-integer packer,
  exhaustive round trips;
* quantizer: hand-derived ties, exact rational brute force on 4x4 states,
  idempotence, scale/sign equivariance, the max-level property, error bound;
* recurrence: the transition-matrix form of the step, exact rationals, the
  delta-rule identities (unit key writes v exactly, basis keys overwrite one
  row, orthogonal directions only decay), read-out through basis queries;
* the quantized loop: the error-propagation identity (error now = transition
  applied to yesterday's error + fresh rounding error), convergence to the
  unquantized FP64 recurrence as the bit width grows, KDA == GDN when all
  channel gates are equal, the beta = 0 / gate = 1 identity.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split("|")])
    return rows


def _rand_state(rng, dk, dv, scale_rows=True, scale_cols=True):
    """Dense state with outliers along rows and columns (dual-axis geometry)."""
    S = rng.standard_normal((dk, dv))
    if scale_rows:
        S *= np.exp(rng.standard_normal(dk))[:, None]
    if scale_cols:
        S *= np.exp(rng.standard_normal(dv))[None, :]
    return S.astype(np.float32)


# ------------------------------------------------------------------ encoding
def test_pack_golden_rows():
    for bits, codes, hexbytes in _golden("pack_examples.txt"):
        bits = int(bits)
        codes = np.array([int(x) for x in codes.split()], np.int32)
        want = bytes.fromhex(hexbytes.replace(" ", ""))
        got = O.pack_row(bits, codes).tobytes()
        assert got == want, (bits, codes, got.hex(), want.hex())
        assert np.array_equal(O.unpack_row(bits, np.frombuffer(want, np.uint8), codes.size), codes)


def _bigint_pack(bits, codes):
    acc = 0
    for j, cde in enumerate(codes):
        acc |= (int(cde) % (1 << bits)) << (bits * j)
    nbytes = (len(codes) * bits + 7) // 8
    return acc.to_bytes(nbytes, "little")


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_pack_matches_bigint_bitstream(bits):
    rng = np.random.default_rng(bits)
    q = O.qmax(bits)
    for n in (8, 16, 64, 128):
        codes = rng.integers(-q, q + 1, n).astype(np.int32)
        assert O.pack_row(bits, codes).tobytes() == _bigint_pack(bits, codes)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_pack_roundtrip_exhaustive(bits):
    """Every code value at every position of a 24-code row (covers every
    position inside the 2-code, 4-code and 1-code groups)."""
    q = O.qmax(bits)
    rng = np.random.default_rng(100 + bits)
    n = 24
    for pos in range(n):
        base = rng.integers(-q, q + 1, n).astype(np.int32)
        for val in range(-q, q + 1):
            base[pos] = val
            packed = O.pack_row(bits, base)
            assert np.array_equal(O.unpack_row(bits, packed, n), base)


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.pack_row(4, np.array([8, 0], np.int32))
    with pytest.raises(ValueError):
        O.pack_row(6, np.array([0, 0, 0, -32], np.int32))  # -2^(b-1) is never produced


def test_record_bytes_and_compression():
    # d = 128: codes 8192 / 12288 / 16384 B + 1024 B of fp32 scales
    assert [O.record_bytes(b, 128, 128) for b in (4, 6, 8)] == [9216, 13312, 17408]
    assert [O.record_bytes(b, 64, 64) for b in (4, 6, 8)] == [2560, 3584, 4608]
    fp32 = 128 * 128 * 4
    ratios = [fp32 / O.record_bytes(b, 128, 128) for b in (4, 6, 8)]
    assert [round(r, 2) for r in ratios] == [7.11, 4.92, 3.76]
    # every record is a whole number of 256-byte units (aligned pool records)
    for b in (4, 6, 8):
        for d in (64, 128):
            assert O.record_bytes(b, d, d) % 256 == 0


# ------------------------------------------------------------------ quantizer
def test_quant_golden_ties():
    for bits, S, codes, r1 in _golden("quant_ties.txt"):
        bits = int(bits)
        S = np.array([float(x) for x in S.split()], np.float32).reshape(2, 2)
        codes = np.array([int(x) for x in codes.split()], np.int32).reshape(2, 2)
        Q, r, c = O.quantize(bits, S)
        assert np.array_equal(Q, codes), (S, Q, codes)
        assert r[1] == np.float32(float(r1))
        assert np.array_equal(c, np.abs(S).max(axis=0))


def _nearest_even(x: Fraction) -> int:
    f = math.floor(x)
    d = x - f
    if d > Fraction(1, 2):
        return f + 1
    if d < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quant_bruteforce_4x4_exact(bits):
    """Each code is the nearest level to S_ij / (r_i c_j) in exact rational
    arithmetic, searched over every level; scales follow the closed rule."""
    q = O.qmax(bits)
    rng = np.random.default_rng(7 + bits)
    near_ties = 0
    for trial in range(200):
        S = _rand_state(rng, 4, 4)
        Q, r, c = O.quantize(bits, S)
        Sf = [[Fraction(float(S[i, j])) for j in range(4)] for i in range(4)]
        for j in range(4):
            assert Fraction(float(c[j])) == max(abs(Sf[i][j]) for i in range(4))
        for i in range(4):
            m = max(abs(Sf[i][j]) / Fraction(float(c[j])) for j in range(4))
            assert abs(Fraction(float(r[i])) - m / q) <= m / q * Fraction(3, 2 ** 24)
            for j in range(4):
                rc = Fraction(float(r[i])) * Fraction(float(c[j]))
                best = min(range(-q, q + 1),
                           key=lambda lv: (abs(Sf[i][j] - lv * rc), lv % 2))
                x = Sf[i][j] / rc
                assert best == _nearest_even(x)
                if abs(x - math.floor(x) - Fraction(1, 2)) < Fraction(1, 10 ** 5):
                    near_ties += 1
                    assert abs(int(Q[i, j]) - best) <= 1
                else:
                    assert int(Q[i, j]) == best, (trial, i, j, float(x))
    assert near_ties < 5


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8, 12, 16])
def test_quant_dequant_idempotent(bits):
    rng = np.random.default_rng(bits)
    for d in (8, 64, 128):
        S = _rand_state(rng, d, d)
        Q, r, c = O.quantize(bits, S)
        Q2, r2, c2 = O.quantize(bits, O.dequantize(Q, r, c))
        assert np.array_equal(Q, Q2)
        np.testing.assert_allclose(r2, r, rtol=4 * 2.0 ** -23)
        np.testing.assert_allclose(c2, c, rtol=4 * 2.0 ** -23)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quant_every_row_and_column_hits_qmax(bits):
    rng = np.random.default_rng(11)
    q = O.qmax(bits)
    S = _rand_state(rng, 128, 128)
    Q, r, c = O.quantize(bits, S)
    assert (np.abs(Q).max(axis=0) == q).all()
    assert (np.abs(Q).max(axis=1) == q).all()
    assert np.abs(Q).max() <= q


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quant_error_bound(bits):
    rng = np.random.default_rng(12)
    S = _rand_state(rng, 128, 128)
    Q, r, c = O.quantize(bits, S)
    step = r.astype(np.float64)[:, None] * c.astype(np.float64)[None, :]
    err = np.abs(S.astype(np.float64) - O.dequantize(Q, r, c).astype(np.float64))
    assert (err <= 0.5 * step * (1 + 1e-5) + 1e-30).all()


def test_quant_equivariance():
    rng = np.random.default_rng(13)
    S = _rand_state(rng, 64, 64)
    Q, r, c = O.quantize(6, S)
    Qn, rn, cn = O.quantize(6, -S)
    assert np.array_equal(Qn, -Q) and np.array_equal(rn, r) and np.array_equal(cn, c)
    Qs, rs, cs = O.quantize(6, S * np.float32(2.0 ** 20))
    assert np.array_equal(Qs, Q) and np.array_equal(rs, r) and np.array_equal(cs, c * 2.0 ** 20)
    # scaling one column by a power of two moves only that column's scale
    S2 = S.copy()
    S2[:, 5] *= 8
    Q2, r2, c2 = O.quantize(6, S2)
    assert np.array_equal(Q2, Q) and np.array_equal(r2, r)
    assert c2[5] == 8 * c[5] and np.array_equal(np.delete(c2, 5), np.delete(c, 5))


def test_quant_zero_row_column_and_tiny():
    S = np.zeros((8, 8), np.float32)
    Q, r, c = O.quantize(6, S)
    assert not Q.any() and not r.any() and not c.any()
    rng = np.random.default_rng(14)
    S = _rand_state(rng, 8, 8)
    S[3, :] = 0
    S[:, 5] = 0
    S[6, 2] = 1e-39  # subnormal entry in an otherwise normal column
    Q, r, c = O.quantize(6, S)
    assert r[3] == 0 and not Q[3].any()
    assert c[5] == 0 and not Q[:, 5].any()
    S = np.zeros((4, 4), np.float32)
    S[1, 1] = 1e-40  # only a subnormal: column max below FLT_MIN -> stored as zero
    Q, r, c = O.quantize(8, S)
    assert not Q.any() and c[1] == 0


def test_dequant_exact_for_power_of_two_scales():
    rng = np.random.default_rng(15)
    Q = rng.integers(-31, 32, (16, 16)).astype(np.int32)
    r = (2.0 ** rng.integers(-20, 5, 16)).astype(np.float32)
    c = (2.0 ** rng.integers(-20, 5, 16)).astype(np.float32)
    want = Q.astype(np.float64) * r[:, None].astype(np.float64) * c[None, :].astype(np.float64)
    assert np.array_equal(O.dequantize(Q, r, c).astype(np.float64), want)
    # general scales: the FP64 reconstruction is the exact rational product for
    # |Q| <= 31 (4- and 6-bit codes) and the fp32 export is its single rounding
    r = rng.random(16).astype(np.float32)
    c = rng.random(16).astype(np.float32)
    S64 = O.reconstruct_f64(Q, r, c)
    for i in range(16):
        for j in range(16):
            exact = Fraction(int(Q[i, j])) * Fraction(float(r[i])) * Fraction(float(c[j]))
            assert Fraction(float(S64[i, j])) == exact
    assert np.array_equal(O.dequantize(Q, r, c), S64.astype(np.float32))
    Q8 = rng.integers(-127, 128, (16, 16)).astype(np.int32)
    exact = Q8.astype(np.float64) * r[:, None].astype(np.float64)
    np.testing.assert_allclose(O.reconstruct_f64(Q8, r, c), exact * c[None, :], rtol=2.0 ** -53,
                               atol=0)


def test_magic_number_rounding_identity():
    """fl(x + 1.5*2^23) - 1.5*2^23 == round_half_even(x) for |x| < 2^22: the
    shortcut the GPU epilogue uses.  Dense grid of k/2^16 over [-256, 256],
    every half-integer, and random fp32 values across the range."""
    M = np.float32(1.5 * 2 ** 23)
    xs = [np.arange(-256 * 2 ** 16, 256 * 2 ** 16 + 1, dtype=np.int64).astype(np.float32)
          / np.float32(2 ** 16),
          np.arange(-2 ** 12, 2 ** 12, dtype=np.float32) + np.float32(0.5)]
    rng = np.random.default_rng(16)
    xs.append((rng.random(2_000_000) * 2 ** 23 - 2 ** 22).astype(np.float32))
    for x in xs:
        got = (x + M) - M
        assert np.array_equal(got, np.rint(x))
        # low bits of the sum's bit pattern are the two's complement code
        bitsum = (x + M).view(np.uint32)
        lo = (bitsum & 0xFF).astype(np.int64)
        assert np.array_equal(lo, np.rint(x).astype(np.int64) & 0xFF)


# ------------------------------------------------------------------ recurrence
def _inputs(rng, dk, dv, kda=False):
    q = rng.standard_normal(dk)
    q /= np.linalg.norm(q)
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    beta = 1 / (1 + math.exp(-rng.standard_normal()))
    alpha = np.exp(-rng.uniform(0.001, 0.5, dk if kda else 1)) * np.ones(dk)
    return q, k, v, beta, alpha


@pytest.mark.parametrize("kda", [False, True])
def test_step_matches_transition_matrix_form(kda):
    """S' = (I - beta k k^T) D S + beta k v^T and y = S'^T q, as matrices."""
    rng = np.random.default_rng(20 + kda)
    for dk, dv in ((4, 4), (16, 32), (64, 64)):
        S = rng.standard_normal((dk, dv))
        q, k, v, beta, alpha = _inputs(rng, dk, dv, kda)
        S1, y = O.gated_delta_f64(S, alpha, q, k, v, beta)
        A = (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(alpha)
        want = A @ S + beta * np.outer(k, v)
        np.testing.assert_allclose(S1, want, rtol=0, atol=1e-13 * np.abs(want).max())
        np.testing.assert_allclose(y, want.T @ q, rtol=0, atol=1e-13 * np.abs(want).max())


def test_step_exact_rational_4x4():
    """Exact rational evaluation of the transition-matrix form on 4x4 inputs."""
    rng = np.random.default_rng(22)
    for _ in range(20):
        S = rng.standard_normal((4, 4))
        q, k, v, beta, alpha = _inputs(rng, 4, 4, True)
        S1, y = O.gated_delta_f64(S, alpha, q, k, v, beta)
        F = Fraction
        Sf = [[F(S[i, j]) for j in range(4)] for i in range(4)]
        kf, qf, vf, af, bf = ([F(x) for x in k], [F(x) for x in q], [F(x) for x in v],
                              [F(x) for x in alpha], F(beta))
        A = [[((1 if i == m else 0) - bf * kf[i] * kf[m]) * af[m] for m in range(4)]
             for i in range(4)]
        want = [[sum(A[i][m] * Sf[m][j] for m in range(4)) + bf * kf[i] * vf[j]
                 for j in range(4)] for i in range(4)]
        yw = [sum(qf[i] * want[i][j] for i in range(4)) for j in range(4)]
        for i in range(4):
            for j in range(4):
                assert abs(F(S1[i, j]) - want[i][j]) <= F(1, 10 ** 14)
        for j in range(4):
            assert abs(F(y[j]) - yw[j]) <= F(1, 10 ** 14)


def test_delta_rule_identities():
    rng = np.random.default_rng(23)
    dk = dv = 64
    S = rng.standard_normal((dk, dv))
    q, k, v, beta, _ = _inputs(rng, dk, dv)
    one = np.ones(dk)
    # unit key, full write strength, no decay: the key now retrieves v exactly
    S1, _ = O.gated_delta_f64(S, one, q, k, v, 1.0)
    np.testing.assert_allclose(S1.T @ k, v, rtol=0, atol=1e-12)
    # partial strength: read-out along k moves a fraction beta toward v
    S1, _ = O.gated_delta_f64(S, one, q, k, v, beta)
    np.testing.assert_allclose(S1.T @ k, (1 - beta) * (S.T @ k) + beta * v, rtol=0, atol=1e-12)
    # directions orthogonal to k are untouched by the write (only decayed)
    w = rng.standard_normal(dk)
    w -= (w @ k) * k
    a = 0.9 * one
    S1, _ = O.gated_delta_f64(S, a, q, k, v, beta)
    np.testing.assert_allclose(S1.T @ w, 0.9 * (S.T @ w), rtol=0, atol=1e-12)
    # basis key: row m is overwritten by v, every other row unchanged bit for bit
    m = 17
    e = np.zeros(dk)
    e[m] = 1.0
    S1, y = O.gated_delta_f64(S, one, q, e, v, 1.0)
    np.testing.assert_allclose(S1[m], v, rtol=0, atol=1e-15)
    assert np.array_equal(np.delete(S1, m, axis=0), np.delete(S, m, axis=0))
    # basis query reads one row of the new state
    S1, y = O.gated_delta_f64(S, a, e, k, v, beta)
    assert np.array_equal(y, S1[m])
    # beta = 0: pure decay, D S
    S1, y = O.gated_delta_f64(S, a, q, k, v, 0.0)
    assert np.array_equal(S1, S * 0.9)


# ------------------------------------------------------------------ step update
def _dyadic_case(rng, dk, dv):
    """Inputs on a coarse binary grid: small integer codes; scales, gates,
    keys, beta and queries powers of two; v a multiple of 1/4.  Every
    intermediate of the step then fits in fp32 exactly, so any correct
    evaluation order returns the exact result."""
    Z = rng.integers(-7, 8, (dk, dv)).astype(np.float32)
    R = 2.0 ** -rng.integers(0, 3, dk)
    C = 2.0 ** -rng.integers(0, 3, dv)
    alpha = 2.0 ** -rng.integers(0, 3, dk)
    k = rng.choice([-1, 1], dk) * 2.0 ** -rng.integers(0, 3, dk)
    q = rng.choice([-1, 1], dk) * 2.0 ** -rng.integers(0, 2, dk)
    v = rng.integers(-32, 33, dv) / 4.0
    beta = 2.0 ** -int(rng.integers(0, 3))
    return Z, R, C, alpha, q, k, v, beta


@pytest.mark.parametrize("dk,dv", [(8, 8), (6, 10), (10, 6)])
def test_step_update_exact_on_dyadic_inputs(dk, dv):
    """On inputs where nothing rounds, the step update equals the exact
    rational value of S' = (I - beta k k^T) D S + beta k v^T with
    S_ij = Z_ij R_i C_j, and y = S'^T q (a dropped term, a wrong sign, a
    transposed scale or a row/column mix-up fails this)."""
    rng = np.random.default_rng(90 + dk)
    F = Fraction
    for _ in range(20):
        Z, R, C, alpha, q, k, v, beta = _dyadic_case(rng, dk, dv)
        Sp, y = O.step_update(Z, R, C, alpha, q, k, v, beta)
        S = [[F(float(Z[i, j])) * F(R[i]) * F(C[j]) for j in range(dv)] for i in range(dk)]
        A = [[((1 if i == m else 0) - F(beta) * F(k[i]) * F(k[m])) * F(alpha[m])
              for m in range(dk)] for i in range(dk)]
        want = [[sum(A[i][m] * S[m][j] for m in range(dk)) + F(beta) * F(k[i]) * F(v[j])
                 for j in range(dv)] for i in range(dk)]
        for i in range(dk):
            for j in range(dv):
                assert F(float(Sp[i, j])) == want[i][j]
        for j in range(dv):
            assert F(float(y[j])) == sum(F(q[i]) * want[i][j] for i in range(dk))


def test_step_update_within_fp32_rounding_of_textbook():
    """On random inputs every S'_ij lies within the rounding bound of its
    fp32 evaluation (u rounded once, the two scale products, k u and the
    fused multiply-add: at most 2^-24 (|S'| + 2|Sd| + 2|k u|) with Sd the
    decayed reconstruction) of the textbook FP64 step."""
    rng = np.random.default_rng(95)
    for dk, dv in ((64, 64), (32, 48)):
        for kda in (False, True):
            Z = rng.integers(-31, 32, (dk, dv)).astype(np.float32)
            R = (rng.uniform(0.5, 2, dk) * 1e-2).astype(np.float32)
            C = rng.uniform(0.5, 2, dv).astype(np.float32)
            q, k, v, beta, alpha = _inputs(rng, dk, dv, kda)
            alpha = alpha.astype(np.float32)
            Sp, y = O.step_update(Z, R, C, alpha, q, k, v, beta)
            k32, v32, q32 = (x.astype(np.float32).astype(np.float64) for x in (k, v, q))
            b32 = float(np.float32(beta))
            S = Z.astype(np.float64) * R.astype(np.float64)[:, None] * C.astype(np.float64)[None]
            T, yT = O.gated_delta_f64(S, alpha.astype(np.float64), q32, k32, v32, b32)
            Sd = alpha.astype(np.float64)[:, None] * S
            ku = np.abs(np.outer(k32, b32 * (v32 - Sd.T @ k32)))
            bound = 2.0 ** -24 * (np.abs(T) + 2 * np.abs(Sd) + 2 * ku) * 1.001 + 1e-300
            err = np.abs(Sp.astype(np.float64) - T)
            assert (err <= bound).all(), float((err / bound).max())
            assert (np.abs(y - yT) <= np.abs(q32) @ bound + 1e-12 * np.abs(yT).max()).all()


# ------------------------------------------------------------------ quantized loop
def _seq(rng, T, dk, dv, kda):
    seq = []
    for _ in range(T):
        q, k, v, beta, _ = _inputs(rng, dk, dv, kda)
        g = -rng.uniform(0.001, 0.5, dk if kda else 1)
        seq.append((q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                    np.float32(beta), g.astype(np.float32)))
    return seq


def _alpha(kda, dk, g):
    return np.array([float(np.float32(math.exp(float(g[i if kda else 0])))) for i in range(dk)])


@pytest.mark.parametrize("kda", [False, True])
def test_error_propagation_identity(kda):
    """E_t = (I - beta k k^T) D_t E_{t-1} + eps_t, with E the gap between the
    quantized and the exact trajectories and eps_t the fresh requantization
    error of step t (the error-propagation proposition, section 3.1)."""
    rng = np.random.default_rng(30 + kda)
    dk = dv = 32
    bits = 6
    S0 = rng.standard_normal((dk, dv)).astype(np.float32)
    Q, r, c = O.quantize(bits, S0)
    Sq = O.reconstruct_f64(Q, r, c)
    St = Sq.copy()  # exact trajectory from the same start: E_0 = 0
    E = np.zeros((dk, dv))
    for q, k, v, beta, g in _seq(rng, 24, dk, dv, kda):
        alpha = _alpha(kda, dk, g)
        Fq, _ = O.gated_delta_f64(Sq, alpha, q, k, v, beta)        # F_t(S^q_{t-1})
        y = O.quant_step_codes(kda, bits, Q, r, c, q, k, v, beta, g)
        Sq = O.reconstruct_f64(Q, r, c)
        eps = Sq - Fq
        St, _ = O.gated_delta_f64(St, alpha, q, k, v, beta)
        k64 = k.astype(np.float64)
        A = (np.eye(dk) - float(beta) * np.outer(k64, k64)) @ np.diag(alpha)
        E_new = Sq - St
        np.testing.assert_allclose(E_new, A @ E + eps, rtol=0,
                                   atol=1e-12 * max(1.0, np.abs(St).max()))
        # y reads the fp32 S' (each element within a few fp32 roundings of Fq)
        np.testing.assert_allclose(y, Fq.T @ q.astype(np.float64), rtol=0,
                                   atol=1e-6 * np.abs(q).sum() * np.abs(Fq).max())
        E = E_new


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("kda", [False, True])
def test_quantized_recurrence_converges_to_fp64(kda):
    """As bits grow by 4, the quantized trajectory's error falls about 16x
    until it reaches the fp32 floor; at 16 bits it is far below 1e-3."""
    rng = np.random.default_rng(40 + kda)
    dk = dv = 64
    T = 64
    seq = _seq(rng, T, dk, dv, kda)
    S0 = np.zeros((dk, dv))
    errs = {}
    for bits in (8, 12, 16, 20, 24):
        St = S0.copy()
        Q, r, c = O.quantize(bits, S0.astype(np.float32))
        worst = 0.0
        for q, k, v, beta, g in seq:
            O.quant_step_codes(kda, bits, Q, r, c, q, k, v, beta, g)
            St, _ = O.gated_delta_f64(St, _alpha(kda, dk, g), q, k, v, beta)
            worst = max(worst, _rel(O.reconstruct_f64(Q, r, c), St))
        errs[bits] = worst
    for b in (8, 12):
        assert 8 < errs[b] / errs[b + 4] < 32, errs
    assert errs[16] < 1e-3 and errs[24] < 2e-6, errs


def test_kda_equals_gdn_with_equal_channel_gates():
    rng = np.random.default_rng(50)
    dk = dv = 64
    S0 = _rand_state(rng, dk, dv)
    for bits in (4, 6, 8):
        Qa, ra, ca = O.quantize(bits, S0)
        Qb, rb, cb = Qa.copy(), ra.copy(), ca.copy()
        for q, k, v, beta, g in _seq(rng, 8, dk, dv, False):
            ya = O.quant_step_codes(False, bits, Qa, ra, ca, q, k, v, beta, g)
            yb = O.quant_step_codes(True, bits, Qb, rb, cb, q, k, v, beta,
                                    np.full(dk, g[0], np.float32))
            assert np.array_equal(ya, yb)
        assert np.array_equal(Qa, Qb) and np.array_equal(ra, rb) and np.array_equal(ca, cb)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_beta0_gate1_keeps_codes(bits):
    """No write (beta = 0) and no decay (log-gate 0): one step leaves every
    code unchanged and the scales within a few ulp; y = S~^T q."""
    rng = np.random.default_rng(60 + bits)
    dk = dv = 128
    Q, r, c = O.quantize(bits, _rand_state(rng, dk, dv))
    Q0, r0, c0 = Q.copy(), r.copy(), c.copy()
    q, k, v, _, _ = _inputs(rng, dk, dv)
    y = O.quant_step_codes(False, bits, Q, r, c, q.astype(np.float32), k.astype(np.float32),
                           v.astype(np.float32), 0.0, np.zeros(1, np.float32))
    assert np.array_equal(Q, Q0)
    np.testing.assert_allclose(r, r0, rtol=4 * 2.0 ** -23)
    np.testing.assert_allclose(c, c0, rtol=4 * 2.0 ** -23)
    St = O.reconstruct_f64(Q0, r0, c0)
    np.testing.assert_allclose(y, St.T @ q.astype(np.float32).astype(np.float64), rtol=0,
                               atol=4 * 2.0 ** -24 * (np.abs(q) @ np.abs(St)).max())


# ------------------------------------------------------------------ batch drivers
def test_records_drivers_match_single_head():
    rng = np.random.default_rng(70)
    dk = dv = 64
    n = 6
    bits = np.array([4, 6, 8, 6, 4, 8], np.uint8)
    sizes = [O.record_bytes(int(b), dk, dv) for b in bits]
    # records laid out in reverse order, so row i is not at the i-th position
    offs = np.zeros(n, np.int64)
    pos = 0
    for i in reversed(range(n)):
        offs[i] = pos
        pos += sizes[i]
    base = np.zeros(sum(sizes), np.uint8)
    S = np.stack([_rand_state(rng, dk, dv) for _ in range(n)])
    O.records_quantize(base, offs, bits, S, dk, dv)
    for kda in (False, True):
        q = rng.standard_normal((n, dk)).astype(np.float32)
        k = rng.standard_normal((n, dk)).astype(np.float32)
        v = rng.standard_normal((n, dv)).astype(np.float32)
        beta = rng.random(n).astype(np.float32)
        g = -rng.uniform(0.001, 0.5, (n, dk) if kda else n).astype(np.float32)
        singles = []
        for i in range(n):
            Qi, ri, ci = O.record_unpack(int(bits[i]), dk, dv, base[offs[i]:offs[i] + sizes[i]])
            assert np.array_equal(O.dequantize(Qi, ri, ci),
                                  O.records_dequantize(base, offs[i:i + 1], bits[i:i + 1],
                                                       dk, dv)[0])
            yi = O.quant_step_codes(kda, int(bits[i]), Qi, ri, ci, q[i], k[i], v[i], beta[i],
                                    g[i] if kda else g[i:i + 1])
            singles.append((O.record_pack(int(bits[i]), Qi, ri, ci), yi))
        y = O.records_step(kda, base, offs, bits, dk, dv, q, k, v, beta, g)
        for i in range(n):
            assert np.array_equal(base[offs[i]:offs[i] + sizes[i]], singles[i][0])
            assert np.array_equal(y[i], singles[i][1])


def test_f32_step_is_rounded_f64_step():
    rng = np.random.default_rng(71)
    n, d = 3, 32
    S = rng.standard_normal((n, d, d)).astype(np.float32)
    q = rng.standard_normal((n, d)).astype(np.float32)
    k = rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    beta = rng.random(n).astype(np.float32)
    g = -rng.uniform(0.001, 0.5, n).astype(np.float32)
    S64 = S.astype(np.float64)
    y64 = O.f64_step(False, S64, q, k, v, beta, g)
    S32 = S.copy()
    y32 = O.f32_step(False, S32, q, k, v, beta, g)
    assert np.array_equal(S32, S64.astype(np.float32))
    assert np.array_equal(y32, y64)


def test_oracle_thread_count_independent(monkeypatch):
    wl = W.custom("gdn", 4, 3, 64, [4, 6, 8], dtype="f32")
    layer = wl.layers[0]
    x = wl.step_inputs(layer, 0)
    rng = np.random.default_rng(72)
    S = np.stack([_rand_state(rng, 64, 64) for _ in range(12)])
    bits = np.tile(layer.head_bits, 4)
    sizes = [O.record_bytes(int(b), 64, 64) for b in bits]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    outs = []
    for nt in (1, 5):
        monkeypatch.setattr(O, "n_threads", lambda nt=nt: nt)
        base = np.zeros(sum(sizes), np.uint8)
        O.records_quantize(base, offs, bits, S, 64, 64)
        y = O.records_step(False, base, offs, bits, 64, 64, x["q"], x["k"], x["v"], x["beta"],
                           x["g"])
        outs.append((base, y))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


# ------------------------------------------------------------------ FP16 pivot records
def test_f16_conversions_match_numpy():
    """binary16 <-> binary32 against numpy's float16 (an independent
    implementation): every half value, and floats at and around every half
    value, halfway points, overflow and subnormal boundaries."""
    h = np.arange(65536, dtype=np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = np.array([O.f16_to_f32(int(x)) for x in h], np.float32)
    same = (ref.view(np.uint32) == got.view(np.uint32)) | (np.isnan(ref) & np.isnan(got))
    assert same.all()
    fin = ref[np.isfinite(ref)].astype(np.float64)
    rng = np.random.default_rng(80)
    xs = np.concatenate([
        (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 12, 50000))),
        fin, fin * (1 + 2.0 ** -11), fin * (1 - 2.0 ** -12), fin * (1 + 2.0 ** -12),
        [65504, 65519.99, 65520, 65536, 1e9, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -25,
         2.0 ** -14 * (1 - 2.0 ** -11), 1e-45, 0.0, -0.0]]).astype(np.float32)
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, want)


def test_f16_record_step():
    """A pivot record holds the state in binary16; one step is the step
    update on the widened values with unit scales, rounded from fp32 to
    binary16, and within a binary16 rounding of the textbook step."""
    rng = np.random.default_rng(81)
    d = 32
    S = (rng.standard_normal((d, d)) * 3).astype(np.float32)
    rec = np.zeros(O.record_bytes(16, d, d), np.uint8)
    assert rec.size == 2 * d * d
    O.records_quantize(rec, np.array([0], np.int64), np.array([16], np.uint8), S[None], d, d)
    assert np.array_equal(rec.view(np.uint16), S.astype(np.float16).view(np.uint16).ravel())
    S16 = O.records_dequantize(rec, np.array([0]), np.array([16], np.uint8), d, d)[0]
    assert np.array_equal(S16, S.astype(np.float16).astype(np.float32))
    q, k, v, beta, _ = _inputs(rng, d, d)
    g = np.array([-0.1], np.float32)
    y = O.records_step(False, rec, np.array([0], np.int64), np.array([16], np.uint8), d, d,
                       q[None].astype(np.float32), k[None].astype(np.float32),
                       v[None].astype(np.float32), np.array([beta], np.float32), g)
    alpha = np.full(d, np.float32(math.exp(-0.1)))
    one = np.ones(d, np.float32)
    want, yw = O.step_update(S16, one, one, alpha, q, k, v, beta)
    assert np.array_equal(rec.view(np.uint16), want.astype(np.float16).view(np.uint16).ravel())
    assert np.array_equal(y[0], yw)
    T, _ = O.gated_delta_f64(S16.astype(np.float64), alpha.astype(np.float64),
                             q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                             np.float32(beta))
    got = rec.view(np.float16).astype(np.float64).reshape(d, d)
    assert (np.abs(got - T) <= 2.0 ** -11 * np.abs(T) + 1e-6 * np.abs(T).max()).all()


# ------------------------------------------------------------------ key-row-aware fit
def _weighted_err(S, imp, Q, r, c):
    R = Q.astype(np.float64) * r.astype(np.float64)[:, None] * c.astype(np.float64)[None, :]
    return (imp.astype(np.float64)[:, None] * (S.astype(np.float64) - R) ** 2).sum(axis=0)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_kra_exact_on_constructed_state(bits):
    """S_ij = R_i C_j K_ij with power-of-two R, C and integer K whose columns
    each reach qmax; with imp_i = 4 mu_i / R_i^2 the row factors are R_i / 2
    exactly, the range-covering column scales 2 C_j are already the weighted
    least-squares scales, and the fit returns K, R / 2, 2 C bit for bit.
    (A wrong root, weight, axis or tie rule breaks this.)"""
    rng = np.random.default_rng(100 + bits)
    dk, dv, q = 16, 12, O.qmax(bits)
    K = rng.integers(-q, q + 1, size=(dk, dv))
    K[rng.integers(0, dk, dv), np.arange(dv)] = q * rng.choice([-1, 1], dv)
    R = 2.0 ** rng.integers(-6, 7, dk)
    C = 2.0 ** rng.integers(-6, 7, dv)
    S = (R[:, None] * C[None, :] * K).astype(np.float32)
    mu = np.abs(S).max(axis=1).astype(np.float64)
    imp = (4 * mu / R ** 2).astype(np.float32)
    Q, r, c = O.quantize_kra(bits, S, imp)
    assert np.array_equal(Q, K)
    assert np.array_equal(r, (R / 2).astype(np.float32))
    assert np.array_equal(c, (2 * C).astype(np.float32))
    assert np.array_equal(O.dequantize(Q, r, c), S)


def test_kra_row_factor_square_root_law():
    """r_i = sqrt(mu_i / imp_i): scaling one row's impact by 4 halves its row
    factor exactly, scaling one row of S by 4 doubles it, other rows keep
    theirs, and the codes of the untouched rows' pattern stay valid."""
    rng = np.random.default_rng(7)
    S = _rand_state(rng, 10, 9)
    imp = rng.uniform(0.2, 3.0, 10).astype(np.float32)
    _, r, _ = O.quantize_kra(6, S, imp)
    imp2 = imp.copy()
    imp2[3] *= 4
    _, r2, _ = O.quantize_kra(6, S, imp2)
    assert r2[3] == r[3] / 2 and np.array_equal(np.delete(r2, 3), np.delete(r, 3))
    S2 = S.copy()
    S2[5] *= 4
    _, r3, _ = O.quantize_kra(6, S2, imp)
    assert r3[5] == 2 * r[5] and np.array_equal(np.delete(r3, 5), np.delete(r, 5))
    mu = np.abs(S).max(axis=1)
    assert np.allclose(r, np.sqrt(mu.astype(np.float64) / imp), rtol=2e-7)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_kra_scale_invariance(bits):
    """S -> 4 S doubles r and c; imp -> 4 imp halves r and doubles c; the codes
    never change (both are exact power-of-two rescalings of every step)."""
    rng = np.random.default_rng(9 + bits)
    S = _rand_state(rng, 24, 20)
    imp = rng.uniform(0.1, 5.0, 24).astype(np.float32)
    Q, r, c = O.quantize_kra(bits, S, imp)
    Q2, r2, c2 = O.quantize_kra(bits, 4 * S, imp)
    assert np.array_equal(Q2, Q) and np.array_equal(r2, 2 * r) and np.array_equal(c2, 2 * c)
    Q3, r3, c3 = O.quantize_kra(bits, S, 4 * imp)
    assert np.array_equal(Q3, Q) and np.array_equal(r3, r / 2) and np.array_equal(c3, 2 * c)
    Q4, r4, c4 = O.quantize_kra(bits, -S, imp)
    assert np.array_equal(Q4, -Q) and np.array_equal(r4, r) and np.array_equal(c4, c)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_kra_fit_properties(bits):
    """Against the range-covering codes P (c0_j = max_i |S_ij / r_i| / qmax,
    P = nearest level): (1) the fitted c_j minimises the impact-weighted
    error of P (perturbing c_j either way by 1e-3 increases it); (2) the
    final codes are each the nearest level in [-qmax, qmax] to S_ij / (r_i
    c_j) (brute force over all levels); (3) the weighted error of the final
    codes is never above that of (c0, P)."""
    rng = np.random.default_rng(20 + bits)
    dk, dv, q = 32, 24, O.qmax(bits)
    S = _rand_state(rng, dk, dv)
    S[rng.integers(0, dk, 5), rng.integers(0, dv, 5)] *= 30      # isolated outliers
    imp = np.exp(rng.normal(0, 1.5, dk)).astype(np.float32)
    Q, r, c = O.quantize_kra(bits, S, imp)
    Sd = S.astype(np.float64)
    x = Sd / r.astype(np.float64)[:, None]
    c0 = np.abs(x).max(axis=0) / q
    P = np.rint(x / c0[None, :])
    w = imp.astype(np.float64) * r.astype(np.float64) ** 2

    def err_s(cc, codes):
        return (w[:, None] * (x - cc[None, :] * codes) ** 2).sum(axis=0)

    base = err_s(c.astype(np.float64), P)
    assert (err_s(c * (1 + 1e-3), P) > base).all()
    assert (err_s(c * (1 - 1e-3), P) > base).all()
    levels = np.arange(-q, q + 1, dtype=np.float64)
    t = x / c.astype(np.float64)[None, :]
    best = levels[np.abs(t[..., None] - levels).argmin(axis=-1)]
    assert np.array_equal(Q, best)
    assert (_weighted_err(S, imp, Q, r, c) <= _weighted_err(S, imp, P, r, c0) * (1 + 1e-9)).all()
    # fitting pays off somewhere: some columns shrink below the covering scale
    assert (c < c0 * (1 - 1e-6)).any()


def test_kra_high_impact_rows_get_finer_steps():
    """Two copies of the same row, impacts 1 and 100: the high-impact copy
    gets a 10x smaller row factor and a smaller reconstruction error."""
    rng = np.random.default_rng(31)
    S = _rand_state(rng, 8, 64)
    S[4] = S[0]
    imp = np.ones(8, np.float32)
    imp[4] = 100.0
    Q, r, c = O.quantize_kra(4, S, imp)
    assert math.isclose(r[0] / r[4], 10.0, rel_tol=1e-6)
    R = O.dequantize(Q, r, c).astype(np.float64)
    e0 = ((R[0] - S[0]) ** 2).sum()
    e4 = ((R[4] - S[4]) ** 2).sum()
    assert e4 < e0 / 4


def test_kra_zero_rows_columns_and_state():
    rng = np.random.default_rng(41)
    S = _rand_state(rng, 6, 5)
    S[2, :] = 0.0
    S[:, 3] = 0.0
    imp = rng.uniform(0.5, 2, 6).astype(np.float32)
    Q, r, c = O.quantize_kra(6, S, imp)
    assert r[2] == 0 and (Q[2] == 0).all() and c[3] == 0 and (Q[:, 3] == 0).all()
    assert np.isfinite(O.dequantize(Q, r, c)).all()
    Q, r, c = O.quantize_kra(8, np.zeros((4, 4), np.float32), np.ones(4, np.float32))
    assert (Q == 0).all() and (r == 0).all() and (c == 0).all()


def test_kra_drivers_and_step_compose():
    """records_quantize / records_step with per-record impacts equal the
    single-head fit, and the quantized step with impacts is the step update
    on the codes, then the key-row-aware fit."""
    rng = np.random.default_rng(51)
    d, bits = 16, [4, 6, 8]
    S = np.stack([_rand_state(rng, d, d) for _ in bits])
    imp = rng.uniform(0.1, 4, (3, d)).astype(np.float32)
    sizes = [O.record_bytes(b, d, d) for b in bits]
    offs = np.array([0, sizes[0], sizes[0] + sizes[1]], np.int64)
    base = np.zeros(sum(sizes), np.uint8)
    b8 = np.array(bits, np.uint8)
    O.records_quantize(base, offs, b8, S, d, d, imp)
    for i, b in enumerate(bits):
        Q, r, c = O.quantize_kra(b, S[i], imp[i])
        assert np.array_equal(base[offs[i]:offs[i] + sizes[i]], O.record_pack(b, Q, r, c))
    x = [_inputs(rng, d, d, kda=True) for _ in bits]
    q = np.stack([t[0] for t in x]).astype(np.float32)
    k = np.stack([t[1] for t in x]).astype(np.float32)
    v = np.stack([t[2] for t in x]).astype(np.float32)
    beta = np.array([t[3] for t in x], np.float32)
    g = np.log(np.stack([t[4] for t in x])).astype(np.float32)
    before = base.copy()
    y = O.records_step(True, base, offs, b8, d, d, q, k, v, beta, g, imp)
    for i, b in enumerate(bits):
        Q, r, c = O.record_unpack(b, d, d, before[offs[i]:offs[i] + sizes[i]])
        alpha = np.exp(g[i].astype(np.float64)).astype(np.float32)
        Sp, yw = O.step_update(Q, r, c, alpha, q[i], k[i], v[i], beta[i])
        Q2, r2, c2 = O.quantize_kra(b, Sp, imp[i])
        assert np.array_equal(base[offs[i]:offs[i] + sizes[i]], O.record_pack(b, Q2, r2, c2))
        assert np.array_equal(y[i], yw)


# ------------------------------------------------------------------ key-row-aware fit, per-row widths
def _width_pattern(rng, dk):
    w = np.array([4] * (dk // 4) + [6] * (dk // 2) + [8] * (dk - dk // 4 - dk // 2), np.uint8)
    return w[rng.permutation(dk)]


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_kra_rows_uniform_widths_is_the_uniform_fit(bits):
    """Every row at the same width: the per-row fit returns the uniform fit's
    codes and scales bit for bit (the widening factors are 1 and the clamp of
    the range-covering codes never acts)."""
    rng = np.random.default_rng(110 + bits)
    S = _rand_state(rng, 32, 24)
    S[rng.integers(0, 32, 4), rng.integers(0, 24, 4)] *= 40
    imp = np.exp(rng.normal(0, 1.5, 32)).astype(np.float32)
    a = O.quantize_kra(bits, S, imp)
    b = O.quantize_kra_rows(np.full(32, bits, np.uint8), S, imp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_kra_rows_each_row_spans_its_own_levels():
    """Rows of comparable magnitude and impact at widths 4, 6 and 8: each
    row's codes stay within its own range and reach close to its own qmax
    (a fit that ignored the widths in the row factors would leave the 8-bit
    rows on the 4-bit rows' coarse grid, or push 4-bit codes out of range)."""
    rng = np.random.default_rng(121)
    dk, dv = 48, 64
    S = rng.standard_normal((dk, dv)).astype(np.float32)
    imp = rng.uniform(0.8, 1.25, dk).astype(np.float32)
    rb = _width_pattern(rng, dk)
    Q, r, c = O.quantize_kra_rows(rb, S, imp)
    qm = np.array([O.qmax(int(b)) for b in rb])
    top = np.abs(Q).max(axis=1)
    assert (top <= qm).all()
    assert (top >= 0.6 * qm).all(), (top, qm)


def test_kra_rows_duplicate_row_error_falls_with_width():
    """The same row stored at 4, 6 and 8 bits (equal impact): the wider copy
    reconstructs it with a smaller error, by roughly the ratio of the level
    counts."""
    rng = np.random.default_rng(131)
    dk, dv = 24, 96
    S = _rand_state(rng, dk, dv)
    S[8] = S[0]
    S[16] = S[0]
    rb = np.array([4] * 8 + [6] * 8 + [8] * 8, np.uint8)
    imp = np.ones(dk, np.float32)
    Q, r, c = O.quantize_kra_rows(rb, S, imp)
    R = O.dequantize(Q, r, c).astype(np.float64)
    e = [((R[i] - S[i]) ** 2).sum() for i in (0, 8, 16)]
    assert e[1] < e[0] / 4 and e[2] < e[1] / 4, e


def test_kra_rows_fit_properties():
    """Per-row level sets: (1) every code is the nearest level in
    [-qmax_i, qmax_i] to S_ij / (r_i c_j) (brute force over each row's
    levels); (2) against the range-covering codes P of the reading (c0_j =
    max_i |x_ij| g_i / qref with x = S / r, P clamped to each row's range),
    the fitted c_j minimises the impact-weighted error of P (a 1e-3
    perturbation either way increases it); (3) the final weighted error is
    never above that of (c0, P)."""
    rng = np.random.default_rng(141)
    dk, dv = 40, 24
    S = _rand_state(rng, dk, dv)
    S[rng.integers(0, dk, 5), rng.integers(0, dv, 5)] *= 30
    imp = np.exp(rng.normal(0, 1.5, dk)).astype(np.float32)
    rb = _width_pattern(rng, dk)
    Q, r, c = O.quantize_kra_rows(rb, S, imp)
    qm = np.array([O.qmax(int(b)) for b in rb], np.float64)
    Sd = S.astype(np.float64)
    x = Sd / r.astype(np.float64)[:, None]
    t = x / c.astype(np.float64)[None, :]
    for i in range(dk):
        levels = np.arange(-qm[i], qm[i] + 1)
        best = levels[np.abs(t[i][:, None] - levels).argmin(axis=-1)]
        assert np.array_equal(Q[i], best), i
    g = qm.max() / qm
    c0 = (np.abs(x) * g[:, None]).max(axis=0) / qm.max()
    P = np.clip(np.rint(x / c0[None, :]), -qm[:, None], qm[:, None])
    w = imp.astype(np.float64) * r.astype(np.float64) ** 2

    def err_s(cc, codes):
        return (w[:, None] * (x - cc[None, :] * codes) ** 2).sum(axis=0)

    base = err_s(c.astype(np.float64), P)
    assert (err_s(c * (1 + 1e-3), P) > base).all()
    assert (err_s(c * (1 - 1e-3), P) > base).all()
    assert (_weighted_err(S, imp, Q, r, c) <= _weighted_err(S, imp, P, r, c0) * (1 + 1e-9)).all()


def test_kra_rows_scale_and_permutation_invariance():
    """S -> 4 S doubles r and c, imp -> 4 imp halves r and doubles c, with the
    codes unchanged; permuting the key rows together with their widths and
    impacts permutes the codes and row factors and keeps the column scales."""
    rng = np.random.default_rng(151)
    dk, dv = 32, 20
    S = _rand_state(rng, dk, dv)
    imp = rng.uniform(0.1, 5.0, dk).astype(np.float32)
    rb = _width_pattern(rng, dk)
    Q, r, c = O.quantize_kra_rows(rb, S, imp)
    Q2, r2, c2 = O.quantize_kra_rows(rb, 4 * S, imp)
    assert np.array_equal(Q2, Q) and np.array_equal(r2, 2 * r) and np.array_equal(c2, 2 * c)
    Q3, r3, c3 = O.quantize_kra_rows(rb, S, 4 * imp)
    assert np.array_equal(Q3, Q) and np.array_equal(r3, r / 2) and np.array_equal(c3, 2 * c)
    p = rng.permutation(dk)
    Q4, r4, c4 = O.quantize_kra_rows(rb[p], S[p], imp[p])
    assert np.array_equal(Q4, Q[p]) and np.array_equal(r4, r[p])
    assert np.allclose(c4, c, rtol=1e-6)


def test_kra_rows_zero_rows_and_columns():
    rng = np.random.default_rng(161)
    S = _rand_state(rng, 8, 6)
    S[3, :] = 0.0
    S[:, 2] = 0.0
    rb = np.array([4, 4, 6, 6, 6, 8, 8, 8], np.uint8)
    Q, r, c = O.quantize_kra_rows(rb, S, rng.uniform(0.5, 2, 8).astype(np.float32))
    assert r[3] == 0 and (Q[3] == 0).all() and c[2] == 0 and (Q[:, 2] == 0).all()
    assert np.isfinite(O.dequantize(Q, r, c)).all()


def test_kra_rows_drivers_and_step_compose():
    """records_quantize / records_step on records with per-row widths and
    impacts equal the single-head per-row fit and its packing; the step is
    the step update on the codes, then that fit."""
    rng = np.random.default_rng(171)
    d = 16
    rbs = np.stack([_width_pattern(rng, d) for _ in range(2)])
    S = np.stack([_rand_state(rng, d, d) for _ in range(2)])
    imp = rng.uniform(0.1, 4, (2, d)).astype(np.float32)
    sizes = [O.record_bytes_rows(rbs[i], d) for i in range(2)]
    offs = np.array([0, sizes[0]], np.int64)
    base = np.zeros(sum(sizes), np.uint8)
    b0 = np.zeros(2, np.uint8)
    O.records_quantize(base, offs, b0, S, d, d, imp, rbs)
    for i in range(2):
        Q, r, c = O.quantize_kra_rows(rbs[i], S[i], imp[i])
        assert np.array_equal(base[offs[i]:offs[i] + sizes[i]], O.record_pack_rows(rbs[i], Q, r, c))
    x = [_inputs(rng, d, d, kda=True) for _ in range(2)]
    q = np.stack([t[0] for t in x]).astype(np.float32)
    k = np.stack([t[1] for t in x]).astype(np.float32)
    v = np.stack([t[2] for t in x]).astype(np.float32)
    beta = np.array([t[3] for t in x], np.float32)
    g = np.log(np.stack([t[4] for t in x])).astype(np.float32)
    before = base.copy()
    y = O.records_step(True, base, offs, b0, d, d, q, k, v, beta, g, imp, rbs)
    for i in range(2):
        Q, r, c = O.record_unpack_rows(rbs[i], d, before[offs[i]:offs[i] + sizes[i]])
        alpha = np.exp(g[i].astype(np.float64)).astype(np.float32)
        Sp, yw = O.step_update(Q, r, c, alpha, q[i], k[i], v[i], beta[i])
        Q2, r2, c2 = O.quantize_kra_rows(rbs[i], Sp, imp[i])
        assert np.array_equal(base[offs[i]:offs[i] + sizes[i]], O.record_pack_rows(rbs[i], Q2, r2, c2))
        assert np.array_equal(y[i], yw)


# ------------------------------------------------------------------ per-key-row widths
def test_rows_quantizer_selects_rows_of_uniform_quantizers():
    """With a width per key row, the column scales do not depend on the
    widths and row i only on its own width: codes and r_i of row i equal
    those of the uniform quantizer at width w_i (a transposed or shifted
    width index fails this)."""
    rng = np.random.default_rng(61)
    dk, dv = 24, 20
    S = _rand_state(rng, dk, dv)
    w = rng.choice([4, 6, 8], dk).astype(np.uint8)
    Q, r, c = O.quantize_rows(w, S)
    for b in (4, 6, 8):
        Qb, rb, cb = O.quantize(b, S)
        assert np.array_equal(c, cb)
        sel = w == b
        assert np.array_equal(Q[sel], Qb[sel]) and np.array_equal(r[sel], rb[sel])
    Qu, ru, cu = O.quantize_rows(np.full(dk, 6, np.uint8), S)
    Q6, r6, c6 = O.quantize(6, S)
    assert np.array_equal(Qu, Q6) and np.array_equal(ru, r6) and np.array_equal(cu, c6)


def test_rows_record_layout_and_roundtrip():
    rng = np.random.default_rng(62)
    dk, dv = 16, 32
    w = np.sort(rng.choice([4, 6, 8], dk)).astype(np.uint8)
    S = _rand_state(rng, dk, dv)
    Q, r, c = O.quantize_rows(w, S)
    rec = O.record_pack_rows(w, Q, r, c)
    assert rec.size == sum(dv * int(b) // 8 for b in w) + 4 * (dk + dv)
    # the rows' streams back to back, each in the uniform row format
    pos = 0
    for i, b in enumerate(w):
        n = dv * int(b) // 8
        assert np.array_equal(rec[pos:pos + n], O.pack_row(int(b), Q[i]))
        pos += n
    assert np.array_equal(rec[pos:pos + 4 * dk].view(np.float32), r)
    Q2, r2, c2 = O.record_unpack_rows(w, dv, rec)
    assert np.array_equal(Q2, Q) and np.array_equal(r2, r) and np.array_equal(c2, c)


def test_rows_drivers_and_step_compose():
    """Records with bits 0 take their key-row widths from row_bits; one step
    is the step update on the codes, then the per-row quantizer."""
    rng = np.random.default_rng(63)
    d = 16
    widths = [np.sort(rng.choice([4, 6, 8], d)).astype(np.uint8) for _ in range(3)]
    bits = np.array([0, 6, 0], np.uint8)
    row_bits = np.stack([widths[0], np.full(d, 6, np.uint8), widths[2]])
    S = np.stack([_rand_state(rng, d, d) for _ in range(3)])
    sizes = [O.record_bytes_rows(row_bits[i], d) for i in range(3)]
    assert sizes[1] == O.record_bytes(6, d, d)
    offs = np.array([0, sizes[0], sizes[0] + sizes[1]], np.int64)
    base = np.zeros(sum(sizes), np.uint8)
    O.records_quantize(base, offs, bits, S, d, d, row_bits=row_bits)
    for i in range(3):
        Q, r, c = O.quantize_rows(row_bits[i], S[i])
        assert np.array_equal(base[offs[i]:offs[i] + sizes[i]], O.record_pack_rows(row_bits[i], Q, r, c))
    back = O.records_dequantize(base, offs, bits, d, d, row_bits=row_bits)
    for i in range(3):
        assert np.array_equal(back[i], O.dequantize(*O.quantize_rows(row_bits[i], S[i])))
    x = [_inputs(rng, d, d, kda=True) for _ in range(3)]
    q = np.stack([t[0] for t in x]).astype(np.float32)
    k = np.stack([t[1] for t in x]).astype(np.float32)
    v = np.stack([t[2] for t in x]).astype(np.float32)
    beta = np.array([t[3] for t in x], np.float32)
    g = np.log(np.stack([t[4] for t in x])).astype(np.float32)
    before = base.copy()
    y = O.records_step(True, base, offs, bits, d, d, q, k, v, beta, g, row_bits=row_bits)
    for i in range(3):
        Q, r, c = O.record_unpack_rows(row_bits[i], d, before[offs[i]:offs[i] + sizes[i]])
        alpha = np.exp(g[i].astype(np.float64)).astype(np.float32)
        Sp, yw = O.step_update(Q, r, c, alpha, q[i], k[i], v[i], beta[i])
        Q2, r2, c2 = O.quantize_rows(row_bits[i], Sp)
        assert np.array_equal(base[offs[i]:offs[i] + sizes[i]],
                              O.record_pack_rows(row_bits[i], Q2, r2, c2))
        assert np.array_equal(y[i], yw)
    with pytest.raises(ValueError):   # bits 0 needs row widths
        O.records_quantize(base, offs, bits, S, d, d)
