/*
 * sq_oracle.c -- CPU oracle for the quantized gated Delta-rule decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the HIP
 * path is checked against.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header or table with the HIP library.
 *
 * Sources (the pages on STEPQuant, arXiv 2609.38169):
 *  - "Paper Explained: STEPQuant" (ta-paperlens), section "The mechanism:
 *    rewriting state with the delta rule" (paper section 2.1): per head a
 *    d_k x d_v state; fade it with the retention gate D_t, look up what k_t
 *    retrieves, write only the difference to v_t with strength beta_t, read
 *    the output with q_t.  GDN: one scalar gate per head; KDA: one gate per
 *    key channel.  The equation itself is missing from the page; the
 *    reading used here is
 *        S_t = (I - beta k k^T) D_t S_{t-1} + beta k v^T,   y_t = S_t^T q_t,
 *    evaluated in the order the words give it (decay, look-up, delta write,
 *    read-out).
 *  - hyper.ai summary, "Method" paragraph 1: the reconstructed state is
 *    updated in floating point and the output computed, then the updated
 *    state is quantized for storage (symmetric uniform quantization).
 *  - hyper.ai summary, "Method" paragraph 4: the state is stored as row
 *    factors x column factors x low-bit integers, each scaled entry going to
 *    the nearest level.  The closed scale rule used here (the impact-weighted
 *    fit has no formula on the pages) is: c_j = max_i |S_ij|, then
 *    r_i = max_j |S_ij / c_j| / qmax.
 *
 * Precision (the pages fix none beyond "floating point"): the step's
 * reductions (what k retrieves) run in FP64 and are rounded once to fp32;
 * the element-wise rank-1 update runs in fp32 in the order stated at
 * sqo_step_update; the quantizer's fp32 order is fixed at sqo_quantize.
 * Build with -ffp-contract=off and without fast-math so that every fp32
 * operation is one correctly rounded IEEE operation.
 *
 * Also here: FP16 pivot records (bits 16), per-key-row widths (records
 * with head width 0) and the key-row-aware dual-axis fit (sqo_quantize_kra).
 *
 * Parity pins: see the oracle tests.  Every function below is pinned by at
 * least one closed form, identity, brute-force or convergence check.  The
 * key-row-aware fit is pinned to the reading written out above it (exact
 * constructed case, square-root law, scale invariance, least-squares
 * optimality, nearest levels); the pages give no formula for it, so against
 * the pages themselves it is parity unpinned.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Storage format of one (slot, head) record                          */
/* ------------------------------------------------------------------ */
/*
 * record = codes[d_k rows][packed d_v codes] | r[d_k] fp32 | c[d_v] fp32
 * Codes are b-bit two's complement integers in [-qmax, qmax],
 * qmax = 2^(b-1) - 1.  Each row is a little-endian bit stream: code j of
 * the row occupies bits [b*j, b*j + b) of the row's bytes.  So
 *   8-bit: byte j is code j;
 *   4-bit: byte n holds code 2n (low nibble) and code 2n+1 (high nibble);
 *   6-bit: bytes 3n..3n+2 hold codes 4n..4n+3 at bits 0, 6, 12, 18 of the
 *          24-bit little-endian word they form.
 */

int sqo_qmax(int bits) { return (1 << (bits - 1)) - 1; }

int64_t sqo_row_bytes(int bits, int dv) { return ((int64_t)dv * bits + 7) / 8; }

/* bits = 16 marks an FP16 pivot record (hyper.ai "Method" paragraph 2: the
 * highest-risk units are kept in FP16 as sparse pivots): the state itself as
 * IEEE binary16, row-major, no scales. */
int64_t sqo_record_bytes(int bits, int dk, int dv) {
    if (bits == 16) return 2 * (int64_t)dk * dv;
    return (int64_t)dk * sqo_row_bytes(bits, dv) + 4 * (int64_t)dk + 4 * (int64_t)dv;
}

/* A record whose key rows have their own widths (in {4, 6, 8}): the rows'
 * code streams back to back, then r[d_k], c[d_v]. */
int64_t sqo_record_bytes_rows(const uint8_t *row_bits, int dk, int dv) {
    int64_t n = 4 * (int64_t)dk + 4 * (int64_t)dv;
    for (int i = 0; i < dk; ++i) n += sqo_row_bytes(row_bits[i], dv);
    return n;
}

/* ------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, from the format's definition             */
/* ------------------------------------------------------------------ */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
 * exponent 0 holds zero and subnormals (fraction * 2^-24), 31 inf / NaN. */
float sqo_f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const int e = (h >> 10) & 31, f = h & 1023;
    float mag;
    if (e == 0)
        mag = ldexpf((float)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + f), e - 25);
    uint32_t u;
    memcpy(&u, &mag, 4);
    u |= sign;
    memcpy(&mag, &u, 4);
    return mag;
}

/* Round a float to the nearest binary16, ties to even (overflow to inf). */
uint16_t sqo_f32_to_f16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7E00u;          /* NaN */
    /* exact rational value |x| = m * 2^(e - 150) */
    const int e = (int)(a >> 23);
    const uint32_t m = e ? ((a & 0x7FFFFFu) | 0x800000u) : (a & 0x7FFFFFu);
    const int ee = e ? e : 1;
    /* target spacing: 2^(E - 25) for a normal half of biased exponent E
     * (value in [2^(E-15), 2^(E-14))), 2^-24 for subnormals */
    int E = ee - 127 + 15;                               /* half biased exponent */
    if (e == 0 || E < 1) E = 1;                          /* subnormal spacing 2^-24 */
    const int shift = (E - 25) - (ee - 150);             /* m * 2^-shift in half units */
    uint32_t q;
    if (shift <= 0) {
        q = m << (-shift);
    } else if (shift > 31) {
        q = 0;
    } else {
        q = m >> shift;
        const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) ++q;
    }
    /* q counts units of 2^(E - 25); q in [1024, 2048] for normals at E */
    uint32_t bitsv;
    if (E == 1 && q < 1024) {
        bitsv = q;                                       /* subnormal (or zero) */
    } else {
        int EE = E;
        if (q >= 2048) {                                 /* rounding carried */
            q >>= 1;
            ++EE;
        }
        if (EE >= 31) return sign | 0x7C00u;             /* overflow */
        bitsv = ((uint32_t)EE << 10) | (q - 1024);
    }
    return sign | (uint16_t)bitsv;
}

/* Pack n codes of one row.  Returns 0, or -1 if a code is out of range. */
int sqo_pack_row(int bits, int n, const int32_t *codes, uint8_t *out) {
    const int64_t nbytes = sqo_row_bytes(bits, n);
    const int32_t q = sqo_qmax(bits);
    memset(out, 0, (size_t)nbytes);
    for (int j = 0; j < n; ++j) {
        if (codes[j] < -q || codes[j] > q) return -1;
        const uint32_t field = (uint32_t)codes[j] & ((1u << bits) - 1u);
        for (int t = 0; t < bits; ++t) {
            const int64_t bit = (int64_t)j * bits + t;
            if (field >> t & 1u) out[bit >> 3] |= (uint8_t)(1u << (bit & 7));
        }
    }
    return 0;
}

/* Unpack n codes of one row (sign-extending each b-bit field). */
void sqo_unpack_row(int bits, int n, const uint8_t *in, int32_t *codes) {
    for (int j = 0; j < n; ++j) {
        uint32_t field = 0;
        for (int t = 0; t < bits; ++t) {
            const int64_t bit = (int64_t)j * bits + t;
            field |= (uint32_t)(in[bit >> 3] >> (bit & 7) & 1u) << t;
        }
        int32_t v = (int32_t)field;
        if (field >> (bits - 1) & 1u) v -= (int32_t)(1u << bits);
        codes[j] = v;
    }
}

/* ------------------------------------------------------------------ */
/* Pinned fp32 quantizer and dequantizer                               */
/* ------------------------------------------------------------------ */
/*
 * Dual-axis symmetric round-to-nearest quantizer (hyper.ai "Method" para 4,
 * closed scale rule).  All in fp32, one rounding per operation:
 *   c_j  = max_i |S_ij|
 *   ic_j = c_j >= FLT_MIN ? 1/c_j : 0        (else c_j stored as 0)
 *   s_ij = S_ij * ic_j                       (rounded to fp32)
 *   m_i  = max_j |s_ij|
 *   r_i  = m_i / qmax
 *   ir_i = r_i >= FLT_MIN ? 1/r_i : 0        (else r_i stored as 0)
 *   Q_ij = clamp(round_half_even(s_ij * ir_i), -qmax, qmax)
 * The last product is taken exactly (in FP64, where the product of two fp32
 * values is exact), so each code is the level nearest to the scaled entry
 * s_ij / r_i.
 * Per-key-row widths (blog.ontle.kr, allocation paragraph: for KDA the unit
 * of the bit allocation is a single key row): row i uses its own qmax_i in
 * r_i = m_i / qmax_i; the column scales do not depend on the widths, so each
 * row's codes and r_i equal those of a uniform quantization of the same
 * state at that row's width.  sqo_quantize is the all-rows-equal case.
 */
void sqo_quantize_rows(const uint8_t *row_bits, int dk, int dv, const float *S, int32_t *Q,
                       float *r, float *c) {
    float *ic = (float *)malloc(sizeof(float) * (size_t)dv);
    for (int j = 0; j < dv; ++j) {
        float m = 0.0f;
        for (int i = 0; i < dk; ++i) {
            const float a = fabsf(S[(size_t)i * dv + j]);
            if (a > m) m = a;
        }
        if (m >= FLT_MIN) {
            c[j] = m;
            ic[j] = 1.0f / m;
        } else {
            c[j] = 0.0f;
            ic[j] = 0.0f;
        }
    }
    for (int i = 0; i < dk; ++i) {
        const float qmax = (float)sqo_qmax(row_bits[i]);
        float m = 0.0f;
        for (int j = 0; j < dv; ++j) {
            const float t = fabsf(S[(size_t)i * dv + j]) * ic[j];
            if (t > m) m = t;
        }
        float ri = m / qmax;
        float iri;
        if (ri >= FLT_MIN) {
            iri = 1.0f / ri;
        } else {
            ri = 0.0f;
            iri = 0.0f;
        }
        r[i] = ri;
        for (int j = 0; j < dv; ++j) {
            const float s = S[(size_t)i * dv + j] * ic[j];
            const double x = (double)s * (double)iri; /* exact */
            double qv = nearbyint(x); /* default rounding mode: half to even */
            if (qv > qmax) qv = qmax;
            if (qv < -qmax) qv = -qmax;
            Q[(size_t)i * dv + j] = (int32_t)qv;
        }
    }
    free(ic);
}

void sqo_quantize(int bits, int dk, int dv, const float *S, int32_t *Q, float *r, float *c) {
    uint8_t *rb = (uint8_t *)malloc((size_t)dk);
    memset(rb, bits, (size_t)dk);
    sqo_quantize_rows(rb, dk, dv, S, Q, r, c);
    free(rb);
}

/*
 * Key-row-aware dual-axis fit (hyper.ai summary, "Method", the Key-Row-Aware
 * Dual-Axis Fitting paragraph; blog.ontle.kr, the paragraph on what is fixed
 * offline).  Each key row i has a row-impact score imp_i > 0, calibrated
 * offline.  The row factor weighs the row's current magnitude against its
 * impact with a square root, so large rows get a wider range and high-impact
 * rows finer steps.  Given the row factors, each column scale is fitted to
 * the impact-weighted reconstruction error, and every scaled entry goes to
 * its nearest level.  The pages give no formulas; the reading used here, in
 * fp32 with one rounding per operation unless FP64 is named:
 *   mu_i  = max_j |S_ij|                         (row magnitude)
 *   r_i   = sqrt(mu_i / imp_i)                   (0 if mu_i < FLT_MIN, or if
 *                                                 r_i is not finite or < FLT_MIN)
 *   ir_i  = r_i > 0 ? 1/r_i : 0
 *   s_ij  = S_ij * ir_i                          (the row-scaled entry)
 *   c0_j  = max_i |s_ij| / qmax                  (the range-covering scale;
 *   ic0_j = c0_j >= FLT_MIN ? 1/c0_j : 0          else c0_j := 0)
 *   P_ij  = round_half_even(s_ij * ic0_j)        (exact product)
 *   w_i   = imp_i * r_i * r_i                    (FP64, exact: the weight of
 *           an s-domain error, since S_ij - r_i c Q = r_i (s_ij - c Q))
 *   A_j   = sum_i w_i s_ij P_ij,  B_j = sum_i w_i P_ij^2          (FP64)
 *   c_j   = B_j > 0 ? (float)(A_j / B_j) : c0_j  (the least-squares scale
 *           for the codes P; 0 if below FLT_MIN)
 *   ic_j  = c_j > 0 ? 1/c_j : 0
 *   Q_ij  = clamp(round_half_even(s_ij * ic_j), -qmax, qmax)  (exact product)
 * With codes P fixed, c_j minimises sum_i imp_i (S_ij - r_i c Q_ij)^2 in the
 * s-domain; the final codes are then the nearest levels for c_j, so the
 * weighted error never exceeds that of the range-covering scale c0_j.
 * One refinement step, not an iteration to convergence.
 */
void sqo_quantize_kra(int bits, int dk, int dv, const float *S, const float *imp, int32_t *Q,
                      float *r, float *c) {
    const float qmax = (float)sqo_qmax(bits);
    float *ir = (float *)malloc(sizeof(float) * (size_t)dk);
    float *sc = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    for (int i = 0; i < dk; ++i) {
        float mu = 0.0f;
        for (int j = 0; j < dv; ++j) {
            const float a = fabsf(S[(size_t)i * dv + j]);
            if (a > mu) mu = a;
        }
        float ri = 0.0f;
        if (mu >= FLT_MIN) ri = sqrtf(mu / imp[i]);
        if (!(ri >= FLT_MIN) || isinf(ri)) ri = 0.0f;
        r[i] = ri;
        ir[i] = ri > 0.0f ? 1.0f / ri : 0.0f;
        for (int j = 0; j < dv; ++j) sc[(size_t)i * dv + j] = S[(size_t)i * dv + j] * ir[i];
    }
    for (int j = 0; j < dv; ++j) {
        float m = 0.0f;
        for (int i = 0; i < dk; ++i) {
            const float a = fabsf(sc[(size_t)i * dv + j]);
            if (a > m) m = a;
        }
        float c0 = m / qmax, ic0 = 0.0f;
        if (c0 >= FLT_MIN)
            ic0 = 1.0f / c0;
        else
            c0 = 0.0f;
        double A = 0.0, B = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double sv = (double)sc[(size_t)i * dv + j];
            const double P = nearbyint(sv * (double)ic0);
            const double w = (double)imp[i] * (double)r[i] * (double)r[i];
            A += w * sv * P;
            B += w * P * P;
        }
        float cj = B > 0.0 ? (float)(A / B) : c0;
        if (!(cj >= FLT_MIN)) cj = 0.0f;
        const float icj = cj > 0.0f ? 1.0f / cj : 0.0f;
        c[j] = cj;
        for (int i = 0; i < dk; ++i) {
            double qv = nearbyint((double)sc[(size_t)i * dv + j] * (double)icj);
            if (qv > qmax) qv = qmax;
            if (qv < -qmax) qv = -qmax;
            Q[(size_t)i * dv + j] = (int32_t)qv;
        }
    }
    free(ir);
    free(sc);
}

/*
 * The key-row-aware fit on a head whose key rows have their own widths
 * (blog.ontle.kr, allocation paragraph: for KDA a single key row is the unit
 * of the bit allocation; the fit as in sqo_quantize_kra).  Row i takes the
 * levels -qmax_i .. qmax_i of its width; qref = max_i qmax_i (the head's
 * widest rows).  Each row's factor is widened by g_i = qref / qmax_i, as the
 * closed rule divides a row's range by its own qmax_i, so that every row
 * spans its own levels on the shared column grid:
 *   g_i   = qref / qmax_i                        (fp32; 1 for the widest rows)
 *   r_i   = sqrt(mu_i / imp_i) * g_i             (0 under the rules above)
 *   s_ij  = S_ij * ir_i
 *   c0_j  = max_i (|s_ij| * g_i) / qref          (covers every row's range)
 *   P_ij  = clamp(round_half_even(s_ij * ic0_j), -qmax_i, qmax_i)
 *   A_j, B_j, c_j as in sqo_quantize_kra
 *   Q_ij  = clamp(round_half_even(s_ij * ic_j), -qmax_i, qmax_i)
 * With all widths equal, g_i = 1 and every step is that of sqo_quantize_kra
 * (the clamp of P never acts there).  The argument that the weighted error
 * never exceeds that of (c0, P) holds row by row with each row's own range.
 */
void sqo_quantize_kra_rows(const uint8_t *row_bits, int dk, int dv, const float *S,
                           const float *imp, int32_t *Q, float *r, float *c) {
    float *qm = (float *)malloc(sizeof(float) * (size_t)dk);
    float *gi = (float *)malloc(sizeof(float) * (size_t)dk);
    float *ir = (float *)malloc(sizeof(float) * (size_t)dk);
    float *sc = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    float qref = 0.0f;
    for (int i = 0; i < dk; ++i) {
        qm[i] = (float)sqo_qmax(row_bits[i]);
        if (qm[i] > qref) qref = qm[i];
    }
    for (int i = 0; i < dk; ++i) {
        gi[i] = qref / qm[i];
        float mu = 0.0f;
        for (int j = 0; j < dv; ++j) {
            const float a = fabsf(S[(size_t)i * dv + j]);
            if (a > mu) mu = a;
        }
        float ri = 0.0f;
        if (mu >= FLT_MIN) ri = sqrtf(mu / imp[i]) * gi[i];
        if (!(ri >= FLT_MIN) || isinf(ri)) ri = 0.0f;
        r[i] = ri;
        ir[i] = ri > 0.0f ? 1.0f / ri : 0.0f;
        for (int j = 0; j < dv; ++j) sc[(size_t)i * dv + j] = S[(size_t)i * dv + j] * ir[i];
    }
    for (int j = 0; j < dv; ++j) {
        float m = 0.0f;
        for (int i = 0; i < dk; ++i) {
            const float a = fabsf(sc[(size_t)i * dv + j]) * gi[i];
            if (a > m) m = a;
        }
        float c0 = m / qref, ic0 = 0.0f;
        if (c0 >= FLT_MIN)
            ic0 = 1.0f / c0;
        else
            c0 = 0.0f;
        double A = 0.0, B = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double sv = (double)sc[(size_t)i * dv + j];
            double P = nearbyint(sv * (double)ic0);
            if (P > qm[i]) P = qm[i];
            if (P < -qm[i]) P = -qm[i];
            const double w = (double)imp[i] * (double)r[i] * (double)r[i];
            A += w * sv * P;
            B += w * P * P;
        }
        float cj = B > 0.0 ? (float)(A / B) : c0;
        if (!(cj >= FLT_MIN)) cj = 0.0f;
        const float icj = cj > 0.0f ? 1.0f / cj : 0.0f;
        c[j] = cj;
        for (int i = 0; i < dk; ++i) {
            double qv = nearbyint((double)sc[(size_t)i * dv + j] * (double)icj);
            if (qv > qm[i]) qv = qm[i];
            if (qv < -qm[i]) qv = -qm[i];
            Q[(size_t)i * dv + j] = (int32_t)qv;
        }
    }
    free(qm);
    free(gi);
    free(ir);
    free(sc);
}

/*
 * Reconstruction (hyper.ai "Method" para 4: the state is the product of row
 * factors, column factors and low-bit integers): S_ij = Q_ij * r_i * c_j,
 * evaluated in FP64 as ((double)Q_ij * r_i) * c_j.  Q_ij * r_i is exact; the
 * second product is exact for |Q| <= 31 (at most 53 significant bits) and
 * rounded once (2^-53 relative) for 8-bit codes.
 */
void sqo_reconstruct_f64(int dk, int dv, const int32_t *Q, const float *r, const float *c,
                         double *S) {
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = ((double)Q[(size_t)i * dv + j] * (double)r[i]) * (double)c[j];
}

/* fp32 export of the reconstruction: (float)(((double)Q_ij * r_i) * c_j). */
void sqo_dequantize(int dk, int dv, const int32_t *Q, const float *r, const float *c, float *S) {
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] =
                (float)(((double)Q[(size_t)i * dv + j] * (double)r[i]) * (double)c[j]);
}

/* ------------------------------------------------------------------ */
/* Gated Delta rule, FP64                                              */
/* ------------------------------------------------------------------ */
/*
 * One step on a double state S (d_k x d_v, row i = key channel i), in the
 * order of the mechanism section: decay, look-up, delta write, read-out.
 *   D     = diag(alpha),  alpha_i = exp(g) (GDN, g scalar) or exp(g_i) (KDA)
 *   Sd    = D S
 *   v_old = Sd^T k                      (what k currently retrieves)
 *   u     = beta (v - v_old)            (the difference, scaled by beta)
 *   S'    = Sd + k u^T                  (write it along k)
 *   y     = S'^T q                      (read-out through q)
 * alpha is supplied by the caller (already exponentiated).
 */
void sqo_gated_delta_f64(int dk, int dv, double *S, const double *alpha, const double *q,
                         const double *k, const double *v, double beta, double *y) {
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];
    for (int j = 0; j < dv; ++j) {
        double vo = 0.0;
        for (int i = 0; i < dk; ++i) vo += k[i] * S[(size_t)i * dv + j];
        u[j] = beta * (v[j] - vo);
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * u[j];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];
        y[j] = acc;
    }
    free(u);
}

/* Retention factors from the log-gate: alpha_i = (float)exp((double)g).
 * The kernels hold the gate in fp32, so the oracle rounds exp(g) to fp32 too. */
static void gate_alpha(int kda, int dk, const float *g, double *alpha) {
    for (int i = 0; i < dk; ++i) {
        const float gi = kda ? g[i] : g[0];
        alpha[i] = (double)(float)exp((double)gi);
    }
}

static void gate_alpha_f32(int kda, int dk, const float *g, float *alpha) {
    for (int i = 0; i < dk; ++i) alpha[i] = (float)exp((double)(kda ? g[i] : g[0]));
}

/*
 * The update of one step on a stored state (paper section 2.1 as the
 * ta-paperlens page explains it: decay, look-up, delta write, read-out;
 * hyper.ai "Method" paragraph 1: the reconstructed state is updated in
 * floating point and the output read before it is requantized).
 * Z holds the stored numbers (integer codes, or widened binary16 values),
 * R and C the row and column scales (r and c of a quantized record; all 1
 * for a binary16 record), alpha the retention factors:
 *   Sd_ij = alpha_i ((Z_ij R_i) C_j)                FP64: decayed reconstruction
 *   u_j   = beta (v_j - sum_i k_i Sd_ij)            FP64: what k retrieves, the difference
 *   u32_j = (float)u_j                              rounded once
 *   W_ij  = (alpha_i R_i) C_j                       fp32, each product rounded
 *   S'_ij = fmaf(Z_ij, W_ij, k_i u32_j)             fp32: k_i u32_j rounded, then one
 *                                                   fused multiply-add (Sd + k u^T)
 *   y_j   = sum_i q_i S'_ij                         FP64 over the fp32 S'
 * The look-up sum is the only reduction over the state; in FP64 and rounded
 * once, its value does not depend on the order of summation except on the
 * rare exact near-ties of that rounding.  Every other step is element-wise
 * and has one result.
 */
void sqo_step_update(int dk, int dv, const float *Z, const float *R, const float *C,
                     const float *alpha, const float *q, const float *k, const float *v,
                     float beta, float *S, double *y) {
    float *u32 = (float *)malloc(sizeof(float) * (size_t)dv);
    for (int j = 0; j < dv; ++j) {
        double vo = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double sd = (double)alpha[i] *
                              (((double)Z[(size_t)i * dv + j] * (double)R[i]) * (double)C[j]);
            vo += (double)k[i] * sd;
        }
        u32[j] = (float)((double)beta * ((double)v[j] - vo));
    }
    for (int i = 0; i < dk; ++i) {
        const float wr = alpha[i] * R[i];
        for (int j = 0; j < dv; ++j) {
            const float w = wr * C[j];
            const float ku = k[i] * u32[j];
            S[(size_t)i * dv + j] = fmaf(Z[(size_t)i * dv + j], w, ku);
        }
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += (double)q[i] * (double)S[(size_t)i * dv + j];
        y[j] = acc;
    }
    free(u32);
}

/* 1 if every key row has the same width */
static int uniform_widths(const uint8_t *row_bits, int dk) {
    for (int i = 1; i < dk; ++i)
        if (row_bits[i] != row_bits[0]) return 0;
    return 1;
}

/*
 * Quantized step on one head with unpacked codes (any bits 2..24):
 * the step update above on the codes -> fp32 S' ->
 * pinned fp32 quantizer (the closed rule, or the key-row-aware fit when
 * imp != NULL gives the row-impact scores).  y receives the read-out of the
 * unrequantized S'.
 */
void sqo_quant_step_codes_rows(int kda, const uint8_t *row_bits, int dk, int dv, int32_t *Q,
                               float *r, float *c, const float *q, const float *k, const float *v,
                               float beta, const float *g, const float *imp, double *y) {
    const size_t n = (size_t)dk * dv;
    float *S = (float *)malloc(sizeof(float) * n);
    float *Z = (float *)malloc(sizeof(float) * n);
    float *alpha = (float *)malloc(sizeof(float) * (size_t)dk);
    for (size_t e = 0; e < n; ++e) Z[e] = (float)Q[e]; /* exact: |Q| < 2^24 */
    gate_alpha_f32(kda, dk, g, alpha);
    sqo_step_update(dk, dv, Z, r, c, alpha, q, k, v, beta, S, y);
    if (imp && uniform_widths(row_bits, dk))
        sqo_quantize_kra(row_bits[0], dk, dv, S, imp, Q, r, c);
    else if (imp)
        sqo_quantize_kra_rows(row_bits, dk, dv, S, imp, Q, r, c);
    else
        sqo_quantize_rows(row_bits, dk, dv, S, Q, r, c);
    free(S);
    free(Z);
    free(alpha);
}

void sqo_quant_step_codes(int kda, int bits, int dk, int dv, int32_t *Q, float *r, float *c,
                          const float *q, const float *k, const float *v, float beta,
                          const float *g, const float *imp, double *y) {
    uint8_t *rb = (uint8_t *)malloc((size_t)dk);
    memset(rb, bits, (size_t)dk);
    sqo_quant_step_codes_rows(kda, rb, dk, dv, Q, r, c, q, k, v, beta, g, imp, y);
    free(rb);
}

/* ------------------------------------------------------------------ */
/* Records                                                             */
/* ------------------------------------------------------------------ */

int sqo_record_unpack_rows(const uint8_t *row_bits, int dk, int dv, const uint8_t *rec, int32_t *Q,
                           float *r, float *c) {
    size_t pos = 0;
    for (int i = 0; i < dk; ++i) {
        sqo_unpack_row(row_bits[i], dv, rec + pos, Q + (size_t)i * dv);
        pos += (size_t)sqo_row_bytes(row_bits[i], dv);
    }
    memcpy(r, rec + pos, sizeof(float) * (size_t)dk);
    memcpy(c, rec + pos + 4 * (size_t)dk, sizeof(float) * (size_t)dv);
    return 0;
}

int sqo_record_pack_rows(const uint8_t *row_bits, int dk, int dv, const int32_t *Q, const float *r,
                         const float *c, uint8_t *rec) {
    size_t pos = 0;
    for (int i = 0; i < dk; ++i) {
        if (sqo_pack_row(row_bits[i], dv, Q + (size_t)i * dv, rec + pos) != 0) return -1;
        pos += (size_t)sqo_row_bytes(row_bits[i], dv);
    }
    memcpy(rec + pos, r, sizeof(float) * (size_t)dk);
    memcpy(rec + pos + 4 * (size_t)dk, c, sizeof(float) * (size_t)dv);
    return 0;
}

/* Uniform-width records.  Returns -1 for dk or dv outside [1, 2^20]. */
int sqo_record_unpack(int bits, int dk, int dv, const uint8_t *rec, int32_t *Q, float *r, float *c) {
    if (dk < 1 || dk > (1 << 20) || dv < 1 || dv > (1 << 20)) return -1;
    uint8_t *rb = (uint8_t *)malloc((size_t)dk);
    memset(rb, bits, (size_t)dk);
    const int st = sqo_record_unpack_rows(rb, dk, dv, rec, Q, r, c);
    free(rb);
    return st;
}

int sqo_record_pack(int bits, int dk, int dv, const int32_t *Q, const float *r, const float *c,
                    uint8_t *rec) {
    if (dk < 1 || dk > (1 << 20) || dv < 1 || dv > (1 << 20)) return -1;
    uint8_t *rb = (uint8_t *)malloc((size_t)dk);
    memset(rb, bits, (size_t)dk);
    const int st = sqo_record_pack_rows(rb, dk, dv, Q, r, c, rec);
    free(rb);
    return st;
}

/* FP16 pivot record: one step.  The step update on the exactly widened
 * binary16 values (unit scales), then S' rounded from fp32 to binary16. */
static void f16_record_step(int kda, int dk, int dv, uint8_t *rec, const float *q,
                            const float *k, const float *v, float beta, const float *g,
                            double *y) {
    const size_t n = (size_t)dk * dv;
    uint16_t *h = (uint16_t *)rec;
    const int nd = dk > dv ? dk : dv;
    float *Z = (float *)malloc(sizeof(float) * n);
    float *S = (float *)malloc(sizeof(float) * n);
    float *alpha = (float *)malloc(sizeof(float) * (size_t)dk);
    float *one = (float *)malloc(sizeof(float) * (size_t)nd);
    for (size_t e = 0; e < n; ++e) Z[e] = sqo_f16_to_f32(h[e]);
    for (int i = 0; i < nd; ++i) one[i] = 1.0f;
    gate_alpha_f32(kda, dk, g, alpha);
    sqo_step_update(dk, dv, Z, one, one, alpha, q, k, v, beta, S, y);
    for (size_t e = 0; e < n; ++e) h[e] = sqo_f32_to_f16(S[e]);
    free(Z);
    free(S);
    free(alpha);
    free(one);
}

/* ------------------------------------------------------------------ */
/* Row-parallel drivers                                                */
/* ------------------------------------------------------------------ */
/*
 * A "row" is one (request, head) unit.  Rows are independent; the drivers
 * only spread them over threads and never change the arithmetic.
 * Inputs are fp32 (bf16 widened exactly by the caller):
 *   q, k, v: [n, d]; beta: [n]; g: [n] (GDN) or [n, d_k] (KDA).
 */
typedef struct {
    int op, kda, dk, dv;
    int n0, n1;
    const uint8_t *bits;
    const int64_t *offs;
    uint8_t *base;
    float *S32;
    double *S64;
    const float *q, *k, *v, *beta, *g;
    double *y;
    const float *imp; /* [n, dk] row-impact scores, or NULL for the closed rule */
    const uint8_t *row_bits; /* [n, dk] per-key-row widths of records with bits 0 */
} job_t;

enum { OP_QUANT = 0, OP_DEQUANT = 1, OP_STEP = 2, OP_F64STEP = 3, OP_F32STEP = 4 };

static void run_row(const job_t *J, int row) {
    const int dk = J->dk, dv = J->dv;
    const size_t n = (size_t)dk * dv;
    const float *g = J->g ? J->g + (J->kda ? (size_t)row * dk : (size_t)row) : NULL;
    const float *imp = J->imp ? J->imp + (size_t)row * dk : NULL;
    /* the record's row widths: per key row (bits 0) or all equal; scratch
     * vectors sized from dk and dv */
    uint8_t *rbw = (uint8_t *)malloc((size_t)dk);
    float *rr = (float *)malloc(sizeof(float) * (size_t)dk);
    float *cc = (float *)malloc(sizeof(float) * (size_t)dv);
    if (J->bits && J->bits[row] == 0)
        memcpy(rbw, J->row_bits + (size_t)row * dk, (size_t)dk);
    else if (J->bits)
        memset(rbw, J->bits[row], (size_t)dk);
    switch (J->op) {
    case OP_QUANT: {
        uint8_t *rec = J->base + J->offs[row];
        if (J->bits[row] == 16) {
            const float *S = J->S32 + (size_t)row * n;
            for (size_t e = 0; e < n; ++e) ((uint16_t *)rec)[e] = sqo_f32_to_f16(S[e]);
            break;
        }
        int32_t *Q = (int32_t *)malloc(sizeof(int32_t) * n);
        if (imp && J->bits[row] != 0)
            sqo_quantize_kra(J->bits[row], dk, dv, J->S32 + (size_t)row * n, imp, Q, rr, cc);
        else if (imp)
            sqo_quantize_kra_rows(rbw, dk, dv, J->S32 + (size_t)row * n, imp, Q, rr, cc);
        else
            sqo_quantize_rows(rbw, dk, dv, J->S32 + (size_t)row * n, Q, rr, cc);
        sqo_record_pack_rows(rbw, dk, dv, Q, rr, cc, rec);
        free(Q);
        break;
    }
    case OP_DEQUANT: {
        const uint8_t *rec = J->base + J->offs[row];
        if (J->bits[row] == 16) {
            float *S = J->S32 + (size_t)row * n;
            for (size_t e = 0; e < n; ++e) S[e] = sqo_f16_to_f32(((const uint16_t *)rec)[e]);
            break;
        }
        int32_t *Q = (int32_t *)malloc(sizeof(int32_t) * n);
        sqo_record_unpack_rows(rbw, dk, dv, rec, Q, rr, cc);
        sqo_dequantize(dk, dv, Q, rr, cc, J->S32 + (size_t)row * n);
        free(Q);
        break;
    }
    case OP_STEP: {
        uint8_t *rec = J->base + J->offs[row];
        const int bits = J->bits[row];
        if (bits == 16) {
            f16_record_step(J->kda, dk, dv, rec, J->q + (size_t)row * dk, J->k + (size_t)row * dk,
                            J->v + (size_t)row * dv, J->beta[row], g, J->y + (size_t)row * dv);
            break;
        }
        int32_t *Q = (int32_t *)malloc(sizeof(int32_t) * n);
        sqo_record_unpack_rows(rbw, dk, dv, rec, Q, rr, cc);
        sqo_quant_step_codes_rows(J->kda, rbw, dk, dv, Q, rr, cc, J->q + (size_t)row * dk,
                                  J->k + (size_t)row * dk, J->v + (size_t)row * dv, J->beta[row],
                                  g, imp, J->y + (size_t)row * dv);
        sqo_record_pack_rows(rbw, dk, dv, Q, rr, cc, rec);
        free(Q);
        break;
    }
    case OP_F64STEP:
    case OP_F32STEP: {
        double *S = J->op == OP_F64STEP ? J->S64 + (size_t)row * n
                                        : (double *)malloc(sizeof(double) * n);
        float *S32 = J->op == OP_F32STEP ? J->S32 + (size_t)row * n : NULL;
        if (S32)
            for (size_t e = 0; e < n; ++e) S[e] = (double)S32[e];
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qd = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kd = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vd = (double *)malloc(sizeof(double) * (size_t)dv);
        gate_alpha(J->kda, dk, g, alpha);
        for (int i = 0; i < dk; ++i) {
            qd[i] = J->q[(size_t)row * dk + i];
            kd[i] = J->k[(size_t)row * dk + i];
        }
        for (int j = 0; j < dv; ++j) vd[j] = J->v[(size_t)row * dv + j];
        sqo_gated_delta_f64(dk, dv, S, alpha, qd, kd, vd, (double)J->beta[row],
                            J->y + (size_t)row * dv);
        if (S32) {
            for (size_t e = 0; e < n; ++e) S32[e] = (float)S[e];
            free(S);
        }
        free(alpha);
        free(qd);
        free(kd);
        free(vd);
        break;
    }
    }
    free(rbw);
    free(rr);
    free(cc);
}

static void *worker(void *arg) {
    const job_t *J = (const job_t *)arg;
    for (int r = J->n0; r < J->n1; ++r) run_row(J, r);
    return NULL;
}

static int run_rows(job_t proto, int n_rows, int n_threads) {
    if (proto.dk <= 0 || proto.dk > 1024 || proto.dv <= 0 || proto.dv > 1024 || n_rows < 0)
        return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 64) n_threads = 64;
    if (n_threads > n_rows) n_threads = n_rows > 0 ? n_rows : 1;
    job_t jobs[64];
    pthread_t th[64];
    for (int w = 0; w < n_threads; ++w) {
        jobs[w] = proto;
        jobs[w].n0 = (int)((int64_t)n_rows * w / n_threads);
        jobs[w].n1 = (int)((int64_t)n_rows * (w + 1) / n_threads);
    }
    for (int w = 1; w < n_threads; ++w) pthread_create(&th[w], NULL, worker, &jobs[w]);
    worker(&jobs[0]);
    for (int w = 1; w < n_threads; ++w) pthread_join(th[w], NULL);
    return 0;
}

/* Record widths 4, 6, 8, 16, or 0 with per-key-row widths in {4, 6, 8}. */
static int check_bits(int n, int dk, const uint8_t *bits, const uint8_t *row_bits) {
    for (int i = 0; i < n; ++i) {
        if (bits[i] == 0) {
            if (!row_bits) return -1;
            for (int r = 0; r < dk; ++r) {
                const uint8_t b = row_bits[(size_t)i * dk + r];
                if (b != 4 && b != 6 && b != 8) return -1;
            }
        } else if (bits[i] != 4 && bits[i] != 6 && bits[i] != 8 && bits[i] != 16) {
            return -1;
        }
    }
    return 0;
}


/* Quantize fp32 states S[n, dk, dv] into the records at base + offs[row];
 * imp [n, dk] selects the key-row-aware fit (NULL: the closed rule);
 * row_bits [n, dk] gives the key-row widths of records with bits 0. */
int sqo_records_quantize(int n, int dk, int dv, const uint8_t *bits, const int64_t *offs,
                         uint8_t *base, const float *S, const float *imp, const uint8_t *row_bits,
                         int n_threads) {
    if (check_bits(n, dk, bits, row_bits)) return -1;
    job_t J = {OP_QUANT, 0, dk, dv, 0, 0, bits, offs, base, (float *)S, NULL,
               NULL, NULL, NULL, NULL, NULL, NULL, imp, row_bits};
    return run_rows(J, n, n_threads);
}

/* Dequantize the records into S[n, dk, dv]. */
int sqo_records_dequantize(int n, int dk, int dv, const uint8_t *bits, const int64_t *offs,
                           const uint8_t *base, float *S, const uint8_t *row_bits, int n_threads) {
    if (check_bits(n, dk, bits, row_bits)) return -1;
    job_t J = {OP_DEQUANT, 0, dk, dv, 0, 0, bits, offs, (uint8_t *)base, S, NULL,
               NULL, NULL, NULL, NULL, NULL, NULL, NULL, row_bits};
    return run_rows(J, n, n_threads);
}

/* One quantized decode step, in place on the records; y[n, dv] in double;
 * imp and row_bits as for sqo_records_quantize. */
int sqo_records_step(int kda, int n, int dk, int dv, const uint8_t *bits, const int64_t *offs,
                     uint8_t *base, const float *q, const float *k, const float *v,
                     const float *beta, const float *g, const float *imp,
                     const uint8_t *row_bits, double *y, int n_threads) {
    if (check_bits(n, dk, bits, row_bits)) return -1;
    job_t J = {OP_STEP, kda, dk, dv, 0, 0, bits, offs, base, NULL, NULL, q, k, v, beta, g, y,
               imp, row_bits};
    return run_rows(J, n, n_threads);
}

/* One unquantized step on FP64 states S[n, dk, dv] (in place). */
int sqo_f64_step(int kda, int n, int dk, int dv, double *S, const float *q, const float *k,
                 const float *v, const float *beta, const float *g, double *y, int n_threads) {
    job_t J = {OP_F64STEP, kda, dk, dv, 0, 0, NULL, NULL, NULL, NULL, S, q, k, v, beta, g, y,
               NULL, NULL};
    return run_rows(J, n, n_threads);
}

/* One step on fp32-stored states S[n, dk, dv]: widen, FP64 step, round back. */
int sqo_f32_step(int kda, int n, int dk, int dv, float *S, const float *q, const float *k,
                 const float *v, const float *beta, const float *g, double *y, int n_threads) {
    job_t J = {OP_F32STEP, kda, dk, dv, 0, 0, NULL, NULL, NULL, S, NULL, q, k, v, beta, g, y,
               NULL, NULL};
    return run_rows(J, n, n_threads);
}
