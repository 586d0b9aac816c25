// HIP kernels for gfx950 (CDNA4): packed low-bit gated Delta-rule state pool.
//
// One workgroup per (request, head) tile.  A d x d tile is spread over the
// workgroup so that each lane holds 4 rows x 16 consecutive columns:
//   lane t: column group cg = t % CG (columns 16 cg .. 16 cg + 15),
//           row band     = t / CG,   rows band + NB * m, m = 0..3
// with CG = d / 16 and NB = d / 4 bands (d = 128: 256 lanes = 4 waves;
// d = 64: 64 lanes = 1 wave).  The CG lanes sharing a band are adjacent in a
// wave, so a load instruction of one wave covers 64 / CG whole consecutive
// rows (contiguous bytes), and the per-row maximum is a DPP reduction over
// adjacent lanes.  Column reductions (over rows) go through LDS: every band
// writes its 16-column partials, then lane j < d folds column j.
//
// The decode step, per tile (STEPQuant pages: ta-paperlens, mechanism
// section; hyper.ai summary, Method paragraphs 1 and 4).  The look-up and
// the update run in FP64 (full rate on CDNA4, like non-packed fp32) so that
// the updated state rounds to the same fp32 value as an FP64 reference: the
// quantized recurrence amplifies any +-1 code difference, so the stored
// codes must not depend on summation order.
//   S_ij    = code_ij r_i c_j                        (exact product, FP64)
//   a_i     = (float) exp(g) or exp(g_i)              (retention gate)
//   v_old_j = c_j * sum_i (k_i a_i r_i) code_ij       (look-up through k, FP64)
//   u_j     = beta (v_j - v_old_j)                    (delta, FP64)
//   S'_ij   = fl32(code_ij (a_i r_i c_j) + k_i u_j)   (decay + delta write)
//   y_j     = sum_i q_i S'_ij                         (read-out, fp32)
//   c'_j    = max_i |S'_ij|,  r'_i = max_j |S'_ij| / c'_j / qmax
//   code'   = round_half_even((S'_ij / c'_j) / r'_i)  (pinned fp32, in place)
#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sq_internal.h"

namespace sqk {
namespace {

template <int D> struct Geo {
    static constexpr int NT = D == 128 ? 256 : 64; // lanes per workgroup
    static constexpr int CG = D / 16;              // column groups
    static constexpr int NB = NT / CG;             // row bands (= D / 4)
    static constexpr int NW = NT / 64;             // waves
};

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u); // round to nearest even (finite values)
    return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld(const T *p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

template <typename T> __device__ __forceinline__ void st(T *p, int64_t i, float v);
template <> __device__ __forceinline__ void st<float>(float *p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<uint16_t>(uint16_t *p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
}

// DPP lane exchange within a row of 16 lanes (row_mask / bank_mask all on).
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141; // row_half_mirror: lane i <-> 7 - i within 8

// Max over the CG adjacent lanes of a band (CG = 4 or 8).
template <int CG> __device__ __forceinline__ float band_max(float v) {
    v = fmaxf(v, dpp<kQuadXor1>(v));
    v = fmaxf(v, dpp<kQuadXor2>(v));
    if constexpr (CG == 8) v = fmaxf(v, dpp<kHalfMirror>(v));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// 16 codes of one row segment: BITS * 16 / 32 dwords.
template <int BITS> struct Seg {
    static constexpr int NWORDS = BITS / 2;
    uint32_t w[NWORDS];
};

template <int BITS> __device__ __forceinline__ Seg<BITS> load_seg(const uint8_t *p) {
    Seg<BITS> s;
    if constexpr (BITS == 8) {
        const uint4 x = *reinterpret_cast<const uint4 *>(p);
        s.w[0] = x.x; s.w[1] = x.y; s.w[2] = x.z; s.w[3] = x.w;
    } else if constexpr (BITS == 4) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        s.w[0] = x.x; s.w[1] = x.y;
    } else {
        const uint32_t *p32 = reinterpret_cast<const uint32_t *>(p);
        s.w[0] = p32[0]; s.w[1] = p32[1]; s.w[2] = p32[2];
    }
    return s;
}

template <int BITS> __device__ __forceinline__ void store_seg(uint8_t *p, const Seg<BITS> &s) {
    if constexpr (BITS == 8) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(s.w[0], s.w[1], s.w[2], s.w[3]);
    } else if constexpr (BITS == 4) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(s.w[0], s.w[1]);
    } else {
        uint32_t *p32 = reinterpret_cast<uint32_t *>(p);
        p32[0] = s.w[0]; p32[1] = s.w[1]; p32[2] = s.w[2];
    }
}

// Code n (0..15) of a segment, sign-extended.
template <int BITS> __device__ __forceinline__ int code_at(const Seg<BITS> &s, int n) {
    const int bit = BITS * n, wd = bit >> 5, off = bit & 31;
    uint32_t f;
    if (off + BITS <= 32)
        f = s.w[wd] >> off;
    else
        f = __builtin_amdgcn_alignbit(s.w[wd + 1], s.w[wd], off);
    return (int32_t)(f << (32 - BITS)) >> (32 - BITS);
}

template <int BITS> __device__ __forceinline__ Seg<BITS> pack_seg(const int *code) {
    Seg<BITS> s;
#pragma unroll
    for (int i = 0; i < Seg<BITS>::NWORDS; ++i) s.w[i] = 0;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        const int bit = BITS * n, wd = bit >> 5, off = bit & 31;
        const uint32_t f = (uint32_t)code[n] & ((1u << BITS) - 1u);
        s.w[wd] |= f << off;
        if (off + BITS > 32) s.w[wd + 1] |= f >> (32 - off);
    }
    return s;
}

template <int BITS> __device__ __forceinline__ int to_code(float x) {
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    const float rq = fminf(fmaxf(__builtin_rintf(x), -QMAX), QMAX);
    return (int)rq;
}

// ---------------------------------------------------------------- quantizer
// Pinned fp32 arithmetic, one rounding per operation (no contraction):
//   c_j = max_i |S_ij|; ic_j = c_j >= FLT_MIN ? 1/c_j : 0 (else c_j := 0)
//   m_i = max_j |S_ij| ic_j; r_i = m_i / qmax; ir_i = r_i >= FLT_MIN ? 1/r_i : 0
//   code = clamp(rint((S_ij ic_j) ir_i))
// Column part: lane j < D folds the band partials of column j.
template <int D>
__device__ __forceinline__ void write_band_partials(float *plane, const float (&v)[16]) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    float4 *dst = reinterpret_cast<float4 *>(plane + band * D + 16 * cg);
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
        dst[n4] = make_float4(v[4 * n4], v[4 * n4 + 1], v[4 * n4 + 2], v[4 * n4 + 3]);
}

template <int D> __device__ __forceinline__ float column_max(const float *plane, int j) {
    float c = 0.0f;
#pragma unroll 8
    for (int b = 0; b < Geo<D>::NB; ++b) c = fmaxf(c, plane[b * D + j]);
    return c;
}

// Column scale of column j from its max: stores c_j, returns 1/c_j (or 0).
__device__ __forceinline__ float column_scale(float cmax, float *cp_j) {
#pragma clang fp contract(off)
    const bool ok = cmax >= FLT_MIN;
    *cp_j = ok ? cmax : 0.0f;
    return ok ? 1.0f / cmax : 0.0f;
}

template <int D>
__device__ __forceinline__ void load16(const float *src, float (&v)[16]) {
    const float4 *p = reinterpret_cast<const float4 *>(src);
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4) {
        const float4 f = p[n4];
        v[4 * n4] = f.x; v[4 * n4 + 1] = f.y; v[4 * n4 + 2] = f.z; v[4 * n4 + 3] = f.w;
    }
}

// Row part: row maxima (DPP over the band's lanes), row scales, codes, store.
template <int D, int BITS>
__device__ __forceinline__ void quantize_rows_store(const float (&x)[4][16], const float (&ic)[16],
                                                    uint8_t *rec) {
#pragma clang fp contract(off)
    using G = Geo<D>;
    constexpr int RB = D * BITS / 8;
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    float *rp = reinterpret_cast<float *>(rec + D * RB);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        float rm = 0.0f;
#pragma unroll
        for (int n = 0; n < 16; ++n) rm = fmaxf(rm, fabsf(x[m][n]) * ic[n]);
        rm = band_max<G::CG>(rm);
        float r = rm / QMAX;
        float ir;
        if (r >= FLT_MIN) {
            ir = 1.0f / r;
        } else {
            r = 0.0f;
            ir = 0.0f;
        }
        if (cg == 0) rp[row] = r;
        int code[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const float sv = x[m][n] * ic[n];
            code[n] = to_code<BITS>(sv * ir);
        }
        store_seg<BITS>(rec + row * RB + cg * (2 * BITS), pack_seg<BITS>(code));
    }
}

// ---------------------------------------------------------------- quant_state
template <int D, int BITS>
__device__ __forceinline__ void quant_tile(uint8_t *rec, const float *S, float *lds) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    float *plane = lds, *lds_ic = lds + G::NB * D;
    float *cp = reinterpret_cast<float *>(rec + D * (D * BITS / 8)) + D;
    float x[4][16];
#pragma unroll
    for (int m = 0; m < 4; ++m) load16<D>(S + (band + G::NB * m) * D + 16 * cg, x[m]);
    float cm[16];
#pragma unroll
    for (int n = 0; n < 16; ++n)
        cm[n] = fmaxf(fmaxf(fabsf(x[0][n]), fabsf(x[1][n])), fmaxf(fabsf(x[2][n]), fabsf(x[3][n])));
    write_band_partials<D>(plane, cm);
    __syncthreads();
    if (t < D) lds_ic[t] = column_scale(column_max<D>(plane, t), cp + t);
    __syncthreads();
    float ic[16];
    load16<D>(lds_ic + 16 * cg, ic);
    quantize_rows_store<D, BITS>(x, ic, rec);
}

template <int D>
__global__ __launch_bounds__(Geo<D>::NT) void quant_state_kernel(PoolView pool, HeadTable tab,
                                                                 const int32_t *slot,
                                                                 const float *S) {
    __shared__ __attribute__((aligned(16))) float lds[Geo<D>::NB * D + D];
    const int H = pool.n_heads;
    const int b = blockIdx.x / H, h = blockIdx.x - b * H;
    uint8_t *rec = pool.base + (int64_t)slot[b] * pool.slot_stride + tab.off[h];
    const float *src = S + (int64_t)blockIdx.x * D * D;
    switch (tab.bits[h]) {
    case 4: quant_tile<D, 4>(rec, src, lds); break;
    case 6: quant_tile<D, 6>(rec, src, lds); break;
    default: quant_tile<D, 8>(rec, src, lds); break;
    }
}

// ---------------------------------------------------------------- dequant_state
template <int D, int BITS>
__device__ __forceinline__ void dequant_tile(const uint8_t *rec, float *S) {
    using G = Geo<D>;
    constexpr int RB = D * BITS / 8;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    const float *rp = reinterpret_cast<const float *>(rec + D * RB);
    const float *cp = rp + D;
    float c[16];
    {
        const float4 *src = reinterpret_cast<const float4 *>(cp + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4) {
            const float4 f = src[n4];
            c[4 * n4] = f.x; c[4 * n4 + 1] = f.y; c[4 * n4 + 2] = f.z; c[4 * n4 + 3] = f.w;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        const Seg<BITS> s = load_seg<BITS>(rec + row * RB + cg * (2 * BITS));
        const double r = (double)rp[row];
        float o[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
#pragma clang fp contract(off)
            // (float)(((double)code * r) * c): the fp32 export of the FP64 product
            const double t0 = (double)code_at<BITS>(s, n) * r;
            o[n] = (float)(t0 * (double)c[n]);
        }
        float4 *dst = reinterpret_cast<float4 *>(S + row * D + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4)
            dst[n4] = make_float4(o[4 * n4], o[4 * n4 + 1], o[4 * n4 + 2], o[4 * n4 + 3]);
    }
}

template <int D>
__global__ __launch_bounds__(Geo<D>::NT) void dequant_state_kernel(PoolView pool, HeadTable tab,
                                                                   const int32_t *slot, float *S) {
    const int H = pool.n_heads;
    const int b = blockIdx.x / H, h = blockIdx.x - b * H;
    const uint8_t *rec = pool.base + (int64_t)slot[b] * pool.slot_stride + tab.off[h];
    float *dst = S + (int64_t)blockIdx.x * D * D;
    switch (tab.bits[h]) {
    case 4: dequant_tile<D, 4>(rec, dst); break;
    case 6: dequant_tile<D, 6>(rec, dst); break;
    default: dequant_tile<D, 8>(rec, dst); break;
    }
}

// ---------------------------------------------------------------- decode step
// LDS: the band-partials region (NB x D doubles in the look-up phase, reused
// as two NB x D fp32 planes for the column maxima and the read-out), then
// u[D] doubles, 1/c'[D] floats and one k.q partial per wave.
template <int D> struct DecodeLds {
    static constexpr int PART_F = 2 * Geo<D>::NB * D; // floats in the partials region
    static constexpr int TOTAL = PART_F + 2 * D + D + 4;
};

template <int D, int BITS, bool KDA, typename TI, typename TO>
__device__ __forceinline__ void decode_tile(uint8_t *rec, int64_t row_io, const StepIO &io,
                                            float *lds) {
    using G = Geo<D>;
    constexpr int RB = D * BITS / 8;
    constexpr int PLANE = G::NB * D;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    double *part64 = reinterpret_cast<double *>(lds);
    float *plane_max = lds, *plane_y = lds + PLANE;
    double *lds_u = reinterpret_cast<double *>(lds + DecodeLds<D>::PART_F);
    float *lds_ic = lds + DecodeLds<D>::PART_F + 2 * D;
    float *lds_kq = lds_ic + D;

    const TI *q = reinterpret_cast<const TI *>(io.q) + row_io * D;
    const TI *k = reinterpret_cast<const TI *>(io.k) + row_io * D;
    const TI *v = reinterpret_cast<const TI *>(io.v) + row_io * D;
    const TI *g = reinterpret_cast<const TI *>(io.g);
    float *rp = reinterpret_cast<float *>(rec + D * RB);
    float *cp = rp + D;

    // ---- loads: codes, scales, inputs
    Seg<BITS> seg[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) seg[m] = load_seg<BITS>(rec + (band + G::NB * m) * RB + cg * (2 * BITS));
    float c[16];
    load16<D>(cp + 16 * cg, c);
    double ar[4], kar[4];
    float kf[4], qf[4], kq_part = 0.0f;
    const float a_head = KDA ? 0.0f : (float)exp((double)ld<TI>(g, row_io));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        const float a = KDA ? (float)exp((double)ld<TI>(g, row_io * D + row)) : a_head;
        kf[m] = ld<TI>(k, row);
        qf[m] = ld<TI>(q, row);
        ar[m] = (double)a * (double)rp[row];   // a_i r_i, exact in FP64
        kar[m] = (double)kf[m] * ar[m];        // k_i a_i r_i
        kq_part += kf[m] * qf[m];
    }
    // ---- look-up: band partials of sum_i (k_i a_i r_i) code_ij, FP64
    {
        double acc[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = 0.0;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 16; ++n) acc[n] = fma(kar[m], (double)code_at<BITS>(seg[m], n), acc[n]);
        double2 *dst = reinterpret_cast<double2 *>(part64 + band * D + 16 * cg);
#pragma unroll
        for (int n2 = 0; n2 < 8; ++n2) dst[n2] = make_double2(acc[2 * n2], acc[2 * n2 + 1]);
    }
    kq_part = wave_sum(cg == 0 ? kq_part : 0.0f);
    if ((t & 63) == 0) lds_kq[t >> 6] = kq_part;
    __syncthreads();
    if (t < D) {
        double P = 0.0;
#pragma unroll 8
        for (int b = 0; b < G::NB; ++b) P += part64[b * D + t];
        const double beta = (double)ld<TI>(reinterpret_cast<const TI *>(io.beta), row_io);
        lds_u[t] = beta * ((double)ld<TI>(v, t) - P * (double)cp[t]);
    }
    __syncthreads();
    // ---- decay + delta write in FP64, rounded once to fp32; read-out and
    //      column maxima partials in fp32
    float x[4][16];
    {
        float cm[16], yp[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const double cn = (double)c[n];
            const double un = lds_u[16 * cg + n];
            cm[n] = 0.0f;
            yp[n] = 0.0f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const double s = fma((double)code_at<BITS>(seg[m], n), ar[m] * cn, (double)kf[m] * un);
                const float sf = (float)s;
                x[m][n] = sf;
                yp[n] = fmaf(qf[m], sf, yp[n]);
                cm[n] = fmaxf(cm[n], fabsf(sf));
            }
        }
        write_band_partials<D>(plane_max, cm);
        write_band_partials<D>(plane_y, yp);
    }
    __syncthreads();
    if (t < D) {
        float yv = 0.0f;
#pragma unroll 8
        for (int b = 0; b < G::NB; ++b) yv += plane_y[b * D + t];
        st<TO>(reinterpret_cast<TO *>(io.y) + row_io * D, t, yv);
        lds_ic[t] = column_scale(column_max<D>(plane_max, t), cp + t);
    }
    __syncthreads();
    float ic[16];
    load16<D>(lds_ic + 16 * cg, ic);
    quantize_rows_store<D, BITS>(x, ic, rec);
}

template <int D, bool KDA, typename TI, typename TO>
__global__ __launch_bounds__(Geo<D>::NT) void decode_kernel(PoolView pool, HeadTable tab, StepIO io) {
    __shared__ __attribute__((aligned(16))) float lds[DecodeLds<D>::TOTAL];
    const int H = pool.n_heads;
    const int b = blockIdx.x / H, h = blockIdx.x - b * H;
    uint8_t *rec = pool.base + (int64_t)io.slot[b] * pool.slot_stride + tab.off[h];
    const int64_t row_io = blockIdx.x; // (b, h) row of the input / output tensors
    switch (tab.bits[h]) {
    case 4: decode_tile<D, 4, KDA, TI, TO>(rec, row_io, io, lds); break;
    case 6: decode_tile<D, 6, KDA, TI, TO>(rec, row_io, io, lds); break;
    default: decode_tile<D, 8, KDA, TI, TO>(rec, row_io, io, lds); break;
    }
}

// ---------------------------------------------------------------- fp32-state step
template <int D, bool KDA, typename TI, typename TO>
__global__ __launch_bounds__(Geo<D>::NT) void f32_decode_kernel(float *state, int64_t slot_stride,
                                                                int32_t H, StepIO io) {
    using G = Geo<D>;
    constexpr int PART = G::NB * D;
    __shared__ __attribute__((aligned(16))) float lds[2 * PART + D + 4];
    float *red0 = lds, *red1 = lds + PART, *lds_u = lds + 2 * PART, *lds_kq = lds_u + D;
    const int b = blockIdx.x / H, h = blockIdx.x - b * H;
    const int64_t row_io = blockIdx.x;
    float *S = state + (int64_t)io.slot[b] * slot_stride + (int64_t)h * D * D;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    const TI *q = reinterpret_cast<const TI *>(io.q) + row_io * D;
    const TI *k = reinterpret_cast<const TI *>(io.k) + row_io * D;
    const TI *v = reinterpret_cast<const TI *>(io.v) + row_io * D;
    const TI *g = reinterpret_cast<const TI *>(io.g);
    const float beta = ld<TI>(reinterpret_cast<const TI *>(io.beta), row_io);

    float x[4][16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float4 *src = reinterpret_cast<const float4 *>(S + (band + G::NB * m) * D + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4) {
            const float4 f = src[n4];
            x[m][4 * n4] = f.x; x[m][4 * n4 + 1] = f.y; x[m][4 * n4 + 2] = f.z; x[m][4 * n4 + 3] = f.w;
        }
    }
    float km[4], am[4], kq_part = 0.0f, ka[4], qa[4];
    const float a_head = KDA ? 0.0f : expf(ld<TI>(g, row_io));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        const float a = KDA ? expf(ld<TI>(g, row_io * D + row)) : a_head;
        const float kr = ld<TI>(k, row), qr = ld<TI>(q, row);
        km[m] = kr;
        am[m] = a;
        ka[m] = kr * a;
        qa[m] = qr * a;
        kq_part += kr * qr;
    }
    float sk[16], sq[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        sk[n] = 0.0f;
        sq[n] = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sk[n] = fmaf(ka[m], x[m][n], sk[n]);
            sq[n] = fmaf(qa[m], x[m][n], sq[n]);
        }
    }
    {
        float4 *d0 = reinterpret_cast<float4 *>(red0 + band * D + 16 * cg);
        float4 *d1 = reinterpret_cast<float4 *>(red1 + band * D + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4) {
            d0[n4] = make_float4(sk[4 * n4], sk[4 * n4 + 1], sk[4 * n4 + 2], sk[4 * n4 + 3]);
            d1[n4] = make_float4(sq[4 * n4], sq[4 * n4 + 1], sq[4 * n4 + 2], sq[4 * n4 + 3]);
        }
    }
    kq_part = wave_sum(cg == 0 ? kq_part : 0.0f);
    if ((t & 63) == 0) lds_kq[t >> 6] = kq_part;
    __syncthreads();
    if (t < D) {
        float SK = 0.0f, SQ = 0.0f;
#pragma unroll 8
        for (int bb = 0; bb < G::NB; ++bb) {
            SK += red0[bb * D + t];
            SQ += red1[bb * D + t];
        }
        float kq = 0.0f;
#pragma unroll
        for (int w = 0; w < G::NW; ++w) kq += lds_kq[w];
        const float u = beta * (ld<TI>(v, t) - SK);
        lds_u[t] = u;
        st<TO>(reinterpret_cast<TO *>(io.y) + row_io * D, t, fmaf(u, kq, SQ));
    }
    __syncthreads();
    float u[16];
    {
        const float4 *src = reinterpret_cast<const float4 *>(lds_u + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4) {
            const float4 f = src[n4];
            u[4 * n4] = f.x; u[4 * n4 + 1] = f.y; u[4 * n4 + 2] = f.z; u[4 * n4 + 3] = f.w;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float o[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) o[n] = fmaf(km[m], u[n], am[m] * x[m][n]);
        float4 *dst = reinterpret_cast<float4 *>(S + (band + G::NB * m) * D + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4)
            dst[n4] = make_float4(o[4 * n4], o[4 * n4 + 1], o[4 * n4 + 2], o[4 * n4 + 3]);
    }
}

// ---------------------------------------------------------------- dispatch
template <int D, bool KDA>
hipError_t decode_dispatch(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                           hipStream_t s) {
    const dim3 grid((unsigned)io.n * (unsigned)pool.n_heads), block(Geo<D>::NT);
    if (!io.in_bf16 && !io.y_bf16)
        hipLaunchKernelGGL((decode_kernel<D, KDA, float, float>), grid, block, 0, s, pool, tab, io);
    else if (!io.in_bf16 && io.y_bf16)
        hipLaunchKernelGGL((decode_kernel<D, KDA, float, uint16_t>), grid, block, 0, s, pool, tab, io);
    else if (io.in_bf16 && !io.y_bf16)
        hipLaunchKernelGGL((decode_kernel<D, KDA, uint16_t, float>), grid, block, 0, s, pool, tab, io);
    else
        hipLaunchKernelGGL((decode_kernel<D, KDA, uint16_t, uint16_t>), grid, block, 0, s, pool, tab, io);
    return hipGetLastError();
}

template <int D, bool KDA>
hipError_t f32_dispatch(float *state, int64_t stride, int32_t H, const StepIO &io, hipStream_t s) {
    const dim3 grid((unsigned)io.n * (unsigned)H), block(Geo<D>::NT);
    if (!io.in_bf16 && !io.y_bf16)
        hipLaunchKernelGGL((f32_decode_kernel<D, KDA, float, float>), grid, block, 0, s, state, stride, H, io);
    else if (!io.in_bf16 && io.y_bf16)
        hipLaunchKernelGGL((f32_decode_kernel<D, KDA, float, uint16_t>), grid, block, 0, s, state, stride, H, io);
    else if (io.in_bf16 && !io.y_bf16)
        hipLaunchKernelGGL((f32_decode_kernel<D, KDA, uint16_t, float>), grid, block, 0, s, state, stride, H, io);
    else
        hipLaunchKernelGGL((f32_decode_kernel<D, KDA, uint16_t, uint16_t>), grid, block, 0, s, state, stride, H, io);
    return hipGetLastError();
}

} // namespace

hipError_t launch_quant_state(const PoolView &pool, const HeadTable &tab, const int32_t *slot,
                              int32_t n, const float *S, hipStream_t stream) {
    const dim3 grid((unsigned)n * (unsigned)pool.n_heads);
    if (pool.d == 128)
        hipLaunchKernelGGL(quant_state_kernel<128>, grid, dim3(Geo<128>::NT), 0, stream, pool, tab, slot, S);
    else
        hipLaunchKernelGGL(quant_state_kernel<64>, grid, dim3(Geo<64>::NT), 0, stream, pool, tab, slot, S);
    return hipGetLastError();
}

hipError_t launch_dequant_state(const PoolView &pool, const HeadTable &tab, const int32_t *slot,
                                int32_t n, float *S, hipStream_t stream) {
    const dim3 grid((unsigned)n * (unsigned)pool.n_heads);
    if (pool.d == 128)
        hipLaunchKernelGGL(dequant_state_kernel<128>, grid, dim3(Geo<128>::NT), 0, stream, pool, tab, slot, S);
    else
        hipLaunchKernelGGL(dequant_state_kernel<64>, grid, dim3(Geo<64>::NT), 0, stream, pool, tab, slot, S);
    return hipGetLastError();
}

hipError_t launch_decode(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                         hipStream_t stream) {
    if (pool.d == 128)
        return io.kda ? decode_dispatch<128, true>(pool, tab, io, stream)
                      : decode_dispatch<128, false>(pool, tab, io, stream);
    return io.kda ? decode_dispatch<64, true>(pool, tab, io, stream)
                  : decode_dispatch<64, false>(pool, tab, io, stream);
}

hipError_t launch_f32_decode(float *state, int64_t slot_stride_floats, int32_t n_heads, int32_t d,
                             const StepIO &io, hipStream_t stream) {
    if (d == 128)
        return io.kda ? f32_dispatch<128, true>(state, slot_stride_floats, n_heads, io, stream)
                      : f32_dispatch<128, false>(state, slot_stride_floats, n_heads, io, stream);
    return io.kda ? f32_dispatch<64, true>(state, slot_stride_floats, n_heads, io, stream)
                  : f32_dispatch<64, false>(state, slot_stride_floats, n_heads, io, stream);
}

} // namespace sqk
