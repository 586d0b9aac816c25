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
// adjacent lanes.  Column maxima (over rows) go through LDS: every band
// writes its 16-column partials, then lane j < d folds column j.  The step's
// two sums over rows (look-up and read-out) run on the matrix cores instead
// (decode_tile); the FP16 pivot step folds FP64 band partials like the maxima.
//
// The decode step, per tile (STEPQuant pages: ta-paperlens, mechanism
// section; hyper.ai summary, Method paragraphs 1 and 4).  The one reduction
// over the state, the look-up, is an exact integer sum on the matrix cores
// (decode_tile) rounded once, so that it does not depend on the order of
// summation: the quantized recurrence amplifies any +-1 code difference, so
// the stored codes must be those of the stated arithmetic.  Everything after
// it is element-wise fp32 with one fixed order.
//   a_i     = (float) exp(g) or exp(g_i)              (retention gate)
//   v_old_j = c_j * sum_i (k_i a_i r_i) code_ij       (look-up through k)
//   u_j     = fl32(beta (v_j - v_old_j))              (delta, FP64, rounded once)
//   S'_ij   = fma(code_ij, (a_i r_i) c_j, k_i u_j)    (decay + delta write, fp32:
//                                                      each product rounded once)
//   y_j     = c_j sum_i (q_i a_i r_i) code_ij + u_j (k.q)   (read-out, = S'^T q)
//   c'_j    = max_i |S'_ij|,  s_ij = S'_ij * (1 / c'_j),  r'_i = max_j |s_ij| / qmax
//   code'   = round half to even of the exact product s_ij * (1 / r'_i)
//             (fp32, each division correctly rounded; stored in place)
//
// Variants of the same body, chosen per launch or per head:
//   - split step (decode_update): S' goes to a workspace instead of being
//     requantized; quant_state of that workspace completes it;
//   - key-row-aware fit (pools with row-impact scores): a different
//     requantizer, kra_quantize_store;
//   - FP16 pivot heads (bits 16): the state kept as binary16;
//   - per-key-row widths (bits 0): each row its own width, see Rows.
#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "sq_internal.h"

#ifndef SQ_DECODE_WAVES
#define SQ_DECODE_WAVES 5
#endif

namespace sqk {
namespace {

// Timeline build (-DSQ_TIMELINE, libsq_timeline.so; never the library's
// default build): lane 0 of each wave of the first kTlTiles tiles of a decode
// launch stores the shader clock (s_memtime) at the phase boundaries of the
// step, kTlSlots slots per wave, read back with sq_timeline_read.  Slots:
// 0 kernel entry, 1 tile start (record address known), 2 the tile's loads
// arrived, 3 codes in LDS, 4 exponent bounds and k.q, 5 / 6 before / after
// barrier 1, 7 / 8 barrier 2, 9 / 10 barrier 3, 11 / 12 barrier 4, 13 end.
#ifdef SQ_TIMELINE
constexpr int kTlTiles = 24576, kTlSlots = 16;
__device__ unsigned long long g_tl[kTlTiles * 4 * kTlSlots];
#define SQ_TL(k)                                                                                  \
    do {                                                                                          \
        if ((threadIdx.x & 63) == 0 && (unsigned)tile < (unsigned)kTlTiles)                       \
            g_tl[((unsigned)tile * 4u + (threadIdx.x >> 6)) * kTlSlots + (k)] = __builtin_amdgcn_s_memtime(); \
    } while (0)
#else
#define SQ_TL(k) do { } while (0)
#endif

template <int D> struct Geo {
    static constexpr int NT = D == 128 ? 256 : 64; // lanes per workgroup
    static constexpr int CG = D / 16;              // column groups
    static constexpr int NB = NT / CG;             // row bands (= D / 4)
    static constexpr int NW = NT / 64;             // waves
};

// ---------------------------------------------------------------- helpers
// Request and head of tile t = b H + h, without a division (scalar ALU).
__device__ __forceinline__ void tile_bh(const PoolView &pool, uint32_t t, int &b, int &h) {
    const uint32_t q = (uint32_t)(((uint64_t)t * pool.h_magic) >> pool.h_shift);
    b = (int)q;
    h = (int)(t - q * (uint32_t)pool.n_heads);
}
__device__ __forceinline__ int info_bits(uint32_t info) { return (int)(info & 0xffu); }
__device__ __forceinline__ int info_n4(uint32_t info) { return (int)((info >> 8) & 0xffu); }
__device__ __forceinline__ int info_n6(uint32_t info) { return (int)((info >> 16) & 0xffu); }
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

// Max of non-negative floats over the CG adjacent lanes of a band (CG = 4
// or 8).  For non-negative IEEE values the order of the bit patterns as
// unsigned integers is the numeric order, so an integer max (which folds the
// DPP exchange into one instruction) gives the float max exactly.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    // old = 0 is the identity of the unsigned max, so the exchange folds into
    // the max instruction as a DPP source
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CG> __device__ __forceinline__ float band_max(float vf) {
    uint32_t v = __float_as_uint(vf);
    v = max(v, dpp_u<kQuadXor1>(v));
    v = max(v, dpp_u<kQuadXor2>(v));
    if constexpr (CG == 8) v = max(v, dpp_u<kHalfMirror>(v));
    return __uint_as_float(v);
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

// Code segments are read once per step: non-temporal loads, word by word
// (a segment is only 4-byte aligned; the words merge into one load).
// Measured about 1 % faster on the 6-bit step than plain loads;
// non-temporal stores of the same segments were slower.
template <int NW> __device__ __forceinline__ void load_words_nt(const uint8_t *p, uint32_t *w) {
    const uint32_t *p32 = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = __builtin_nontemporal_load(p32 + i);
}
template <int BITS> __device__ __forceinline__ Seg<BITS> load_seg(const uint8_t *p) {
    Seg<BITS> s;
    load_words_nt<Seg<BITS>::NWORDS>(p, s.w);
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

// Code of a scaled entry: round half to even of the exact product s * ir,
// by one fused multiply-add with the magic number 1.5 * 2^23: for
// |s * ir| < 2^22, fl(s * ir + 1.5 * 2^23) = 1.5 * 2^23 + rint(s * ir)
// (a single rounding at unit spacing), whose low bits are the code in two's
// complement.  Returns that bit pattern (code in the low BITS bits).
__device__ __forceinline__ uint32_t code_bits(float s, float ir) {
    return __float_as_uint(__builtin_fmaf(s, ir, 12582912.0f));
}
// The same with the magic number passed in: from a vector register (below),
// the FMA has no literal operand and can pair with another fp32 instruction
// in the same issue cycle, which a literal or scalar operand prevents.
__device__ __forceinline__ uint32_t code_bits(float s, float ir, float magic) {
    return __float_as_uint(__builtin_fmaf(s, ir, magic));
}
// 1.5 * 2^23 in a vector register the compiler does not fold back into a
// literal
__device__ __forceinline__ float magic_vgpr() {
    float m = 12582912.0f;
    asm volatile("" : "+v"(m));
    return m;
}

// Pack 16 codes (low BITS bits of f[n], garbage above) into a row segment
// with funnel shifts: alignbit(f, acc, s) = (acc >> s) | (f << (32 - s))
// appends the s low bits of f at the top of acc; everything above them in f
// falls out of the word.  A code split across two words is appended with the
// bits that fit, then appended whole to the next word, whose accumulated
// shift (32 + bits already written) drops the part written before.
template <int BITS> __device__ __forceinline__ Seg<BITS> pack_stream(const uint32_t (&f)[16]) {
    Seg<BITS> s;
    if constexpr (BITS == 8) {
        // whole bytes: the low bytes of four codes gathered by two byte
        // permutes and an OR per word (three instructions for four codes)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            s.w[q] = __builtin_amdgcn_perm(f[4 * q + 1], f[4 * q], 0x0c0c0400u) |
                     __builtin_amdgcn_perm(f[4 * q + 3], f[4 * q + 2], 0x04000c0cu);
        return s;
    }
    uint32_t acc = 0;
    int fill = 0, word = 0;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        if (fill + BITS <= 32) {
            acc = __builtin_amdgcn_alignbit(f[n], acc, BITS);
            fill += BITS;
            if (fill == 32) {
                s.w[word++] = acc;
                fill = 0;
            }
        } else {
            const int part = 32 - fill;
            acc = __builtin_amdgcn_alignbit(f[n], acc, part);
            s.w[word++] = acc;
            acc = __builtin_amdgcn_alignbit(f[n], acc, BITS);
            fill = BITS - part;
        }
    }
    return s;
}

// 16 codes of a BITS-wide segment as one sign-extended byte each (the 8-bit
// segment layout).
template <int BITS> __device__ __forceinline__ Seg<8> widen_seg(const Seg<BITS> &s) {
    Seg<8> o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o.w[q] = ((uint32_t)code_at<BITS>(s, 4 * q) & 0xFFu) |
                 (((uint32_t)code_at<BITS>(s, 4 * q + 1) & 0xFFu) << 8) |
                 (((uint32_t)code_at<BITS>(s, 4 * q + 2) & 0xFFu) << 16) |
                 ((uint32_t)code_at<BITS>(s, 4 * q + 3) << 24);
    return o;
}

// The first W / 2 words of a raw 16-byte segment as a W-wide segment.
template <int W> __device__ __forceinline__ Seg<W> as_seg(const Seg<8> &raw) {
    Seg<W> s;
#pragma unroll
    for (int i = 0; i < Seg<W>::NWORDS; ++i) s.w[i] = raw.w[i];
    return s;
}

// Where a record's key rows are and how wide.  Uniform heads (MIXED = false):
// every row BITS wide.  Heads with per-key-row widths (MIXED = true,
// instantiated with BITS = 8; quant / dequant widen each segment to the
// 8-bit layout, the decode step reads it at its own width): rows
// [0, n4) are 4-bit, [n4, n4 + n6) 6-bit, the rest 8-bit, each row's code
// stream right after the previous one.  The widths change only at multiples
// of the rows one wavefront holds per m (8 at d = 128, 16 at d = 64), so a
// row's width is uniform over the wavefront and the branches on it are
// scalar.
template <int D, int BITS, bool MIXED> struct Rows {
    int n4, n6;
    __device__ __forceinline__ int width(int row) const {
        if constexpr (!MIXED) return BITS;
        return row < n4 ? 4 : (row < n4 + n6 ? 6 : 8);
    }
    __device__ __forceinline__ int offset(int row) const {
        if constexpr (!MIXED) return row * (D * BITS / 8);
        const int a = min(row, n4), b = min(max(row - n4, 0), n6), c = max(row - n4 - n6, 0);
        return a * (D / 2) + b * (3 * D / 4) + c * D;
    }
    __device__ __forceinline__ int codes_bytes() const { return offset(D); }
    __device__ __forceinline__ float qmax(int row) const {
        return (float)((1 << (width(row) - 1)) - 1);
    }
    // 1 / qmax rounded to nearest
    __device__ __forceinline__ float inv_qmax(int row) const {
        const int w = width(row);
        return w == 4 ? 1.0f / 7.0f : (w == 6 ? 1.0f / 31.0f : 1.0f / 127.0f);
    }
    // MIXED: the widest segment (16 bytes, 4-byte aligned) is read whatever
    // the row's width, so the four rows' loads issue back to back before any
    // width branch.  A narrower row's extra bytes lie in the next row or in
    // r[] of the same record (which the same workgroup only writes later).
    __device__ __forceinline__ Seg<8> load_raw(const uint8_t *rec, int row, int cg) const {
        Seg<8> s;
        load_words_nt<4>(rec + (uint32_t)(offset(row) + cg * (2 * width(row))), s.w);
        return s;
    }
    __device__ __forceinline__ Seg<8> widen(const Seg<8> &raw, int row) const {
        const int w = __builtin_amdgcn_readfirstlane(width(row));
        if (w == 4) {
            Seg<4> s4;
            s4.w[0] = raw.w[0]; s4.w[1] = raw.w[1];
            return widen_seg<4>(s4);
        }
        if (w == 6) {
            Seg<6> s6;
            s6.w[0] = raw.w[0]; s6.w[1] = raw.w[1]; s6.w[2] = raw.w[2];
            return widen_seg<6>(s6);
        }
        return raw;
    }
    __device__ __forceinline__ Seg<BITS> load(const uint8_t *rec, int row, int cg) const {
        if constexpr (!MIXED) {
            // unsigned 32-bit offsets: the load takes the record's (scalar)
            // base directly
            return load_seg<BITS>(rec + (uint32_t)(offset(row) + cg * (2 * BITS)));
        } else {
            return widen(load_raw(rec, row, cg), row);
        }
    }
    // f: code bit patterns whose low bits are the two's-complement codes
    __device__ __forceinline__ void store(uint8_t *rec, int row, int cg,
                                         const uint32_t (&f)[16]) const {
        if constexpr (!MIXED) {
            // unsigned 32-bit offset from the record base, as for the loads
            store_seg<BITS>(rec + (uint32_t)(offset(row) + cg * (2 * BITS)), pack_stream<BITS>(f));
        } else {
            const int w = __builtin_amdgcn_readfirstlane(width(row));
            uint8_t *p = rec + (uint32_t)(offset(row) + cg * (2 * w));
            if (w == 4)
                store_seg<4>(p, pack_stream<4>(f));
            else if (w == 6)
                store_seg<6>(p, pack_stream<6>(f));
            else
                store_seg<8>(p, pack_stream<8>(f));
        }
    }
};

// ---------------------------------------------------------------- quantizer
// Pinned fp32 arithmetic, one rounding per operation (no contraction):
//   c_j = max_i |S_ij|; ic_j = c_j >= FLT_MIN ? 1/c_j : 0 (else c_j := 0)
//   s_ij = S_ij ic_j (rounded); m_i = max_j |s_ij|; r_i = m_i / qmax;
//   ir_i = r_i >= FLT_MIN ? 1/r_i : 0;  code = clamp(rint(s_ij * ir_i)),
//   the last product exact (not rounded before rint)
// The three divisions are correctly rounded, by short sequences in their
// input ranges (every value of each range checked against the IEEE division
// on MI355X by sq_arith_selfcheck):
//   1/x, x in [FLT_MIN, 2^126): the hardware reciprocal y, refined once,
//     fma(fma(-x, y, 1), y, y)  (outside the range: the IEEE division);
//   m / qmax, m in [0, 2], qmax in {7, 31, 127}: q = m z with z = 1/qmax
//     rounded, then fma(fma(-q, qmax, m), z, q), the correction step of a
//     faithful quotient with a correctly rounded reciprocal (Markstein).
//     |s| <= 1 + 2^-23 for every scaled entry, so m stays in range.
__device__ __forceinline__ float recip_rn(float x) {
    const float y = __builtin_amdgcn_rcpf(x);
    return __builtin_fmaf(__builtin_fmaf(-x, y, 1.0f), y, y);
}
__device__ __forceinline__ float div_qmax(float m, float qmax, float z) {
#pragma clang fp contract(off)
    const float q = m * z;
    return __builtin_fmaf(__builtin_fmaf(-q, qmax, m), z, q);
}
// LDS layouts.  A band's 16-column group is written by one lane as 16-byte
// chunks; eight consecutive lanes write the same chunk index at the same
// time, and the 32 x 4-byte LDS banks repeat every 128 bytes.  The chunk
// index is therefore XOR-swizzled with the writer's lane & 7 so that the
// eight lanes land on eight different 16-byte bank groups.
//   fp32 plane [NB][D]:  float4 chunk c4 of lane t stored at c4 ^ ((t >> 1) & 3)
//   FP64 plane [NB][D]:  double2 chunk c2 of lane t stored at c2 ^ (t & 7)
//   per-column vectors read by column group cg: element n at n ^ cg (8- or
//   16-byte elements), or float4 chunk c4 at c4 ^ ((cg >> 1) & 3) (floats)
template <int D> __device__ __forceinline__ int plane_idx(int band, int cg, int n) {
    const int key = ((band * Geo<D>::CG + cg) >> 1) & 3;
    return band * D + 16 * cg + (((n >> 2) ^ key) << 2) + (n & 3);
}
template <int D> __device__ __forceinline__ int part_idx(int band, int cg, int n) {
    const int key = (band * Geo<D>::CG + cg) & 7;
    return band * D + 16 * cg + (((n >> 1) ^ key) << 1) + (n & 1);
}
__device__ __forceinline__ int colvec2_idx(int j) { return (j & ~15) | ((j & 15) ^ ((j >> 4) & 7)); }
__device__ __forceinline__ int colvec4_idx(int j) {
    const int cg = j >> 4, n = j & 15;
    return 16 * cg + (((n >> 2) ^ ((cg >> 1) & 3)) << 2) + (n & 3);
}

// Column part: every lane writes its 16 column partials; lane j < D then
// folds column j over the bands.
template <int D>
__device__ __forceinline__ void write_band_partials(float *plane, const float (&v)[16]) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
        *reinterpret_cast<float4 *>(plane + plane_idx<D>(band, cg, 4 * n4)) =
            make_float4(v[4 * n4], v[4 * n4 + 1], v[4 * n4 + 2], v[4 * n4 + 3]);
}

// Max over the band partials of column j (non-negative: integer max, exact).
template <int D> __device__ __forceinline__ float column_max(const float *plane, int j) {
    uint32_t c = 0;
#pragma unroll 8
    for (int b = 0; b < Geo<D>::NB; ++b)
        c = max(c, __float_as_uint(plane[plane_idx<D>(b, j >> 4, j & 15)]));
    return __uint_as_float(c);
}

// The 16 per-column floats of column group cg from a colvec4-swizzled vector.
__device__ __forceinline__ void load_colvec16(const float *vec, int cg, float (&v)[16]) {
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4) {
        const float4 f = *reinterpret_cast<const float4 *>(vec + colvec4_idx(16 * cg + 4 * n4));
        v[4 * n4] = f.x; v[4 * n4 + 1] = f.y; v[4 * n4 + 2] = f.z; v[4 * n4 + 3] = f.w;
    }
}

// Column scale of column j from its max: stores c_j, returns 1/c_j (or 0).
__device__ __forceinline__ float column_scale(float cmax, float *cp_j) {
#pragma clang fp contract(off)
    const bool ok = cmax >= FLT_MIN;
    *cp_j = ok ? cmax : 0.0f;
    float ic = recip_rn(cmax);
    // maxima of 2^126 and above (reciprocal subnormal): the IEEE division,
    // on a wavefront-uniform branch (the empty asm keeps the compiler from
    // computing the division on every path and selecting)
    if (__builtin_amdgcn_ballot_w64(cmax >= 0x1p126f) != 0) {
        float x = cmax;
        asm volatile("" : "+v"(x));
        if (x >= 0x1p126f) ic = 1.0f / x;
    }
    return ok ? ic : 0.0f;
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

// Row part.  x holds S' on entry and ic_vec the reciprocal column scales
// (colvec4 layout), read four columns at a time so that they are not all live
// next to the 64 entries.  s = S' ic is formed once: |s| is the pinned |S'| ic
// of the row maximum and s * ir is the pinned scaled entry.
// The row maxima are reduced over the band's lanes with DPP; lane cg < 4 of
// a band then computes the two correctly rounded divisions of row cg, and
// the results are broadcast back with ds_swizzle.  Codes: round half to even
// of the exact product s * ir (code_bits); |s * ir| <= qmax (1 + 2 eps), so
// the clamp to [-qmax, qmax] can never act and is omitted.
template <int D, int BITS, bool MIXED = false>
__device__ __forceinline__ void quantize_rows_store(float (&x)[4][16], const float *ic_vec,
                                                    uint8_t *rec, Rows<D, BITS, MIXED> rows = {}) {
#pragma clang fp contract(off)
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    float *rp = reinterpret_cast<float *>(rec + rows.codes_bytes());
    float rm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4) {
        const float4 f = *reinterpret_cast<const float4 *>(ic_vec + colvec4_idx(16 * cg + 4 * n4));
        const float ic[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 4 * n4 + i;
                x[m][n] = x[m][n] * ic[i];
                rm[m] = fmaxf(rm[m], fabsf(x[m][n]));
            }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) rm[m] = band_max<G::CG>(rm[m]);
    // lane cg (< 4) of the band owns row band + NB * cg
    const float sel01 = (cg & 1) ? rm[1] : rm[0];
    const float sel23 = (cg & 1) ? rm[3] : rm[2];
    const float mrow = (cg & 2) ? sel23 : sel01;
    const int row_own = band + G::NB * (cg & 3);
    float r = div_qmax(mrow, rows.qmax(row_own), rows.inv_qmax(row_own));
    float ir;
    if (r >= FLT_MIN) {
        ir = recip_rn(r); // r <= (1 + 2^-23) / 7
    } else {
        r = 0.0f;
        ir = 0.0f;
    }
    if (cg < 4) rp[(uint32_t)(band + G::NB * cg)] = r;
    float irm[4];
    // broadcast lane (band base + m) to the band: ds_swizzle bit mode,
    // lane' = (lane & and_mask) | or_mask within 32 lanes
    constexpr int AND_MASK = 0x1F & ~(G::CG - 1);
    irm[0] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ir), AND_MASK | (0 << 5)));
    irm[1] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ir), AND_MASK | (1 << 5)));
    irm[2] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ir), AND_MASK | (2 << 5)));
    irm[3] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ir), AND_MASK | (3 << 5)));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        uint32_t f[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) f[n] = code_bits(x[m][n], irm[m]);
        rows.store(rec, row, cg, f);
    }
}

// ---------------------------------------------------------------- quant_state
template <int D, int BITS, bool MIXED = false>
__device__ __forceinline__ void quant_tile(uint8_t *rec, const float *S, float *lds,
                                           Rows<D, BITS, MIXED> rows = {}) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    float *plane = lds, *lds_ic = lds + G::NB * D;
    float *cp = reinterpret_cast<float *>(rec + rows.codes_bytes()) + D;
    float x[4][16];
#pragma unroll
    for (int m = 0; m < 4; ++m) load16<D>(S + (band + G::NB * m) * D + 16 * cg, x[m]);
    float cm[16];
#pragma unroll
    for (int n = 0; n < 16; ++n)
        cm[n] = fmaxf(fmaxf(fabsf(x[0][n]), fabsf(x[1][n])), fmaxf(fabsf(x[2][n]), fabsf(x[3][n])));
    write_band_partials<D>(plane, cm);
    __syncthreads();
    if (t < D) lds_ic[colvec4_idx(t)] = column_scale(column_max<D>(plane, t), cp + t);
    __syncthreads();
    quantize_rows_store<D, BITS, MIXED>(x, lds_ic, rec, rows);
}

// ---------------------------------------------------------------- FP16 pivot records
// bits = 16: the record is the state itself as IEEE binary16, row-major, no
// scales (the highest-risk heads kept in FP16 as pivots).  Conversions are
// round-to-nearest-even (v_cvt_f16_f32) and exact widening (v_cvt_f32_f16).
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float half_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float half_at(const uint32_t (&w)[8], int n) {
    return (n & 1) ? half_hi(w[n >> 1]) : half_lo(w[n >> 1]);
}

template <int D>
__device__ __forceinline__ void load_half16(const uint8_t *rec, int row, int cg, uint32_t (&w)[8]) {
    const uint4 *p = reinterpret_cast<const uint4 *>(rec + 2 * (row * D + 16 * cg));
    const uint4 a = p[0], b = p[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <int D>
__device__ __forceinline__ void store_half16(uint8_t *rec, int row, int cg, const float (&v)[16]) {
    uint4 *p = reinterpret_cast<uint4 *>(rec + 2 * (row * D + 16 * cg));
    p[0] = make_uint4(pack_half2(v[0], v[1]), pack_half2(v[2], v[3]), pack_half2(v[4], v[5]),
                      pack_half2(v[6], v[7]));
    p[1] = make_uint4(pack_half2(v[8], v[9]), pack_half2(v[10], v[11]), pack_half2(v[12], v[13]),
                      pack_half2(v[14], v[15]));
}

template <int D> __device__ __forceinline__ void quant_tile_f16(uint8_t *rec, const float *S) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float v[16];
        load16<D>(S + (band + G::NB * m) * D + 16 * cg, v);
        store_half16<D>(rec, band + G::NB * m, cg, v);
    }
}

template <int D> __device__ __forceinline__ void dequant_tile_f16(const uint8_t *rec, float *S) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        uint32_t w[8];
        load_half16<D>(rec, row, cg, w);
        float4 *dst = reinterpret_cast<float4 *>(S + row * D + 16 * cg);
#pragma unroll
        for (int n4 = 0; n4 < 4; ++n4)
            dst[n4] = make_float4(half_at(w, 4 * n4), half_at(w, 4 * n4 + 1), half_at(w, 4 * n4 + 2),
                                  half_at(w, 4 * n4 + 3));
    }
}

template <int D>
__global__ __launch_bounds__(Geo<D>::NT) void quant_state_kernel(PoolView pool, HeadTable tab,
                                                                 const int32_t *slot,
                                                                 const float *S) {
    __shared__ __attribute__((aligned(16))) float lds[Geo<D>::NB * D + D];
    int b, h;
    tile_bh(pool, blockIdx.x, b, h);
    const uint32_t info = tab.info[h];
    uint8_t *rec = pool.base + (int64_t)slot[b] * pool.slot_stride + tab.off[h];
    const float *src = S + (int64_t)blockIdx.x * D * D;
    switch (info_bits(info)) {
    case 0: quant_tile<D, 8, true>(rec, src, lds, {info_n4(info), info_n6(info)}); break;
    case 4: quant_tile<D, 4>(rec, src, lds); break;
    case 6: quant_tile<D, 6>(rec, src, lds); break;
    case 16: quant_tile_f16<D>(rec, src); break;
    default: quant_tile<D, 8>(rec, src, lds); break;
    }
}

// ---------------------------------------------------------------- dequant_state
template <int D, int BITS, bool MIXED = false>
__device__ __forceinline__ void dequant_tile(const uint8_t *rec, float *S,
                                             Rows<D, BITS, MIXED> rows = {}) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    const float *rp = reinterpret_cast<const float *>(rec + rows.codes_bytes());
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
        const Seg<BITS> s = rows.load(rec, row, cg);
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
    int b, h;
    tile_bh(pool, blockIdx.x, b, h);
    const uint32_t info = tab.info[h];
    const uint8_t *rec = pool.base + (int64_t)slot[b] * pool.slot_stride + tab.off[h];
    float *dst = S + (int64_t)blockIdx.x * D * D;
    switch (info_bits(info)) {
    case 0: dequant_tile<D, 8, true>(rec, dst, {info_n4(info), info_n6(info)}); break;
    case 4: dequant_tile<D, 4>(rec, dst); break;
    case 6: dequant_tile<D, 6>(rec, dst); break;
    case 16: dequant_tile_f16<D>(rec, dst); break;
    default: dequant_tile<D, 8>(rec, dst); break;
    }
}

// ---------------------------------------------------------------- decode step
// LDS of the decode step (floats from the base):
//   [0, MAIN_F)           the tile's codes as bytes (D x D); after the step has
//                         read them, the column-maximum partials of S' in the
//                         same dwords (the dword of column j and key quad band
//                         holds that band's partial of column j).  The FP16
//                         pivot step uses it for its pair-summed FP64 look-up
//                         partials and then its read-out partials.  WIDE (the
//                         key-row-aware fit): 2 NB x D floats, its two FP64
//                         column sums.
//   [XCH_F, +3 NW BPW 32) the FP64 digit-sum exchange of the look-up
//   [DIG_F, +4 D + 32)    digit rows of the look-up and read-out factors (16 rows of
//                         D bytes, row pitch D + 8 bytes)
//   [IC_F, +D)            1/c'_j
//   [CU_F, +2 D + 32)     {c_j, u_j}, padded to 18 per 16 columns
//   [MISC_F, +16)         the GDN gate
// Without WIDE that is 23.3 KB at d = 128, so LDS does not limit a CU to
// fewer workgroups than the register budget does.
template <int D, bool WIDE = false> struct DecodeLds {
    static constexpr int MAIN_F = WIDE ? 2 * Geo<D>::NB * D : D * D / 4;
    static constexpr int XCH_F = MAIN_F;
    static constexpr int DIG_F = XCH_F + 3 * Geo<D>::NW * (Geo<D>::CG / Geo<D>::NW) * 32;
    static constexpr int IC_F = DIG_F + 4 * D + 32, CU_F = IC_F + D, MISC_F = CU_F + 2 * D + 32;
    static constexpr int TOTAL = MISC_F + 16;
};

// Lane t of a band of CG lanes reads lane (band base + m) with ds_swizzle
// (bit mode: lane' = (lane & and_mask) | or_mask, within 32 lanes).
template <int CG, int M> __device__ __forceinline__ float band_bcast(float v) {
    constexpr int AND_MASK = 0x1F & ~(CG - 1);
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), AND_MASK | (M << 5)));
}

// v plus the value of the lane holding the other band of the lane's band pair
// (lanes t and t ^ CG within a wave): DPP row rotation by 8 for CG = 8,
// ds_swizzle with xor mask 4 for CG = 4.  Both lanes get the same sum.
template <int CG> __device__ __forceinline__ double pair_sum(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
    if constexpr (CG == 8) {
        lo = __builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, false); // row_ror:8
        hi = __builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, false);
    } else {
        static_assert(CG == 4, "band pairs of 4 or 8 lanes");
        lo = __builtin_amdgcn_ds_swizzle(lo, 0x1F | (4 << 10));
        hi = __builtin_amdgcn_ds_swizzle(hi, 0x1F | (4 << 10));
    }
    return v + __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// ---------------------------------------------------------------- key-row-aware fit
// Requantization with the key-row-aware dual-axis fit (hyper.ai summary,
// "Method", the Key-Row-Aware Dual-Axis Fitting paragraph): per key row a
// row-impact score imp_i > 0 (calibrated offline), in fp32 with one rounding
// per operation unless FP64 is named:
//   r_i = sqrt(max_j |S'_ij| / imp_i), ir_i = 1 / r_i      (0 for zero rows)
//   s_ij = S'_ij ir_i; c0_j = max_i |s_ij| / qmax           (range-covering)
//   P_ij = nearest level of s_ij / c0_j (exact product s * (1 / c0))
//   w_i = imp_i r_i^2; A_j = sum_i w_i s_ij P_ij, B_j = sum_i w_i P_ij^2  (FP64)
//   c_j = B_j > 0 ? (float)(A_j / B_j) : c0_j   (the impact-weighted least-
//          squares scale for the codes P)
//   Q_ij = nearest level of s_ij / c_j, clamped to [-qmax, qmax]
// The FP64 sums run in one pass: each lane sums its 4 rows, lane pairs add
// their two bands, and the A and B pair sums share the 32 KB partials
// region.  c_j >= c0_j / 2 (a weighted average of s / P over |P| >= 1), so
// |s / c_j| <= 2 qmax and the magic-number rounding stays exact.
// Per-key-row widths (MIXED, blog.ontle.kr allocation paragraph): row i
// takes its own qmax_i; with qref the head's largest, its row factor is
// widened by g_i = qref / qmax_i (fp32) and the range-covering scale is
// c0_j = max_i (|s_ij| g_i) / qref, so each row spans its own levels on the
// shared column grid; the final codes clamp to each row's range.  Rounding
// errors keep |s ic0| <= qmax_i (1 + 4 eps) < qmax_i + 1/2, so P needs no
// clamp.  With uniform widths g_i = 1 and this is the rule above.
template <int D, int BITS, bool MIXED = false>
__device__ __forceinline__ void kra_quantize_store(float (&x)[4][16], const float *imp,
                                                   uint8_t *rec, float *lds,
                                                   Rows<D, BITS, MIXED> rows = {}) {
#pragma clang fp contract(off)
    using G = Geo<D>;
    const float MAGIC = magic_vgpr(); // 1.5 * 2^23
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    double *part64 = reinterpret_cast<double *>(lds);
    float *plane = lds; // column maxima; used (and reduced) before part64
    float *lds_c0 = lds + DecodeLds<D, true>::DIG_F + 2 * D; // digit rows: dead by now
    float *lds_ic = lds + DecodeLds<D, true>::IC_F;
    float *rp = reinterpret_cast<float *>(rec + rows.codes_bytes());
    float *cp = rp + D;
    // the head's widest rows (widths never decrease along the rows)
    const float QREF = rows.qmax(D - 1);
    float gm[4]; // g of the lane's rows (wavefront-uniform: scalar registers)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        gm[m] = QREF / rows.qmax(band + G::NB * m);
        if constexpr (MIXED)
            gm[m] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gm[m])));
    }
    // ---- row magnitudes, reduced over the band's lanes
    float mu[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        mu[m] = 0.0f;
#pragma unroll
        for (int n = 0; n < 16; ++n) mu[m] = fmaxf(mu[m], fabsf(x[m][n]));
        mu[m] = band_max<G::CG>(mu[m]);
    }
    // ---- row factors: lane cg (< 4) of the band owns row band + NB * cg
    const float sel01 = (cg & 1) ? mu[1] : mu[0];
    const float sel23 = (cg & 1) ? mu[3] : mu[2];
    const float mrow = (cg & 2) ? sel23 : sel01;
    const int row_own = band + G::NB * (cg & 3);
    const float im = imp[row_own];
    float r = 0.0f;
    if (mrow >= FLT_MIN) r = sqrtf(mrow / im) * (QREF / rows.qmax(row_own));
    if (!(r >= FLT_MIN) || r == INFINITY) r = 0.0f;
    const float ir = r > 0.0f ? 1.0f / r : 0.0f;
    if (cg < 4) rp[(uint32_t)(band + G::NB * cg)] = r;
    constexpr int AND_MASK = 0x1F & ~(G::CG - 1);
    float irm[4], wm_r[4], wm_i[4];
#define SQ_BCAST(v, m) __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), AND_MASK | ((m) << 5)))
    irm[0] = SQ_BCAST(ir, 0); irm[1] = SQ_BCAST(ir, 1); irm[2] = SQ_BCAST(ir, 2); irm[3] = SQ_BCAST(ir, 3);
    wm_r[0] = SQ_BCAST(r, 0); wm_r[1] = SQ_BCAST(r, 1); wm_r[2] = SQ_BCAST(r, 2); wm_r[3] = SQ_BCAST(r, 3);
    wm_i[0] = SQ_BCAST(im, 0); wm_i[1] = SQ_BCAST(im, 1); wm_i[2] = SQ_BCAST(im, 2); wm_i[3] = SQ_BCAST(im, 3);
#undef SQ_BCAST
    double w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) w[m] = (double)wm_i[m] * (double)wm_r[m] * (double)wm_r[m];
    // ---- row-scaled entries and their column maxima
    {
        float cm[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) cm[n] = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                x[m][n] = x[m][n] * irm[m];
                cm[n] = fmaxf(cm[n], fabsf(x[m][n]) * gm[m]);
            }
        write_band_partials<D>(plane, cm);
    }
    __syncthreads();
    if (t < D) {
        float c0 = column_max<D>(plane, t) / QREF;
        float ic0 = 0.0f;
        if (c0 >= FLT_MIN)
            ic0 = 1.0f / c0;
        else
            c0 = 0.0f;
        lds_c0[t] = c0;
        lds_ic[colvec4_idx(t)] = ic0;
    }
    __syncthreads();
    float ic[16];
    load_colvec16(lds_ic, cg, ic);
    // ---- the two FP64 column sums in one pass: each lane sums its 4 rows,
    //      the two bands of a lane pair (lanes t and t ^ CG of one wave) are
    //      added by a lane exchange, and the pair sums go through LDS (A in
    //      the first half of part64, B in the second, NB / 2 rows each)
    double *partA = part64, *partB = part64 + (G::NB / 2) * D;
#pragma unroll
    for (int n2 = 0; n2 < 8; ++n2) {
        double a[2] = {0.0, 0.0}, q[2] = {0.0, 0.0};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int n = 2 * n2 + e;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float P = __builtin_fmaf(x[m][n], ic[n], MAGIC) - MAGIC; // exact
                const double wp = w[m] * (double)P;
                a[e] = fma(wp, (double)x[m][n], a[e]);
                q[e] = fma(wp, (double)P, q[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            a[e] = pair_sum<G::CG>(a[e]);
            q[e] = pair_sum<G::CG>(q[e]);
        }
        if ((band & 1) == 0) {
            const int i = part_idx<D>(band >> 1, cg, 2 * n2);
            *reinterpret_cast<double2 *>(partA + i) = make_double2(a[0], a[1]);
            *reinterpret_cast<double2 *>(partB + i) = make_double2(q[0], q[1]);
        }
    }
    __syncthreads();
    if (t < D) {
        double A = 0.0, Bq = 0.0;
#pragma unroll 8
        for (int b = 0; b < G::NB / 2; ++b) {
            const int i = part_idx<D>(b, t >> 4, t & 15);
            A += partA[i];
            Bq += partB[i];
        }
        float c = Bq > 0.0 ? (float)(A / Bq) : lds_c0[t];
        if (!(c >= FLT_MIN)) c = 0.0f;
        cp[t] = c;
        lds_ic[colvec4_idx(t)] = c > 0.0f ? 1.0f / c : 0.0f;
    }
    __syncthreads();
    load_colvec16(lds_ic, cg, ic);
    constexpr uint32_t MB = 0x4B400000u; // bit pattern of MAGIC
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        uint32_t qm = (uint32_t)rows.qmax(row);
        if constexpr (MIXED) qm = __builtin_amdgcn_readfirstlane(qm);
        uint32_t f[16];
#pragma unroll
        for (int n = 0; n < 16; ++n)
            f[n] = min(max(code_bits(x[m][n], ic[n], MAGIC), MB - qm), MB + qm);
        rows.store(rec, row, cg, f);
    }
}

template <int D, int BITS, bool MIXED = false>
__device__ __forceinline__ void quant_tile_kra(uint8_t *rec, const float *S, const float *imp,
                                               float *lds, Rows<D, BITS, MIXED> rows = {}) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    float x[4][16];
#pragma unroll
    for (int m = 0; m < 4; ++m) load16<D>(S + (band + G::NB * m) * D + 16 * cg, x[m]);
    kra_quantize_store<D, BITS, MIXED>(x, imp, rec, lds, rows);
}

// ROWS: the pool has heads with per-key-row widths (their own kernel, so that
// the uniform bodies keep their register budget).
template <int D, bool ROWS>
__global__ __launch_bounds__(Geo<D>::NT) __attribute__((amdgpu_waves_per_eu(ROWS ? 3 : 4)))
void quant_state_kra_kernel(PoolView pool, HeadTable tab, const int32_t *slot, const float *S) {
    __shared__ __attribute__((aligned(16))) float lds[DecodeLds<D, true>::TOTAL];
    int b, h;
    tile_bh(pool, blockIdx.x, b, h);
    uint8_t *rec = pool.base + (int64_t)slot[b] * pool.slot_stride + tab.off[h];
    const float *src = S + (int64_t)blockIdx.x * D * D;
    const float *imp = pool.impact + (int64_t)h * D;
    const uint32_t info = tab.info[h];
    switch (info_bits(info)) {
    case 0:
        if constexpr (ROWS)
            quant_tile_kra<D, 8, true>(rec, src, imp, lds, {info_n4(info), info_n6(info)});
        break;
    case 4: quant_tile_kra<D, 4>(rec, src, imp, lds); break;
    case 6: quant_tile_kra<D, 6>(rec, src, imp, lds); break;
    case 16: quant_tile_f16<D>(rec, src); break;
    default: quant_tile_kra<D, 8>(rec, src, imp, lds); break;
    }
}

// Retention factor a = exp(g) rounded once to fp32 (through FP64 exp).
__device__ __forceinline__ float gate_factor(float g) { return (float)exp((double)g); }

// What one lane reads of one tile.
struct TileIn {
    uint32_t w[4][4];    // the lane's 4 row segments (BITS / 2 dwords used)
    float r[4];          // row scales of the lane's rows
    float k[4];          // k at the lane's rows
    float g;             // KDA: log-gate of row band + NB (cg & 3); GDN: the head's
    float beta;          // beta of the (b, h) row
    float cj, vj;        // c_j, v_j of the column whose look-up this lane completes
    float fk, fq, fr;    // k, q and r of the lane's factor row band + NB (cg & 3)
    float kb[2], qb[2], rb[2], gb[2]; // rows (t & 63) + 64 i, i < D / 64: every wave sees all rows
    uint8_t *rec;        // the tile's record
};

template <int D, int BITS, bool KDA, typename TI, bool MIXED>
__device__ __forceinline__ void load_tile(TileIn &in, int tile, uint8_t *rec, const StepIO &io,
                                          Rows<D, BITS, MIXED> rows) {
    using G = Geo<D>;
    constexpr int BPW = G::CG / G::NW;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    in.rec = rec;
    if constexpr (MIXED) {
        // raw segments, each in its row's own width (the step writes each
        // code as a byte with a branch on the row's width)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const Seg<8> raw = rows.load_raw(rec, band + G::NB * m, cg);
#pragma unroll
            for (int i = 0; i < 4; ++i) in.w[m][i] = raw.w[i];
        }
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const Seg<BITS> sg = rows.load(rec, band + G::NB * m, cg);
#pragma unroll
            for (int i = 0; i < Seg<BITS>::NWORDS; ++i) in.w[m][i] = sg.w[i];
        }
    }
    const float *rp = reinterpret_cast<const float *>(rec + rows.codes_bytes());
    const int64_t row_io = tile;
    const TI *k = reinterpret_cast<const TI *>(io.k) + row_io * D;
    const TI *q = reinterpret_cast<const TI *>(io.q) + row_io * D;
    const TI *g = reinterpret_cast<const TI *>(io.g);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        in.r[m] = rp[row];
        in.k[m] = ld<TI>(k, row);
    }
    in.g = KDA ? ld<TI>(g, row_io * D + band + G::NB * (cg & 3)) : ld<TI>(g, row_io);
    in.beta = ld<TI>(reinterpret_cast<const TI *>(io.beta), row_io);
    // the column this lane completes in the look-up: 16 (w BPW + b) + (lane & 15)
    // with b = (lane >> 4) & 3 (lanes with b >= BPW load a duplicate)
    const int jl = 16 * (BPW * (t >> 6) + (((t >> 4) & 3) % BPW)) + (t & 15);
    in.cj = rp[D + jl];
    in.vj = ld<TI>(reinterpret_cast<const TI *>(io.v) + row_io * D, jl);
    const int rowf = band + G::NB * (cg & 3);
    in.fk = ld<TI>(k, (uint32_t)rowf);
    in.fq = ld<TI>(q, (uint32_t)rowf);
    in.fr = rp[(uint32_t)rowf];
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
        const int row = (t & 63) + 64 * i;
        in.kb[i] = ld<TI>(k, row);
        in.qb[i] = ld<TI>(q, row);
        in.rb[i] = rp[row];
        in.gb[i] = KDA ? ld<TI>(g, row_io * D + row) : 0.0f;
    }
}

template <int BITS> __device__ __forceinline__ Seg<BITS> seg_of(const TileIn &in, int m) {
    Seg<BITS> s;
#pragma unroll
    for (int i = 0; i < Seg<BITS>::NWORDS; ++i) s.w[i] = in.w[m][i];
    return s;
}

// Codes in LDS during a step: column j holds its D codes as bytes in key
// order k = 4 band + m (row band + NB m), four keys per dword.  The dword
// index within the column is XOR-swizzled with bits 0..2 and 4..6 of j (bits
// 2..4 of the index), so that every half-wave access touches 32 distinct
// banks: the byte writes and phase-2 reads of one code position (lanes: 4
// bands x 8 column groups) and the matrix-core fragment reads (16 columns x
// 2 key groups x 2 dwords).
template <int D> __device__ __forceinline__ int code_sw(int j) {
    return (((((j & 3) ^ (j >> 4)) & 3) << 3) | ((((j >> 2) ^ (j >> 6)) & 1) << 2));
}
template <int D> __device__ __forceinline__ int code_word(int j, int kq) {
    constexpr int NQ = D / 4;
    return j * NQ + (kq ^ (code_sw<D>(j) & (NQ - 1)));
}
// Digit rows: row d holds digit d of every key's factor, four keys per
// dword in the code columns' key order, rows D / 4 + 2 dwords apart.  The
// pitch (not a swizzle) keeps the matrix-core fragment reads (16 rows x 2
// key dwords) on distinct banks, so a lane's eight digit writes and its
// fragment reads all sit at fixed offsets from one base address.
template <int D> __device__ __forceinline__ int digit_word(int d, int kq) {
    return d * (D / 4 + 2) + kq;
}

// Wavefront maximum of non-negative ints and sum of floats: DPP within rows of
// 16 lanes (quad exchanges, then mirrors within 8 and 16), after which every
// lane holds its row's result; then row_bcast:15 folds row 0 into row 1 and
// row 2 into row 3, row_bcast:31 folds row 1 into rows 2 and 3, and lane 63
// holds the wavefront's result (sum order ((r2 + r3) + (r0 + r1))).
constexpr int kRowMirror = 0x140;   // row_mirror: lane i <-> 15 - i within 16
constexpr int kRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kRowBcast31 = 0x143;  // lane 31 to rows 2 and 3
template <int CTRL, int ROW_MASK> __device__ __forceinline__ uint32_t dpp_rows(uint32_t v) {
    // rows outside ROW_MASK keep v itself (the identity of max and of the
    // fold below, which adds 0 for them)
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
    v = max(v, dpp_u<kQuadXor1>(v));
    v = max(v, dpp_u<kQuadXor2>(v));
    v = max(v, dpp_u<kHalfMirror>(v));
    v = max(v, dpp_u<kRowMirror>(v));
    v = max(v, dpp_rows<kRowBcast15, 0xA>(v));
    v = max(v, dpp_rows<kRowBcast31, 0xC>(v));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_i(int v) {
    v = max(v, (int)dpp_u<kQuadXor1>((uint32_t)v));
    v = max(v, (int)dpp_u<kQuadXor2>((uint32_t)v));
    v = max(v, (int)dpp_u<kHalfMirror>((uint32_t)v));
    v = max(v, (int)dpp_u<kRowMirror>((uint32_t)v));
    v = max(v, (int)dpp_rows<kRowBcast15, 0xA>((uint32_t)v));
    v = max(v, (int)dpp_rows<kRowBcast31, 0xC>((uint32_t)v));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __uint_as_float(dpp_u<kQuadXor1>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u<kQuadXor2>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u<kHalfMirror>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u<kRowMirror>(__float_as_uint(v)));
    // rows 1 and 3: + lane 15 of rows 0 and 2; then rows 2 and 3: + lane 31
    const int lane = threadIdx.x & 63;
    const float b15 = __uint_as_float(dpp_rows<kRowBcast15, 0xA>(__float_as_uint(v)));
    v = (lane & 16) ? v + b15 : v;
    const float b31 = __uint_as_float(dpp_rows<kRowBcast31, 0xC>(__float_as_uint(v)));
    v = (lane & 32) ? v + b31 : v;
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Signed base-256 digits d_0..d_7 of an integer-valued X, |X| < 2^62: the
// bytes of (X + C) xor C with C = 0x8080...80, each read as int8, so that
// sum_i d_i 256^i = X exactly (each byte is u_i - 128 for the bytes u_i of
// X + C, and the range of such sums contains every |X| < 2^62).
__device__ __forceinline__ uint64_t digits8(double X) {
    const double hi = floor(X * 0x1p-32);
    const double lo = fma(hi, -0x1p32, X); // exact, in [0, 2^32)
    uint64_t K = ((uint64_t)(uint32_t)(int32_t)hi << 32) | (uint64_t)(uint32_t)lo;
    K += 0x8080808080808080ull;
    return K ^ 0x8080808080808080ull;
}

// 4 x 4 byte transpose: byte m of o[e] = byte e of row word m (a, b, c, d
// for m = 0..3), by two rounds of byte permutes.
__device__ __forceinline__ void byte_transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                uint32_t (&o)[4]) {
    const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u); // a0 b0 a1 b1
    const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u); // a2 b2 a3 b3
    const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u); // c0 d0 c1 d1
    const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u); // c2 d2 c3 d3
    o[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);          // a0 b0 c0 d0
    o[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);          // a1 b1 c1 d1
    o[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);          // a2 b2 c2 d2
    o[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);          // a3 b3 c3 d3
}

// Each byte's low nibble, a 4-bit two's-complement code n, sign-extended to
// the whole byte: n ^ 8 is in [0, 15], + 0x78 stays below 0x100 (no carry
// into the next byte), and flipping bit 7 of (n ^ 8) + 0x78 = c + 0x80
// gives c mod 256 for the code c.
__device__ __forceinline__ uint32_t sext_low_nibbles(uint32_t x) {
    return (((x & 0x0F0F0F0Fu) ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) volatile uint8_t lds_u8;

// One step of one (request, head) tile.
// Look-up and read-out: v_old_j = c_j sum_i a_i r_i k_i code_ij and the
// read-out's old-state term c_j sum_i a_i r_i q_i code_ij are exact integer
// sums on the matrix cores (int8 x int8 -> int32): the factors k_i r_i (a_i)
// of a tile are written as fixed-point integers on one exponent (an upper
// bound of the tile's largest), split into 8 signed base-256 digits (4 for
// the q factor), and the digit rows multiply the code bytes.  The digit sums,
// combined with one FP64 rounding, give the look-up at least as accurately as
// an FP64 sum; u_j is then rounded once to fp32.  y = S_d^T q + u (k.q) (the
// update's rank-1 term folded), to about 2^-27 relative before its output
// rounding.
// SPLIT: write S' (fp32) to io.s_out instead of requantizing; the record
// is only read.  The requantization then runs as its own launch.
// KRA: requantize with the key-row-aware fit (row-impact scores imp[D]).
// MIXED: per-key-row widths (instantiated with BITS = 8; each row's raw
// segment is read at its own width when its codes go to LDS).
template <int D, int BITS, bool KDA, bool SPLIT, bool KRA, typename TI, typename TO,
          bool MIXED = false>
__device__ __forceinline__ void decode_tile(uint8_t *rec_in, int tile, const StepIO &io,
                                            const float *imp, float *lds,
                                            Rows<D, BITS, MIXED> rows = {}) {
    using G = Geo<D>;
    using L = DecodeLds<D, KRA>;
    constexpr int NQ = D / 4;              // dwords per code column
    constexpr int BPW = G::CG / G::NW;     // 16-column blocks per wave
    constexpr int KS = D / 64;             // key steps of the matrix-core look-up (64 keys)
    static_assert(G::CG % G::NW == 0 && BPW <= 4, "column blocks per wave");
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    const int w = t >> 6, lg = (t >> 4) & 3, ln = t & 15;
    uint8_t *code_b = reinterpret_cast<uint8_t *>(lds);
    double *xch = reinterpret_cast<double *>(lds + L::XCH_F); // digit-sum exchange
    uint8_t *dig_b = reinterpret_cast<uint8_t *>(lds + L::DIG_F);
    float *lds_ic = lds + L::IC_F;
    float2 *lds_cu = reinterpret_cast<float2 *>(lds + L::CU_F); // {c_j, u_j} at 18 (j / 16) + j % 16
    float *misc = lds + L::MISC_F; // [15]: GDN gate
    SQ_TL(1);
    TileIn cur;
    load_tile<D, BITS, KDA, TI, MIXED>(cur, tile, rec_in, io, rows);
#ifdef SQ_TIMELINE
    asm volatile("" ::"v"(cur.w[0][0]), "v"(cur.w[3][0]), "v"(cur.kb[1]), "v"(cur.qb[1]), "v"(cur.cj),
                 "v"(cur.vj), "v"(cur.fk), "v"(cur.fq), "v"(cur.fr), "v"(cur.beta));
#endif
    SQ_TL(2);
    uint8_t *rec = cur.rec;
    float *cp = reinterpret_cast<float *>(rec + rows.codes_bytes()) + D;
    const int64_t row_io = tile;
    // byte addresses of the lane's codes of columns 16 cg + n, one per value
    // of (n & 7): 4 code_word(16 cg + n, band) = cbase[n & 7] + 4 n NQ.  For
    // n < 8 the swizzle splits, code_sw(16 cg + n) = code_sw(16 cg) ^
    // code_sw(n), and it only touches the bits below NQ, so the lane part is
    // formed once and each n & 7 is one XOR with a constant.
    const int cb0 = 4 * (16 * cg * NQ + (band ^ (code_sw<D>(16 * cg) & (NQ - 1))));
    int cbase[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) cbase[q] = cb0 ^ (4 * (code_sw<D>(q) & (NQ - 1)));
    // ---- retention factors: GDN one per head (one lane, shared through LDS
    //      after the first barrier); KDA one per key row, computed by lane
    //      cg & 3 of each band for row band + NB (cg & 3) and broadcast.
    float am[4];
    float ga = 0.0f; // KDA: the gate of row band + NB (cg & 3)
    if constexpr (KDA) {
        ga = gate_factor(cur.g);
        am[0] = band_bcast<G::CG, 0>(ga);
        am[1] = band_bcast<G::CG, 1>(ga);
        am[2] = band_bcast<G::CG, 2>(ga);
        am[3] = band_bcast<G::CG, 3>(ga);
    } else {
        if (t == 0) misc[15] = gate_factor(cur.g);
    }
    // ---- the lane's codes into LDS: per column n a dword of its four rows'
    //      code bytes, at d = 128 also kept in cws[n] for the update after the
    //      matrix cores (no second read of LDS; at d = 64 the register budget
    //      does not allow it and the update reads them back)
    uint32_t cws[16];
    if constexpr (MIXED) {
        // per row, one wavefront-uniform branch on its width; rows 0, 1 and
        // then 2, 3 are gathered into the column dwords, which go to LDS as
        // in the uniform case below
        uint32_t pk[16];
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
            int c[2][16];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int m = 2 * mp + e;
                const int wd = __builtin_amdgcn_readfirstlane(rows.width(band + G::NB * m));
                const Seg<8> raw = seg_of<8>(cur, m);
                if (wd == 4) {
                    const Seg<4> sg = as_seg<4>(raw);
#pragma unroll
                    for (int n = 0; n < 16; ++n) c[e][n] = code_at<4>(sg, n);
                } else if (wd == 6) {
                    const Seg<6> sg = as_seg<6>(raw);
#pragma unroll
                    for (int n = 0; n < 16; ++n) c[e][n] = code_at<6>(sg, n);
                } else {
#pragma unroll
                    for (int n = 0; n < 16; ++n) c[e][n] = code_at<8>(raw, n);
                }
            }
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                if (mp == 0)
                    pk[n] = __builtin_amdgcn_perm((uint32_t)c[1][n], (uint32_t)c[0][n], 0x0c0c0400u);
                else
                    pk[n] |= __builtin_amdgcn_perm((uint32_t)c[1][n], (uint32_t)c[0][n], 0x04000c0cu);
            }
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            uint32_t *cw = reinterpret_cast<uint32_t *>(code_b + cbase[n] + 4 * n * NQ);
            cw[0] = pk[n];
            cw[8 * NQ] = pk[n + 8];
        }
        if constexpr (D == 128) {
#pragma unroll
            for (int n = 0; n < 16; ++n) cws[n] = pk[n];
        }
    } else if constexpr (BITS == 8 || BITS == 4) {
        // 8 and 4 bits: the code fields sit on byte (nibble) boundaries, so
        // the column dwords are a 4 x 4 byte transpose of the rows' segment
        // words (8 byte permutes per 4 dwords), at 4 bits followed by the
        // sign extension of each byte's low or high nibble (SWAR, 7
        // instructions per 8 codes) instead of one bit-field extract per code
        uint32_t cd[16]; // cd[n]: the dword of column 16 cg + n
        if constexpr (BITS == 8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t o[4];
                byte_transpose4(cur.w[0][q], cur.w[1][q], cur.w[2][q], cur.w[3][q], o);
#pragma unroll
                for (int e = 0; e < 4; ++e) cd[4 * q + e] = o[e];
            }
        } else {
#pragma unroll
            for (int hw = 0; hw < 2; ++hw) {
                uint32_t o[4]; // byte m of o[e]: the two codes of columns 8 hw + 2 e, + 1 of row m
                byte_transpose4(cur.w[0][hw], cur.w[1][hw], cur.w[2][hw], cur.w[3][hw], o);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cd[8 * hw + 2 * e] = sext_low_nibbles(o[e]);
                    cd[8 * hw + 2 * e + 1] = sext_low_nibbles(o[e] >> 4);
                }
            }
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            uint32_t *cw = reinterpret_cast<uint32_t *>(code_b + cbase[n] + 4 * n * NQ);
            cw[0] = cd[n];
            cw[8 * NQ] = cd[n + 8];
            if constexpr (D == 128) {
                cws[n] = cd[n];
                cws[n + 8] = cd[n + 8];
            }
        }
    } else {
        Seg<BITS> seg[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) seg[m] = seg_of<BITS>(cur, m);
        // one dword per column: the four rows' codes gathered by two byte
        // permutes and an OR, one LDS write (single-byte writes, four per
        // column, kept the LDS busy longer than the three instructions take)
        // columns n and n + 8 share the address base cbase[n & 7], 8 d / 4
        // dwords apart, so their two writes issue as one paired write
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            uint32_t wd[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t b[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) b[m] = (uint32_t)code_at<BITS>(seg[m], n + 8 * h);
                const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u); // b0, b1 in bytes 0, 1
                const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu); // b2, b3 in bytes 2, 3
                wd[h] = lo | hi;
            }
            uint32_t *cw = reinterpret_cast<uint32_t *>(code_b + cbase[n] + 4 * n * NQ);
            cw[0] = wd[0];
            cw[8 * NQ] = wd[1];
            if constexpr (D == 128) {
                cws[n] = wd[0];
                cws[n + 8] = wd[1];
            }
        }
    }
    SQ_TL(3);
    // ---- factors of key k = 4 band + m in FP64: look-up k_i r_i, read-out
    //      q_i r_i (times a_i for KDA; the GDN gate scales the sums).  D = 128:
    //      lane cg < 4 takes the k factor of row m = cg, cg >= 4 the q factor of
    //      row cg - 4; D = 64: both factors of row m = cg.
    constexpr int NJOB = 8 / G::CG;
    double fx[NJOB];
    const int jm = cg & 3;
#pragma unroll
    for (int jb = 0; jb < NJOB; ++jb) {
        const int vec = G::CG == 8 ? (cg >> 2) : jb;
        double x = (double)(vec ? cur.fq : cur.fk) * (double)cur.fr;
        if constexpr (KDA) x *= (double)ga; // the gate of the same row
        fx[jb] = x;
    }
    // ---- the tile's exponents, computed by every wave over all D rows (no
    //      exchange between waves): Ek >= the biased FP64 exponent of every k
    //      factor, Eq of every q factor, from the fp32 exponent fields e(.)
    //      of k (or q) and r: |k r| < 2^(e(k) + e(r) - 252) (zero and
    //      subnormal fields 0 included), so the FP64 field of k r is at most
    //      e(k) + e(r) + 770, at most one above the exact one.  The fields
    //      are added in place (bits 23..31) and shifted once after the
    //      reduction.  KDA: the gate enters through a bound, a_i = exp(g_i) <
    //      2^(ceil(g_i log2 e) + 1).  A larger E only drops bits far below
    //      the 53 the look-up needs (|X| < 2^62).  And k.q.
    constexpr uint32_t EXPM = 0x7F800000u;
    int Ek, Eq;
    float kq = 0.0f;
    if constexpr (KDA) {
        int ek = 0, eq = 0;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const uint32_t er = __float_as_uint(cur.rb[i]) & EXPM;
            const int ea = (int)ceilf(cur.gb[i] * 1.44269504f) + 2;
            ek = max(ek, (int)(((__float_as_uint(cur.kb[i]) & EXPM) + er) >> 23) + ea);
            eq = max(eq, (int)(((__float_as_uint(cur.qb[i]) & EXPM) + er) >> 23) + ea);
            kq = fmaf(cur.kb[i], cur.qb[i], kq);
        }
        Ek = wave_max_i(ek) + 770;
        Eq = wave_max_i(eq) + 770;
    } else {
        uint32_t ek = 0, eq = 0;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const uint32_t er = __float_as_uint(cur.rb[i]) & EXPM;
            ek = max(ek, (__float_as_uint(cur.kb[i]) & EXPM) + er);
            eq = max(eq, (__float_as_uint(cur.qb[i]) & EXPM) + er);
            kq = fmaf(cur.kb[i], cur.qb[i], kq);
        }
        Ek = (int)(wave_max_u(ek) >> 23) + 770;
        Eq = (int)(wave_max_u(eq) >> 23) + 770;
    }
    kq = wave_sum_dpp(kq);
#ifdef SQ_TIMELINE
    asm volatile("" ::"v"(kq), "s"(Ek), "s"(Eq));
#endif
    SQ_TL(4);
    // ---- digit rows: the k factors as integers X_i = rint(x_i 2^(61 - e)) on
    //      the tile's exponent e (|X| < 2^62, 8 digits, rows 0..7); the q
    //      factors likewise with |X| < 2^30 (4 digits, rows 8..11).  One code
    //      path for both: a q factor's digits 4..7 are zero and land in rows
    //      12..15, which the matrix cores never read.
#pragma unroll
    for (int jb = 0; jb < NJOB; ++jb) {
        const int vec = G::CG == 8 ? (cg >> 2) : jb;
        const uint64_t dg = digits8(rint(ldexp(fx[jb], vec ? 1052 - Eq : 1084 - Ek)));
        const int r0 = vec ? 8 : 0;
#pragma unroll
        for (int d = 0; d < 8; ++d)
            dig_b[4 * digit_word<D>(r0 + d, band) + jm] = (uint8_t)(dg >> (8 * d));
    }
    SQ_TL(5);
    __syncthreads();
    SQ_TL(6);
    if constexpr (!KDA) {
        const float a = misc[15];
        am[0] = am[1] = am[2] = am[3] = a;
    }
    // ---- matrix cores: digit sums D[d][j] = sum_k digit_d(X_k) code_kj for the
    //      wave's column blocks, all keys (rows 12..15 of A are zero)
    v4i acc[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b) acc[b] = v4i{0, 0, 0, 0};
    // byte addresses of key step 0; lane group lg takes keys 16 lg .. 16 lg
    // + 15 of each step, in A and in B alike (the sum does not depend on how
    // the matrix core orders the keys within a group, as long as both
    // operands use the same keys).  Code fragments: 16 aligned bytes (the
    // swizzle moves whole 4-dword groups); key step s2 moves only address
    // bit 6 (index bit 4 of 16 s2, which the swizzle XORs but never
    // carries), so step s2 is step 0 XOR (s2 << 6); the code swizzle splits
    // as above (column 16 c + ln is column ln XOR the wave-uniform part of
    // c).  Digit fragments: 8-byte aligned (row pitch d + 8 bytes), read as
    // two 8-byte halves; step s2 is 64 s2 bytes on.
    const int a_dig = 4 * digit_word<D>(ln, 4 * lg);
    const int a_cw = 4 * code_word<D>(ln, 4 * lg);
    const int wu = __builtin_amdgcn_readfirstlane(w);
    int a_code[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        const int c = wu * BPW + b;
        a_code[b] = (a_cw ^ (4 * (code_sw<D>(16 * c) & (NQ - 1)))) + 64 * c * NQ;
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
        v4i A = v4i{0, 0, 0, 0};
        if (ln < 12) {
            const long *pa = reinterpret_cast<const long *>(dig_b + a_dig + 64 * s2);
            const long a0 = pa[0], a1 = pa[1];
            A = v4i{(int)a0, (int)(a0 >> 32), (int)a1, (int)(a1 >> 32)};
        }
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const v4i B = *reinterpret_cast<const v4i *>(code_b + (a_code[b] ^ (s2 << 6)));
            acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc[b], 0, 0, 0);
        }
    }
    // lane (lg, ln) holds digits 4 lg .. 4 lg + 3 of column 16 cb + ln: their
    // weighted sum is exact in FP64 (|sum| < 2^46); lanes lg = 1 (digits 4..7)
    // and lg = 2 (q digits) hand theirs to lane lg = 0 through LDS
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        const double part = fma((double)acc[b][3], 0x1p24,
                                fma((double)acc[b][2], 0x1p16, fma((double)acc[b][1], 0x1p8, (double)acc[b][0])));
        if (lg < 3) xch[((w * BPW + b) * 3 + lg) * 16 + ln] = part;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane (b, ln), b < BPW, completes column 16 (w BPW + b) + ln
    if (lg < BPW) {
        const int cbk = w * BPW + lg, j = 16 * cbk + ln;
        const double *px = xch + cbk * 48 + ln;
        double P = ldexp(fma(px[16], 0x1p32, px[0]), Ek - 1084); // sum_i k_i r_i (a_i) code_ij
        double Y = ldexp(px[32], Eq - 1052);                      // sum_i q_i r_i (a_i) code_ij
        if constexpr (!KDA) {
            P *= (double)am[0];
            Y *= (double)am[0];
        }
        const double cj = (double)cur.cj;
        // u_j in FP64, rounded once to fp32
        const float u = (float)((double)cur.beta * ((double)cur.vj - P * cj));
        lds_cu[18 * cbk + ln] = make_float2(cur.cj, u);
        st<TO>(reinterpret_cast<TO *>(io.y) + row_io * D, j, (float)fma((double)u, (double)kq, Y * cj));
    }
    SQ_TL(7);
    __syncthreads();
    SQ_TL(8);
    // ---- decay + delta write in fp32: S'_mn = fma(code, (a_m r_m) c_n, k_m u_n),
    //      each product rounded once; the column-maximum partial of the lane's
    //      four rows replaces the code dword it was computed from (only this
    //      lane reads that dword after the matrix cores, which finished before
    //      the last barrier)
    float x[4][16];
    {
        float ar[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ar[m] = am[m] * cur.r[m];
        // the lane's 16 {c, u} pairs: 8 aligned 16-byte reads (stride 18 pairs
        // per column group: 4 cg + 2 n mod 32 words, no bank conflicts)
        const float4 *cu4 = reinterpret_cast<const float4 *>(lds_cu + 18 * cg);
        if constexpr (D != 128) {
            // all 16 code dwords are read before the first partial overwrites
            // one (the compiler cannot tell the addresses apart, so reads placed
            // after a write would each wait for the LDS round trip)
#pragma unroll
            for (int n = 0; n < 16; ++n)
                cws[n] = *reinterpret_cast<const uint32_t *>(code_b + cbase[n & 7] + 4 * n * NQ);
        }
        if constexpr (D == 128) {
            // columns n and n + 8 one after the other, so that their two
            // partials (same address base, 8 d / 4 dwords apart) are written
            // as one paired write
#pragma unroll
            for (int n2 = 0; n2 < 4; ++n2) {
                const float4 pa = cu4[n2], pb = cu4[n2 + 4];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int n = 2 * n2 + e;
                    float cmv[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int nn = n + 8 * h;
                        const float4 p = h ? pb : pa;
                        const float2 cu = e ? make_float2(p.z, p.w) : make_float2(p.x, p.y);
                        const uint32_t cw = cws[nn];
                        float cm = 0.0f;
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const float code = (float)(int8_t)(cw >> (8 * m));
                            const float sf = fmaf(code, ar[m] * cu.x, cur.k[m] * cu.y);
                            x[m][nn] = sf;
                            cm = fmaxf(cm, fabsf(sf));
                        }
                        cmv[h] = cm;
                    }
                    if constexpr (!SPLIT && !KRA) {
                        uint32_t *cwp = reinterpret_cast<uint32_t *>(code_b + cbase[n] + 4 * n * NQ);
                        cwp[0] = __float_as_uint(cmv[0]);
                        cwp[8 * NQ] = __float_as_uint(cmv[1]);
                    }
                }
            }
        } else {
            // d = 64 (one wave): column by column, which keeps its
            // register budget without spills
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const float2 cu = reinterpret_cast<const float2 *>(cu4)[n];
                uint32_t *cwp = reinterpret_cast<uint32_t *>(code_b + cbase[n & 7] + 4 * n * NQ);
                const uint32_t cw = cws[n];
                float cm = 0.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float code = (float)(int8_t)(cw >> (8 * m));
                    const float sf = fmaf(code, ar[m] * cu.x, cur.k[m] * cu.y);
                    x[m][n] = sf;
                    cm = fmaxf(cm, fabsf(sf));
                }
                if constexpr (!SPLIT && !KRA) *cwp = __float_as_uint(cm);
            }
        }
    }
    if constexpr (SPLIT) {
        // each lane's 64 contiguous bytes of a row back to back (interleaving
        // the rows per 16-byte chunk measured 1.8x slower on MI355X)
        float *s_out = io.s_out + (int64_t)tile * D * D;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float4 *dst = reinterpret_cast<float4 *>(s_out + (band + G::NB * m) * D + 16 * cg);
#pragma unroll
            for (int n4 = 0; n4 < 4; ++n4)
                dst[n4] = make_float4(x[m][4 * n4], x[m][4 * n4 + 1], x[m][4 * n4 + 2],
                                      x[m][4 * n4 + 3]);
        }
        return;
    }
    SQ_TL(9);
    __syncthreads();
    SQ_TL(10);
    if constexpr (KRA) {
        kra_quantize_store<D, BITS, MIXED>(x, imp, rec, lds, rows);
    } else {
        if (t < D) {
            // the 32 band partials of column t: its code dwords, 16 bytes at a
            // time, in the order of the column's own swizzle (chunk i XOR the
            // swizzle's chunk bits: eight consecutive columns' swizzles differ
            // in index bits 2..4, so each 16-byte read of eight lanes covers
            // all banks; in plain order every lane would read the same four)
            const uint4 *col = reinterpret_cast<const uint4 *>(code_b + 4 * t * NQ);
            const int sc = (code_sw<D>(t) & (NQ - 1)) >> 2;
            uint32_t cmax = 0;
#pragma unroll
            for (int i = 0; i < NQ / 4; ++i) {
                const uint4 v = col[i ^ sc];
                cmax = max(cmax, max(max(v.x, v.y), max(v.z, v.w)));
            }
            lds_ic[colvec4_idx(t)] = column_scale(__uint_as_float(cmax), cp + (uint32_t)t);
        }
        SQ_TL(11);
        __syncthreads();
        SQ_TL(12);
        quantize_rows_store<D, BITS, MIXED>(x, lds_ic, rec, rows);
        SQ_TL(13);
    }
}

// FP16 pivot record: the same FP64 look-up on the exactly widened state and
// the same fp32 update with unit scales, S' = fma(h_ij, a_i, k_i u_j), then
// rounded to binary16.
template <int D, bool KDA, bool SPLIT, typename TI, typename TO>
__device__ __forceinline__ void decode_tile_f16(uint8_t *rec, int tile, const StepIO &io,
                                                float *lds) {
    using G = Geo<D>;
    const int t = threadIdx.x, cg = t % G::CG, band = t / G::CG;
    double *part64 = reinterpret_cast<double *>(lds); // NB / 2 x D pair sums
    float *plane_y = lds;                               // NB x D, after part64 is read
    float2 *lds_cu = reinterpret_cast<float2 *>(lds + DecodeLds<D>::CU_F);
    float *lds_misc = lds + DecodeLds<D>::MISC_F;
    const int64_t row_io = tile;
    const TI *k = reinterpret_cast<const TI *>(io.k) + row_io * D;
    const TI *q = reinterpret_cast<const TI *>(io.q) + row_io * D;
    const TI *g = reinterpret_cast<const TI *>(io.g);

    float kf[4], qf[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int row = band + G::NB * m;
        kf[m] = ld<TI>(k, row);
        qf[m] = ld<TI>(q, row);
    }
    const float beta = ld<TI>(reinterpret_cast<const TI *>(io.beta), row_io);
    float vj = 0.0f;
    if (t < D) vj = ld<TI>(reinterpret_cast<const TI *>(io.v) + row_io * D, t);
    float am[4];
    if constexpr (KDA) {
        const float a = gate_factor(ld<TI>(g, row_io * D + band + G::NB * (cg & 3)));
        am[0] = band_bcast<G::CG, 0>(a);
        am[1] = band_bcast<G::CG, 1>(a);
        am[2] = band_bcast<G::CG, 2>(a);
        am[3] = band_bcast<G::CG, 3>(a);
    } else {
        if (t == 0) lds_misc[0] = gate_factor(ld<TI>(g, row_io));
    }
    {
        uint32_t w[4][8];
#pragma unroll
        for (int m = 0; m < 4; ++m) load_half16<D>(rec, band + G::NB * m, cg, w[m]);
        double ka[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ka[m] = KDA ? (double)kf[m] * (double)am[m] : (double)kf[m];
        // each lane sums its 4 rows, the two bands of a lane pair (lanes t
        // and t ^ CG) are added by a lane exchange, and the even band writes
#pragma unroll
        for (int n2 = 0; n2 < 8; ++n2) {
            double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                acc0 = fma(ka[m], (double)half_lo(w[m][n2]), acc0);
                acc1 = fma(ka[m], (double)half_hi(w[m][n2]), acc1);
            }
            acc0 = pair_sum<G::CG>(acc0);
            acc1 = pair_sum<G::CG>(acc1);
            if ((band & 1) == 0)
                *reinterpret_cast<double2 *>(part64 + part_idx<D>(band >> 1, cg, 2 * n2)) =
                    make_double2(acc0, acc1);
        }
    }
    __syncthreads();
    if constexpr (!KDA) {
        const float a = lds_misc[0];
        am[0] = am[1] = am[2] = am[3] = a;
    }
    if (t < D) {
        double P = 0.0;
#pragma unroll 8
        for (int b = 0; b < G::NB / 2; ++b) P += part64[part_idx<D>(b, t >> 4, t & 15)];
        if constexpr (!KDA) P *= (double)am[0];
        lds_cu[colvec2_idx(t)] = make_float2(1.0f, (float)((double)beta * ((double)vj - P)));
    }
    __syncthreads();
    {
        // each lane reads and writes only its own 4 x 16 elements, so the row
        // segments are loaded again here (after the barriers) rather than
        // held in registers across them
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            uint32_t wm[8];
            load_half16<D>(rec, band + G::NB * m, cg, wm);
            float o[16];
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const float un = lds_cu[colvec2_idx(16 * cg + n)].y;
                o[n] = fmaf(half_at(wm, n), am[m], kf[m] * un);
                // S' is rounded to fp32 first and binary16 second; the empty
                // asm keeps the compiler from fusing the fma with the
                // conversion (a mixed-precision fma rounds once, to binary16,
                // which differs on near-ties)
                asm volatile("" : "+v"(o[n]));
            }
            if constexpr (SPLIT) {
                float4 *dst = reinterpret_cast<float4 *>(io.s_out + (int64_t)tile * D * D +
                                                         (band + G::NB * m) * D + 16 * cg);
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4)
                    dst[n4] = make_float4(o[4 * n4], o[4 * n4 + 1], o[4 * n4 + 2], o[4 * n4 + 3]);
            } else {
                store_half16<D>(rec, band + G::NB * m, cg, o);
            }
            float ypart[16];
#pragma unroll
            for (int n = 0; n < 16; ++n) ypart[n] = qf[m] * o[n];
            if (m == 0) {
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4)
                    *reinterpret_cast<float4 *>(plane_y + plane_idx<D>(band, cg, 4 * n4)) =
                        make_float4(ypart[4 * n4], ypart[4 * n4 + 1], ypart[4 * n4 + 2],
                                    ypart[4 * n4 + 3]);
            } else {
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4) {
                    float4 *pp = reinterpret_cast<float4 *>(plane_y + plane_idx<D>(band, cg, 4 * n4));
                    float4 f = *pp;
                    f.x += ypart[4 * n4]; f.y += ypart[4 * n4 + 1];
                    f.z += ypart[4 * n4 + 2]; f.w += ypart[4 * n4 + 3];
                    *pp = f;
                }
            }
        }
    }
    __syncthreads();
    if (t < D) {
        float yv = 0.0f;
#pragma unroll 8
        for (int b = 0; b < G::NB; ++b) yv += plane_y[plane_idx<D>(b, t >> 4, t & 15)];
        st<TO>(reinterpret_cast<TO *>(io.y) + row_io * D, t, yv);
    }
}

// One workgroup per (request, head) tile, as many resident per CU as the
// register budget allows: five 4-wave workgroups (96 VGPRs, 23.3 KB of LDS
// each), which hides the loads, barriers and reduction phases of one tile
// behind the others.  Four with the key-row-aware fit (its FP64 column sums
// take 32 KB of LDS) and in pools with per-key-row widths (whose mixed-width
// body needs more than 96 VGPRs without spilling); three with both (about
// 140 VGPRs).  d = 64 tiles (one wave each, small heads) keep four waves
// per SIMD too: their body spills a few registers at 96.
template <int D, bool KRA, bool ROWS> constexpr int decode_waves_per_eu() {
    return KRA && ROWS ? 3 : (KRA || ROWS || D == 64 ? 4 : SQ_DECODE_WAVES);
}
// ROWS: the pool has heads with per-key-row widths (their own kernel, so
// that pools without them keep the register budget of the uniform bodies).
template <int D, bool KDA, bool SPLIT, bool KRA, bool ROWS, typename TI, typename TO>
__global__ __launch_bounds__(Geo<D>::NT) __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<D, KRA, ROWS>())))
void decode_kernel(PoolView pool, HeadTable tab, StepIO io) {
    __shared__ __attribute__((aligned(16))) float lds[DecodeLds<D, KRA>::TOTAL];
    const int tile = blockIdx.x;
    SQ_TL(0);
    // Two rounds of scalar loads before the record's address is known: the
    // pool and step arguments, then slot, offset and widths together (the
    // empty asm statements keep the compiler from spreading them over more
    // rounds).
    const int32_t *slot_idx = io.slot;
    uint8_t *base = pool.base;
    const int64_t stride = pool.slot_stride;
    asm volatile("" ::"s"(slot_idx), "s"(base), "s"(stride), "s"(pool.h_magic), "s"(pool.h_shift),
                 "s"(pool.n_heads));
    int b, h;
    tile_bh(pool, tile, b, h);
    // slot_idx is read-only for the kernel: a scalar (constant-space) load
    const int32_t slot =
        *(const __attribute__((address_space(4))) int32_t *)(uintptr_t)(slot_idx + b);
    const int64_t head_off = tab.off[h];
    const uint32_t info = tab.info[h];
    asm volatile("" ::"s"(slot), "s"(head_off), "s"(info));
    uint8_t *rec = base + (int64_t)slot * stride + head_off;
    const float *imp = KRA ? pool.impact + (int64_t)h * D : nullptr;
    switch (info_bits(info)) {
    case 0:
        if constexpr (ROWS)
            decode_tile<D, 8, KDA, SPLIT, KRA, TI, TO, true>(rec, tile, io, imp, lds,
                                                             {info_n4(info), info_n6(info)});
        break;
    case 4: decode_tile<D, 4, KDA, SPLIT, KRA, TI, TO>(rec, tile, io, imp, lds); break;
    case 6: decode_tile<D, 6, KDA, SPLIT, KRA, TI, TO>(rec, tile, io, imp, lds); break;
    case 16: decode_tile_f16<D, KDA, SPLIT, TI, TO>(rec, tile, io, lds); break;
    default: decode_tile<D, 8, KDA, SPLIT, KRA, TI, TO>(rec, tile, io, imp, lds); break;
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
template <int D, bool KDA, bool SPLIT, bool KRA, bool ROWS>
hipError_t decode_dispatch(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                           hipStream_t s) {
    const dim3 grid((unsigned)io.n * (unsigned)pool.n_heads), block(Geo<D>::NT);
    if (!io.in_bf16 && !io.y_bf16)
        hipLaunchKernelGGL((decode_kernel<D, KDA, SPLIT, KRA, ROWS, float, float>), grid, block, 0, s,
                           pool, tab, io);
    else if (!io.in_bf16 && io.y_bf16)
        hipLaunchKernelGGL((decode_kernel<D, KDA, SPLIT, KRA, ROWS, float, uint16_t>), grid, block, 0,
                           s, pool, tab, io);
    else if (io.in_bf16 && !io.y_bf16)
        hipLaunchKernelGGL((decode_kernel<D, KDA, SPLIT, KRA, ROWS, uint16_t, float>), grid, block, 0,
                           s, pool, tab, io);
    else
        hipLaunchKernelGGL((decode_kernel<D, KDA, SPLIT, KRA, ROWS, uint16_t, uint16_t>), grid, block,
                           0, s, pool, tab, io);
    return hipGetLastError();
}

template <bool SPLIT, bool KRA, bool ROWS>
hipError_t decode_gate_dispatch(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                                hipStream_t stream) {
    if (pool.d == 128)
        return io.kda ? decode_dispatch<128, true, SPLIT, KRA, ROWS>(pool, tab, io, stream)
                      : decode_dispatch<128, false, SPLIT, KRA, ROWS>(pool, tab, io, stream);
    return io.kda ? decode_dispatch<64, true, SPLIT, KRA, ROWS>(pool, tab, io, stream)
                  : decode_dispatch<64, false, SPLIT, KRA, ROWS>(pool, tab, io, stream);
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
    if (pool.impact) {
        if (pool.d == 128 && pool.row_mixed)
            hipLaunchKernelGGL((quant_state_kra_kernel<128, true>), grid, dim3(Geo<128>::NT), 0,
                               stream, pool, tab, slot, S);
        else if (pool.d == 128)
            hipLaunchKernelGGL((quant_state_kra_kernel<128, false>), grid, dim3(Geo<128>::NT), 0,
                               stream, pool, tab, slot, S);
        else if (pool.row_mixed)
            hipLaunchKernelGGL((quant_state_kra_kernel<64, true>), grid, dim3(Geo<64>::NT), 0,
                               stream, pool, tab, slot, S);
        else
            hipLaunchKernelGGL((quant_state_kra_kernel<64, false>), grid, dim3(Geo<64>::NT), 0,
                               stream, pool, tab, slot, S);
    } else if (pool.d == 128) {
        hipLaunchKernelGGL(quant_state_kernel<128>, grid, dim3(Geo<128>::NT), 0, stream, pool, tab, slot, S);
    } else {
        hipLaunchKernelGGL(quant_state_kernel<64>, grid, dim3(Geo<64>::NT), 0, stream, pool, tab, slot, S);
    }
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
    // a pool with row-impact scores requantizes with the key-row-aware fit
    if (pool.impact)
        return pool.row_mixed ? decode_gate_dispatch<false, true, true>(pool, tab, io, stream)
                              : decode_gate_dispatch<false, true, false>(pool, tab, io, stream);
    return pool.row_mixed ? decode_gate_dispatch<false, false, true>(pool, tab, io, stream)
                          : decode_gate_dispatch<false, false, false>(pool, tab, io, stream);
}

hipError_t launch_decode_update(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                                hipStream_t stream) {
    return pool.row_mixed ? decode_gate_dispatch<true, false, true>(pool, tab, io, stream)
                          : decode_gate_dispatch<true, false, false>(pool, tab, io, stream);
}

// ---------------------------------------------------------------- arithmetic self-check
// Every input of the quantizer's short division sequences (recip_rn on
// [FLT_MIN, 2^126), div_qmax on [0, 2] for qmax = 7, 31, 127) against the
// IEEE division; counts[k] += the number of results that differ.
__global__ void clear_counts_kernel(unsigned long long *counts) {
    if (threadIdx.x < 4) counts[threadIdx.x] = 0;
}
__global__ __launch_bounds__(256) void arith_selfcheck_kernel(unsigned long long *counts) {
#pragma clang fp contract(off)
    unsigned long long bad[4] = {0, 0, 0, 0};
    const uint32_t stride = gridDim.x * blockDim.x;
    const uint32_t first = blockIdx.x * blockDim.x + threadIdx.x;
    // i < 0x7e000000 and stride < 2^21: i + stride never wraps
    for (uint32_t i = first; i < 0x7e000000u; i += stride) {
        const float x = __uint_as_float(0x00800000u + i);
        bad[0] += __float_as_uint(recip_rn(x)) != __float_as_uint(1.0f / x);
    }
    for (uint32_t i = first; i <= 0x40000000u; i += stride) {
        const float m = __uint_as_float(i);
        bad[1] += __float_as_uint(div_qmax(m, 7.0f, 1.0f / 7.0f)) != __float_as_uint(m / 7.0f);
        bad[2] += __float_as_uint(div_qmax(m, 31.0f, 1.0f / 31.0f)) != __float_as_uint(m / 31.0f);
        bad[3] += __float_as_uint(div_qmax(m, 127.0f, 1.0f / 127.0f)) != __float_as_uint(m / 127.0f);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (bad[k]) atomicAdd(&counts[k], bad[k]);
}

hipError_t launch_arith_selfcheck(unsigned long long *counts, hipStream_t stream) {
    clear_counts_kernel<<<1, 64, 0, stream>>>(counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    arith_selfcheck_kernel<<<2048, 256, 0, stream>>>(counts);
    return hipGetLastError();
}

// ---------------------------------------------------------------- streaming copy
// The HBM rate a plain read-and-write stream reaches (the practical ceiling
// the decode step is compared with): 16-byte non-temporal loads and stores,
// four in flight per lane, grid-stride over 32768 workgroups of 256 lanes
// (the fastest of the shapes measured on MI355X).
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_copy_kernel(const u4v *__restrict__ src,
                                                          u4v *__restrict__ dst, uint64_t n) {
    constexpr int U = 4;
    const uint64_t stride = (uint64_t)gridDim.x * 256 * U;
    uint64_t i = (uint64_t)blockIdx.x * 256 * U + threadIdx.x;
    for (; i + 256 * (U - 1) < n; i += stride) {
        u4v v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + 256 * u);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + 256 * u);
    }
    // tail: the last partial group of 1024 vectors, one vector per lane
    for (; i < n; i += 256) dst[i] = src[i];
}

hipError_t launch_stream_copy(const void *src, void *dst, uint64_t n16, hipStream_t stream) {
    hipLaunchKernelGGL(stream_copy_kernel, dim3(32768), dim3(256), 0, stream,
                       static_cast<const u4v *>(src), static_cast<u4v *>(dst), n16);
    return hipGetLastError();
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

// ---------------------------------------------------------------- split step without allocation
// Staging buffer of sq_split_step_noalloc: the split step's S' (fp32
// [n, H, d, d]) between its two launches.  One copy per GPU, placed by the
// runtime with the code object and held until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: host code
// uses only the per-device address from hipGetSymbolAddress below.
static __device__ __align__(256) float scratch[SQ_SPLIT_SCRATCH_BYTES / sizeof(float)];

namespace sqk {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_dev[kMaxDevices]; // device address of `scratch` per device, once looked up
} // namespace

hipError_t scratch_address(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        // first call on this device, with it current: look up this device's copy
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_dev[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

hipError_t launch_split_step_scratch(const PoolView &pool, const HeadTable &tab, const StepIO &io_in,
                                     hipStream_t stream) {
    float *S = nullptr;
    hipError_t e = scratch_address(&S);
    if (e != hipSuccess) return e;
    // every tile writes its whole d x d block of S' before the second launch
    // (same stream) reads it, so nothing needs clearing between calls
    StepIO io = io_in;
    io.s_out = S;
    e = launch_decode_update(pool, tab, io, stream);
    if (e != hipSuccess) return e;
    return launch_quant_state(pool, tab, io.slot, io.n, S, stream);
}
} // namespace sqk

#ifdef SQ_TIMELINE
// Timeline build only: copy the stamps out (bytes <= the buffer's size) or
// clear them; both synchronous, on the null stream.  Return hipError_t codes.
extern "C" int sq_timeline_read(void *dst, size_t bytes) {
    if (bytes > sizeof(sqk::g_tl)) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(sqk::g_tl), bytes, 0, hipMemcpyDeviceToHost);
}
extern "C" int sq_timeline_clear() {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(sqk::g_tl));
    if (e != hipSuccess) return (int)e;
    return (int)hipMemset(p, 0, sizeof(sqk::g_tl));
}
#endif
