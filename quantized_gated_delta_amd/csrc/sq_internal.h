// Internal interface between the C-ABI layer (sq_api.cpp) and the HIP
// kernels (sq_kernels.hip).  Not installed; the public boundary is sq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sq.h"

namespace sqk {

constexpr int kMaxHeads = 64;

// Per-head record placement inside one slot of the pool.  One 32-bit word of
// widths per head, so that a kernel reads it with a scalar load:
//   bits = info & 0xff: 4, 6, 8, 16 (FP16 pivot), or 0 (per-key-row widths);
//   n4 = (info >> 8) & 0xff, n6 = (info >> 16) & 0xff: for bits 0, rows
//   [0, n4) are 4-bit, [n4, n4 + n6) 6-bit, the rest 8-bit.
struct HeadTable {
    int64_t off[kMaxHeads];   // byte offset of head h's record within a slot
    uint32_t info[kMaxHeads]; // widths, as above
};
inline uint32_t head_info(int bits, int n4, int n6) {
    return (uint32_t)bits | ((uint32_t)n4 << 8) | ((uint32_t)n6 << 16);
}

struct PoolView {
    uint8_t *base;       // device pointer to slot 0
    int64_t slot_stride; // bytes per slot
    int32_t n_heads;
    // request of tile t (t < 2^31): (t * h_magic) >> h_shift = t / n_heads,
    // with h_shift = 31 + ceil(log2 n_heads), h_magic = ceil(2^h_shift / n_heads)
    uint32_t h_magic;
    int32_t h_shift;
    int32_t d;           // d_k == d_v
    const float *impact; // row-impact scores [n_heads, d] (key-row-aware fit) or null
    int32_t row_mixed;   // some head has per-key-row widths (head bits 0)
};

// Step inputs; dtype flags: 0 = fp32, 1 = bf16.
struct StepIO {
    const int32_t *slot;
    const void *q, *k, *v, *beta, *g;
    void *y;
    int32_t n;
    int32_t in_bf16, y_bf16;
    int32_t kda;
    float *s_out;   // split step only: S' as fp32 [n, H, d, d]
};

// Bytes of one record: d rows of d * bits / 8 code bytes, then r[d], c[d]
// fp32; bits = 16 is an FP16 pivot record (the state as binary16, no scales).
inline int64_t record_bytes(int bits, int d) {
    if (bits == 16) return 2 * (int64_t)d * d;
    return (int64_t)d * d * bits / 8 + 8 * (int64_t)d;
}

// Bytes of a record with per-key-row widths (n4 4-bit, n6 6-bit, the rest
// 8-bit rows), then r[d], c[d] fp32, padded to a multiple of 256 bytes.
inline int64_t record_bytes_rows(int n4, int n6, int d) {
    const int64_t n8 = d - n4 - n6;
    const int64_t raw = (int64_t)d * (4 * n4 + 6 * n6 + 8 * n8) / 8 + 8 * (int64_t)d;
    return (raw + 255) / 256 * 256;
}

hipError_t launch_quant_state(const PoolView &pool, const HeadTable &tab, const int32_t *slot,
                              int32_t n, const float *S, hipStream_t stream);
hipError_t launch_dequant_state(const PoolView &pool, const HeadTable &tab, const int32_t *slot,
                                int32_t n, float *S, hipStream_t stream);
hipError_t launch_decode(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                         hipStream_t stream);
// The decode step without its requantization: S' (fp32) goes to io.s_out.
hipError_t launch_decode_update(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                                hipStream_t stream);
// The split step with S' staged in the library's static per-device buffer
// (sq_split_step_noalloc): launch_decode_update into it, then
// launch_quant_state from it, both on `stream`.  io.s_out is ignored.  The
// caller has checked n * n_heads * d * d * 4 <= SQ_SPLIT_SCRATCH_BYTES.
hipError_t launch_split_step_scratch(const PoolView &pool, const HeadTable &tab, const StepIO &io,
                                     hipStream_t stream);
// Device address of that buffer on the current device (looked up once per
// device).
hipError_t scratch_address(float **out);
hipError_t launch_f32_decode(float *state, int64_t slot_stride_floats, int32_t n_heads, int32_t d,
                             const StepIO &io, hipStream_t stream);

// Streaming copy of n16 16-byte vectors (a measurement of the HBM rate).
hipError_t launch_stream_copy(const void *src, void *dst, uint64_t n16, hipStream_t stream);
// issue-rate probes (sq_probe.hip): SQ_PROBE_OPS_PER_LAUNCH operations of one
// class per launch
constexpr int kProbeWorkgroups = 8192;
constexpr int kProbeIters = 1024;
static_assert((long long)kProbeWorkgroups * 256 * kProbeIters * 8 == SQ_PROBE_OPS_PER_LAUNCH,
              "probe shape");
hipError_t launch_issue_probe(int op, float *sink, hipStream_t stream);

// Exhaustive check of the quantizer's division sequences: counts[0..4)
// (device) receive the mismatches against the IEEE division.
hipError_t launch_arith_selfcheck(unsigned long long *counts, hipStream_t stream);

} // namespace sqk
