// C ABI of the packed low-bit recurrent-state pool (declared in include/sq.h).
//
// Host side only: argument validation, the pool layout, error text and
// kernel launches on the caller's stream.  The library owns no device
// memory; every device buffer comes from the caller.
#include "sq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "sq_internal.h"

struct sq_pool {
    sq_pool_desc desc;          // head_bits points at bits below
    uint8_t bits[sqk::kMaxHeads];
    sqk::PoolView view;
    sqk::HeadTable tab;
    int64_t rec_bytes[sqk::kMaxHeads];
    size_t bytes;               // n_slots * slot_stride
    bool row_mixed;             // some head has per-key-row widths
};

namespace {

thread_local char g_err[512] = "";

sq_status fail(sq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

sq_status hip_fail(hipError_t e, const char *what) {
    return fail(SQ_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Rows of one head with per-key-row widths: non-decreasing widths in
// {4, 6, 8} that change only at multiples of the rows a wavefront holds per
// row slot (d / 16 at d = 128, d / 4 at d = 64).  Returns the 4- and 6-bit
// row counts.
sq_status row_split(const sq_pool_desc *d, const uint8_t *row_bits, int h, uint8_t *n4,
                    uint8_t *n6) {
    const int dk = d->d_k, grain = dk == 128 ? 8 : 16;
    const uint8_t *w = row_bits + (size_t)h * dk;
    int c4 = 0, c6 = 0;
    for (int i = 0; i < dk; ++i) {
        if (w[i] != 4 && w[i] != 6 && w[i] != 8)
            return fail(SQ_EUNSUPPORTED, "row_bits[%d][%d] = %d, must be 4, 6 or 8", h, i, w[i]);
        if (i > 0 && w[i] < w[i - 1])
            return fail(SQ_EUNSUPPORTED, "row_bits[%d] must be non-decreasing (row %d)", h, i);
        if (i > 0 && w[i] != w[i - 1] && i % grain != 0)
            return fail(SQ_EUNSUPPORTED,
                        "row_bits[%d] changes width at row %d, not a multiple of %d", h, i, grain);
        c4 += w[i] == 4;
        c6 += w[i] == 6;
    }
    *n4 = (uint8_t)c4;
    *n6 = (uint8_t)c6;
    return SQ_OK;
}

sq_status check_desc(const sq_pool_desc *d, const uint8_t *row_bits = nullptr) {
    if (!d) return fail(SQ_EINVAL, "desc is NULL");
    if (d->n_slots < 1) return fail(SQ_EINVAL, "n_slots must be >= 1 (got %d)", d->n_slots);
    if (d->n_heads < 1 || d->n_heads > sqk::kMaxHeads)
        return fail(SQ_EUNSUPPORTED, "n_heads must be in [1, %d] (got %d)", sqk::kMaxHeads, d->n_heads);
    if (d->d_k != d->d_v)
        return fail(SQ_EUNSUPPORTED, "d_k must equal d_v (got %d, %d)", d->d_k, d->d_v);
    if (d->d_k != 64 && d->d_k != 128)
        return fail(SQ_EUNSUPPORTED, "d_k = d_v must be 64 or 128 (got %d)", d->d_k);
    if (d->gate != SQ_GATE_GDN && d->gate != SQ_GATE_KDA)
        return fail(SQ_EINVAL, "gate must be SQ_GATE_GDN or SQ_GATE_KDA (got %d)", (int)d->gate);
    if (!d->head_bits) return fail(SQ_EINVAL, "head_bits is NULL");
    for (int h = 0; h < d->n_heads; ++h) {
        const int b = d->head_bits[h];
        if (b == 0) {
            if (!row_bits)
                return fail(SQ_EINVAL, "head_bits[%d] = 0 needs per-row widths (row_bits)", h);
            uint8_t n4, n6;
            sq_status st = row_split(d, row_bits, h, &n4, &n6);
            if (st) return st;
        } else if (b != 4 && b != 6 && b != 8 && b != 16) {
            return fail(SQ_EUNSUPPORTED, "head_bits[%d] = %d, must be 4, 6, 8 or 16", h, b);
        }
    }
    return SQ_OK;
}

// Layout: per slot, head records back to back in head order.  row_bits is
// read only for heads whose head_bits is 0 (already validated).
int64_t layout(const sq_pool_desc *d, const uint8_t *row_bits, int64_t *off, int64_t *rec,
               uint8_t *n4 = nullptr, uint8_t *n6 = nullptr) {
    int64_t pos = 0;
    for (int h = 0; h < d->n_heads; ++h) {
        int64_t rb;
        uint8_t a = 0, b = 0;
        if (d->head_bits[h] == 0) {
            row_split(d, row_bits, h, &a, &b);
            rb = sqk::record_bytes_rows(a, b, d->d_k);
        } else {
            rb = sqk::record_bytes(d->head_bits[h], d->d_k);
        }
        if (n4) n4[h] = a;
        if (n6) n6[h] = b;
        if (off) off[h] = pos;
        if (rec) rec[h] = rb;
        pos += rb;
    }
    return pos;
}

sq_status check_rows(const sq_pool *p, const int32_t *slot_idx, int32_t n) {
    if (!p) return fail(SQ_EINVAL, "pool is NULL");
    if (n < 0) return fail(SQ_EINVAL, "n must be >= 0 (got %d)", n);
    if (n > p->desc.n_slots)
        return fail(SQ_EINVAL, "n = %d exceeds n_slots = %d (slots must be distinct)", n, p->desc.n_slots);
    if ((int64_t)n * p->desc.n_heads > 0x7FFFFFFFll)
        return fail(SQ_EUNSUPPORTED, "n * n_heads exceeds the grid limit");
    if (n > 0 && !slot_idx) return fail(SQ_EINVAL, "slot_idx is NULL");
    if (n > 0 && !aligned(slot_idx, 4)) return fail(SQ_EINVAL, "slot_idx is not 4-byte aligned");
    return SQ_OK;
}

// Debug mode: with SQ_DEBUG set to a value other than "0" in the
// environment (read at each call), every compute entry point on a pool first
// runs sq_check_slots on its slot indices (which synchronises the stream) and
// enqueues nothing if one is out of range or repeated: overlapping slots would
// make the in-place update race.
bool debug_slots() {
    const char *v = std::getenv("SQ_DEBUG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

sq_status check_io(const char *name, const void *p, bool need) {
    if (!need) return SQ_OK;
    if (!p) return fail(SQ_EINVAL, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(SQ_EINVAL, "%s is not 16-byte aligned", name);
    return SQ_OK;
}

sq_status check_step_io(const void *q, const void *k, const void *v, const void *beta,
                        const void *g, sq_dtype in_dtype, const void *y, sq_dtype y_dtype) {
    if (in_dtype != SQ_F32 && in_dtype != SQ_BF16)
        return fail(SQ_EINVAL, "in_dtype must be SQ_F32 or SQ_BF16 (got %d)", (int)in_dtype);
    if (y_dtype != SQ_F32 && y_dtype != SQ_BF16)
        return fail(SQ_EINVAL, "y_dtype must be SQ_F32 or SQ_BF16 (got %d)", (int)y_dtype);
    sq_status st;
    if ((st = check_io("q", q, true)) || (st = check_io("k", k, true)) ||
        (st = check_io("v", v, true)) || (st = check_io("beta", beta, true)) ||
        (st = check_io("g", g, true)) || (st = check_io("y", y, true)))
        return st;
    return SQ_OK;
}

} // namespace

extern "C" {

const char *sq_last_error(void) { return g_err; }

const char *sq_version(void) { return "sq 0.1 (gfx950)"; }

sq_status sq_pool_bytes_rows(const sq_pool_desc *desc, const uint8_t *row_bits, size_t *bytes) {
    sq_status st = check_desc(desc, row_bits);
    if (st) return st;
    if (!bytes) return fail(SQ_EINVAL, "bytes is NULL");
    const int64_t stride = layout(desc, row_bits, nullptr, nullptr);
    if ((uint64_t)desc->n_slots > (uint64_t)INT64_MAX / (uint64_t)stride)
        return fail(SQ_ENOMEM, "pool size overflows");
    *bytes = (size_t)((int64_t)desc->n_slots * stride);
    return SQ_OK;
}

sq_status sq_pool_bytes(const sq_pool_desc *desc, size_t *bytes) {
    return sq_pool_bytes_rows(desc, nullptr, bytes);
}

sq_status sq_pool_create_rows(const sq_pool_desc *desc, const uint8_t *row_bits, void *dev_buf,
                              size_t bytes, sq_pool **out) {
    if (!out) return fail(SQ_EINVAL, "out is NULL");
    *out = nullptr;
    size_t need = 0;
    sq_status st = sq_pool_bytes_rows(desc, row_bits, &need);
    if (st) return st;
    if (!dev_buf) return fail(SQ_EINVAL, "dev_buf is NULL");
    if (!aligned(dev_buf, 256)) return fail(SQ_EINVAL, "dev_buf is not 256-byte aligned");
    if (bytes < need) return fail(SQ_ENOMEM, "buffer has %zu bytes, pool needs %zu", bytes, need);
    sq_pool *p = new (std::nothrow) sq_pool;
    if (!p) return fail(SQ_ENOMEM, "host allocation failed");
    std::memset(p, 0, sizeof *p);
    p->desc = *desc;
    std::memcpy(p->bits, desc->head_bits, (size_t)desc->n_heads);
    p->desc.head_bits = p->bits;
    uint8_t n4[sqk::kMaxHeads] = {}, n6[sqk::kMaxHeads] = {};
    const int64_t stride = layout(desc, row_bits, p->tab.off, p->rec_bytes, n4, n6);
    for (int h = 0; h < desc->n_heads; ++h) {
        p->tab.info[h] = sqk::head_info(desc->head_bits[h], n4[h], n6[h]);
        p->row_mixed |= desc->head_bits[h] == 0;
    }
    int s = 0;
    while ((1 << s) < desc->n_heads) ++s;
    p->view.h_shift = 31 + s;
    p->view.h_magic = (uint32_t)((((uint64_t)1 << (31 + s)) + (uint64_t)desc->n_heads - 1) /
                                 (uint64_t)desc->n_heads);
    p->view.row_mixed = p->row_mixed;
    p->view.base = static_cast<uint8_t *>(dev_buf);
    p->view.slot_stride = stride;
    p->view.n_heads = desc->n_heads;
    p->view.d = desc->d_k;
    p->bytes = need;
    *out = p;
    return SQ_OK;
}

sq_status sq_pool_create(const sq_pool_desc *desc, void *dev_buf, size_t bytes, sq_pool **out) {
    return sq_pool_create_rows(desc, nullptr, dev_buf, bytes, out);
}

sq_status sq_pool_destroy(sq_pool *pool) {
    delete pool;
    return SQ_OK;
}

sq_status sq_pool_layout(const sq_pool *pool, int64_t *slot_stride, int64_t *head_off,
                         int64_t *record_bytes) {
    if (!pool) return fail(SQ_EINVAL, "pool is NULL");
    if (slot_stride) *slot_stride = pool->view.slot_stride;
    for (int h = 0; h < pool->desc.n_heads; ++h) {
        if (head_off) head_off[h] = pool->tab.off[h];
        if (record_bytes) record_bytes[h] = pool->rec_bytes[h];
    }
    return SQ_OK;
}

sq_status sq_pool_set_row_impact(sq_pool *pool, const float *impact) {
    if (!pool) return fail(SQ_EINVAL, "pool is NULL");
    if (impact && !aligned(impact, 16)) return fail(SQ_EINVAL, "impact is not 16-byte aligned");
    pool->view.impact = impact;
    return SQ_OK;
}

sq_status sq_quant_state(sq_pool *pool, const int32_t *slot_idx, int32_t n, const float *S,
                         hipStream_t stream) {
    sq_status st = check_rows(pool, slot_idx, n);
    if (st) return st;
    if (n == 0) return SQ_OK;
    if (debug_slots() && (st = sq_check_slots(pool, slot_idx, n, stream))) return st;
    if ((st = check_io("S", S, true))) return st;
    const hipError_t e = sqk::launch_quant_state(pool->view, pool->tab, slot_idx, n, S, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "quant_state launch");
}

sq_status sq_dequant_state(const sq_pool *pool, const int32_t *slot_idx, int32_t n, float *S,
                           hipStream_t stream) {
    sq_status st = check_rows(pool, slot_idx, n);
    if (st) return st;
    if (n == 0) return SQ_OK;
    if (debug_slots() && (st = sq_check_slots(pool, slot_idx, n, stream))) return st;
    if ((st = check_io("S", S, true))) return st;
    const hipError_t e = sqk::launch_dequant_state(pool->view, pool->tab, slot_idx, n, S, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "dequant_state launch");
}

sq_status sq_decode_step(sq_pool *pool, const int32_t *slot_idx, int32_t n, const void *q,
                         const void *k, const void *v, const void *beta, const void *g,
                         sq_dtype in_dtype, void *y, sq_dtype y_dtype, hipStream_t stream) {
    sq_status st = check_rows(pool, slot_idx, n);
    if (st) return st;
    if (n == 0) return SQ_OK;
    if (debug_slots() && (st = sq_check_slots(pool, slot_idx, n, stream))) return st;
    if ((st = check_step_io(q, k, v, beta, g, in_dtype, y, y_dtype))) return st;
    sqk::StepIO io;
    io.slot = slot_idx;
    io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.y = y;
    io.n = n;
    io.in_bf16 = in_dtype == SQ_BF16;
    io.y_bf16 = y_dtype == SQ_BF16;
    io.kda = pool->desc.gate == SQ_GATE_KDA;
    io.s_out = nullptr;
    const hipError_t e = sqk::launch_decode(pool->view, pool->tab, io, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "decode_step launch");
}

sq_status sq_decode_update(const sq_pool *pool, const int32_t *slot_idx, int32_t n, const void *q,
                           const void *k, const void *v, const void *beta, const void *g,
                           sq_dtype in_dtype, void *y, sq_dtype y_dtype, float *S_out,
                           hipStream_t stream) {
    sq_status st = check_rows(pool, slot_idx, n);
    if (st) return st;
    if (n == 0) return SQ_OK;
    if (debug_slots() && (st = sq_check_slots(pool, slot_idx, n, stream))) return st;
    if ((st = check_step_io(q, k, v, beta, g, in_dtype, y, y_dtype))) return st;
    if ((st = check_io("S_out", S_out, true))) return st;
    sqk::StepIO io;
    io.slot = slot_idx;
    io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.y = y;
    io.n = n;
    io.in_bf16 = in_dtype == SQ_BF16;
    io.y_bf16 = y_dtype == SQ_BF16;
    io.kda = pool->desc.gate == SQ_GATE_KDA;
    io.s_out = S_out;
    const hipError_t e = sqk::launch_decode_update(pool->view, pool->tab, io, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "decode_update launch");
}

sq_status sq_split_step_noalloc(sq_pool *pool, const int32_t *slot_idx, int32_t n, const void *q,
                                const void *k, const void *v, const void *beta, const void *g,
                                sq_dtype in_dtype, void *y, sq_dtype y_dtype, hipStream_t stream) {
    sq_status st = check_rows(pool, slot_idx, n);
    if (st) return st;
    if (n == 0) return SQ_OK;
    if (debug_slots() && (st = sq_check_slots(pool, slot_idx, n, stream))) return st;
    const uint64_t need = (uint64_t)n * (uint64_t)pool->desc.n_heads * (uint64_t)pool->desc.d_k *
                          (uint64_t)pool->desc.d_v * sizeof(float);
    if (need > (uint64_t)SQ_SPLIT_SCRATCH_BYTES)
        return fail(SQ_ENOMEM,
                    "S' of %d requests x %d heads needs %llu bytes, the static buffer holds %llu "
                    "(at most %llu requests of this pool per call)",
                    n, pool->desc.n_heads, (unsigned long long)need,
                    (unsigned long long)SQ_SPLIT_SCRATCH_BYTES,
                    (unsigned long long)(SQ_SPLIT_SCRATCH_BYTES /
                                         ((uint64_t)pool->desc.n_heads * pool->desc.d_k *
                                          pool->desc.d_v * sizeof(float))));
    if ((st = check_step_io(q, k, v, beta, g, in_dtype, y, y_dtype))) return st;
    sqk::StepIO io;
    io.slot = slot_idx;
    io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.y = y;
    io.n = n;
    io.in_bf16 = in_dtype == SQ_BF16;
    io.y_bf16 = y_dtype == SQ_BF16;
    io.kda = pool->desc.gate == SQ_GATE_KDA;
    io.s_out = nullptr;
    const hipError_t e = sqk::launch_split_step_scratch(pool->view, pool->tab, io, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "split_step_noalloc launch");
}

sq_status sq_f32_decode_step(float *state_pool, int32_t n_slots, int32_t n_heads, int32_t d_k,
                             int32_t d_v, sq_gate gate, const int32_t *slot_idx, int32_t n,
                             const void *q, const void *k, const void *v, const void *beta,
                             const void *g, sq_dtype in_dtype, void *y, sq_dtype y_dtype,
                             hipStream_t stream) {
    if (n_slots < 1) return fail(SQ_EINVAL, "n_slots must be >= 1 (got %d)", n_slots);
    if (n_heads < 1) return fail(SQ_EINVAL, "n_heads must be >= 1 (got %d)", n_heads);
    if (d_k != d_v) return fail(SQ_EUNSUPPORTED, "d_k must equal d_v (got %d, %d)", d_k, d_v);
    if (d_k != 64 && d_k != 128) return fail(SQ_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d_k);
    if (gate != SQ_GATE_GDN && gate != SQ_GATE_KDA)
        return fail(SQ_EINVAL, "gate must be SQ_GATE_GDN or SQ_GATE_KDA (got %d)", (int)gate);
    if (n < 0) return fail(SQ_EINVAL, "n must be >= 0 (got %d)", n);
    if (n > n_slots) return fail(SQ_EINVAL, "n = %d exceeds n_slots = %d", n, n_slots);
    if ((int64_t)n * n_heads > 0x7FFFFFFFll) return fail(SQ_EUNSUPPORTED, "grid too large");
    if (n == 0) return SQ_OK;
    if (!slot_idx) return fail(SQ_EINVAL, "slot_idx is NULL");
    sq_status st;
    if ((st = check_io("state_pool", state_pool, true))) return st;
    if ((st = check_step_io(q, k, v, beta, g, in_dtype, y, y_dtype))) return st;
    sqk::StepIO io;
    io.slot = slot_idx;
    io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.y = y;
    io.n = n;
    io.in_bf16 = in_dtype == SQ_BF16;
    io.y_bf16 = y_dtype == SQ_BF16;
    io.kda = gate == SQ_GATE_KDA;
    const int64_t stride = (int64_t)n_heads * d_k * d_v;
    const hipError_t e = sqk::launch_f32_decode(state_pool, stride, n_heads, d_k, io, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "f32_decode_step launch");
}

sq_status sq_check_slots(const sq_pool *pool, const int32_t *slot_idx, int32_t n,
                         hipStream_t stream) {
    sq_status st = check_rows(pool, slot_idx, n);
    if (st) return st;
    if (n == 0) return SQ_OK;
    std::vector<int32_t> host((size_t)n);
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    e = hipMemcpy(host.data(), slot_idx, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(slot_idx)");
    std::vector<uint8_t> seen((size_t)pool->desc.n_slots, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t s = host[(size_t)i];
        if (s < 0 || s >= pool->desc.n_slots)
            return fail(SQ_EINVAL, "slot_idx[%d] = %d is outside [0, %d)", i, s, pool->desc.n_slots);
        if (seen[(size_t)s]) return fail(SQ_EINVAL, "slot_idx[%d] = %d is repeated", i, s);
        seen[(size_t)s] = 1;
    }
    return SQ_OK;
}

sq_status sq_device_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return SQ_OK;
    if (!src || !dst) return fail(SQ_EINVAL, "src or dst is NULL");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(SQ_EINVAL, "buffers are not 16-byte aligned");
    if (bytes % 16) return fail(SQ_EINVAL, "bytes (%zu) is not a multiple of 16", bytes);
    const hipError_t e = sqk::launch_stream_copy(src, dst, (uint64_t)(bytes / 16), stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "stream copy launch");
}

sq_status sq_issue_probe(int op, float *sink, hipStream_t stream) {
    if (op < 0 || op >= SQ_PROBE_COUNT) return fail(SQ_EINVAL, "op = %d is not a probe class", op);
    if (!sink) return fail(SQ_EINVAL, "sink is NULL");
    if (!aligned(sink, 4)) return fail(SQ_EINVAL, "sink is not 4-byte aligned");
    const hipError_t e = sqk::launch_issue_probe(op, sink, stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "issue probe launch");
}

sq_status sq_arith_selfcheck(uint64_t *counts, hipStream_t stream) {
    if (!counts) return fail(SQ_EINVAL, "counts is NULL");
    if (!aligned(counts, 8)) return fail(SQ_EINVAL, "counts is not 8-byte aligned");
    const hipError_t e =
        sqk::launch_arith_selfcheck(reinterpret_cast<unsigned long long *>(counts), stream);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "arith_selfcheck launch");
}

} // extern "C"
