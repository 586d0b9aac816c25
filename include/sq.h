/*
 * sq.h -- C ABI of the packed low-bit recurrent-state pool and its fused
 * gated Delta-rule decode step on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages on STEPQuant, arXiv 2609.38169):
 *  - "Paper Explained: STEPQuant" (ta-paperlens), section "The mechanism:
 *    rewriting state with the delta rule": per (request, head) a d_k x d_v
 *    state S is faded by the retention gate, the key's current look-up is
 *    formed, the beta-scaled difference to v is written along k, and the
 *    head output is read through q.  GDN has one scalar gate per head, KDA
 *    one gate per key channel.  Reading of the dropped equation:
 *        S' = (I - beta k k^T) diag(a) S + beta k v^T,   y = S'^T q,
 *        a = exp(g)   (g: log-gate, one per head or one per key channel).
 *  - hyper.ai summary, "Method", first paragraph: the reconstructed state is
 *    updated in floating point, the output is computed, and the updated
 *    state is then quantized for storage (symmetric uniform quantization).
 *  - hyper.ai summary, "Method", Key-Row-Aware Dual-Axis Fitting paragraph:
 *    the state is stored as row factors x column factors x low-bit integers,
 *    each scaled entry rounded to the nearest level.  Scale rule used here,
 *    in fp32 with one correctly rounded operation per step:
 *        c_j  = max_i |S'_ij|,             ic_j = 1 / c_j   (0 if c_j < FLT_MIN)
 *        s_ij = S'_ij * ic_j,              r_i  = max_j |s_ij| / qmax
 *        ir_i = 1 / r_i (0 if r_i < FLT_MIN)
 *        code = round-half-even of the exact product s_ij * ir_i, that is
 *               the level nearest to s_ij / r_i,   qmax = 2^(bits-1) - 1.
 *    Scales below FLT_MIN are stored as 0 and their codes are 0.
 *  - hyper.ai summary, "Method", last paragraph: packed-state kernels sit in
 *    a per-request recurrent-state pool; a fused kernel reconstructs tiles,
 *    applies the delta update and reads out the output.  Here the
 *    requantization and packed write-back are fused into the same kernel.
 *  - blog.ontle.kr (efficiency paragraph): serving pre-allocates spare
 *    slots, so requests reach their state through a slot index.
 *
 * Memory and ownership
 *  - Every tensor argument is a DEVICE pointer to contiguous row-major
 *    memory that the caller owns (e.g. a torch tensor); the library never
 *    allocates or frees device memory (its one buffer of its own, the static
 *    per-GPU array behind sq_split_step_noalloc, comes with the code object).
 *    Pointers must be 16-byte aligned and the pool buffer 256-byte aligned.
 *  - Host pointers: the descriptor, head_bits, and the layout outputs.
 *  - An sq_pool is a small host-side handle describing how a caller-owned
 *    device buffer is laid out; destroying it never touches the buffer.
 *
 * Pool layout (little-endian):
 *   pool[slot] = record(h = 0) | record(h = 1) | ... | record(H - 1)
 *   slot_stride = sum_h record_bytes(bits_h)
 *   record      = codes[d_k][d_v * bits / 8] | r[d_k] fp32 | c[d_v] fp32
 *   Each code row is a little-endian bit stream, code j at bits
 *   [bits*j, bits*j + bits), b-bit two's complement in [-qmax, qmax]:
 *   8-bit one code per byte; 4-bit code 2n in the low nibble of byte n;
 *   6-bit four codes per three bytes.  Record sizes at d = 128:
 *   9216 / 13312 / 17408 bytes for 4 / 6 / 8 bits (d = 64: 2560/3584/4608),
 *   all multiples of 256 bytes.
 *   bits = 16 marks an FP16 pivot head (hyper.ai summary, "Method", second
 *   paragraph: the highest-risk state units stay in FP16 as sparse
 *   pivots): its record is the state itself as IEEE binary16, row-major
 *   [d_k][d_v], 2 d_k d_v bytes, no scales; the decode step updates the
 *   widened values with the arithmetic of sq_decode_step (unit scales),
 *   then rounds S' from fp32 to binary16 (nearest even; values beyond the
 *   binary16 range become infinite).
 *
 * Execution
 *  - Compute entry points only validate their arguments on the host and
 *    enqueue work on the given stream; they return before the work runs.
 *    Device faults surface at the caller's next synchronisation.
 *  - Argument errors return a non-zero status synchronously and enqueue
 *    nothing; sq_last_error() then describes the problem (thread-local).
 *  - The decode step updates the listed slots in place.  The entries of
 *    slot_idx must be distinct and in [0, n_slots); slots not listed are
 *    never read or written.  Overlapping calls on the same slots race.
 *    Debug mode: with the environment variable SQ_DEBUG set (to anything
 *    but "0"; read at each call), every compute entry point on a pool first
 *    runs sq_check_slots on its slot indices, which synchronises the stream,
 *    and returns SQ_EINVAL without enqueueing anything if one is out of
 *    range or repeated.
 *  - n = 0 is a valid no-op.
 *  - Supported shapes: d_k = d_v = d in {64, 128}; bits in {4, 6, 8, 16},
 *    or 0 with per-key-row widths (sq_pool_create_rows);
 *    1 <= n_heads <= 64.  Others return SQ_EUNSUPPORTED.
 *  - NaN or infinite inputs give undefined (but memory-safe) results.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_EINVAL = 1,        /* bad argument (null, misaligned, out of range) */
    SQ_EUNSUPPORTED = 2,  /* shape or bit width the library does not handle */
    SQ_ENOMEM = 3,        /* buffer too small / host allocation failed */
    SQ_EHIP = 4           /* a HIP runtime call failed (text in sq_last_error) */
} sq_status;

typedef enum { SQ_GATE_GDN = 0, SQ_GATE_KDA = 1 } sq_gate;

typedef enum { SQ_F32 = 0, SQ_BF16 = 1 } sq_dtype;

/* Opcode classes of sq_issue_probe (the decode step's per-element vector
 * operations): fp32 FMA and fp32 multiply with every operand in a vector
 * register (a scalar or literal operand halves their rate), fp32 max3 of
 * absolute values, int32 to fp32 conversion (the class of the byte-to-fp32
 * widening), signed bit-field extract, funnel shift, FP64 FMA, and fp32 FMA
 * and int32 to fp32 conversion interleaved half and half (a conversion cannot
 * issue beside another conversion, but can beside an FMA of another wave). */
typedef enum {
    SQ_PROBE_FMA_F32 = 0,
    SQ_PROBE_MUL_F32 = 1,
    SQ_PROBE_MAX3_F32 = 2,
    SQ_PROBE_CVT_BYTE = 3,
    SQ_PROBE_BFE = 4,
    SQ_PROBE_ALIGNBIT = 5,
    SQ_PROBE_FMA_F64 = 6,
    SQ_PROBE_FMA_CVT_PAIR = 7,
    SQ_PROBE_COUNT = 8
} sq_probe_op;

/* Operations of its class that one sq_issue_probe launch performs
 * (8192 workgroups x 256 lanes x 1024 iterations x 8 chains). */
#define SQ_PROBE_OPS_PER_LAUNCH 17179869184LL

typedef struct {
    int32_t n_slots;          /* pool capacity in requests (>= 1) */
    int32_t n_heads;          /* heads per request, 1..64 */
    int32_t d_k;              /* key dimension (rows of the state) */
    int32_t d_v;              /* value dimension (columns), must equal d_k */
    const uint8_t *head_bits; /* host array [n_heads], each 4, 6, 8 or 16 (0: per-row
                                 widths, sq_pool_create_rows only); copied */
    sq_gate gate;             /* GDN: g is [n, H]; KDA: g is [n, H, d_k] */
} sq_pool_desc;

typedef struct sq_pool sq_pool;

/* Bytes of device memory a pool with this descriptor needs
 * (n_slots * slot_stride).  Defines the layout above: a per-request
 * recurrent-state pool (hyper.ai summary, "Method", last paragraph) with
 * spare slots reached through a slot index (blog.ontle.kr, efficiency
 * paragraph).  Errors: SQ_EINVAL for a NULL or inconsistent descriptor,
 * SQ_EUNSUPPORTED for shapes or widths outside the supported set. */
sq_status sq_pool_bytes(const sq_pool_desc *desc, size_t *bytes);

/* Wrap the caller's device buffer dev_buf (>= sq_pool_bytes, 256-byte
 * aligned) as a pool (the per-request state pool of hyper.ai summary,
 * "Method", last paragraph).  Host-side only: the buffer's contents are not
 * touched (initialise slots with sq_quant_state).  *out receives a handle
 * to release with sq_pool_destroy.  Errors: as sq_pool_bytes, plus
 * SQ_EINVAL for a NULL or misaligned buffer and SQ_ENOMEM if bytes is too
 * small or the host handle cannot be allocated. */
sq_status sq_pool_create(const sq_pool_desc *desc, void *dev_buf, size_t bytes, sq_pool **out);

/* Per-key-row bit widths (blog.ontle.kr, allocation paragraph: for KDA
 * models the unit of the bit allocation is a single key row).  Same as
 * sq_pool_bytes / sq_pool_create, except that a head with head_bits[h] = 0
 * gives each key row its own width row_bits[h * d_k + i] in {4, 6, 8}
 * (host array [n_heads][d_k], read during the call; only rows of width-0
 * heads are read, so it may be NULL when there are none).  Within such a
 * head the widths must be non-decreasing in i and may change only at rows
 * that are multiples of 8 (d_k = 128) or 16 (d_k = 64), so that the rows
 * one wavefront holds share a width.  Grouping the key channels by width is
 * an offline permutation of the model's key channels (q, k and the KDA gate
 * alike), which leaves every output unchanged.  Record of such a head: the
 * rows' code streams back to back (each row in the format of its width),
 * then r[d_k], c[d_v] fp32, padded to a multiple of 256 bytes.  Row i's
 * codes use the closed rule with its own qmax (r_i = max_j |s_ij| / qmax_i),
 * or the key-row-aware fit with per-row levels (sq_pool_set_row_impact).
 * Errors: SQ_EINVAL if a
 * width-0 head has no row_bits, SQ_EUNSUPPORTED for widths outside
 * {4, 6, 8}, decreasing widths or a change off the 8/16-row grid. */
sq_status sq_pool_bytes_rows(const sq_pool_desc *desc, const uint8_t *row_bits, size_t *bytes);
sq_status sq_pool_create_rows(const sq_pool_desc *desc, const uint8_t *row_bits, void *dev_buf,
                              size_t bytes, sq_pool **out);

/* Release the host handle of a pool (hyper.ai summary, "Method", last
 * paragraph: the pool is the serving system's; this library only describes
 * its layout).  Never frees or touches dev_buf.  NULL is a no-op. */
sq_status sq_pool_destroy(sq_pool *pool);

/* Layout of a pool: slot stride in bytes, and per head its record's byte
 * offset within a slot and its record size.  Output arrays are host arrays
 * of n_heads entries; any output pointer may be NULL. */
sq_status sq_pool_layout(const sq_pool *pool, int64_t *slot_stride, int64_t *head_off,
                         int64_t *record_bytes);

/* Switch the pool's requantization (in sq_decode_step and sq_quant_state)
 * to the key-row-aware dual-axis fit (hyper.ai summary, "Method", the
 * Key-Row-Aware Dual-Axis Fitting paragraph; blog.ontle.kr, the paragraph on
 * what is fixed offline): per key row i of head h a row-impact score
 * impact[h][i], calibrated offline, sets the row factor
 * r_i = sqrt(max_j |S'_ij| / impact_i), and each column scale is fitted by one
 * impact-weighted least-squares step from the range-covering scale; entries go
 * to the nearest level, clamped to +-qmax.  Heads with per-key-row widths
 * keep each row's own levels +-qmax_i: with qref the head's largest qmax,
 * row i's factor is widened by g_i = qref / qmax_i (fp32, 1 for the widest
 * rows) and the range-covering scale is max_i (|s_ij| g_i) / qref, so every
 * row spans its own levels on the shared column grid.  The record format is
 * unchanged.
 *   impact: DEVICE pointer to fp32 [n_heads][d_k], 16-byte aligned, every
 *           value finite and > 0 (others give undefined but memory-safe
 *           codes); owned by the caller and read by every later launch on
 *           this pool, so it must outlive them.  NULL restores the closed
 *           max rule.  FP16 pivot heads ignore it.
 * Host-only: enqueues nothing.  Must not race with calls using the pool. */
sq_status sq_pool_set_row_impact(sq_pool *pool, const float *impact);

/* Quantize fp32 states S [n, H, d_k, d_v] (device) into the slots
 * slot_idx[0..n) (device int32) with each head's bit width (hyper.ai
 * summary, "Method", Key-Row-Aware Dual-Axis Fitting paragraph: row factors
 * x column factors x low-bit integers, nearest level).  Arithmetic: the
 * scale rule written out at the top of this file (or the key-row-aware fit
 * of sq_pool_set_row_impact); FP16 pivot heads store the nearest binary16.
 * Bit-exact with that arithmetic.  Errors: SQ_EINVAL for NULL or misaligned
 * pointers or n < 0; nothing is enqueued then. */
sq_status sq_quant_state(sq_pool *pool, const int32_t *slot_idx, int32_t n, const float *S,
                         hipStream_t stream);

/* Reconstruct fp32 states S [n, H, d_k, d_v] from the slots slot_idx[0..n)
 * (hyper.ai summary, "Method", Key-Row-Aware Dual-Axis Fitting paragraph:
 * the state is the product of the row factor, the column factor and the
 * integer).  Arithmetic: S_ij = (float)(((double)code_ij * r_i) * c_j), one
 * FP64 product chain rounded once to fp32 (the FP64 value is exact for
 * |code| <= 31 and rounded once, by at most 2^-53 relative, for 8-bit
 * codes).  FP16 pivot heads widen their binary16 values exactly.  Errors:
 * SQ_EINVAL for NULL or misaligned pointers or n < 0. */
sq_status sq_dequant_state(const sq_pool *pool, const int32_t *slot_idx, int32_t n, float *S,
                           hipStream_t stream);

/* One fused decode step for n requests (request b lives in slot slot_idx[b];
 * "Paper Explained: STEPQuant" (ta-paperlens), section "The mechanism:
 * rewriting state with the delta rule"; hyper.ai summary, "Method", first and
 * last paragraphs): for every (b, h): dequantize, decay by a = exp(g), look up
 * v_old = Sd^T k, u = beta (v - v_old), S' = Sd + k u^T, y = S'^T q (from the
 * unrequantized S'), then requantize S' to the head's bit width and store it
 * in place.  Arithmetic (the pages say only "floating point"):
 * a_i = (float)exp(g_i); v_old and u to FP64 accuracy (the kernel forms v_old
 * as an exact integer sum and rounds it once), u_j then rounded once to fp32;
 * the rank-1 write in fp32 as S'_ij = fma(code_ij, (a_i r_i) c_j, k_i u_j),
 * each product rounded once; then the scale rule at the top of this file.
 * y is formed from the update before S' is rounded to fp32,
 * y_j = c_j sum_i q_i a_i r_i code_ij + u_j (k . q), to about 2^-27 relative
 * before its rounding to y_dtype.  Codes are bit-exact with this arithmetic
 * except where an FP64 evaluation of the look-up lands within its own
 * rounding error of an fp32 rounding boundary of u_j; against the
 * order-independent definition (FP64 step, S' rounded once to fp32, then the
 * scale rule) they agree within 1 LSB on all but a few in 10^5 entries.
 *   q, k: [n, H, d_k]   v: [n, H, d_v]   beta: [n, H]
 *   g (log-gate): [n, H] for GDN, [n, H, d_k] for KDA
 *   y: [n, H, d_v] output
 * in_dtype gives the type of q, k, v, beta, g; y_dtype the type of y. */
sq_status sq_decode_step(sq_pool *pool, const int32_t *slot_idx, int32_t n, const void *q,
                         const void *k, const void *v, const void *beta, const void *g,
                         sq_dtype in_dtype, void *y, sq_dtype y_dtype, hipStream_t stream);

/* First half of the split step (hyper.ai summary, "Method", last paragraph,
 * and blog.ontle.kr: once the head output exists, scale fitting and packed
 * write-back run on a separate stream).  Does what sq_decode_step does up to
 * and including the read-out: y is written, and S' rounded to fp32 is written
 * to S_out [n, H, d_k, d_v] (device, 16-byte aligned, request order like y);
 * the pool is only read.  Calling sq_quant_state(pool, slot_idx, n, S_out, s2)
 * afterwards (s2 may be another stream, ordered after this one by the caller,
 * e.g. with an event) stores exactly the records sq_decode_step would have
 * stored.  Until that call the listed slots still hold the previous state.
 * Same argument conventions and errors as sq_decode_step; S_out NULL or
 * misaligned gives SQ_EINVAL. */
sq_status sq_decode_update(const sq_pool *pool, const int32_t *slot_idx, int32_t n, const void *q,
                           const void *k, const void *v, const void *beta, const void *g,
                           sq_dtype in_dtype, void *y, sq_dtype y_dtype, float *S_out,
                           hipStream_t stream);

/* Bytes of the static per-GPU buffer behind sq_split_step_noalloc. */
#define SQ_SPLIT_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the split
 * step (sq_decode_update, then sq_quant_state of its S') with S' staged in
 * a buffer of the library's own instead of a caller workspace.  Both
 * launches go on `stream`, in that order; afterwards the listed slots hold
 * exactly the records, and y exactly the values, that sq_decode_update
 * followed by sq_quant_state of its S_out would give (and so sq_decode_step).
 * The call allocates nothing: the buffer is a static device array of
 * SQ_SPLIT_SCRATCH_BYTES (64 MiB) per GPU, which each GPU the library runs
 * on holds until the process ends; its device address is looked up once per
 * device on the first call there (make that first call outside graph
 * capture; later calls record into a graph like any other launch).  Limit: n * n_heads * d_k * d_v * 4 bytes
 * of S' must fit, i.e. n * n_heads <= 1024 at d = 128 (4096 at d = 64);
 * larger n returns SQ_ENOMEM and enqueues nothing.  Every call on one GPU
 * shares its buffer: calls on one stream are ordered, but calls that
 * overlap on one GPU (other streams, other threads, other pools) race and
 * corrupt each other's S'.  The buffer keeps the last call's S'; each call
 * writes all of the S' it reads, so nothing is cleared.  Arguments, errors
 * and in-place semantics otherwise as sq_decode_step. */
sq_status sq_split_step_noalloc(sq_pool *pool, const int32_t *slot_idx, int32_t n, const void *q,
                                const void *k, const void *v, const void *beta, const void *g,
                                sq_dtype in_dtype, void *y, sq_dtype y_dtype, hipStream_t stream);

/* The same step on an fp32 state pool state_pool [n_slots, H, d_k, d_v], in
 * place on the listed slots: the unquantized serving default the pages
 * compare against (bayesiansapien page, TL;DR: the state is kept per
 * request in FP32).  Arithmetic: fp32 throughout (a = expf(g); the two sums
 * over the state by fp32 partial sums folded through LDS; S'_ij =
 * fma(k_i, u_j, a_i S_ij) with a_i S_ij rounded first).  Same argument conventions and errors as sq_decode_step;
 * state_pool NULL or misaligned gives SQ_EINVAL. */
sq_status sq_f32_decode_step(float *state_pool, int32_t n_slots, int32_t n_heads, int32_t d_k,
                             int32_t d_v, sq_gate gate, const int32_t *slot_idx, int32_t n,
                             const void *q, const void *k, const void *v, const void *beta,
                             const void *g, sq_dtype in_dtype, void *y, sq_dtype y_dtype,
                             hipStream_t stream);

/* Debug check: copy slot_idx[0..n) (device) to the host, synchronising the
 * stream, and verify every entry is in [0, n_slots) and distinct.  Returns
 * SQ_EINVAL with the first offending index in sq_last_error() otherwise. */
sq_status sq_check_slots(const sq_pool *pool, const int32_t *slot_idx, int32_t n,
                         hipStream_t stream);

/* Self-check of the hardware arithmetic the quantizer relies on.  The
 * quantizer's divisions (the dual-axis scale rule above) are computed by
 * short sequences that are correctly rounded only because of how this GPU's
 * reciprocal instruction rounds; this call re-checks them on every input
 * they can receive: 1/x for every float x in [FLT_MIN, 2^126) (counts[0])
 * and m / qmax for every float m in [0, 2] and qmax = 7, 31, 127
 * (counts[1..3]), each against the IEEE division.  counts: 4 uint64 in
 * device memory (8-byte aligned), cleared and then filled on `stream` with
 * the number of differing results (all zero on a conforming GPU); read them
 * after synchronising the stream.  About 5 * 10^9 evaluations, tens of
 * milliseconds.  counts NULL gives SQ_EINVAL. */
sq_status sq_arith_selfcheck(uint64_t *counts, hipStream_t stream);

/* Measurement helper: copy `bytes` (a multiple of 16) from src to dst, both
 * DEVICE pointers, 16-byte aligned and not overlapping, with a plain
 * streaming kernel (16-byte non-temporal loads and stores).  Its rate is the
 * HBM bandwidth a read-and-write stream actually reaches on this GPU, which
 * the benchmark reports next to the published peak; the pages define no such
 * call.  bytes = 0 is a no-op.  Errors: SQ_EINVAL for NULL or misaligned
 * pointers or a size that is not a multiple of 16. */
sq_status sq_device_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* Measurement helper: one launch of the issue-rate probe of opcode class op
 * (sq_probe_op) on `stream`.  It performs SQ_PROBE_OPS_PER_LAUNCH operations
 * of that class in eight independent dependency chains per lane over a
 * whole-chip grid, so SQ_PROBE_OPS_PER_LAUNCH / (launch duration, timed by
 * the caller with events on `stream`) is the rate at which the GPU issues
 * that class: the vector-ALU ceiling the benchmark prices the decode step's
 * per-element operations at, next to the streaming copy's bandwidth ceiling.
 * The pages define no such call.  sink: DEVICE pointer to 4 bytes, 4-byte
 * aligned; the probe's one store is guarded by an equality with a NaN,
 * which never holds, so nothing is written (the guard keeps the chains'
 * work from being removed).  Errors: SQ_EINVAL
 * for op outside [0, SQ_PROBE_COUNT) or a NULL or misaligned sink. */
sq_status sq_issue_probe(int op, float *sink, hipStream_t stream);

/* Text describing the last non-OK status returned on this thread (error
 * reporting of this library; the pages define no interface).  Never NULL. */
const char *sq_last_error(void);

/* Library version string. */
const char *sq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
