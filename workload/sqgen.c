/*
 * Seeded synthetic inputs for the gated Delta-rule decode step.
 *
 * This file holds no arithmetic of the method itself: it only draws the
 * per-step inputs (q, k, v, beta, log-gate), the per-head gate rates, the
 * per-head bit widths and the slot permutation.  Both the CPU oracle and the
 * HIP path consume what it writes; neither side re-implements it.
 *
 * Generator: counter-based SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): the 64-bit finaliser
 *   z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *   z *= 0x94D049BB133111EB; z ^= z >> 31
 * applied to key + (i + 1) * 0x9E3779B97F4A7C15.  The key chains the seed,
 * a stream id, the layer, the step t, the request b and the head h through
 * the same finaliser, so every value depends only on its coordinates and
 * never on thread count or generation order.
 *
 * Uniform: top 53 bits * 2^-53, in [0, 1).
 * Normal: Box-Muller in double, one normal per pair of draws (2i, 2i + 1):
 *   sqrt(-2 ln(1 - U0)) * cos(2 pi U1).
 *
 * Value recipe (the hybrid GDN / KDA decode workloads):
 *   q, k : N(0,1) per channel, L2-normalised in double
 *   v    : N(0,1)
 *   beta : sigmoid(N(0,1))
 *   g    : log-gate = -a with a ~ U(0.001, 0.5), drawn once per head
 *          (per head and key channel for KDA) and repeated at every step
 * Rounding to the storage dtype: double -> float (round to nearest even),
 * then float -> bfloat16 (round to nearest even) when the dtype is bf16.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

enum { ST_Q = 1, ST_K = 2, ST_V = 3, ST_BETA = 4, ST_GATE = 5, ST_BITS = 6,
       ST_SLOTS = 7, ST_STATE = 8 };

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t sqg_key(uint64_t seed, uint64_t stream, int64_t layer, int64_t t,
                 int64_t b, int64_t h) {
    uint64_t k = mix64(seed + GOLDEN);
    k = mix64(k ^ stream);
    k = mix64(k ^ (uint64_t)layer);
    k = mix64(k ^ (uint64_t)t);
    k = mix64(k ^ (uint64_t)b);
    k = mix64(k ^ (uint64_t)h);
    return k;
}

uint64_t sqg_draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

double sqg_uniform(uint64_t key, uint64_t i) {
    return (double)(sqg_draw(key, i) >> 11) * 0x1.0p-53;
}

double sqg_normal(uint64_t key, uint64_t i) {
    const double u0 = sqg_uniform(key, 2 * i);
    const double u1 = sqg_uniform(key, 2 * i + 1);
    return sqrt(-2.0 * log(1.0 - u0)) * cos(6.283185307179586 * u1);
}

/* float -> bfloat16, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline void store(void *dst, int dtype, size_t idx, double x) {
    const float f = (float)x;
    if (dtype == 0)
        ((float *)dst)[idx] = f;
    else
        ((uint16_t *)dst)[idx] = f32_to_bf16(f);
}

/* Per-head (GDN: per_channel == 0) or per-(head, channel) gate rates
 * a ~ U(0.001, 0.5), drawn once for a layer; out has H or H*d entries. */
void sqg_gate_rates(uint64_t seed, int64_t layer, int H, int d, int per_channel,
                    double *out) {
    for (int h = 0; h < H; ++h) {
        const uint64_t key = sqg_key(seed, ST_GATE, layer, 0, 0, h);
        const int n = per_channel ? d : 1;
        for (int i = 0; i < n; ++i)
            out[(size_t)h * n + i] = 0.001 + 0.499 * sqg_uniform(key, (uint64_t)i);
    }
}

/* In-place Fisher-Yates shuffle of perm[0..n) driven by stream `stream`. */
void sqg_shuffle(uint64_t seed, uint64_t stream, int64_t layer, int n, int32_t *perm) {
    const uint64_t key = sqg_key(seed, stream, layer, 0, 0, 0);
    for (int i = n - 1; i > 0; --i) {
        const uint64_t j = (uint64_t)(sqg_uniform(key, (uint64_t)i) * (double)(i + 1));
        const int32_t tmp = perm[i];
        perm[i] = perm[j];
        perm[j] = tmp;
    }
}

typedef struct {
    uint64_t seed;
    int64_t layer, t;
    int H, d, per_channel_gate, dtype;
    int n_rows;
    const int32_t *b_list; /* n_rows request ids, or NULL: rows are b*H + h */
    const int32_t *h_list;
    const double *gate_rates;
    void *q, *k, *v, *beta, *g;
    int row0, row1;
} job_t;

static void gen_row(const job_t *J, int row) {
    int b, h;
    if (J->b_list) {
        b = J->b_list[row];
        h = J->h_list[row];
    } else {
        b = row / J->H;
        h = row % J->H;
    }
    const int d = J->d;
    const size_t base = (size_t)row * d;
    double buf[512];
    for (int which = 0; which < 2; ++which) { /* q, then k: L2-normalised */
        const uint64_t key = sqg_key(J->seed, which == 0 ? ST_Q : ST_K, J->layer, J->t, b, h);
        double ss = 0.0;
        for (int i = 0; i < d; ++i) {
            buf[i] = sqg_normal(key, (uint64_t)i);
            ss += buf[i] * buf[i];
        }
        const double inv = 1.0 / sqrt(ss);
        void *dst = which == 0 ? J->q : J->k;
        for (int i = 0; i < d; ++i) store(dst, J->dtype, base + i, buf[i] * inv);
    }
    {
        const uint64_t key = sqg_key(J->seed, ST_V, J->layer, J->t, b, h);
        for (int i = 0; i < d; ++i) store(J->v, J->dtype, base + i, sqg_normal(key, (uint64_t)i));
    }
    {
        const uint64_t key = sqg_key(J->seed, ST_BETA, J->layer, J->t, b, h);
        const double x = sqg_normal(key, 0);
        store(J->beta, J->dtype, (size_t)row, 1.0 / (1.0 + exp(-x)));
    }
    if (J->per_channel_gate) {
        for (int i = 0; i < d; ++i)
            store(J->g, J->dtype, base + i, -J->gate_rates[(size_t)h * d + i]);
    } else {
        store(J->g, J->dtype, (size_t)row, -J->gate_rates[h]);
    }
}

static void *worker(void *arg) {
    const job_t *J = (const job_t *)arg;
    for (int r = J->row0; r < J->row1; ++r) gen_row(J, r);
    return NULL;
}

/*
 * Fill one step's inputs for n_rows (request, head) rows.
 * Row r is (b_list[r], h_list[r]) when b_list is given, else (r / H, r % H).
 * Layout: q, k, v, (KDA) g: [n_rows, d]; beta, (GDN) g: [n_rows].
 * dtype 0 = float32, 1 = bfloat16 (raw uint16).  Returns 0, or -1 on bad args.
 */
int sqg_step_inputs(uint64_t seed, int64_t layer, int64_t t, int H, int d,
                    int per_channel_gate, int dtype, int n_rows,
                    const int32_t *b_list, const int32_t *h_list,
                    const double *gate_rates, void *q, void *k, void *v,
                    void *beta, void *g, int n_threads) {
    if (d <= 0 || d > 512 || H <= 0 || n_rows < 0 || (dtype != 0 && dtype != 1)) return -1;
    if ((b_list == NULL) != (h_list == NULL)) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 64) n_threads = 64;
    if (n_threads > n_rows) n_threads = n_rows > 0 ? n_rows : 1;
    job_t jobs[64];
    pthread_t th[64];
    for (int w = 0; w < n_threads; ++w) {
        job_t J = {seed, layer, t, H, d, per_channel_gate, dtype, n_rows, b_list, h_list,
                   gate_rates, q, k, v, beta, g, 0, 0};
        J.row0 = (int)((int64_t)n_rows * w / n_threads);
        J.row1 = (int)((int64_t)n_rows * (w + 1) / n_threads);
        jobs[w] = J;
    }
    for (int w = 1; w < n_threads; ++w) pthread_create(&th[w], NULL, worker, &jobs[w]);
    worker(&jobs[0]);
    for (int w = 1; w < n_threads; ++w) pthread_join(th[w], NULL);
    return 0;
}

/* n normals of stream ST_STATE at coordinates (layer, t, b, h), as doubles:
 * used for arbitrary dense test states. */
void sqg_normals(uint64_t seed, int64_t layer, int64_t t, int64_t b, int64_t h,
                 int64_t n, double *out) {
    const uint64_t key = sqg_key(seed, ST_STATE, layer, t, b, h);
    for (int64_t i = 0; i < n; ++i) out[i] = sqg_normal(key, (uint64_t)i);
}
