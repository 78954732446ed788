/*
 * oracle.c -- CPU oracle for the 4-bit group-256 weight-quantized matmul
 * (dequant-fused GEMV and Q8_1 "MMQ" prefill).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the HIP library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or constant with the HIP library and includes none of
 * its files.
 *
 * What is computed, and where it is described:
 *   - The weight format (4-bit codes, groups of 256 along K, one fp16 scale and
 *     one fp16 minimum per group, two codes per byte) is the "HFQ4-G256" format
 *     named in the hipfire MMQ-prefill note (ai-navigate-news.com article on the
 *     HFQ4-G256 MMQ prefill path, list of changes and benchmark table heading).
 *     The page names the format without a byte layout; the layout below is the
 *     reading this project fixed (see the "Readings" list in the design notes).
 *   - Q8_1 activations (int8 blocks of 32 with an fp16 scale d and an fp16 sum
 *     s) are the "Q8_1 MMQ layout" the same note pre-quantizes prefill
 *     activations into (same page, list of changes).
 *   - Integer dot products per block are the "keep-quant integer core" that the
 *     vllm.cpp TG150 campaign keeps bit-exact against the CPU (vllm.cpp pull
 *     request 4, "Design", correctness policy).
 *   - The fp64 naive sum is the CPU oracle that op-level NMSE is measured
 *     against (vllm.cpp issue 5, "Working rules", rule 3).
 *
 * Arithmetic rules:
 *   - Where floating point decides an integer (a 4-bit code, an int8 code, an
 *     fp16 rounding) the decision is taken in IEEE fp32 with round-to-nearest-
 *     even, no contraction (build with -ffp-contract=off), exactly as the GPU
 *     must take it.
 *   - Every output sum is an fp64 sum over k in ascending order, of products
 *     of exactly dequantized values, one output at a time.  Threads split the
 *     output rows only, so results do not depend on the thread count.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORC_VERSION 1

/* ------------------------------------------------------------------ */
/* test-only planted mistakes (mutation check of the pins)             */
/* ------------------------------------------------------------------ */
/* 0 = none.  Each non-zero value plants one plausible mistake; the pin tests
 * must fail for every one of them.  Never set outside tests. */
enum {
    MUT_NONE = 0,
    MUT_NIBBLE_SEQUENTIAL = 1, /* codes 2i / 2i+1 share a byte instead of i / i+16 */
    MUT_DEQUANT_NO_MIN = 2,    /* dequantization drops the group minimum        */
    MUT_SCALE_OVER_16 = 3,     /* scale = (max-min)/16 instead of /15           */
    MUT_Q8_ROUND_AWAY = 4,     /* int8 codes round half away from zero          */
    MUT_Q8_UNROUNDED_D = 5,    /* int8 codes use the fp32 d, not the fp16 one   */
    MUT_GEMV_TRANSPOSED = 6,   /* GEMV reads weight [k][n] instead of [n][k]    */
    MUT_MMQ_NO_D = 7,          /* MMQ forgets the activation block scale d      */
    MUT_DOTS_CENTERED = 8,     /* block dots use (q-8) instead of q             */
    MUT_F16_TRUNCATE = 9,      /* fp32->fp16 truncates instead of RNE           */
    MUT_GROUP_OFF_BY_ONE = 10, /* dequant takes the scale of the next group     */
    MUT_LAST = 10
};
static int g_mutation = 0;
static int g_threads = 0;

int orc_version(void) { return ORC_VERSION; }
void orc_set_mutation(int m) { g_mutation = (m >= 0 && m <= MUT_LAST) ? m : 0; }
int orc_get_mutation(void) { return g_mutation; }
void orc_set_threads(int n) { g_threads = n > 0 ? n : 0; }
int orc_get_threads(void)
{
    if (g_threads > 0) return g_threads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, from the IEEE 754 definition            */
/* ------------------------------------------------------------------ */
/* Nearest binary16 value to f, ties to even; overflow to infinity.
 * Written from the format's definition: binary16 has 10 fraction bits,
 * exponent bias 15, smallest normal 2^-14, subnormal quantum 2^-24, largest
 * finite 65504. */
uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);      /* a in [2^(e-1), 2^e) */
    int E = e - 1;     /* a in [2^E, 2^(E+1)) */
    if (E < -14) E = -14;           /* subnormal range: quantum 2^-24 */
    double quantum = ldexp(1.0, E - 10);
    double n = a / quantum;          /* exact: division by a power of two */
    if (g_mutation == MUT_F16_TRUNCATE) n = floor(n);
    else n = nearbyint(n);           /* round half to even (default mode) */
    double v = n * quantum;
    if (v > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    int e2;
    double m = frexp(v, &e2);        /* v = m 2^e2, m in [0.5, 1) */
    uint16_t biased = (uint16_t)(e2 - 1 + 15);
    uint16_t frac = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (biased << 10) | frac);
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int biased = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (biased == 0) v = ldexp((double)frac, -24);
    else if (biased == 31) v = frac ? NAN : INFINITY;
    else v = ldexp((double)(1024 + frac), biased - 25);
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------ */
/* thread helper: split [0, n) into contiguous ranges                  */
/* ------------------------------------------------------------------ */
typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void *ctx; int64_t lo, hi; } range_job;

static void *range_thread(void *p)
{
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_rows(int64_t n, range_fn fn, void *ctx)
{
    int T = orc_get_threads();
    if (T > n) T = (int)(n > 0 ? n : 1);
    if (T <= 1) { fn(ctx, 0, n); return; }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)T);
    range_job *jobs = (range_job *)malloc(sizeof(range_job) * (size_t)T);
    for (int t = 0; t < T; ++t) {
        jobs[t].fn = fn; jobs[t].ctx = ctx;
        jobs[t].lo = n * t / T; jobs[t].hi = n * (t + 1) / T;
        pthread_create(&th[t], NULL, range_thread, &jobs[t]);
    }
    for (int t = 0; t < T; ++t) pthread_join(th[t], NULL);
    free(th); free(jobs);
}

/* ------------------------------------------------------------------ */
/* 4-bit weights, groups of 256 (and of 32)                            */
/* ------------------------------------------------------------------ */
/* Layout (the project's reading; the pages name the format only):
 *   qs  u8  [N][K/2]   group g of row n occupies bytes [128 g, 128 g + 128).
 *                       Inside a group, sub-block j (32 consecutive k) takes
 *                       bytes [16 j, 16 j + 16); byte i of it holds the code of
 *                       element 32 j + i in its low nibble and the code of
 *                       element 32 j + i + 16 in its high nibble.
 *   sm  f16 [N][K/256][2]   (scale, minimum) per group.
 * Dequantized weight: w' = scale * q + minimum, with scale and minimum taken
 * from their fp16 values.
 * The group-32 variant (the *_g functions with group = 32) keeps qs exactly
 * as above and carries one (scale, minimum) pair per 32 weights,
 * sm f16 [N][K/32][2]; packing and dequantization are the same steps over
 * groups of 32. */
#define GROUP 256
#define BLOCK 32

/* byte offset and nibble (0 = low, 1 = high) of element k of one row; the
 * layout is the same for both group sizes (a group of 256 is eight runs of 32) */
static inline void code_position(int64_t k, int64_t *byte, int *hi)
{
    if (g_mutation == MUT_NIBBLE_SEQUENTIAL) {
        *byte = k / 2;
        *hi = (int)(k & 1);
        return;
    }
    int64_t j = k / BLOCK, i = k % BLOCK;
    *byte = j * 16 + (i & 15);
    *hi = i >= 16;
}

/* the two group sizes of (scale, minimum) pairs: 256 and 32 weights */
static inline int valid_group(int64_t group) { return group == GROUP || group == BLOCK; }

static inline int read_code(const uint8_t *row, int64_t k)
{
    int64_t b; int hi;
    code_position(k, &b, &hi);
    return hi ? (row[b] >> 4) & 15 : row[b] & 15;
}

typedef struct {
    const float *W; int64_t K; uint8_t *qs; uint16_t *sm; int64_t group;
} pack_ctx;

static void pack_rows(void *p, int64_t lo, int64_t hi)
{
    pack_ctx *c = (pack_ctx *)p;
    const int64_t K = c->K, GS = c->group, G = K / GS;
    for (int64_t n = lo; n < hi; ++n) {
        const float *w = c->W + n * K;
        uint8_t *row = c->qs + n * (K / 2);
        uint16_t *sm = c->sm + n * G * 2;
        memset(row, 0, (size_t)(K / 2));
        for (int64_t g = 0; g < G; ++g) {
            const float *wg = w + g * GS;
            float mn = wg[0], mx = wg[0];
            for (int k = 1; k < GS; ++k) {
                if (wg[k] < mn) mn = wg[k];
                if (wg[k] > mx) mx = wg[k];
            }
            /* a zero minimum or maximum counts as +0 whatever its sign bit */
            mn = mn + 0.0f;
            mx = mx + 0.0f;
            float range = mx - mn;                       /* fp32, RN */
            float denom = (g_mutation == MUT_SCALE_OVER_16) ? 16.0f : 15.0f;
            uint16_t s16 = orc_f32_to_f16(range / denom); /* fp32 divide, RN */
            uint16_t m16 = orc_f32_to_f16(mn);
            float sf = orc_f16_to_f32(s16), mf = orc_f16_to_f32(m16);
            sm[2 * g] = s16;
            sm[2 * g + 1] = m16;
            for (int k = 0; k < GS; ++k) {
                int q = 0;
                if (sf != 0.0f) {
                    float t = (wg[k] - mf) / sf;          /* fp32 sub, fp32 divide */
                    float r = rintf(t);                   /* half to even */
                    q = r < 0.0f ? 0 : (r > 15.0f ? 15 : (int)r);
                }
                int64_t b; int h;
                code_position(g * GS + k, &b, &h);
                row[b] |= (uint8_t)(h ? (q << 4) : q);
            }
        }
    }
}

/* Pack W [N][K] fp32 into qs/sm with one (scale, minimum) pair per group of
 * `group` (256 or 32) weights along K.  Returns 0, or -1 on bad arguments. */
int orc_q4_pack_g(const float *W, int64_t N, int64_t K, int64_t group, uint8_t *qs, uint16_t *sm)
{
    if (!W || !qs || !sm || N < 0 || K <= 0 || !valid_group(group) || K % GROUP) return -1;
    pack_ctx c = {W, K, qs, sm, group};
    parallel_rows(N, pack_rows, &c);
    return 0;
}

int orc_q4_pack(const float *W, int64_t N, int64_t K, uint8_t *qs, uint16_t *sm)
{
    return orc_q4_pack_g(W, N, K, GROUP, qs, sm);
}

/* Exact dequantization of one row into fp64. */
static void dequant_row(const uint8_t *row, const uint16_t *sm, int64_t K, int64_t GS, double *out)
{
    const int64_t G = K / GS;
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / GS;
        if (g_mutation == MUT_GROUP_OFF_BY_ONE && g + 1 < G) g += 1;
        double s = (double)orc_f16_to_f32(sm[2 * g]);
        double m = (double)orc_f16_to_f32(sm[2 * g + 1]);
        if (g_mutation == MUT_DEQUANT_NO_MIN) m = 0.0;
        out[k] = s * (double)read_code(row, k) + m;
    }
}

int orc_q4_dequant_g(const uint8_t *qs, const uint16_t *sm, int64_t N, int64_t K, int64_t group,
                     double *Wd)
{
    if (!qs || !sm || !Wd || N < 0 || K <= 0 || !valid_group(group) || K % GROUP) return -1;
    for (int64_t n = 0; n < N; ++n)
        dequant_row(qs + n * (K / 2), sm + n * (K / group) * 2, K, group, Wd + n * K);
    return 0;
}

int orc_q4_dequant(const uint8_t *qs, const uint16_t *sm, int64_t N, int64_t K, double *Wd)
{
    return orc_q4_dequant_g(qs, sm, N, K, GROUP, Wd);
}

/* Unpack the 4-bit codes of W (as integers 0..15) into codes [N][K]. */
int orc_q4_codes(const uint8_t *qs, int64_t N, int64_t K, uint8_t *codes)
{
    if (!qs || !codes || N < 0 || K <= 0 || K % GROUP) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)read_code(qs + n * (K / 2), k);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Q8_1 activations                                                    */
/* ------------------------------------------------------------------ */
/* qa i8 [M][K]; ds f16 [M][K/32][2] = (d, s) per block of 32 along K.
 *   amax = max |x|,  d = fp16(amax / 127),  a = clamp(rint(x / d), -127, 127)
 *   (a = 0 when d == 0),  s = fp16(d * sum(a)). */
int orc_q8_1_quantize(const float *x, int64_t M, int64_t K, int8_t *qa, uint16_t *ds)
{
    if (!x || !qa || !ds || M < 0 || K <= 0 || K % BLOCK) return -1;
    const int64_t B = K / BLOCK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < B; ++b) {
            const float *xb = x + m * K + b * BLOCK;
            int8_t *ab = qa + m * K + b * BLOCK;
            float amax = 0.0f;
            for (int i = 0; i < BLOCK; ++i) {
                float v = fabsf(xb[i]);
                if (v > amax) amax = v;
            }
            float dq = amax / 127.0f;                   /* fp32 divide, RN */
            uint16_t d16 = orc_f32_to_f16(dq);
            float df = orc_f16_to_f32(d16);
            if (g_mutation == MUT_Q8_UNROUNDED_D) df = dq;
            int sum = 0;
            for (int i = 0; i < BLOCK; ++i) {
                int a = 0;
                if (df != 0.0f) {
                    float t = xb[i] / df;                  /* fp32 divide, RN */
                    float r = (g_mutation == MUT_Q8_ROUND_AWAY) ? roundf(t) : rintf(t);
                    a = r < -127.0f ? -127 : (r > 127.0f ? 127 : (int)r);
                }
                ab[i] = (int8_t)a;
                sum += a;
            }
            /* df * sum is exact in fp32 (11-bit times 13-bit significands) */
            ds[(m * B + b) * 2] = d16;
            ds[(m * B + b) * 2 + 1] = orc_f32_to_f16(orc_f16_to_f32(d16) * (float)sum);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* GEMV: y[m][n] = sum_k x[m][k] * w'[n][k]   (fp64, k ascending)       */
/* ------------------------------------------------------------------ */
typedef struct {
    const float *x; int64_t M; const uint8_t *qs; const uint16_t *sm;
    int64_t N, K; double *y; int64_t group;
} gemv_ctx;

static void gemv_rows(void *p, int64_t lo, int64_t hi)
{
    gemv_ctx *c = (gemv_ctx *)p;
    const int64_t K = c->K;
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t n = lo; n < hi; ++n) {
        if (g_mutation == MUT_GEMV_TRANSPOSED) {
            /* planted mistake: weight element (n, k) read from row k, column n */
            for (int64_t k = 0; k < K; ++k) {
                int64_t rn = k % c->N, rk = n % K;
                int64_t g = rk / c->group;
                const uint8_t *row = c->qs + rn * (K / 2);
                const uint16_t *sm = c->sm + rn * (K / c->group) * 2;
                w[k] = (double)orc_f16_to_f32(sm[2 * g]) * read_code(row, rk) +
                       (double)orc_f16_to_f32(sm[2 * g + 1]);
            }
        } else {
            dequant_row(c->qs + n * (K / 2), c->sm + n * (K / c->group) * 2, K, c->group, w);
        }
        for (int64_t m = 0; m < c->M; ++m) {
            const float *xm = c->x + m * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += (double)xm[k] * w[k];
            c->y[m * c->N + n] = acc;
        }
    }
    free(w);
}

int orc_q4_gemv_g(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm,
                  int64_t N, int64_t K, int64_t group, double *y)
{
    if (!x || !qs || !sm || !y || M < 0 || N < 0 || K <= 0 || !valid_group(group) || K % GROUP) return -1;
    gemv_ctx c = {x, M, qs, sm, N, K, y, group};
    parallel_rows(N, gemv_rows, &c);
    return 0;
}

int orc_q4_gemv(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm,
                int64_t N, int64_t K, double *y)
{
    return orc_q4_gemv_g(x, M, qs, sm, N, K, GROUP, y);
}

/* ------------------------------------------------------------------ */
/* Per-block integer dots: idot[m][n][b] = sum_{k in b} a[m][k] q[n][k] */
/* ------------------------------------------------------------------ */
int orc_q4_block_dots(const int8_t *qa, int64_t M, const uint8_t *qs, int64_t N, int64_t K,
                      int32_t *idot)
{
    if (!qa || !qs || !idot || M < 0 || N < 0 || K <= 0 || K % GROUP) return -1;
    const int64_t B = K / BLOCK;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *row = qs + n * (K / 2);
            for (int64_t b = 0; b < B; ++b) {
                int64_t acc = 0;
                for (int i = 0; i < BLOCK; ++i) {
                    int64_t k = b * BLOCK + i;
                    int q = read_code(row, k);
                    if (g_mutation == MUT_DOTS_CENTERED) q -= 8;
                    acc += (int64_t)qa[m * K + k] * q;
                }
                idot[(m * N + n) * B + b] = (int32_t)acc;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* MMQ: y[m][n] = sum_k x'[m][k] * w'[n][k],  x' = d * a  (fp64)        */
/* ------------------------------------------------------------------ */
typedef struct {
    const int8_t *qa; const uint16_t *ds; int64_t M;
    const uint8_t *qs; const uint16_t *sm; int64_t N, K; double *y;
    const double *xd;   /* dequantized activations [M][K] */
    int64_t group;
} mmq_ctx;

static void mmq_rows(void *p, int64_t lo, int64_t hi)
{
    mmq_ctx *c = (mmq_ctx *)p;
    const int64_t K = c->K;
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t n = lo; n < hi; ++n) {
        dequant_row(c->qs + n * (K / 2), c->sm + n * (K / c->group) * 2, K, c->group, w);
        for (int64_t m = 0; m < c->M; ++m) {
            const double *xm = c->xd + m * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xm[k] * w[k];
            c->y[m * c->N + n] = acc;
        }
    }
    free(w);
}

/* Exact dequantization of Q8_1 activations into fp64: x' = d * a. */
int orc_q8_1_dequant(const int8_t *qa, const uint16_t *ds, int64_t M, int64_t K, double *xd)
{
    if (!qa || !ds || !xd || M < 0 || K <= 0 || K % BLOCK) return -1;
    const int64_t B = K / BLOCK;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double d = (double)orc_f16_to_f32(ds[(m * B + k / BLOCK) * 2]);
            if (g_mutation == MUT_MMQ_NO_D) d = 1.0;
            xd[m * K + k] = d * (double)qa[m * K + k];
        }
    return 0;
}

int orc_q4_mmq_g(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                 const uint16_t *sm, int64_t N, int64_t K, int64_t group, double *y)
{
    if (!qa || !ds || !qs || !sm || !y || M < 0 || N < 0 || K <= 0 || !valid_group(group) || K % GROUP)
        return -1;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xd) return -2;
    orc_q8_1_dequant(qa, ds, M, K, xd);
    mmq_ctx c = {qa, ds, M, qs, sm, N, K, y, xd, group};
    parallel_rows(N, mmq_rows, &c);
    free(xd);
    return 0;
}

int orc_q4_mmq(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
               const uint16_t *sm, int64_t N, int64_t K, double *y)
{
    return orc_q4_mmq_g(qa, ds, M, qs, sm, N, K, GROUP, y);
}
