/*
 * Driver of the sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer,
 * host code only): the C-ABI runtime of libwqmm and the CPU oracle, compiled
 * instrumented and linked into this program, which exercises every host-side
 * path that runs without a GPU -- argument validation of each entry point,
 * the startup error when no device is present, the kernel planner over a
 * spread of shapes (its index and size arithmetic), the status strings -- and
 * runs the oracle on small seeded problems, checking invariants that hold by
 * construction (a zero scale gives 0, A >= |y|, the group-scaled form with one
 * group equals the per-row form). Any sanitizer report aborts with a
 * non-zero status. Test infrastructure: built and run by
 * tests/test_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wqmm.h"

long oracle_row_bytes(int fmt, long I);
int oracle_matmul(int fmt, long O, long I, const unsigned char *w, long row_stride, const float *scales,
                  const float *x, long S, float *y, double *absb, int nthreads);
int oracle_matmul_gs(int fmt, long O, long I, const unsigned char *w, long row_stride, const float *scales,
                     long gs, const float *x, long S, float *y, double *absb, int nthreads);
void oracle_silu_mul(const float *g, const float *u, long n, float *h);

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64*: deterministic test data */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float rndf(void) { return ((float)(rnd() & 0xFFFFFF) / 16777216.0f) * 2.0f - 1.0f; }

static void api_checks(void) {
    /* status strings */
    for (int c = 1; c >= -9; --c) CHECK(wq_strerror(c) != NULL && strlen(wq_strerror(c)) > 0);
    /* row bytes */
    CHECK(wq_row_bytes(WQ_F32, 9) == 36 && wq_row_bytes(WQ_I8, 9) == 9 && wq_row_bytes(WQ_I4, 9) == 5 &&
          wq_row_bytes(WQ_I2, 9) == 3 && wq_row_bytes(7, 9) == -1 && wq_row_bytes(WQ_I4, -1) == -1);
    /* init: bad lists are refused before any device query; no GPU -> WQ_E_NODEV */
    int dup[2] = {0, 0}, neg[1] = {-1}, big[1] = {WQ_MAX_DEVICES};
    CHECK(wq_init(dup, 2) == WQ_E_INVAL);
    CHECK(wq_init(neg, 1) == WQ_E_INVAL);
    CHECK(wq_init(big, 1) == WQ_E_INVAL);
    CHECK(wq_init(NULL, 1) == WQ_E_INVAL);
    CHECK(wq_init(NULL, -1) == WQ_E_INVAL);
    int rc = wq_init(NULL, 0);
    CHECK(rc == WQ_E_NODEV || rc == WQ_OK);
    int has_gpu = rc == WQ_OK;
    size_t f = 0, t = 0;
    CHECK(wq_mem_info(-1, &f, &t) == WQ_E_INVAL);
    if (!has_gpu) CHECK(wq_mem_info(0, &f, &t) == WQ_E_NOTINIT);
    /* uploads: argument errors first */
    unsigned char w[64] = {0};
    float sc[4] = {1, 1, 1, 1};
    wq_tensor *tp = NULL;
    CHECK(wq_tensor_upload(NULL, 0, WQ_I4, 4, 8, w, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload(&tp, 0, 9, 4, 8, w, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload(&tp, 0, WQ_I4, 0, 8, w, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload(&tp, 0, WQ_I4, 4, -3, w, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload(&tp, 0, WQ_I4, 4, 8, NULL, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload(&tp, 0, WQ_I4, 4, 8, w, NULL) == WQ_E_INVAL);
    CHECK(wq_tensor_upload(&tp, -1, WQ_I4, 4, 8, w, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload_gs(&tp, 0, WQ_I4, 4, 8, 0, w, sc) == WQ_E_INVAL);
    CHECK(wq_tensor_upload_gs(&tp, 0, WQ_I4, 4, 128, 32, w, sc) == WQ_E_UNSUPPORTED);
    CHECK(wq_tensor_upload_gs(&tp, 0, WQ_F32, 4, 128, 64, w, sc) == WQ_E_INVAL);
    if (!has_gpu) CHECK(wq_tensor_upload(&tp, 0, WQ_I4, 4, 8, w, sc) == WQ_E_NOTINIT);
    CHECK(tp == NULL);
    /* matmul entry points with bad handles or sizes */
    float x[16] = {0}, y[16] = {0};
    CHECK(wq_matmul_t(NULL, x, 1, y) == WQ_E_INVAL);
    CHECK(wq_matmul_dev(NULL, x, 1, y, NULL) == WQ_E_INVAL);
    CHECK(wq_matmul_dev_noalloc(NULL, x, 1, y, NULL) == WQ_E_INVAL);
    CHECK(wq_matmul(&tp, 0, WQ_I4, 4, 8, w, sc, x, -1, y) == WQ_E_INVAL);
    CHECK(wq_matmul(&tp, 0, WQ_I4, 4, 8, w, sc, NULL, 1, y) == WQ_E_INVAL);
    CHECK(wq_noalloc_scratch_bytes() == (size_t)WQ_NOALLOC_SCRATCH_BYTES);
    /* groups */
    wq_group *g = NULL;
    CHECK(wq_grouped_create(NULL, 1, &g) == WQ_E_INVAL);
    wq_tensor *none[1] = {NULL};
    CHECK(wq_grouped_create(none, 1, &g) == WQ_E_INVAL);
    CHECK(wq_grouped_create(none, 0, &g) == WQ_E_INVAL);
    CHECK(wq_swiglu_create(none, NULL, 1, &g) == WQ_E_INVAL);
    CHECK(wq_grouped_free(NULL) == WQ_OK && wq_tensor_free(NULL) == WQ_OK);
    const float *xs[1] = {x};
    float *ys[1] = {y};
    int S1[1] = {1};
    CHECK(wq_grouped_matmul_dev(NULL, xs, S1, ys, NULL) == WQ_E_INVAL);
    CHECK(wq_swiglu_matmul_dev(NULL, xs, S1, ys, NULL) == WQ_E_INVAL);
    CHECK(wq_swiglu_ffn_dev(NULL, NULL, xs, S1, ys, ys, NULL) == WQ_E_INVAL);
    /* measurement helper: argument checks only */
    unsigned out[64];
    CHECK(wq_stream_read_dev(NULL, 1024, 4, 4, out, NULL) == WQ_E_INVAL);
    CHECK(wq_stream_read_dev((void *)0x20000, 1024, 5, 4, out, NULL) == WQ_E_INVAL);
    CHECK(wq_stream_read_dev((void *)0x20000, 1024, 4, 3, out, NULL) == WQ_E_INVAL);
    /* the planner over a spread of shapes, every format and S bucket */
    char buf[256];
    const int Os[] = {1, 3, 64, 1000, 2048, 6144, 12288, 16384, 100000};
    const int Is[] = {1, 5, 63, 512, 1027, 2048, 6144, 8192, 40000, 65536, 200000};
    const int Ss[] = {0, 1, 2, 3, 4, 5, 8, 9, 16, 17, 64, 512, 2048};
    for (int fmt = 0; fmt <= 3; ++fmt)
        for (size_t a = 0; a < sizeof Os / sizeof *Os; ++a)
            for (size_t b = 0; b < sizeof Is / sizeof *Is; ++b)
                for (size_t c = 0; c < sizeof Ss / sizeof *Ss; ++c) {
                    memset(buf, 0x55, sizeof buf);
                    CHECK(wq_describe_plan(fmt, Os[a], Is[b], Ss[c], buf, sizeof buf) == WQ_OK);
                    CHECK(memchr(buf, 0, sizeof buf) != NULL);
                }
    CHECK(wq_describe_plan(0, 4, 4, 1, buf, 8) == WQ_OK && strlen(buf) < 8); /* truncated, terminated */
    CHECK(wq_describe_plan(9, 4, 4, 1, buf, sizeof buf) == WQ_E_INVAL);
    CHECK(wq_describe_plan(0, 4, 4, 1, NULL, sizeof buf) == WQ_E_INVAL);
}

static void oracle_checks(void) {
    for (int fmt = 0; fmt <= 3; ++fmt) {
        for (int trial = 0; trial < 6; ++trial) {
            const long O = 1 + rnd() % 40, I = 1 + rnd() % 300, S = 1 + rnd() % 4;
            const long rb = oracle_row_bytes(fmt, I), stride = rb + (rnd() % 3);
            unsigned char *w = malloc((size_t)(O * stride));
            float *sc = malloc(sizeof(float) * (size_t)O), *x = malloc(sizeof(float) * (size_t)(S * I));
            float *y = malloc(sizeof(float) * (size_t)(S * O)), *y1 = malloc(sizeof(float) * (size_t)(S * O));
            double *a = malloc(sizeof(double) * (size_t)(S * O));
            for (long i = 0; i < O * stride; ++i) w[i] = (unsigned char)rnd();
            if (fmt == 0) /* finite f32 weights */
                for (long o = 0; o < O; ++o)
                    for (long i = 0; i < I; ++i) {
                        float v = rndf();
                        memcpy(w + o * stride + 4 * i, &v, 4);
                    }
            for (long o = 0; o < O; ++o) sc[o] = (o % 5 == 2) ? 0.0f : 0.01f + 0.04f * fabsf(rndf());
            for (long i = 0; i < S * I; ++i) x[i] = rndf();
            CHECK(oracle_matmul(fmt, O, I, w, stride, sc, x, S, y, a, 1) == 0);
            for (long s = 0; s < S; ++s)
                for (long o = 0; o < O; ++o) {
                    CHECK(a[s * O + o] >= fabs((double)y[s * O + o]) * (1.0 - 1e-7));
                    if (o % 5 == 2) CHECK(y[s * O + o] == 0.0f && a[s * O + o] == 0.0);
                }
            if (fmt != 0) { /* one group spanning the row is the per-row form (+0 and -0 equal) */
                CHECK(oracle_matmul_gs(fmt, O, I, w, stride, sc, I, x, S, y1, NULL, 1) == 0);
                for (long j = 0; j < S * O; ++j) CHECK(y[j] == y1[j]);
            }
            free(w), free(sc), free(x), free(y), free(y1), free(a);
        }
    }
    float g[5] = {-3, -0.5f, 0, 0.5f, 3}, u[5] = {1, 2, 3, 4, 5}, h[5];
    oracle_silu_mul(g, u, 5, h);
    CHECK(h[2] == 0.0f && h[3] > 0 && h[0] < 0);
    CHECK(oracle_matmul(1, 2, 4, NULL, 1, NULL, NULL, 1, NULL, NULL, 1) == -1); /* stride < row bytes */
}

int main(void) {
    api_checks();
    oracle_checks();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitized host build: all checks passed\n");
    return 0;
}
