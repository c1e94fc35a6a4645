/*
 * Drives the CPU oracle (oracle/rbq_oracle.c) over small seeded inputs so
 * that it can run under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Test infrastructure: built and run by tests/test_sanitizers_cpu.py.
 *
 * Besides running every entry point (encode, dequant, gemm, refit, the fp16
 * conversions) on ragged and degenerate shapes, it checks facts that need no
 * second implementation: the layer output equals the dequantised matrix
 * times x, every scale is finite for finite W, non-finite W is flagged, and
 * bad arguments return -1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16(double v);
void oracle_f64_to_f16_array(const double *v, int64_t n, uint16_t *out);
int oracle_encode(const float *W, int64_t out, int64_t in, int K, int64_t group_size,
                  uint32_t *planes, uint16_t *scales);
int oracle_dequant(const uint32_t *planes, const uint16_t *scales, int64_t out, int64_t in,
                   int K, int64_t group_size, double *What);
int oracle_gemm(const uint32_t *planes, const uint16_t *scales, int64_t out, int64_t in,
                int K, int64_t group_size, const uint16_t *X, int64_t M, double *Y);
int oracle_refit(const float *W, int64_t out, int64_t in, int K, int64_t group_size,
                 const uint32_t *planes, uint16_t *scales);

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double uniform(void)            /* splitmix64 -> [0, 1) */
{
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fputc('\n', stderr);                           \
            ++failures;                                    \
        }                                                  \
    } while (0)

static void run_shape(int64_t out, int64_t in, int K, int64_t group, int64_t M)
{
    const int64_t G = in == 0 ? 0 : (group ? in / group : 1);
    float *W = malloc(sizeof(float) * (size_t)(out * in + 1));
    uint32_t *planes = malloc(sizeof(uint32_t) * (size_t)(K * out * (in / 32) + 1));
    uint16_t *scales = malloc(sizeof(uint16_t) * (size_t)(K * out * G + 1));
    double *What = malloc(sizeof(double) * (size_t)(out * in + 1));
    uint16_t *X = malloc(sizeof(uint16_t) * (size_t)(M * in + 1));
    double *Y = malloc(sizeof(double) * (size_t)(M * out + 1));
    for (int64_t i = 0; i < out * in; ++i)
        W[i] = (float)((uniform() - 0.5) * 0.08);
    if (out > 1)                                   /* an all-zero row */
        memset(W + in, 0, sizeof(float) * (size_t)in);
    for (int64_t i = 0; i < M * in; ++i)
        X[i] = oracle_f64_to_f16((uniform() - 0.5) * 4.0);

    int flags = oracle_encode(W, out, in, K, group, planes, scales);
    CHECK(flags == 0, "encode flags %d (out %ld in %ld K %d)", flags, (long)out, (long)in, K);
    for (int64_t i = 0; i < K * out * G; ++i)
        CHECK(isfinite(oracle_f16_to_f64(scales[i])), "scale %ld not finite", (long)i);
    CHECK(oracle_dequant(planes, scales, out, in, K, group, What) == 0, "dequant");
    CHECK(oracle_gemm(planes, scales, out, in, K, group, X, M, Y) == 0, "gemm");
    for (int64_t m = 0; m < M; ++m)
        for (int64_t r = 0; r < out; ++r) {
            double ref = 0.0, mag = 0.0;
            for (int64_t j = 0; j < in; ++j) {
                ref += What[r * in + j] * oracle_f16_to_f64(X[m * in + j]);
                mag += fabs(What[r * in + j] * oracle_f16_to_f64(X[m * in + j]));
            }
            CHECK(fabs(Y[m * out + r] - ref) <= 1e-12 * (mag + 1e-300), "gemm row %ld token %ld", (long)r,
                  (long)m);
        }
    int rf = oracle_refit(W, out, in, K, group, planes, scales);
    CHECK(rf >= 0 && (rf & 1) == 0, "refit flags %d", rf);

    free(W); free(planes); free(scales); free(What); free(X); free(Y);
}

int main(void)
{
    /* fp16 conversions over every bit pattern and back */
    for (uint32_t h = 0; h < 65536; ++h) {
        double v = oracle_f16_to_f64((uint16_t)h);
        if (!isnan(v)) {
            uint16_t back = oracle_f64_to_f16(v);
            CHECK(back == h, "fp16 round trip %04x -> %04x", h, back);
        }
    }
    double vals[5] = {0.0, -0.0, 65520.0, 1e-9, -3.25};
    uint16_t outv[5];
    oracle_f64_to_f16_array(vals, 5, outv);
    CHECK(outv[2] == 0x7c00, "65520 rounds to +inf");

    /* shapes: ragged, degenerate, grouped, every K */
    run_shape(1, 32, 1, 0, 1);
    run_shape(5, 96, 2, 0, 3);
    run_shape(17, 256, 3, 128, 2);
    run_shape(16, 512, 4, 128, 4);
    run_shape(3, 384, 8, 128, 1);
    run_shape(0, 64, 2, 0, 1);
    run_shape(4, 0, 2, 0, 1);

    /* non-finite W is flagged; bad arguments are refused */
    {
        float W[64];
        uint32_t p[4];
        uint16_t s[4];
        for (int i = 0; i < 64; ++i)
            W[i] = 0.01f * (float)(i - 30);
        W[7] = NAN;
        W[40] = INFINITY;
        CHECK(oracle_encode(W, 2, 32, 2, 0, p, s) & 1, "non-finite W flagged");
        CHECK(oracle_encode(W, 2, 48, 2, 0, p, s) == -1, "in %% 32");
        CHECK(oracle_encode(W, 2, 32, 9, 0, p, s) == -1, "K > 8");
        CHECK(oracle_encode(W, 1, 64, 2, 48, p, s) == -1, "group does not divide in");
        CHECK(oracle_gemm(p, s, 2, 32, 2, 0, NULL, -1, NULL) == -1, "M < 0");
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle host checks passed\n");
    return 0;
}
