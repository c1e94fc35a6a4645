/*
 * rbq_oracle.c -- plain, slow CPU oracle for the residual-binarized linear
 * layer.  TEST INFRASTRUCTURE ONLY: it exists so the tests, the smoke check
 * and the benchmark's CPU-baseline leg can check and time the HIP library.
 * Nothing in the product path may call it, and it shares no code, header or
 * table with the HIP library.
 *
 * What it computes (sources: "RaBiT: Residual-Aware Binarization Training
 * for Accurate and Efficient LLMs", paperlayer.ai summary, sections 4.1, 4.2,
 * A, B, G and D "GPU implementation"; "QBB: Quantization with Binary Bases
 * for LLMs", atlas.scime.ai summary, "Approach" and "Key results"):
 *
 *   W ~= sum_k a_k (.) B_k, each B_k a +-1 matrix ("binary core", RaBiT 4.1)
 *   with a scale per output row (RaBiT) or per row per group of 128 input
 *   columns (QBB "W(4x1)A16g128").  The cores are derived one after another
 *   from one full-precision weight: B_1 = sign(W), the residual
 *   R_1 = W - a_1 B_1, B_2 = sign(R_1), ... (RaBiT 4.2, A "RaBiT",
 *   B "RaBiT residual coupling", G "RaBiT training"; QBB "cascaded
 *   analytical residual binarization").  The closed-form scale for a fixed
 *   sign pattern is the mean absolute residual (the XNOR-Net binarization
 *   that QBB lists under "Builds on").
 *
 *   y = sum_k a_k (.) (B_k x): the layer output as a plain fp64
 *   dequantize-and-multiply (RaBiT 4.1 "additions and subtractions").
 *
 *   Optional refinement of the scales for fixed planes: the joint
 *   least-squares fit of the K scales of each (row, group) (QBB
 *   "Approach", the data-free part of its refinement of the bases).
 *
 * Readings where the pages are silent (each also listed in the design doc):
 *   - sign(0) = +1, decided by comparison (R >= 0), so -0.0 gives +1.
 *   - packed layout: plane k, row r, word w, bit b (LSB first) holds column
 *     32w + b; bit 1 means +1 (RaBiT D "GPU implementation": 32 columns per
 *     uint32).  Planes are [K][out][in/32], scales fp16 bits [K][out][G].
 *   - the mean |R| of a (row, group) is one serial fp64 sum in ascending
 *     column order, one correctly rounded fp64 division by the count, then
 *     ONE rounding fp64 -> binary16 to nearest, ties to even.
 *   - the residual subtracts the stored (fp16-rounded) scale, computed in
 *     fp32 with one rounding: R <- R - (+-a).
 *   - groups are consecutive runs of group_size columns starting at
 *     column 0; group_size 0 means one group of the whole row.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * OpenMP only spreads rows over threads; each row's arithmetic order is
 * fixed, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* IEEE binary16 <-> binary64                                          */
/* ------------------------------------------------------------------ */

/* binary16 bit pattern -> its exact value as a double. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0x1f)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1.f) * 2^(e-15)     */
    return sign ? -v : v;
}

/* double -> binary16 bit pattern, rounded once, to nearest, ties to even.
 * The value is scaled by the power-of-two quantum of its binade (exact),
 * rounded to an integer with rint() (default mode: ties to even), and the
 * integer is placed in the bit pattern; a carry out of the significand
 * moves into the exponent field, which is the correct next binade. */
uint16_t oracle_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00);
    /* 65520 is halfway between 65504 (largest finite, odd significand) and
     * 2^16; ties go to the even neighbour, which is out of range: infinity. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24 */
        double n = rint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)n);   /* n == 1024 is the smallest normal */
    }
    int ex;
    frexp(a, &ex);                  /* a = f * 2^ex, f in [0.5, 1): leading bit 2^(ex-1) */
    int lead = ex - 1;              /* -14 .. 15 */
    double n = rint(ldexp(a, 10 - lead));        /* 1024 .. 2048 */
    uint32_t bits = (uint32_t)((lead + 15) << 10) + (uint32_t)n - 1024u;
    return (uint16_t)(sign | bits);
}

/* Array form of oracle_f64_to_f16 (one call per element). */
void oracle_f64_to_f16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_f16(v[i]);
}

/* ------------------------------------------------------------------ */
/* Encoder: sequential residual binarization                            */
/* ------------------------------------------------------------------ */

/*
 * W: fp32 [out][in].  planes: uint32 [K][out][in/32] (fully written).
 * scales: fp16 bits [K][out][G], G = group_size ? in/group_size : 1.
 * Returns a flag word: bit 0 = some W entry is not finite, bit 1 = some
 * scale rounded to infinity.  Returns -1 on bad arguments.
 */
int oracle_encode(const float *W, int64_t out, int64_t in, int K, int64_t group_size,
                  uint32_t *planes, uint16_t *scales)
{
    if (out < 0 || in < 0 || in % 32 || K < 1 || K > 8 || group_size < 0)
        return -1;
    if (group_size && in % group_size)
        return -1;
    int64_t n = group_size ? group_size : in;   /* columns per group */
    int64_t G = (in == 0) ? 0 : (group_size ? in / group_size : 1);
    int64_t words = in / 32;
    int flags = 0;

    #pragma omp parallel for schedule(static) reduction(|:flags)
    for (int64_t r = 0; r < out; ++r) {
        float *R = (float *)malloc(sizeof(float) * (size_t)(in ? in : 1));
        memcpy(R, W + r * in, sizeof(float) * (size_t)in);
        for (int64_t j = 0; j < in; ++j)
            if (!isfinite(R[j]))
                flags |= 1;
        for (int k = 0; k < K; ++k) {
            uint32_t *prow = planes + ((int64_t)k * out + r) * words;
            memset(prow, 0, sizeof(uint32_t) * (size_t)words);
            for (int64_t t = 0; t < G; ++t) {
                int64_t c0 = t * n;
                /* B_k = sign(R_{k-1}) with sign(0) = +1, and the closed-form
                 * scale mean|R_{k-1}| of this group. */
                double S = 0.0;
                for (int64_t j = c0; j < c0 + n; ++j)
                    S += (double)fabsf(R[j]);
                double m = S / (double)n;
                uint16_t h = oracle_f64_to_f16(m);
                if ((h & 0x7fff) == 0x7c00)
                    flags |= 2;
                scales[((int64_t)k * out + r) * G + t] = h;
                float a = (float)oracle_f16_to_f64(h);   /* exact */
                for (int64_t j = c0; j < c0 + n; ++j) {
                    int plus = (R[j] >= 0.0f);
                    if (plus)
                        prow[j / 32] |= (uint32_t)1 << (j % 32);
                    /* residual against the stored path: R - a * (+-1) */
                    R[j] = R[j] - (plus ? a : -a);
                }
            }
        }
        free(R);
    }
    return flags;
}

/* ------------------------------------------------------------------ */
/* Dequantize and multiply (plain definition of the layer output)       */
/* ------------------------------------------------------------------ */

/* What[r][j] = sum_k a_k[r][group(j)] * (bit ? +1 : -1), in fp64 (exact for
 * K <= 8: every term is an fp16 value, and the sum of at most eight fp16
 * values fits in a double's significand). */
int oracle_dequant(const uint32_t *planes, const uint16_t *scales, int64_t out, int64_t in,
                   int K, int64_t group_size, double *What)
{
    if (out < 0 || in < 0 || in % 32 || K < 1 || K > 8 || group_size < 0)
        return -1;
    if (group_size && in % group_size)
        return -1;
    int64_t G = group_size ? in / group_size : 1;
    int64_t words = in / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < out; ++r) {
        for (int64_t j = 0; j < in; ++j) {
            int64_t t = group_size ? j / group_size : 0;
            double w = 0.0;
            for (int k = 0; k < K; ++k) {
                double a = oracle_f16_to_f64(scales[((int64_t)k * out + r) * G + t]);
                uint32_t word = planes[((int64_t)k * out + r) * words + j / 32];
                int bit = (word >> (j % 32)) & 1u;
                w += bit ? a : -a;
            }
            What[r * in + j] = w;
        }
    }
    return 0;
}

/* Y[m][r] = sum_j What[r][j] * X[m][j], fp64, j ascending.
 * X: fp16 bits [M][in].  Y: double [M][out]. */
int oracle_gemm(const uint32_t *planes, const uint16_t *scales, int64_t out, int64_t in,
                int K, int64_t group_size, const uint16_t *X, int64_t M, double *Y)
{
    if (out < 0 || in < 0 || in % 32 || K < 1 || K > 8 || group_size < 0 || M < 0)
        return -1;
    if (group_size && in % group_size)
        return -1;
    int64_t G = group_size ? in / group_size : 1;
    int64_t words = in / 32;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * in + 1));
    for (int64_t i = 0; i < M * in; ++i)
        xd[i] = oracle_f16_to_f64(X[i]);

    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < out; ++r) {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(in + 1));
        for (int64_t j = 0; j < in; ++j) {
            int64_t t = group_size ? j / group_size : 0;
            double w = 0.0;
            for (int k = 0; k < K; ++k) {
                double a = oracle_f16_to_f64(scales[((int64_t)k * out + r) * G + t]);
                uint32_t word = planes[((int64_t)k * out + r) * words + j / 32];
                w += ((word >> (j % 32)) & 1u) ? a : -a;
            }
            wrow[j] = w;
        }
        for (int64_t m = 0; m < M; ++m) {
            const double *x = xd + m * in;
            double acc = 0.0;
            for (int64_t j = 0; j < in; ++j)
                acc += wrow[j] * x[j];
            Y[m * out + r] = acc;
        }
        free(wrow);
    }
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Joint least-squares refit of the K scales for fixed planes           */
/* ------------------------------------------------------------------ */

/*
 * The cascade picks each scale for its own step only; the refinement the
 * QBB summary describes ("Approach": the binary bases are refined after
 * the analytical initialisation) starts from there.  Its part that needs no
 * data is the joint least-squares fit of the K scales of every (row, group)
 * to W with the planes held fixed:
 *     minimise sum_j (W_j - sum_k a_k B_kj)^2  over a = (a_1 .. a_K).
 * Normal equations G a = b with
 *     G_kl = sum_j B_kj B_lj = n - 2 * (columns where planes k, l differ),
 *     b_k  = sum_j B_kj W_j   (one serial fp64 sum, ascending columns).
 * G is factored as L D L^T (unit lower L, no square roots) in the fixed
 * order below, and the solve runs forward, diagonal, backward.  A pivot
 * D_i <= n * 2^-30 (dependent planes, e.g. all-zero rows where every plane
 * is +1), a non-finite b, or a solution that is not finite in binary16
 * keeps the given scales of that (row, group).  Each solved scale is rounded
 * once to binary16.  For K = 1 this is b / n = mean |W|, the cascade's own
 * first scale.
 *
 * scales: in = the scales kept where no refit is made (normally the
 * encoder's), out = the refit.  Returns flags: bit 0 = a non-finite W,
 * bit 2 = some (row, group) kept its scales; -1 on bad arguments.
 */
int oracle_refit(const float *W, int64_t out, int64_t in, int K, int64_t group_size,
                 const uint32_t *planes, uint16_t *scales)
{
    if (out < 0 || in < 0 || in % 32 || K < 1 || K > 8 || group_size < 0)
        return -1;
    if (group_size && in % group_size)
        return -1;
    int64_t n = group_size ? group_size : in;
    int64_t G = (in == 0) ? 0 : (group_size ? in / group_size : 1);
    int64_t words = in / 32;
    int flags = 0;

    #pragma omp parallel for schedule(static) reduction(|:flags)
    for (int64_t r = 0; r < out; ++r) {
        const float *w = W + r * in;
        for (int64_t j = 0; j < in; ++j)
            if (!isfinite(w[j]))
                flags |= 1;
        for (int64_t t = 0; t < G; ++t) {
            int64_t c0 = t * n;
            double g[8][8], b[8], L[8][8], D[8], z[8], a[8];
            /* normal equations */
            for (int k = 0; k < K; ++k) {
                const uint32_t *pk = planes + ((int64_t)k * out + r) * words;
                b[k] = 0.0;
                for (int64_t j = c0; j < c0 + n; ++j) {
                    int plus = (pk[j / 32] >> (j % 32)) & 1u;
                    b[k] += plus ? (double)w[j] : -(double)w[j];
                }
                for (int l = 0; l <= k; ++l) {
                    const uint32_t *pl = planes + ((int64_t)l * out + r) * words;
                    int64_t differ = 0;
                    for (int64_t j = c0; j < c0 + n; ++j)
                        differ += ((pk[j / 32] ^ pl[j / 32]) >> (j % 32)) & 1u;
                    g[k][l] = g[l][k] = (double)(n - 2 * differ);
                }
            }
            /* G = L D L^T */
            int ok = 1;
            for (int i = 0; i < K && ok; ++i) {
                for (int j = 0; j < i; ++j) {
                    double s = g[i][j];
                    for (int p = 0; p < j; ++p)
                        s = s - (L[i][p] * D[p]) * L[j][p];
                    L[i][j] = s / D[j];
                }
                double s = g[i][i];
                for (int p = 0; p < i; ++p)
                    s = s - (L[i][p] * D[p]) * L[i][p];
                D[i] = s;
                if (!(s > (double)n * 0x1p-30))
                    ok = 0;
            }
            for (int k = 0; k < K && ok; ++k)
                if (!isfinite(b[k]))
                    ok = 0;
            uint16_t h[8];
            if (ok) {
                for (int i = 0; i < K; ++i) {      /* L z = b */
                    double s = b[i];
                    for (int p = 0; p < i; ++p)
                        s = s - L[i][p] * z[p];
                    z[i] = s;
                }
                for (int i = K - 1; i >= 0; --i) { /* D L^T a = z */
                    double s = z[i] / D[i];
                    for (int p = i + 1; p < K; ++p)
                        s = s - L[p][i] * a[p];
                    a[i] = s;
                }
                for (int k = 0; k < K; ++k) {
                    h[k] = oracle_f64_to_f16(a[k]);
                    if ((h[k] & 0x7c00) == 0x7c00)  /* inf or nan */
                        ok = 0;
                }
            }
            if (ok) {
                for (int k = 0; k < K; ++k)
                    scales[((int64_t)k * out + r) * G + t] = h[k];
            } else {
                flags |= 4;
            }
        }
    }
    return flags;
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
