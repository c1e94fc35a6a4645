// refit.hip -- joint least-squares refit of the K scales of every (row,
// group) for fixed sign planes.
//
// The cascade of the encoder fits each scale for its own step only; the
// refinement in the QBB summary (atlas.scime.ai, "Approach": the binary
// bases are refined after the analytical initialisation) has a part that
// needs no data, the least-squares fit of all K scales together with the
// planes held fixed:
//     minimise sum_j (W_j - sum_k a_k B_kj)^2,
// whose normal equations are G a = b with
//     G_kl = sum_j B_kj B_lj = n - 2 * (columns where planes k and l differ)
//     b_k  = sum_j B_kj W_j.
// G is integer (counted exactly with popcounts); b is summed in fp64 in
// parallel; G = L D L^T (unit lower L, no square roots) and the solve run in
// fp64 in a fixed order, and each scale is rounded once to binary16.  A
// pivot D_i <= n 2^-30 (dependent planes, such as the identical all-+1
// planes of an all-zero row), a non-finite W, or a scale that is not finite
// in binary16 keeps the given scales of that (row, group) and sets a status
// bit.  With one plane the refit is sum_j |W_j| / n, the encoder's scale.
//
// Work: a segment (row, group of n columns) is handled by LPS lanes (4 for
// 128-column groups, so 16 segments per wave; 64 for whole rows).  Each lane
// reads 8 consecutive columns at a time (two 16-byte loads of W and one byte
// of every plane's word), adds +-W_j into K fp64 sums and counts plane
// differences with popcounts; the lanes of a segment then combine with
// shuffles, and the segment's first lane solves and writes.  The serial
// solve runs once per wave for all its segments, so fewer lanes per group
// means fewer solves: 13824 x 5120, K = 4, took 169 us with 16 lanes per
// group, 85 us with 4, 88 us with 2 and 162 us with 1 (whose loads no longer
// fill whole cache lines).  The kernel reads W once (HBM-bound, like the
// encoder).
#include "rbq.h"
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int RF_THREADS = 256;
constexpr int RF_GROUP_LPS = 4;                 // lanes per 128-column group

template <int LPS>
__device__ __forceinline__ double seg_sum_f64(double v) {
#pragma unroll
    for (int m = 1; m < LPS; m <<= 1)
        v += __shfl_xor(v, m, RBQ_WAVE);
    return v;
}

template <int LPS>
__device__ __forceinline__ int seg_sum_i32(int v) {
#pragma unroll
    for (int m = 1; m < LPS; m <<= 1)
        v += __shfl_xor(v, m, RBQ_WAVE);
    return v;
}

// L D L^T solve of the K x K normal equations, in the fixed order the
// definition above gives (no contraction into fused multiply-adds, so the
// pivots of an integer G come out the same wherever this runs).  Returns
// false for a pivot <= n 2^-30.
template <int K>
__device__ bool ldl_solve(const double (&g)[K][K], const double (&b)[K], double n, double (&a)[K]) {
#pragma clang fp contract(off)
    double L[K][K], D[K], z[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
#pragma unroll
        for (int j = 0; j < i; ++j) {
            double s = g[i][j];
#pragma unroll
            for (int p = 0; p < j; ++p)
                s = s - (L[i][p] * D[p]) * L[j][p];
            L[i][j] = s / D[j];
        }
        double s = g[i][i];
#pragma unroll
        for (int p = 0; p < i; ++p)
            s = s - (L[i][p] * D[p]) * L[i][p];
        D[i] = s;
        if (!(s > n * 0x1p-30))
            return false;
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
        double s = b[i];
#pragma unroll
        for (int p = 0; p < i; ++p)
            s = s - L[i][p] * z[p];
        z[i] = s;
    }
#pragma unroll
    for (int i = K - 1; i >= 0; --i) {
        double s = z[i] / D[i];
#pragma unroll
        for (int p = i + 1; p < K; ++p)
            s = s - L[p][i] * a[p];
        a[i] = s;
    }
    return true;
}

// Grid: RF_THREADS threads = RF_THREADS / LPS segments per workgroup;
// segment id = row * G + group.
template <int K, int LPS>
__global__ __launch_bounds__(RF_THREADS) void refit_kernel(const float *__restrict__ W, int out, int in, int n,
                                                           const uint32_t *__restrict__ planes,
                                                           uint16_t *__restrict__ scales,
                                                           int32_t *__restrict__ status) {
    const int G = in / n;
    const long nseg = (long)out * G;
    const long seg = (long)blockIdx.x * (RF_THREADS / LPS) + threadIdx.x / LPS;
    const int sl = threadIdx.x % LPS;                       // lane within the segment
    const bool live = seg < nseg;
    const int r = live ? (int)(seg / G) : 0;
    const int t = live ? (int)(seg - (long)r * G) : 0;
    const int words = in >> 5;
    const size_t plane_stride = (size_t)out * words;

    double b[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        b[k] = 0.0;
    int differ[K * (K - 1) / 2 + 1];
#pragma unroll
    for (int p = 0; p < K * (K - 1) / 2 + 1; ++p)
        differ[p] = 0;
    bool finite = true;
    if (live) {
        const float *wrow = W + (size_t)r * in + (size_t)t * n;
        const uint32_t *prow = planes + (size_t)r * words;
        for (int c = 8 * sl; c < n; c += 8 * LPS) {
            const int col = t * n + c;                      // column in the row
            const v4f w0 = *reinterpret_cast<const v4f *>(wrow + c);
            const v4f w1 = *reinterpret_cast<const v4f *>(wrow + c + 4);
            const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                finite = finite && __builtin_isfinite(w[e]);
            uint32_t byte[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                byte[k] = (prow[k * plane_stride + (col >> 5)] >> (col & 31)) & 0xFFu;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    b[k] += ((byte[k] >> e) & 1u) ? (double)w[e] : -(double)w[e];
            int p = 0;
#pragma unroll
            for (int k = 1; k < K; ++k)
#pragma unroll
                for (int l = 0; l < k; ++l)
                    differ[p++] += __builtin_popcount(byte[k] ^ byte[l]);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
        b[k] = seg_sum_f64<LPS>(b[k]);
#pragma unroll
    for (int p = 0; p < K * (K - 1) / 2; ++p)
        differ[p] = seg_sum_i32<LPS>(differ[p]);
    const int all_finite = seg_sum_i32<LPS>(finite ? 0 : 1) == 0;

    if (live && sl == 0) {
        const double nd = (double)n;
        double g[K][K];
        int p = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            g[k][k] = nd;
#pragma unroll
            for (int l = 0; l < k; ++l) {
                g[k][l] = g[l][k] = (double)(n - 2 * differ[p]);
                ++p;
            }
        }
        double a[K];
        bool ok = all_finite && ldl_solve<K>(g, b, nd, a);
        uint16_t h[K];
        if (ok) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                h[k] = f64_to_f16_rne(a[k]);
                if ((h[k] & 0x7C00u) == 0x7C00u)
                    ok = false;
            }
        }
        if (ok) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                scales[((size_t)k * out + r) * G + t] = h[k];
        } else if (status != nullptr) {
            atomicOr(status, (all_finite ? 0 : (int)RBQ_STATUS_NONFINITE_W) | (int)RBQ_STATUS_REFIT_KEPT);
        }
    }
}

template <int K, int LPS>
hipError_t launch_kl(const float *W, int out, int in, int n, const uint32_t *planes, uint16_t *scales,
                     int32_t *status, hipStream_t st) {
    const long nseg = (long)out * (in / n);
    const long per = RF_THREADS / LPS;
    const long blocks = (nseg + per - 1) / per;
    if (blocks > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((refit_kernel<K, LPS>), dim3((unsigned)blocks), dim3(RF_THREADS), 0, st, W, out, in, n,
                       planes, scales, status);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const float *W, int out, int in, int n, const uint32_t *planes, uint16_t *scales,
                    int32_t *status, hipStream_t st) {
    // 4 lanes for 128-column groups (8 columns at a time), 64 for longer segments
    if (n <= 128)
        return launch_kl<K, RF_GROUP_LPS>(W, out, in, n, planes, scales, status, st);
    return launch_kl<K, 64>(W, out, in, n, planes, scales, status, st);
}

}  // namespace

hipError_t launch_refit(const float *W, int out, int in, int K, int group_size, const uint32_t *planes,
                        uint16_t *scales, int32_t *status, hipStream_t st) {
    const int n = group_size ? group_size : in;
    if (out <= 0 || in <= 0 || n % 8 != 0 || in % n != 0)
        return hipErrorInvalidValue;
    switch (K) {
    case 1: return launch_k<1>(W, out, in, n, planes, scales, status, st);
    case 2: return launch_k<2>(W, out, in, n, planes, scales, status, st);
    case 3: return launch_k<3>(W, out, in, n, planes, scales, status, st);
    case 4: return launch_k<4>(W, out, in, n, planes, scales, status, st);
    case 5: return launch_k<5>(W, out, in, n, planes, scales, status, st);
    case 6: return launch_k<6>(W, out, in, n, planes, scales, status, st);
    case 7: return launch_k<7>(W, out, in, n, planes, scales, status, st);
    case 8: return launch_k<8>(W, out, in, n, planes, scales, status, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rbq
