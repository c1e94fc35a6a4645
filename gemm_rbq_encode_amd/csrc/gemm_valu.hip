// gemm_valu.hip -- y = sum_k a_k (.) (B_k x) with a plain fp32 VALU bit loop.
//
// The correctness baseline and the fallback for shapes the MFMA kernels do
// not take.  Each +-1 dot product is formed as 2 * (sum of x where the bit
// is set) - (sum of x over the word), so only additions touch x ("RaBiT"
// summary, paperlayer.ai, section 4.1: binary cores with per-channel
// scales, computed by additions and subtractions).
//
// One wave per output row and token; lane l takes words l, l+64, ... of the
// row, reads the 32 matching fp16 activations, and accumulates
// a_k[r][t] * (2 S_k - sum x) over the K planes; a wave reduction gives y.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

__global__ __launch_bounds__(256) void gemm_valu_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    int K, int group_size, const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y, int silu) {
    const int wave = threadIdx.x / RBQ_WAVE;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    // one output per wave: row r, or with the SiLU-mul epilogue the (gate,
    // up) rows 2r, 2r + 1 giving column r of a Y of out / 2 columns
    const int r = blockIdx.x * 4 + wave;
    const int nout = silu ? out / 2 : out;
    if (r >= nout)
        return;
    const int nr = silu ? 2 : 1;
    const int words = in >> 5;
    const int G = group_size ? in / group_size : 1;
    for (int m = blockIdx.y; m < M; m += gridDim.y) {
        const uint16_t *x = X + (size_t)m * in;
        float acc[2] = {0.0f, 0.0f};
        for (int w = lane; w < words; w += RBQ_WAVE) {
            float xv[32];
            const uint4 *xp = reinterpret_cast<const uint4 *>(x + 32 * w);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = xp[q];
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xv[8 * q + 2 * e] = h2f((uint16_t)(u[e] & 0xFFFFu));
                    xv[8 * q + 2 * e + 1] = h2f((uint16_t)(u[e] >> 16));
                }
            }
            float sx = 0.0f;
#pragma unroll
            for (int b = 0; b < 32; ++b)
                sx += xv[b];
            const int t = group_size ? (32 * w) / group_size : 0;
            for (int q = 0; q < nr; ++q) {
                const int row = nr * r + q;
                for (int k = 0; k < K; ++k) {
                    const uint32_t bits = planes[((size_t)k * out + row) * words + w];
                    float s = 0.0f;
#pragma unroll
                    for (int b = 0; b < 32; ++b)
                        s += ((bits >> b) & 1u) ? xv[b] : 0.0f;
                    const float a = h2f(scales[((size_t)k * out + row) * G + t]);
                    acc[q] += a * (2.0f * s - sx);
                }
            }
        }
        acc[0] = wave_sum_f32(acc[0]);
        if (silu)
            acc[1] = wave_sum_f32(acc[1]);
        if (lane == 0)
            Y[(size_t)m * nout + r] = silu ? silu_mul_f16(acc[0], acc[1]) : f2h(acc[0]);
    }
}

// Dual scales for M tokens: Y[m][r] = sum_k g_k[r] sum_j (bit ? +1 : -1)
// h_k[j] X[m][j] ("RaBiT" summary, section 4.1: a scaling vector on each
// side of every binary core).  One wave per output row and token; lane l
// takes words l, l+64, ...; the products h_k[j] x[j] of two binary16
// values are exact in fp32, summed in fp32 per lane, then by a wave
// reduction; each plane's sum takes its row scale once.
__global__ __launch_bounds__(256) void gemm_valu_dual_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ g, const uint16_t *__restrict__ h,
    int out, int in, int K, const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y) {
    const int wave = threadIdx.x / RBQ_WAVE;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int r = blockIdx.x * 4 + wave;
    if (r >= out)
        return;
    const int words = in >> 5;
    for (int m = blockIdx.y; m < M; m += gridDim.y) {
        const uint16_t *x = X + (size_t)m * in;
        float y = 0.0f;
        for (int k = 0; k < K; ++k) {
            float acc = 0.0f;
            for (int w = lane; w < words; w += RBQ_WAVE) {
                const uint32_t bits = planes[((size_t)k * out + r) * words + w];
                const uint4 *xp = reinterpret_cast<const uint4 *>(x + 32 * w);
                const uint4 *hp = reinterpret_cast<const uint4 *>(h + (size_t)k * in + 32 * w);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 xv = xp[q], hv = hp[q];
                    const uint32_t xu[4] = {xv.x, xv.y, xv.z, xv.w}, hu[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint16_t xb = (uint16_t)(xu[e >> 1] >> (16 * (e & 1)));
                        const uint16_t hb = (uint16_t)(hu[e >> 1] >> (16 * (e & 1)));
                        const float p = h2f(xb) * h2f(hb);
                        acc += ((bits >> (8 * q + e)) & 1u) ? p : -p;
                    }
                }
            }
            acc = wave_sum_f32(acc);
            y = __builtin_fmaf(h2f(g[(size_t)k * out + r]), acc, y);
        }
        if (lane == 0)
            Y[(size_t)m * out + r] = f2h(y);
    }
}

__global__ void fill_zero_u16_kernel(uint16_t *Y, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        Y[i] = 0;
}

}  // namespace

hipError_t launch_gemm_valu(const uint32_t *planes, const uint16_t *scales, int out, int in,
                            int K, int group_size, const uint16_t *X, int M, uint16_t *Y, int silu,
                            hipStream_t st) {
    if (silu && out % 2 != 0)
        return hipErrorInvalidValue;
    const int gy = M < 65535 ? M : 65535;
    const int nout = silu ? out / 2 : out;
    hipLaunchKernelGGL(gemm_valu_kernel, dim3((nout + 3) / 4, gy), dim3(256), 0, st, planes,
                       scales, out, in, K, group_size, X, M, Y, silu);
    return hipGetLastError();
}

hipError_t launch_gemm_valu_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                                 int K, const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    const int gy = M < 65535 ? M : 65535;
    hipLaunchKernelGGL(gemm_valu_dual_kernel, dim3((out + 3) / 4, gy), dim3(256), 0, st, planes, g, h, out, in, K,
                       X, M, Y);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t *Y, int64_t n, hipStream_t st) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(fill_zero_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, Y, n);
    return hipGetLastError();
}

}  // namespace rbq
