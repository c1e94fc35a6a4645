// qat.hip -- the coupled (QAT-style) forward and its straight-through
// backward ("RaBiT" summary, paperlayer.ai: section 4.2 "Coupled Training"
// and the "RaBiT training" procedure of section G).
//
// Training keeps one shared fp32 weight W and learnable binary16 scales a_k;
// every forward pass derives the binary cores again, path by path, from W:
// B_1 = sign(W), R_1 = W - a_1 B_1, B_2 = sign(R_1), ... (sign(0) = +1).
// The backward passes the gradient straight through sign():
//   dW      = dY^T X                          (the gradient of What, whole)
//   da_k    = sum over the columns j of a scale's group of B_k[r][j] dW[r][j]
//   dX      = dY What,  What = sum_k a_k B_k
//
// Four kernels:
//  * qat_cascade_kernel: the cores for given scales.  One wave per row reads
//    the row 64 columns at a time (one fp32 per lane, 256 coalesced bytes,
//    8 chunks in flight), steps the residual through the K paths in fp32
//    (one rounding per step, the same operations as the definition), and the
//    ballot of each step is two plane words; v_writelane gathers 64 words
//    per plane into one VGPR, stored coalesced.  Bound by the read of W.
//  * qat_dw_kernel: dW = dY^T X on v_mfma_f32_16x16x32_f16.  fp16 products
//    are exact in fp32, so dW carries only the fp32 accumulation error.  A
//    workgroup computes a 128 x 128 tile of dW; the token dimension is the
//    contraction, staged 32 tokens at a time through LDS transposed (rows
//    of dW and columns of X along the LDS rows, tokens contiguous) so that
//    each lane's 8-token fragment is one 16-byte LDS read.
//  * qat_dscales_kernel: one wave per (row, scale group) reads that part of
//    dW with the sign words and sums B_k dW in fp64 in a fixed order.
//  * qat_dx_kernel: dX = dY What on the same MFMA.  What is formed per tile
//    from the sign words and scales in fp32 and split into two fp16 parts
//    hi = fp16(w), lo = fp16(w - hi), so dY hi + dY lo carries w to 2^-22
//    relative (an absolute 2^-25 where lo is subnormal) with fp32
//    accumulation; a formed weight beyond the fp16 range is reported.
#include <algorithm>

#include "rbq.h"
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

// v_writelane_b32 (write one lane of a VGPR from a uniform value).
extern "C" __device__ int rbq_qat_writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// cores for given scales

constexpr int QC_THREADS = 256;
constexpr int QC_WAVES = QC_THREADS / RBQ_WAVE;
constexpr int QC_UNROLL = 8;

template <int K>
__global__ __launch_bounds__(QC_THREADS) void qat_cascade_kernel(const float *__restrict__ W, int out, int in,
                                                                 int group_size,
                                                                 const uint16_t *__restrict__ scales,
                                                                 uint32_t *__restrict__ planes,
                                                                 int32_t *__restrict__ status) {
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / RBQ_WAVE));
    const int r = blockIdx.x * QC_WAVES + wave;
    if (r >= out)
        return;                               // whole wave
    const int words = in >> 5;
    const int G = group_size ? in / group_size : 1;
    const size_t plane_stride = (size_t)out * words;
    const float *wr = W + (size_t)r * in;
    uint32_t *pr = planes + (size_t)r * words;

    uint32_t acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        acc[k] = 0u;
    int slot = 0, wbase = 0;
    bool bad = false;
    float a[K];
    int cur_g = -1;
    for (int c0 = 0; c0 < in; c0 += RBQ_WAVE * QC_UNROLL) {
        float w[QC_UNROLL];
#pragma unroll
        for (int u = 0; u < QC_UNROLL; ++u) {
            const int c = c0 + u * RBQ_WAVE + lane;
            w[u] = c < in ? wr[c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < QC_UNROLL; ++u) {
            const int c = c0 + u * RBQ_WAVE;   // uniform
            if (c >= in)
                break;
            // a chunk of 64 columns lies in one group (groups of 128 start at
            // multiples of 128), so the scales are uniform over the wave
            const int g = group_size ? c / group_size : 0;
            if (g != cur_g) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    a[k] = h2f(scales[((size_t)k * out + r) * G + g]);
                cur_g = g;
            }
            const bool half = c + 32 >= in;    // the row ends after 32 more columns
            float R = w[u];
            bad = bad || ((!half || lane < 32) && !__builtin_isfinite(R));
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const bool b = R >= 0.0f;      // -0.0 gives +1; NaN gives -1
                const uint64_t m = __ballot(b);
                R = b ? R - a[k] : R + a[k];
                acc[k] = (uint32_t)rbq_qat_writelane_i32((int)(uint32_t)m, slot, (int)acc[k]);
                if (!half)
                    acc[k] = (uint32_t)rbq_qat_writelane_i32((int)(uint32_t)(m >> 32), slot + 1, (int)acc[k]);
            }
            slot += half ? 1 : 2;
            if (slot == RBQ_WAVE) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    pr[(size_t)k * plane_stride + wbase + lane] = acc[k];
                wbase += RBQ_WAVE;
                slot = 0;
            }
        }
    }
    if (slot != 0 && lane < slot) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            pr[(size_t)k * plane_stride + wbase + lane] = acc[k];
    }
    if (status != nullptr) {
        const bool any_bad = __ballot(bad) != 0;
        if (lane == 0 && any_bad)
            atomicOr(status, (int)RBQ_STATUS_NONFINITE_W);
    }
}

// ---------------------------------------------------------------------------
// dense tiles on the fp16 matrix cores

constexpr int QT_THREADS = 256;               // 4 waves, 2 x 2 over the tile
constexpr int QT_TILE = 128;                  // output tile edge
constexpr int QT_BK = 32;                     // contraction step
constexpr int QT_LDP = QT_BK + 8;             // padded LDS row pitch (halves)

// C tile of one wave: 4 x 4 MFMA tiles of 16 x 16; C[i][j] of an MFMA tile
// sits in lane j + 16 (i / 4), register i % 4 (i from the A fragment's row,
// j from the B fragment's).
__device__ __forceinline__ void mma_step(const _Float16 *As, const _Float16 *Bs, int arow0, int brow0, int li,
                                         int lg, v4f (&acc)[4][4]) {
    v8h af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const v8h *>(&As[(arow0 + i * 16 + li) * QT_LDP + 8 * lg]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const v8h *>(&Bs[(brow0 + j * 16 + li) * QT_LDP + 8 * lg]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// 16 consecutive fp16 values of row `row` (pitch `pitch` halves) from column
// `col`; zero outside [0, rows) x [0, cols).  `vec`: 16-byte loads are aligned.
__device__ __forceinline__ void load16(const uint16_t *__restrict__ base, int row, int rows, int col, int cols,
                                       size_t pitch, bool vec, uint16_t (&v)[16]) {
    if (row < rows && vec && col + 16 <= cols) {
        const uint4 *p = reinterpret_cast<const uint4 *>(base + (size_t)row * pitch + col);
        const uint4 x0 = p[0], x1 = p[1];
        const uint32_t u[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = (uint16_t)(u[i] & 0xFFFFu);
            v[2 * i + 1] = (uint16_t)(u[i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = (row < rows && col + i < cols) ? base[(size_t)row * pitch + col + i] : (uint16_t)0;
    }
}

// dW[r][j] = sum_m dY[m][r] X[m][j]: grid (ceil(in / 128), ceil(out / 128)).
__global__ __launch_bounds__(QT_THREADS) void qat_dw_kernel(const uint16_t *__restrict__ dY,
                                                            const uint16_t *__restrict__ X, int M, int out,
                                                            int in, float *__restrict__ dW) {
    __shared__ __align__(16) _Float16 As[QT_TILE * QT_LDP];   // [dW row][token]
    __shared__ __align__(16) _Float16 Bs[QT_TILE * QT_LDP];   // [X column][token]
    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = tid / RBQ_WAVE;
    const int wr = wave & 1, wc = wave >> 1;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = blockIdx.y * QT_TILE, j0 = blockIdx.x * QT_TILE;
    // staging: thread (q, mm) moves 16 values of token mm, tile columns 16 q ..
    const int mm = tid & 31, q = tid >> 5;
    const bool vec_a = (out & 7) == 0 && ((uintptr_t)dY & 15) == 0;
    const bool vec_b = ((uintptr_t)X & 15) == 0;      // in is a multiple of 32

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    for (int m0 = 0; m0 < M; m0 += QT_BK) {
        uint16_t a[16], b[16];
        const int m = m0 + mm < M ? m0 + mm : M;      // M: a row that reads as zero
        load16(dY, m, M, r0 + 16 * q, out, out, vec_a, a);
        load16(X, m, M, j0 + 16 * q, in, in, vec_b, b);
        __syncthreads();                               // the previous step's reads are done
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            As[(16 * q + i) * QT_LDP + mm] = __builtin_bit_cast(_Float16, a[i]);
            Bs[(16 * q + i) * QT_LDP + mm] = __builtin_bit_cast(_Float16, b[i]);
        }
        __syncthreads();
        mma_step(As, Bs, 64 * wr, 64 * wc, li, lg, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = j0 + 64 * wc + 16 * j + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = r0 + 64 * wr + 16 * i + 4 * lg + v;
                if (r < out && c < in)
                    dW[(size_t)r * in + c] = acc[i][j][v];
            }
        }
}

// dX[m][j] = sum_r dY[m][r] What[r][j]: grid (ceil(in / 128), ceil(M / 128)).
template <int K>
__global__ __launch_bounds__(QT_THREADS) void qat_dx_kernel(const uint16_t *__restrict__ dY,
                                                            const uint32_t *__restrict__ planes,
                                                            const uint16_t *__restrict__ scales, int M, int out,
                                                            int in, int group_size, int r_slice,
                                                            float *__restrict__ dX, int32_t *__restrict__ status) {
    __shared__ __align__(16) _Float16 As[QT_TILE * QT_LDP];   // [token][r]
    __shared__ __align__(16) _Float16 Bh[QT_TILE * QT_LDP];   // [column][r], hi part
    __shared__ __align__(16) _Float16 Bl[QT_TILE * QT_LDP];   // lo part
    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = tid / RBQ_WAVE;
    const int wm = wave & 1, wc = wave >> 1;
    const int li = lane & 15, lg = lane >> 4;
    const int m_base = blockIdx.y * QT_TILE, j0 = blockIdx.x * QT_TILE;
    const int words = in >> 5;
    const int G = group_size ? in / group_size : 1;
    const size_t plane_stride = (size_t)out * words;
    const bool vec_a = (out & 7) == 0 && ((uintptr_t)dY & 15) == 0;
    // staging of dY: thread (am, ah) moves 16 values of token am
    const int am = tid >> 1, ah = tid & 1;
    // forming What: thread (q, rr) forms 16 columns 16 q .. of row rr
    const int rr = tid & 31, q = tid >> 5;
    const int wq = (j0 >> 5) + (q >> 1);          // its sign word
    const int sh = 16 * (q & 1);
    const bool col_ok = wq < words;
    const int g = group_size ? (j0 + 16 * q) / group_size : 0;
    bool ovf = false;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    // slice blockIdx.z of the contraction: rows [r_lo, r_hi) of What, its
    // partial dX at dX + z M in (one slice: dX itself)
    const int r_lo = blockIdx.z * r_slice;
    const int r_hi = min(out, r_lo + r_slice);
    dX += (size_t)blockIdx.z * M * in;
    for (int r0 = r_lo; r0 < r_hi; r0 += QT_BK) {
        uint16_t a[16];
        load16(dY, m_base + am, M, r0 + 16 * ah, r_hi, out, vec_a, a);
        const int r = r0 + rr;
        uint32_t bits[K];
        float sc[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool ok = col_ok && r < r_hi;
            bits[k] = ok ? planes[(size_t)k * plane_stride + (size_t)r * words + wq] >> sh : 0u;
            sc[k] = ok ? h2f(scales[((size_t)k * out + r) * G + g]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            As[am * QT_LDP + 16 * ah + i] = __builtin_bit_cast(_Float16, a[i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float w = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k)
                w += ((bits[k] >> i) & 1u) ? sc[k] : -sc[k];
            ovf = ovf || !(__builtin_fabsf(w) < 65520.0f);
            const _Float16 hi = (_Float16)w;
            const _Float16 lo = (_Float16)(w - (float)hi);
            Bh[(16 * q + i) * QT_LDP + rr] = hi;
            Bl[(16 * q + i) * QT_LDP + rr] = lo;
        }
        __syncthreads();
        mma_step(As, Bl, 64 * wm, 64 * wc, li, lg, acc);
        mma_step(As, Bh, 64 * wm, 64 * wc, li, lg, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = j0 + 64 * wc + 16 * j + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m_base + 64 * wm + 16 * i + 4 * lg + v;
                if (m < M && c < in)
                    dX[(size_t)m * in + c] = acc[i][j][v];
            }
        }
    if (status != nullptr) {
        const bool any = __ballot(ovf) != 0;
        if (lane == 0 && any)
            atomicOr(status, (int)RBQ_STATUS_SCALE_OVERFLOW);
    }
}

// ---------------------------------------------------------------------------
// scale gradients: one wave per (row, group)

template <int K>
__global__ __launch_bounds__(QC_THREADS) void qat_dscales_kernel(const float *__restrict__ dW,
                                                                 const uint32_t *__restrict__ planes, int out,
                                                                 int in, int group_size,
                                                                 float *__restrict__ dscales) {
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / RBQ_WAVE));
    const int G = group_size ? in / group_size : 1;
    const int n = group_size ? group_size : in;
    const long seg = (long)blockIdx.x * QC_WAVES + wave;
    if (seg >= (long)out * G)
        return;                               // whole wave
    const int r = (int)(seg / G), t = (int)(seg - (long)r * G);
    const int words = in >> 5;
    const size_t plane_stride = (size_t)out * words;
    const float *wrow = dW + (size_t)r * in;
    double s[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        s[k] = 0.0;
    for (int c = t * n + lane; c < (t + 1) * n; c += RBQ_WAVE) {
        const double w = (double)wrow[c];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t word = planes[(size_t)k * plane_stride + (size_t)r * words + (c >> 5)];
            s[k] += ((word >> (c & 31)) & 1u) ? w : -w;
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const double tot = wave_sum_f64(s[k]);
        if (lane == 0)
            dscales[((size_t)k * out + r) * G + t] = (float)tot;
    }
}

// dX = the sum of the S partial slices, in slice order (deterministic).
__global__ void qat_sum_slices(const float *__restrict__ parts, int S, size_t n, float *__restrict__ dX) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    float v = parts[i];
    for (int z = 1; z < S; ++z)
        v += parts[(size_t)z * n + i];
    dX[i] = v;
}

__global__ void qat_fill_zero_f32(float *p, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0.0f;
}

hipError_t fill_zero(float *p, size_t n, hipStream_t st) {
    if (n == 0)
        return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(qat_fill_zero_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace

bool qat_supports(int K) { return K >= 1 && K <= 4; }

// Contraction slices of dX: enough workgroups for about two per compute
// unit, at most 16 slices and at least 256 rows of What per slice.
int qat_dx_slices(int M, int out, int in) {
    if (M <= 0 || in <= 0 || out <= 0)
        return 1;
    const long tiles = (long)((in + QT_TILE - 1) / QT_TILE) * ((M + QT_TILE - 1) / QT_TILE);
    long S = (512 + tiles - 1) / tiles;
    S = std::min(S, 16L);
    S = std::min(S, (long)std::max(1, out / 256));
    return (int)std::max(S, 1L);
}

size_t qat_backward_workspace_bytes(int M, int out, int in) {
    const int S = qat_dx_slices(M, out, in);
    return S > 1 ? (size_t)S * M * in * sizeof(float) : 0;
}

hipError_t launch_qat_encode(const float *W, int out, int in, int K, int group_size, const uint16_t *scales,
                             uint32_t *planes, int32_t *status, hipStream_t st) {
    if (out == 0 || in == 0)
        return hipSuccess;
    const dim3 grid((out + QC_WAVES - 1) / QC_WAVES);
    switch (K) {
    case 1: hipLaunchKernelGGL(qat_cascade_kernel<1>, grid, dim3(QC_THREADS), 0, st, W, out, in, group_size, scales, planes, status); break;
    case 2: hipLaunchKernelGGL(qat_cascade_kernel<2>, grid, dim3(QC_THREADS), 0, st, W, out, in, group_size, scales, planes, status); break;
    case 3: hipLaunchKernelGGL(qat_cascade_kernel<3>, grid, dim3(QC_THREADS), 0, st, W, out, in, group_size, scales, planes, status); break;
    default: hipLaunchKernelGGL(qat_cascade_kernel<4>, grid, dim3(QC_THREADS), 0, st, W, out, in, group_size, scales, planes, status); break;
    }
    return hipGetLastError();
}

hipError_t launch_qat_backward(const uint32_t *planes, const uint16_t *scales, int out, int in, int K,
                               int group_size, const uint16_t *X, const uint16_t *dY, int M, float *dX,
                               float *dW, float *dscales, void *workspace, size_t ws_bytes, int32_t *status,
                               hipStream_t st) {
    hipError_t e = hipSuccess;
    if (dW != nullptr) {
        if (M == 0) {
            e = fill_zero(dW, (size_t)out * in, st);
        } else if (out > 0 && in > 0) {
            const dim3 grid((in + QT_TILE - 1) / QT_TILE, (out + QT_TILE - 1) / QT_TILE);
            hipLaunchKernelGGL(qat_dw_kernel, grid, dim3(QT_THREADS), 0, st, dY, X, M, out, in, dW);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
    }
    if (dscales != nullptr && out > 0 && in > 0) {
        const int G = group_size ? in / group_size : 1;
        const dim3 grid((unsigned)(((long)out * G + QC_WAVES - 1) / QC_WAVES));
        switch (K) {
        case 1: hipLaunchKernelGGL(qat_dscales_kernel<1>, grid, dim3(QC_THREADS), 0, st, dW, planes, out, in, group_size, dscales); break;
        case 2: hipLaunchKernelGGL(qat_dscales_kernel<2>, grid, dim3(QC_THREADS), 0, st, dW, planes, out, in, group_size, dscales); break;
        case 3: hipLaunchKernelGGL(qat_dscales_kernel<3>, grid, dim3(QC_THREADS), 0, st, dW, planes, out, in, group_size, dscales); break;
        default: hipLaunchKernelGGL(qat_dscales_kernel<4>, grid, dim3(QC_THREADS), 0, st, dW, planes, out, in, group_size, dscales); break;
        }
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    if (dX != nullptr && M > 0 && in > 0) {
        if (out == 0)
            return fill_zero(dX, (size_t)M * in, st);
        // few output tiles (small M): split the contraction over slices whose
        // partial sums go to the workspace, added in order by a second kernel
        int S = qat_dx_slices(M, out, in);
        if ((size_t)S * M * in * sizeof(float) > ws_bytes || workspace == nullptr)
            S = 1;
        const int r_slice = S > 1 ? ((out + S - 1) / S + QT_BK - 1) / QT_BK * QT_BK : out;
        S = (out + r_slice - 1) / r_slice;
        float *dst = S > 1 ? static_cast<float *>(workspace) : dX;
        const dim3 grid((in + QT_TILE - 1) / QT_TILE, (M + QT_TILE - 1) / QT_TILE, S);
        switch (K) {
        case 1: hipLaunchKernelGGL(qat_dx_kernel<1>, grid, dim3(QT_THREADS), 0, st, dY, planes, scales, M, out, in, group_size, r_slice, dst, status); break;
        case 2: hipLaunchKernelGGL(qat_dx_kernel<2>, grid, dim3(QT_THREADS), 0, st, dY, planes, scales, M, out, in, group_size, r_slice, dst, status); break;
        case 3: hipLaunchKernelGGL(qat_dx_kernel<3>, grid, dim3(QT_THREADS), 0, st, dY, planes, scales, M, out, in, group_size, r_slice, dst, status); break;
        default: hipLaunchKernelGGL(qat_dx_kernel<4>, grid, dim3(QT_THREADS), 0, st, dY, planes, scales, M, out, in, group_size, r_slice, dst, status); break;
        }
        if ((e = hipGetLastError()) != hipSuccess || S == 1)
            return e;
        const size_t n = (size_t)M * in;
        hipLaunchKernelGGL(qat_sum_slices, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const float *>(workspace), S, n, dX);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace rbq
