// gemm_prefill.hip -- prefill-batch residual-binary GEMM on the fp16 matrix
// cores of gfx950: Y[m][r] = sum_j What[r][j] X[m][j] with
// What[r][j] = sum_k a_k[r][t(j)] (bit ? +1 : -1) ("RaBiT" summary,
// paperlayer.ai, section 4.1: binary cores with per-channel scales;
// "QBB" summary, atlas.scime.ai, "Key results": per-group scales).
//
// With thousands of tokens the layer is a dense contraction, so each weight
// tile is unpacked once into LDS as fp16 values of What (the per-row sum of
// the K signed scales, rounded once to fp16) and multiplied with
// v_mfma_f32_16x16x32_f16 against fp16 activation tiles (kept exact); fp32
// accumulation, one fp16 rounding of each output.  fp16 rather than bf16:
// the activations stay exact in fp16, and the single rounding of What costs
// a relative error of at most 2^-11 per weight.
//
// Tiling: a workgroup (8 waves) computes a 256-token x 128-row output tile;
// wave (wm, wn) owns 64 x 64 of it as 4 x 4 MFMA tiles of 16 x 16.  The K
// loop steps 64 columns at a time through double-buffered LDS; the next
// step's activation words and weight bits are requested before the current
// step's MFMAs are issued.  Rows of both LDS tiles are padded to 72 halves
// so that the 16-byte fragment reads of 16 lanes fall in distinct banks.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = PF_WAVES * RBQ_WAVE;
constexpr int BM = 256;            // tokens per tile
constexpr int BN = 128;            // weight rows per tile
constexpr int BK = 64;             // columns per step
constexpr int LDP = BK + 8;        // padded LDS row pitch (halves)

template <int K>
__global__ __launch_bounds__(PF_THREADS, 1) void gemm_prefill_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    int group_size, const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y) {
    __shared__ __align__(16) _Float16 As[2][BM * LDP];
    __shared__ __align__(16) _Float16 Bs[2][BN * LDP];

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int wm = wave & 3, wn = wave >> 2;          // 4 x 2 waves
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int words = in >> 5;
    const int G = group_size ? in / group_size : 1;
    const int nsteps = in / BK;

    // ---- global -> register assignments
    // activations: 256 rows x 64 columns = 2048 x 16 bytes; thread: 4 pieces
    // (row = piece / 8, 8 halves at column 8 * (piece % 8))
    int a_row[4], a_col[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int piece = tid + p * PF_THREADS;
        a_row[p] = piece >> 3;
        a_col[p] = (piece & 7) * 8;
    }
    const uint16_t *a_src[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        a_src[p] = X + (size_t)min(m0 + a_row[p], M - 1) * in + a_col[p];
    // weights: 128 rows x 64 columns; thread: row tid / 4, 16 columns at 16 * (tid % 4)
    const int b_row = tid >> 2, b_q = tid & 3;
    const int b_r = min(n0 + b_row, out - 1);
    const uint32_t *b_src = planes + (size_t)b_r * words + (b_q >> 1);
    const int b_shift = 16 * (b_q & 1);
    const size_t plane_stride = (size_t)out * words;

    uint4 a_reg[4];
    uint32_t b_reg[K];
    uint16_t s_reg[K];
    auto fetch = [&](int step) {
        const int k0 = min(step, nsteps - 1) * BK;
        const int t = group_size ? (k0 + 16 * b_q) / group_size : 0;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a_reg[p] = *reinterpret_cast<const uint4 *>(a_src[p] + k0);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            b_reg[k] = b_src[k * plane_stride + k0 / 32];
            s_reg[k] = scales[((size_t)k * out + b_r) * G + t];
        }
    };
    // What for 16 columns of one row: sum_k (+-a_k), rounded once to fp16
    auto stash = [&](int step, int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<uint4 *>(&As[buf][a_row[p] * LDP + a_col[p]]) = a_reg[p];
        (void)step;
        float sc[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            sc[k] = h2f(s_reg[k]);
        v8h v0, v1;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float w = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k)
                w += ((b_reg[k] >> (b_shift + j)) & 1u) ? sc[k] : -sc[k];
            if (j < 8)
                v0[j] = (_Float16)w;
            else
                v1[j - 8] = (_Float16)w;
        }
        v8h *dst = reinterpret_cast<v8h *>(&Bs[buf][b_row * LDP + 16 * b_q]);
        dst[0] = v0;
        dst[1] = v1;
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    fetch(0);
    stash(0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        fetch(step + 1);           // in flight during the MFMAs (a clamped repeat at the end)
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            v8h af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const v8h *>(
                    &As[buf][(wm * 64 + i * 16 + li) * LDP + ks * 32 + 8 * lg]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const v8h *>(
                    &Bs[buf][(wn * 64 + j * 16 + li) * LDP + ks * 32 + 8 * lg]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (step + 1 < nsteps)
            stash(step + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- C[i][j] of an MFMA tile sits in lane j + 16*(i/4), register i%4:
    // i = token (A row), j = weight row (B column)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = n0 + wn * 64 + j * 16 + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 64 + i * 16 + 4 * lg + v;
                if (m < M && r < out)
                    Y[(size_t)m * out + r] = f2h(acc[i][j][v]);
            }
        }
}

template <int K>
hipError_t launch_k(const uint32_t *planes, const uint16_t *scales, int out, int in,
                    int group_size, const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    dim3 grid((out + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL(gemm_prefill_kernel<K>, grid, dim3(PF_THREADS), 0, st, planes, scales,
                       out, in, group_size, X, M, Y);
    return hipGetLastError();
}

}  // namespace

bool prefill_supports(int in, int K, int group_size, int M) {
    return K >= 1 && K <= 4 && in % BK == 0 && in > 0 && M >= 1 && (M + BM - 1) / BM <= 65535 &&
           (group_size == 0 || group_size % BK == 0);
}

hipError_t launch_gemm_prefill(const uint32_t *planes, const uint16_t *scales, int out, int in,
                               int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                               hipStream_t st) {
    if (!prefill_supports(in, K, group_size, M))
        return hipErrorInvalidValue;
    switch (K) {
    case 1: return launch_k<1>(planes, scales, out, in, group_size, X, M, Y, st);
    case 2: return launch_k<2>(planes, scales, out, in, group_size, X, M, Y, st);
    case 3: return launch_k<3>(planes, scales, out, in, group_size, X, M, Y, st);
    case 4: return launch_k<4>(planes, scales, out, in, group_size, X, M, Y, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rbq
