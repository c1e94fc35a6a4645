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

// ---------------------------------------------------------------------------
// One and two planes: the weights never pass through LDS.
//
// What takes only 2^K values per row (per row and group with group scales):
// with v = b_1 + 2 b_2 the value is sum_k (b_k ? a_k : -a_k), one fp32 sum
// rounded once to fp16, the same value the kernel above writes to LDS.  Each
// lane keeps the four values of its weight row as a byte table (low bytes in
// one register, high bytes in another), and a B fragment of 8 fp16 weights
// comes out of four v_perm_b32 lookups whose selectors are built from the
// sign bits with a few shifts, masks and byte permutes (about 4 VALU
// operations per 2 weights).  Only the activations are staged through LDS,
// which halves the LDS traffic per MFMA compared with unpacking into LDS.
//
// Tiling: a workgroup (4 waves) computes 128 tokens x 256 weight rows; wave w
// owns rows [64 w, 64 w + 64) of it for all 128 tokens, as 4 x 2 tiles of
// v_mfma_f32_32x32x16_f16 (A = activations, B = weights).  The K loop steps
// 64 columns per stage.  Within a stage, lane half h of sub-step ks holds
// columns 32 h + 8 ks + e (e = 0..7) on both operands, so a lane needs byte
// ks of word h of its row's 64-column span -- one 32-bit load per plane and
// stage -- and 16 contiguous bytes of an activation row per sub-step.
// Workgroups are numbered so that each XCD gets a contiguous run of tiles
// (row tiles fastest), so concurrent workgroups on one XCD share activation
// tiles in its L2.
constexpr int PB_THREADS = 256;
constexpr int PB_BM = 128;             // tokens per tile
constexpr int PB_BN = 256;             // weight rows per tile (64 per wave)
constexpr int PB_BK = 64;              // columns per stage
constexpr int PB_PITCH = PB_BK + 8;    // halves per LDS token row (144 B: conflict-free 16 B reads)

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int K, bool GROUPED>
__global__ __launch_bounds__(PB_THREADS, 2) void gemm_prefill_bits_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    int group_size, const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y, int tiles_n,
    int total) {
    __shared__ __align__(16) _Float16 As[2][PB_BM * PB_PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int l32 = lane & 31, h = lane >> 5;

    // Workgroups go to the XCDs round-robin: give XCD x the tiles
    // [x per, (x + 1) per) (the remainder keeps its own numbering).
    int id = blockIdx.x;
    const int per = total >> 3;
    if (id < per * 8)
        id = (id & 7) * per + (id >> 3);
    const int tm = id / tiles_n, tn = id - tm * tiles_n;
    const int m0 = tm * PB_BM, n0 = tn * PB_BN;
    const int words = in >> 5;
    const int nst = in / PB_BK;
    const int G = GROUPED ? in / group_size : 1;
    const int spg = GROUPED ? group_size / PB_BK : 1;

    // activations: 128 tokens x 64 columns = 1024 pieces of 16 B, 4 per thread
    uint32_t a_goff[4];
    int a_loff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int piece = tid + p * PB_THREADS;
        const int tok = piece >> 3, col = (piece & 7) * 8;
        a_goff[p] = (uint32_t)(min(m0 + tok, M - 1) * in + col);
        a_loff[p] = tok * PB_PITCH + col;
    }
    // this lane's weight rows (clamped; rows past out are computed, not stored)
    int rowc[2];
    uint32_t b_goff[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        rowc[b] = min(n0 + 64 * wave + 32 * b + l32, out - 1);
        b_goff[b] = (uint32_t)(rowc[b] * words + h);
    }
    const uint32_t pstride = (uint32_t)out * (uint32_t)words;

    uint32_t plo[2], phi[2];
    uint16_t sreg[2][K];
    auto load_scales = [&](int t) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int k = 0; k < K; ++k)
                sreg[b][k] = scales[((size_t)k * out + rowc[b]) * G + t];
    };
    // byte tables of V[v] = sum_k (bit k of v ? a_k : -a_k), v = 0..3
    auto make_tables = [&]() {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float a[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                a[k] = h2f(sreg[b][k]);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float w = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k)
                    w += ((v >> k) & 1) ? a[k] : -a[k];
                const uint32_t hv = f2h(w);
                lo |= (hv & 0xFFu) << (8 * v);
                hi |= (hv >> 8) << (8 * v);
            }
            plo[b] = lo;
            phi[b] = hi;
        }
    };

    v4u a_reg[4];
    uint32_t bw[2][K];
    auto fetch = [&](int st) {
        const uint32_t k0 = (uint32_t)st * PB_BK;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a_reg[p] = *reinterpret_cast<const v4u *>(X + a_goff[p] + k0);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int k = 0; k < K; ++k)
                bw[b][k] = planes[b_goff[b] + k * pstride + 2u * (uint32_t)st];
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<v4u *>(&As[buf][a_loff[p]]) = a_reg[p];
    };

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][b][r] = 0.0f;

    load_scales(0);
    make_tables();
    fetch(0);
    stash(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        uint32_t cw[2][K];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int k = 0; k < K; ++k)
                cw[b][k] = bw[b][k];
        if (GROUPED && st > 0 && st % spg == 0)
            make_tables();
        if (st + 1 < nst) {
            fetch(st + 1);
            if (GROUPED && (st + 1) % spg == 0)
                load_scales((st + 1) / spg);
        }
        // B fragments of the four sub-steps: dword p of sub-step ks holds
        // the weights of columns 32 h + 8 ks + 2p and + 2p + 1.
        v4u bf[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t w1 = cw[b][0], w2 = K > 1 ? cw[b][K > 1 ? 1 : 0] : 0u;
            // 2-bit table index v of every even column (Z) and odd column (Zo)
            const uint32_t z = (w1 & 0x55555555u) | ((w2 & 0x55555555u) << 1);
            const uint32_t zo = ((w1 >> 1) & 0x55555555u) | (w2 & 0xAAAAAAAAu);
            const uint32_t y01 = __builtin_amdgcn_perm(zo, z, 0x05040100u);   // [z.b0 z.b1 zo.b0 zo.b1]
            const uint32_t y23 = __builtin_amdgcn_perm(zo, z, 0x07060302u);   // [z.b2 z.b3 zo.b2 zo.b3]
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t ym = ((half ? y23 : y01) >> (2 * p)) & 0x03030303u;
                    const uint32_t ym4 = ym | 0x04040404u;
                    // selectors [v, v + 4, v', v' + 4] of the two sub-steps
                    const uint32_t s0 = __builtin_amdgcn_perm(ym4, ym, 0x06020400u);
                    const uint32_t s1 = __builtin_amdgcn_perm(ym4, ym, 0x07030501u);
                    bf[b][2 * half][p] = __builtin_amdgcn_perm(phi[b], plo[b], s0);
                    bf[b][2 * half + 1][p] = __builtin_amdgcn_perm(phi[b], plo[b], s1);
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            v8h af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const v8h *>(
                    &As[buf][(i * 32 + l32) * PB_PITCH + 32 * h + 8 * ks]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        af[i], __builtin_bit_cast(v8h, bf[b][ks]), acc[i][b], 0, 0, 0);
        }
        if (st + 1 < nst)
            stash(buf ^ 1);
        __syncthreads();
    }

    // C register r of a 32 x 32 tile: token 8 (r / 4) + 4 h + r % 4, weight row l32
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int row = n0 + 64 * wave + 32 * b + l32;
        if (row < out) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (m < M)
                        Y[(size_t)m * out + row] = f2h(acc[i][b][r]);
                }
        }
    }
}

template <int K, bool GROUPED>
hipError_t launch_bits(const uint32_t *planes, const uint16_t *scales, int out, int in,
                       int group_size, const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    const int tiles_n = (out + PB_BN - 1) / PB_BN;
    const int tiles_m = (M + PB_BM - 1) / PB_BM;
    const long long total = (long long)tiles_n * tiles_m;
    if (total > 0x7FFFFFFFLL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_prefill_bits_kernel<K, GROUPED>), dim3((unsigned)total), dim3(PB_THREADS), 0,
                       st, planes, scales, out, in, group_size, X, M, Y, tiles_n, (int)total);
    return hipGetLastError();
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
    // 32-bit element offsets in the bit-unpacking kernel
    const bool small = (size_t)M * in < (1ull << 31) && (size_t)out * (in / 32) * K < (1ull << 31);
    if (K <= 2 && small) {
        if (group_size == 0)
            return K == 1 ? launch_bits<1, false>(planes, scales, out, in, 0, X, M, Y, st)
                          : launch_bits<2, false>(planes, scales, out, in, 0, X, M, Y, st);
        return K == 1 ? launch_bits<1, true>(planes, scales, out, in, group_size, X, M, Y, st)
                      : launch_bits<2, true>(planes, scales, out, in, group_size, X, M, Y, st);
    }
    switch (K) {
    case 1: return launch_k<1>(planes, scales, out, in, group_size, X, M, Y, st);
    case 2: return launch_k<2>(planes, scales, out, in, group_size, X, M, Y, st);
    case 3: return launch_k<3>(planes, scales, out, in, group_size, X, M, Y, st);
    case 4: return launch_k<4>(planes, scales, out, in, group_size, X, M, Y, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rbq
