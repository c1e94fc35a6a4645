// gemm_split.hip -- residual-binary GEMM for a few tokens (2 .. 16), the
// input columns split over workgroups.
//
// y[m][r] = sum_k a_k[r] * (2 S_k - sum x), S_k = sum of x over the set bits
// of row r of plane k ("RaBiT" summary, paperlayer.ai, sections 4.1 and 4.2:
// binary cores with per-channel scales, the K paths side by side).
//
// Why split the columns.  With several tokens every workgroup that covers a
// whole row has to quantise every token over the whole row, and that
// per-workgroup VALU work (about 6 operations per column and token) grows
// with the token count until it dominates: 16 tokens of 11008 columns take
// ~7 us of one compute unit.  Here workgroup (r, c) covers the 16-row tiles
// of row group r but only the 512-column chunks of slice c, so it quantises
// only its slice, with its own power-of-two scale per token (each partial sum
// is converted back to float before slices are added).  The slices' fp32
// partial outputs go to a workspace and a second kernel adds them in slice
// order and rounds once to fp16.
//
// Inside a workgroup (16 waves, one per compute unit), in three phases
// separated by barriers that wait for LDS traffic only:
//   * every wave requests its share of the slice of x (16-column pieces of
//     single tokens), then the weights of its first two (tile, chunk) units;
//   * all waves quantise x into an LDS image laid out like the B operand of
//     v_mfma_i32_16x16x64_i8 (token groups of 4 tokens x 3 limbs = 12
//     columns), per-token maxima and sums of q meeting in LDS atomics (the
//     sums as 64-bit integers, so exact and order-free);
//   * all waves stream their units.  The A operand is the weight word shifted
//     right by the bit position s and masked with 0x01010101 (bytes 0 or 1),
//     so every bit position adds into one accumulator per plane and token
//     group, and the masks are shared by the token groups.  Partial sums of a
//     tile meet in LDS as int32 additions (exact), and one thread per (row,
//     token) converts them with the row's scales.
// An earlier version left the quantisation to 4 waves (one per SIMD), one
// token group at a time: 16 tokens took ~8 us there, latency rather than
// arithmetic.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int SP_WAVES = 16;
constexpr int SP_THREADS = SP_WAVES * RBQ_WAVE;
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;                        // 512 columns
constexpr int NLIMB = 3;
constexpr int TOK = 4;                                 // tokens per group
constexpr int NC = NLIMB * TOK;                        // MFMA columns per group
constexpr int ENTRY_ROW = NC * 16;                     // one lane group, one bit position
constexpr int IMG_CHUNK = 8 * 4 * ENTRY_ROW + 64;      // one chunk of one group (padded)
constexpr int SP_MAX_CPS = 8;                          // chunks per slice
#ifndef SP_TARGET_CPS
#define SP_TARGET_CPS 2
#endif
constexpr int SP_MAX_M = 16;
constexpr int SP_MAX_TILES = SP_THREADS / TILE_ROWS;

size_t split_lds_bytes(int cps, int ng, int K, int tpw) {
    return (size_t)cps * ng * IMG_CHUNK + 16 + (size_t)tpw * ng * K * NC * TILE_ROWS * 4;
}

// Workgroup barrier that waits for this wave's LDS operations only: global
// loads already requested stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Grid: x = row group (tiles [x T / NR, (x+1) T / NR)), y = column slice
// (chunks [y C / S, (y+1) C / S)).  P = fp32 partial outputs [S][M][out].
// IPT = (half-word, token) items per thread in the quantisation phase.
template <int K, int NG, int IPT>
__global__ __launch_bounds__(SP_THREADS, 1) void gemm_split_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    const uint16_t *__restrict__ X, int M, float *__restrict__ P) {
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ uint32_t tmax[NG * TOK];
    __shared__ unsigned long long tsum[NG * TOK];   // sum of q per token, exact

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int li = lane & 15, lg = lane >> 4;
    const int words = in >> 5;
    const int nchunks = (words + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int S = gridDim.y;
    const int c0 = (int)(((long)blockIdx.y * nchunks) / S);
    const int c1 = (int)(((long)(blockIdx.y + 1) * nchunks) / S);
    const int cps = c1 - c0;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int NR = gridDim.x;
    const int t0 = (int)(((long)blockIdx.x * T) / NR);
    const int t1 = (int)(((long)(blockIdx.x + 1) * T) / NR);
    const int ntl = t1 - t0;
    const int img_group = cps * IMG_CHUNK;            // one token group's image
    const int pad = NG * img_group;                   // 16 zero bytes for unused MFMA columns
    int *red = reinterpret_cast<int *>(lds + pad + 16);   // [ntl][NG][K][NC][16]

    // ---- activations first (their wait must not include the weights):
    // item i = token i / nhs, half-word i % nhs of the slice (16 columns);
    // half-words past the row end load its last one and get the scale 0
    const int nhs = cps * CHUNK_WORDS * 2;                                   // half-words of the slice
    const int nh = min(cps * CHUNK_WORDS, words - c0 * CHUNK_WORDS) * 2;    // those inside the row
    const int nitems = M * nhs;
    v4u xw[IPT][2];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = min(tid + j * SP_THREADS, nitems - 1);
        const int m = it / nhs, h = it - m * nhs;
        const v4u *xp = reinterpret_cast<const v4u *>(X + (size_t)m * in + 16 * (c0 * CHUNK_WORDS * 2 + min(h, nh - 1)));
        xw[j][0] = xp[0];
        xw[j][1] = xp[1];
    }

    // ---- then each wave's first two (tile, chunk) units; units are split
    // evenly, in order, over all 16 waves
    const int U = ntl * cps;
    const int u0 = (wave * U) / SP_WAVES;
    const int u1 = ((wave + 1) * U) / SP_WAVES;
    const int n = u1 - u0;
    const int ulast = max(min(u0, U - 1), u1 - 1);
    const size_t plane_stride = (size_t)out * words;
    // u -> (tile u / cps, chunk u % cps): exact for u < 2^11 and cps <= 32
    const uint32_t magic = ((1u << 21) + cps - 1) / cps;
    // lane (li, lg): words 4lg .. 4lg+3 of the chunk in row li of the tile
    // (rows past the end read the last row, words past the row end its last
    // four words, which meet zeros in the image)
    int lnext = u0;
    v4u ring[2][K];
    auto load_unit = [&](v4u (&slot)[K]) {
        const int u = min(lnext, ulast);
        const int tq = (int)(((uint32_t)u * magic) >> 21);
        const int row = min((t0 + tq) * TILE_ROWS + li, out - 1);
        const int wi = min((c0 + u - tq * cps) * CHUNK_WORDS + 4 * lg, words - 4);
        const uint32_t *p = planes + (size_t)row * words + wi;
#pragma unroll
        for (int k = 0; k < K; ++k)
            slot[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + k * plane_stride));
        ++lnext;
    };
    load_unit(ring[0]);
    load_unit(ring[1]);

    if (tid < NG * TOK) {
        tmax[tid] = 0u;
        tsum[tid] = 0ull;
    }
    for (int i = tid; i < ntl * NG * K * NC * TILE_ROWS; i += SP_THREADS)
        red[i] = 0;
    if (tid < 4)
        reinterpret_cast<uint32_t *>(lds + pad)[tid] = 0u;
    lds_barrier();

    // ---- quantisation by all waves: per-token maximum of |x| over the slice
    // (fp16 bit patterns without the sign compare like magnitudes)
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = tid + j * SP_THREADS;
        if (it < nitems) {
            v2u16 mx2 = (v2u16){0, 0};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, xw[j][hh][c] & 0x7FFF7FFFu));
            __hip_atomic_fetch_max(&tmax[it / nhs], max((uint32_t)mx2.x, (uint32_t)mx2.y), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    lds_barrier();
    // q = round(x * 2^sh), |x| < 2^E, sh = 22 - E, |q| <= 2^22; v = q + 0x808080
    // from fma(x, 2^sh, 1.5*2^23); its bytes xor 0x80 are the limbs.  Image
    // entry (word w, bit s) of token group g: columns 32w + 8kk + s, one byte
    // each, at [g][chunk w/16][s][lane group (w/4)%4][column 3 (m%4) + l][4 (w%4) + kk]
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = tid + j * SP_THREADS;
        if (it < nitems) {
            const int m = it / nhs, h = it - m * nhs;
            const int e = (int)(tmax[m] >> 10);
            const int sh = 22 - ((e == 0 ? 1 : e) - 14);
            const float scale = h < nh ? __builtin_ldexpf(1.0f, sh) : 0.0f;
            const int w = h >> 1, eh = h & 1;   // word of the slice
            unsigned char *dst = lds + (m / TOK) * img_group + (w / CHUNK_WORDS) * IMG_CHUNK +
                                 ((w >> 2) & 3) * ENTRY_ROW + (w & 3) * 4 + 2 * eh + (NLIMB * (m % TOK)) * 16;
            int psum = 0;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t uu0 = xw[j][0][s >> 1], uu1 = xw[j][1][s >> 1];
                const uint16_t h0 = (s & 1) ? (uint16_t)(uu0 >> 16) : (uint16_t)uu0;
                const uint16_t h1 = (s & 1) ? (uint16_t)(uu1 >> 16) : (uint16_t)uu1;
                const uint32_t v0 =
                    __builtin_bit_cast(uint32_t, __builtin_fmaf(h2f(h0), scale, 12582912.0f)) - 0x4ABF7F80u;
                const uint32_t v1 =
                    __builtin_bit_cast(uint32_t, __builtin_fmaf(h2f(h1), scale, 12582912.0f)) - 0x4ABF7F80u;
                psum += (int)(v0 + v1) - 2 * 0x808080;
                const uint32_t l01 = __builtin_amdgcn_perm(v1, v0, 0x05010400u) ^ 0x80808080u;
                const uint32_t l2 = __builtin_amdgcn_perm(v1, v0, 0x0C0C0602u) ^ 0x8080u;
                unsigned char *d = dst + s * (4 * ENTRY_ROW);
                *reinterpret_cast<uint16_t *>(d) = (uint16_t)l01;
                *reinterpret_cast<uint16_t *>(d + 16) = (uint16_t)(l01 >> 16);
                *reinterpret_cast<uint16_t *>(d + 32) = (uint16_t)l2;
            }
            __hip_atomic_fetch_add(&tsum[m], (unsigned long long)(long long)psum, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    lds_barrier();

    // ---- streaming by all waves.  A operand: the word shifted right by the
    // bit position s, masked with 0x01010101 (bytes 0 or 1), shared by the
    // token groups; one accumulator per plane and token group.
    v4i acc[NG][K];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k)
            acc[g][k] = (v4i){0, 0, 0, 0};
    const bool bl = li < NC;
    const int b_off = bl ? (lg * NC + li) * 16 : pad;
    const int b_stride = bl ? 4 * ENTRY_ROW : 0;
    const int b_chunk = bl ? IMG_CHUNK : 0;
    const int b_group = bl ? img_group : 0;
    int ptile = t0 + (int)(((uint32_t)u0 * magic) >> 21);
    int pchunk = u0 - (ptile - t0) * cps;
    auto chunk = [&](const v4u (&wv)[K]) {
        const unsigned char *bp = lds + b_off + pchunk * b_chunk;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            v4i av[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                av[k] = (v4i){(int)((wv[k].x >> s) & 0x01010101u), (int)((wv[k].y >> s) & 0x01010101u),
                              (int)((wv[k].z >> s) & 0x01010101u), (int)((wv[k].w >> s) & 0x01010101u)};
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const v4i b = *reinterpret_cast<const v4i *>(bp + g * b_group + s * b_stride);
#pragma unroll
                for (int k = 0; k < K; ++k)
                    acc[g][k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[k], b, acc[g][k], 0, 0, 0);
            }
        }
    };
    // at a tile's end or at the wave's last unit, add the sums into LDS
    // (lane (li, lg) holds rows 4lg + v of MFMA column li)
    auto step = [&](int i) {
        const bool tile_end = ++pchunk == cps;
        if (tile_end || i == n - 1) {
            if (li < NC) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        int *rp = red + ((((ptile - t0) * NG + g) * K + k) * NC + li) * TILE_ROWS + 4 * lg;
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            __hip_atomic_fetch_add(rp + v, acc[g][k][v], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
            }
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int k = 0; k < K; ++k)
                    acc[g][k] = (v4i){0, 0, 0, 0};
        }
        if (tile_end) {
            pchunk = 0;
            ++ptile;
        }
    };
    const int nbk = (n + 1) / 2;
    for (int bi = 0; bi + 1 < nbk; ++bi) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            chunk(ring[d]);
            load_unit(ring[d]);
            step(bi * 2 + d);
        }
    }
    if (nbk > 0) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const int i = (nbk - 1) * 2 + d;
            if (i < n) {
                chunk(ring[d]);
                step(i);
            }
        }
    }
    __syncthreads();

    // ---- one thread per (row, token): column 3m + l of a group holds
    // sum(bit l_j); sum(bit q) = T_0 + 2^8 T_1 + 2^16 T_2 (exact in fp64) and
    // the slice's partial y = sum_k a_k (2 sum(bit q) - sum q) 2^-sh
    const int rows = min(ntl * TILE_ROWS, out - t0 * TILE_ROWS);
    for (int idx = tid; idx < rows * M; idx += SP_THREADS) {
        const int m = idx / rows, rr = idx - m * rows;
        const int tl = rr / TILE_ROWS, i = rr % TILE_ROWS;
        const int g = m / TOK, mm = m % TOK;
        const int row = t0 * TILE_ROWS + rr;
        const int e = (int)(tmax[m] >> 10);
        const int sh = 22 - ((e == 0 ? 1 : e) - 14);
        const double sx = (double)(long long)tsum[m];
        float y = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int *rp = red + (((tl * NG + g) * K + k) * NC + NLIMB * mm) * TILE_ROWS + i;
            const double t = (double)rp[0] + 256.0 * (double)rp[TILE_ROWS] + 65536.0 * (double)rp[2 * TILE_ROWS];
            y += h2f(scales[(size_t)k * out + row]) * (float)(2.0 * t - sx);
        }
        P[((size_t)blockIdx.y * M + m) * out + row] = __builtin_ldexpf(y, -sh);
    }
}

// Y[m][r] = fp16(sum over slices of P[s][m][r]), slices in order.
__global__ __launch_bounds__(256) void split_combine_kernel(const float *__restrict__ P, int S,
                                                            int n, uint16_t *__restrict__ Y) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        float y = 0.0f;
        for (int s = 0; s < S; ++s)
            y += P[(size_t)s * n + i];
        Y[i] = f2h(y);
    }
}

int split_num_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    return cus;
}

size_t split_lds_limit() {
    static size_t lim = 0;
    if (lim == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        lim = (size_t)v - 1024;   // the kernel's static LDS comes on top
    }
    return lim;
}

struct SplitPlan {
    int S = 0, NR = 0, tpw = 0, cps = 0, ng = 0;
    size_t lds = 0;
};

// About one workgroup per compute unit; slices of SP_TARGET_CPS chunks when
// the image and the partial sums of the then taller row groups fit in LDS
// (narrow slices keep the per-workgroup quantisation short), wider ones
// otherwise.
SplitPlan split_plan(int out, int in, int K, int M) {
    SplitPlan p;
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int ng = (M + TOK - 1) / TOK;
    const int s_hi = (nchunks + SP_TARGET_CPS - 1) / SP_TARGET_CPS;
    const int s_lo = (nchunks + SP_MAX_CPS - 1) / SP_MAX_CPS;
    for (int S = s_hi; S >= s_lo; --S) {
        const int cps = (nchunks + S - 1) / S;
        int NR = split_num_cus() / S;
        NR = NR < 1 ? 1 : (NR > T ? T : NR);
        const int tpw = (T + NR - 1) / NR;
        const size_t lds = split_lds_bytes(cps, ng, K, tpw);
        if (tpw <= SP_MAX_TILES && lds <= split_lds_limit()) {
            p.S = S;
            p.NR = NR;
            p.tpw = tpw;
            p.cps = cps;
            p.ng = ng;
            p.lds = lds;
            return p;
        }
    }
    return p;
}

template <int K, int NG>
hipError_t launch_kg(const uint32_t *planes, const uint16_t *scales, int out, int in, const uint16_t *X,
                     int M, uint16_t *Y, float *P, const SplitPlan &pl, hipStream_t st) {
    const int ipt = (M * pl.cps * CHUNK_WORDS * 2 + SP_THREADS - 1) / SP_THREADS;
    if (ipt <= 1)
        hipLaunchKernelGGL((gemm_split_kernel<K, NG, 1>), dim3(pl.NR, pl.S), dim3(SP_THREADS), pl.lds, st,
                           planes, scales, out, in, X, M, P);
    else if (ipt <= 2)
        hipLaunchKernelGGL((gemm_split_kernel<K, NG, 2>), dim3(pl.NR, pl.S), dim3(SP_THREADS), pl.lds, st,
                           planes, scales, out, in, X, M, P);
    else if (ipt <= 4)
        hipLaunchKernelGGL((gemm_split_kernel<K, NG, 4>), dim3(pl.NR, pl.S), dim3(SP_THREADS), pl.lds, st,
                           planes, scales, out, in, X, M, P);
    else
        hipLaunchKernelGGL((gemm_split_kernel<K, NG, 8>), dim3(pl.NR, pl.S), dim3(SP_THREADS), pl.lds, st,
                           planes, scales, out, in, X, M, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int n = M * out;
    hipLaunchKernelGGL(split_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, st, P, pl.S, n, Y);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const uint32_t *planes, const uint16_t *scales, int out, int in, const uint16_t *X,
                    int M, uint16_t *Y, float *P, const SplitPlan &pl, hipStream_t st) {
    switch (pl.ng) {
    case 1: return launch_kg<K, 1>(planes, scales, out, in, X, M, Y, P, pl, st);
    case 2: return launch_kg<K, 2>(planes, scales, out, in, X, M, Y, P, pl, st);
    case 3: return launch_kg<K, 3>(planes, scales, out, in, X, M, Y, P, pl, st);
    default: return launch_kg<K, 4>(planes, scales, out, in, X, M, Y, P, pl, st);
    }
}

}  // namespace

bool split_supports(int out, int in, int K, int group_size, int M) {
    return group_size == 0 && K >= 1 && K <= 2 && in % 128 == 0 && in > 0 && M >= 2 &&
           M <= SP_MAX_M && out >= 1 && split_plan(out, in, K, M).S > 0;
}

// Measured on MI355X (K = 2, Llama-2-7B shapes): ahead of the flat and
// decode kernels from 8 tokens on for tall (at least two 16-row tiles per
// compute unit) or wide (more than 8192 columns) layers -- 16 tokens:
// 11008 x 4096 20.9 us (flat 26.4), 4096 x 11008 23.5 us (flat 39.5) --
// and behind them with 4 tokens or on 4096 x 4096.
bool split_preferred(int out, int in, int K, int group_size, int M) {
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    return M >= 8 && (T >= 2 * split_num_cus() || in > 8192) && split_supports(out, in, K, group_size, M);
}

size_t split_workspace_bytes(int out, int in, int K, int group_size, int M) {
    if (!split_supports(out, in, K, group_size, M))
        return 0;
    return (size_t)split_plan(out, in, K, M).S * M * out * sizeof(float);
}

hipError_t launch_gemm_split(const uint32_t *planes, const uint16_t *scales, int out, int in, int K,
                             int group_size, const uint16_t *X, int M, uint16_t *Y, void *workspace,
                             size_t ws_bytes, hipStream_t st) {
    if (!split_supports(out, in, K, group_size, M) ||
        ws_bytes < split_workspace_bytes(out, in, K, group_size, M) || workspace == nullptr ||
        ((uintptr_t)workspace & 3u) != 0)
        return hipErrorInvalidValue;
    const SplitPlan pl = split_plan(out, in, K, M);
    float *P = static_cast<float *>(workspace);
    return K == 1 ? launch_k<1>(planes, scales, out, in, X, M, Y, P, pl, st)
                  : launch_k<2>(planes, scales, out, in, X, M, Y, P, pl, st);
}

}  // namespace rbq
