// gemm_split.hip -- residual-binary GEMM for a few tokens (2 .. 16), the
// input columns split over workgroups, on the fp16 matrix cores.
//
// Y = X What^T with What[r][j] = sum_k a_k[r] (bit ? +1 : -1) ("RaBiT"
// summary, paperlayer.ai, section 4.1: binary cores with per-channel scales,
// the K paths side by side), rounded once to fp16, fp32 accumulation, one
// fp16 rounding of each output.
//
// Why not the int8 route of the one-token kernels.  Those quantise x into
// signed 8-bit limbs per workgroup, and with several tokens that work (about
// 6 VALU operations per column and token), the per-token maxima and the
// limb image grow with the token count until they dominate.  Here x goes to
// LDS unchanged as fp16, and What is formed in registers from the sign words
// by byte-table lookups: the four values sum_k +-a_k of a row held as a byte
// table (low bytes in one register, high bytes in another), 8 weights from
// four v_perm_b32 whose selectors come from the sign bits (about 4 VALU
// operations per 2 weights, the same for any token count).  An int8 version
// of this kernel measured 487 GB/s for 16 tokens on the Llama-2-7B shapes,
// this one 753 GB/s.
//
// Why split the columns.  16 tokens x 4096 columns of x are 128 KB, the most
// one workgroup's LDS holds next to its partial sums.  Workgroup (r, c)
// covers the 16-row tiles of row group r and the 512-column chunks of slice
// c (up to 8 chunks per slice, fewer while LDS does not fit).  With one slice
// the workgroup writes Y; with several, fp32 partial outputs go to the
// workspace and a second kernel adds them in slice order (adding them in the
// last workgroup to finish, behind device-coherent stores, measured slower).
//
// Inside a workgroup (16 waves, one per compute unit):
//   * every wave requests the scales of its first two tiles, its share of
//     the slice of x (direct global-to-LDS loads, 16 tokens padded with
//     copies of the last one), then the weights of its first two units;
//   * a barrier once its x loads have landed (the weight loads stay in
//     flight); pieces past the row end are then zeroed;
//   * each wave streams its contiguous range of (tile, chunk) units: 16
//     v_mfma_f32_16x16x32_f16 per unit (A = x, B = What).  Lane (li, lg)
//     loads words 4lg .. 4lg+3 of row li of the chunk, and MFMA t of the
//     unit takes byte t % 4 of word 4lg + t / 4 (x columns 128 lg + 8 t ..
//     + 7 of the chunk), so no data crosses lanes;
//   * the fp32 sums of a wave's run of units in one tile go to one LDS slot
//     per run, and one thread per (row, token) adds a tile's slots in unit
//     order (deterministic).
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int SP_WAVES = 16;
constexpr int SP_THREADS = SP_WAVES * RBQ_WAVE;
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;                        // 512 columns
constexpr int SP_MAX_CPS = 8;                          // chunks per slice
constexpr int SP_MAX_M = 16;
constexpr int SP_MAX_TILES = SP_THREADS / TILE_ROWS;

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

// x slot layout: [chunk][token][64 pieces of 16 B], piece q of token m at
// position q ^ m (m < 16), so the A-fragment reads of 16 lanes (16 tokens,
// one piece) hit distinct banks; one load instruction writes one token's
// 1 KB chunk row, lane i the 16 bytes at position i.
constexpr int SF_XCHUNK = 16 * 1024;                  // 16 tokens x 512 fp16

size_t splitf_lds_bytes(int cps, int tpw) {
    return (size_t)cps * SF_XCHUNK + (size_t)tpw * cps * 1024;
}

__device__ __forceinline__ uint32_t sf_lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int K>
__global__ __launch_bounds__(SP_THREADS, 1) void gemm_splitf_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    const uint16_t *__restrict__ X, int M, float *__restrict__ P, uint16_t *__restrict__ Y) {
    extern __shared__ __align__(16) unsigned char lds[];
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
    const int U = ntl * cps;
    float *slots = reinterpret_cast<float *>(lds + cps * SF_XCHUNK);   // [U][64 lanes][4]
    __shared__ uint32_t run_start[16];                                   // bit u: a wave's range starts at u
    if (tid < 16)
        run_start[tid] = 0u;

    // this wave's contiguous unit range, and the scales of this lane's row in
    // its first two tiles (a run rarely spans more; later tiles load theirs
    // when they start), requested before the x loads so that the wait for
    // those below counts only the weight loads after them
    const int u0 = (wave * U) / SP_WAVES;
    const int u1 = ((wave + 1) * U) / SP_WAVES;
    const int n = u1 - u0;
    const uint32_t magic = ((1u << 21) + cps - 1) / cps;   // u / cps for u < 2^11
    int ptile = t0 + (int)(((uint32_t)u0 * magic) >> 21);
    // (packed: plane k in bits 16k; scalars, not an array, so that they stay
    // in registers)
    auto row_scales = [&](int t) __attribute__((always_inline)) {
        const int row = min(t * TILE_ROWS + li, out - 1);
        uint32_t v = scales[row];
        if (K > 1)
            v |= (uint32_t)scales[(size_t)out + row] << 16;
        return v;
    };
    const uint32_t sc0 = row_scales(ptile), sc1 = row_scales(ptile + 1);

    // ---- x slice into LDS: load i (of 16 cps) = token i % 16, chunk i / 16;
    // pieces past the row end read its last piece and are zeroed below
    const uint32_t xl = __builtin_amdgcn_readfirstlane(sf_lds_addr(lds));
    const int npieces = in / 8;                         // 16-byte pieces of a row
    for (int i = wave; i < 16 * cps; i += SP_WAVES) {
        const int m = i & 15, c = i >> 4;
        const int q = lane ^ m;
        const int piece = min((c0 + c) * 64 + q, npieces - 1);
        const uint32_t voff = (uint32_t)((min(m, M - 1) * in + 8 * piece) * 2);
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(X),
                     "s"(xl + (uint32_t)(c * SF_XCHUNK + m * 1024))
                     : "memory");
    }

    // ---- then the weights of each wave's first two units
    const int ulast = max(min(u0, U - 1), u1 - 1);
    const size_t plane_stride = (size_t)out * words;
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
    // this wave's x loads have landed (only its 2K weight loads are younger)
    // and its LDS stores are done
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * K) : "memory");
    if (lane == 0 && n > 0)
        __hip_atomic_fetch_or(&run_start[u0 >> 5], 1u << (u0 & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if ((c0 + cps) * 64 > npieces) {
        // zero the pieces past the row end in the slice's last chunk
        const int c = cps - 1, q0 = npieces - (c0 + c) * 64;
        for (int i = tid; i < 16 * 64; i += SP_THREADS) {
            const int m = i >> 6, q = i & 63;
            if (q >= q0)
                *reinterpret_cast<v4u *>(lds + c * SF_XCHUNK + m * 1024 + 16 * (q ^ m)) = (v4u){0, 0, 0, 0};
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // ---- streaming
    const int tfirst = ptile;
    int pchunk = u0 - (ptile - t0) * cps;
    int seg = u0;                      // first unit of the current run
    uint32_t plo = 0, phi = 0;
    auto tables = [&]() __attribute__((always_inline)) {
        const uint32_t sv = ptile == tfirst ? sc0 : ptile == tfirst + 1 ? sc1 : row_scales(ptile);
        float a[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            a[k] = h2f((uint16_t)(sv >> (16 * k)));
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
        plo = lo;
        phi = hi;
    };
    if (n > 0)
        tables();
    v4f acc = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    const int a_row = li * 1024;
    auto chunk = [&](const v4u (&wv)[K]) {
        const unsigned char *xb = lds + pchunk * SF_XCHUNK + a_row;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w1 = wv[0][j], w2 = K > 1 ? wv[K > 1 ? 1 : 0][j] : 0u;
            // 2-bit table index of every even (z) and odd (zo) column
            const uint32_t z = (w1 & 0x55555555u) | ((w2 & 0x55555555u) << 1);
            const uint32_t zo = ((w1 >> 1) & 0x55555555u) | (w2 & 0xAAAAAAAAu);
            const uint32_t y01 = __builtin_amdgcn_perm(zo, z, 0x05040100u);   // bytes 0, 1
            const uint32_t y23 = __builtin_amdgcn_perm(zo, z, 0x07060302u);   // bytes 2, 3
            v4u wf[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t ym = ((half ? y23 : y01) >> (2 * p)) & 0x03030303u;
                    const uint32_t ym4 = ym | 0x04040404u;
                    wf[2 * half][p] = __builtin_amdgcn_perm(phi, plo, __builtin_amdgcn_perm(ym4, ym, 0x06020400u));
                    wf[2 * half + 1][p] = __builtin_amdgcn_perm(phi, plo, __builtin_amdgcn_perm(ym4, ym, 0x07030501u));
                }
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int t = 4 * j + b;      // columns 128 lg + 8 t .. + 7
                const v8h xa = *reinterpret_cast<const v8h *>(xb + 16 * ((16 * lg + t) ^ li));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, __builtin_bit_cast(v8h, wf[b]), acc, 0, 0, 0);
            }
        }
    };
    // at a tile's end or the wave's last unit: the run's sums to its slot
    auto step = [&](int i) {
        const bool tile_end = ++pchunk == cps;
        if (tile_end || i == n - 1) {
            *reinterpret_cast<v4f *>(slots + ((size_t)seg * 64 + lane) * 4) = acc;
            acc = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
            seg = u0 + i + 1;
        }
        if (tile_end) {
            pchunk = 0;
            ++ptile;
            if (i + 1 < n)
                tables();
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

    // ---- one thread per (row, token): the tile's runs in unit order (a run
    // starts where its tile or some wave's range starts).  C of a 16 x 16
    // MFMA tile: token i, row j in lane j + 16 (i / 4), register i % 4.
    const int rows = min(ntl * TILE_ROWS, out - t0 * TILE_ROWS);
    for (int idx = tid; idx < rows * M; idx += SP_THREADS) {
        const int m = idx / rows, rr = idx - m * rows;
        const int tl = rr >> 4, i = rr & 15;
        const int row = t0 * TILE_ROWS + rr;
        const float *sp = slots + i * 4 + 16 * 4 * (m >> 2) + (m & 3);
        float y = 0.0f;
        for (int u = tl * cps; u < (tl + 1) * cps; ++u)
            if (u == tl * cps || (run_start[u >> 5] >> (u & 31)) & 1u)
                y += sp[(size_t)u * 256];
        if (S == 1)
            Y[(size_t)m * out + row] = f2h(y);
        else
            P[((size_t)blockIdx.y * M + m) * out + row] = y;
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
    int S = 0, NR = 0, tpw = 0, cps = 0;
    size_t lds = 0;
};

// About one workgroup per compute unit; slices of SP_MAX_CPS chunks (one
// slice, no second kernel, for in <= 4096), narrower while the x slice and
// the partial-sum slots do not fit in LDS.  (Slices of 2 or 4 chunks
// measured slower: 632 and 672 GB/s against 753 for 16 tokens.)
SplitPlan split_plan(int out, int in) {
    SplitPlan p;
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    for (int want = SP_MAX_CPS; want >= 1; --want) {
        const int S = (nchunks + want - 1) / want;
        const int cps = (nchunks + S - 1) / S;
        int NR = split_num_cus() / S;
        NR = NR < 1 ? 1 : (NR > T ? T : NR);
        const int tpw = (T + NR - 1) / NR;
        const size_t lds = splitf_lds_bytes(cps, tpw);
        if (tpw <= SP_MAX_TILES && lds <= split_lds_limit()) {
            p.S = S;
            p.NR = NR;
            p.tpw = tpw;
            p.cps = cps;
            p.lds = lds;
            return p;
        }
    }
    return p;
}

template <int K>
hipError_t launch_f(const uint32_t *planes, const uint16_t *scales, int out, int in, const uint16_t *X,
                    int M, uint16_t *Y, float *P, const SplitPlan &pl, hipStream_t st) {
    hipLaunchKernelGGL((gemm_splitf_kernel<K>), dim3(pl.NR, pl.S), dim3(SP_THREADS), pl.lds, st, planes, scales,
                       out, in, X, M, P, Y);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.S == 1)
        return e;
    const int n = M * out;
    hipLaunchKernelGGL(split_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, st, P, pl.S, n, Y);
    return hipGetLastError();
}

}  // namespace

bool split_supports(int out, int in, int K, int group_size, int M) {
    return group_size == 0 && K >= 1 && K <= 2 && in % 128 == 0 && in > 0 && M >= 2 &&
           M <= SP_MAX_M && out >= 1 && split_plan(out, in).S > 0;
}

// Measured on MI355X (K = 2, Llama-2-7B shapes): ahead of the flat and
// decode kernels from 8 tokens on for layers of at least one 16-row tile
// per compute unit or more than 8192 columns -- 16 tokens: 4096 x 4096
// 10.0 us (decode 14.7), 11008 x 4096 13.0 us (flat 27.0), 4096 x 11008
// 15.6 us (flat 38.2) -- and behind the flat kernel with 4 tokens.
bool split_preferred(int out, int in, int K, int group_size, int M) {
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    return M >= 8 && (T >= split_num_cus() || in > 8192) && split_supports(out, in, K, group_size, M);
}

// fp32 partial outputs of the slices when there are several; none with one
size_t split_workspace_bytes(int out, int in, int K, int group_size, int M) {
    if (!split_supports(out, in, K, group_size, M))
        return 0;
    const SplitPlan pl = split_plan(out, in);
    return pl.S > 1 ? (size_t)pl.S * M * out * sizeof(float) : 0;
}

hipError_t launch_gemm_split(const uint32_t *planes, const uint16_t *scales, int out, int in, int K,
                             int group_size, const uint16_t *X, int M, uint16_t *Y, void *workspace,
                             size_t ws_bytes, hipStream_t st) {
    const size_t need = split_workspace_bytes(out, in, K, group_size, M);
    if (!split_supports(out, in, K, group_size, M) || ws_bytes < need || (need > 0 && workspace == nullptr) ||
        ((uintptr_t)workspace & 3u) != 0)
        return hipErrorInvalidValue;
    const SplitPlan pl = split_plan(out, in);
    float *P = static_cast<float *>(workspace);
    return K == 1 ? launch_f<1>(planes, scales, out, in, X, M, Y, P, pl, st)
                  : launch_f<2>(planes, scales, out, in, X, M, Y, P, pl, st);
}

}  // namespace rbq
