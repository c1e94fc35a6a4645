// gemm_group.hip -- residual-binary GEMV for one token with one scale per
// (row, 128-column group) and up to four planes ("QBB" summary,
// atlas.scime.ai, "Approach": binary bases with their own scales; the
// W(4x1)A16g128 layout of its results tables).
//
// y[r] = sum_k sum_t a_k[r][t] (2 S_k[r][t] - sum_t x), S_k[r][t] = sum of x over
// the set bits of row r of plane k inside group t.  The per-group sums come
// from v_mfma_i32_16x16x64_i8:
//   * x is quantised once per token, q = round(x * 2^sh) (|q| <= 2^22), and
//     split into three signed bytes l_0, l_1, l_2, q = l_0 + 2^8 l_1 + 2^16 l_2;
//   * the A operand is a weight word shifted right by the bit position s and
//     masked with 0x01010101: byte kk holds bit 8kk + s (0 or 1), so every
//     bit position adds into the same accumulator;
//   * in the 16 x 64 operand layout, lane group g of a 512-column chunk holds
//     words 4g..4g+3, i.e. exactly the chunk's group g.  MFMA column
//     n = 3t + l (t < 4, l < 3) takes limb l of group t and is zero in every
//     other lane group, so C[i][n] is row i's bit sum of limb l over group t
//     alone: the group sums come out separated, and the lanes that hold them
//     apply the group's scales before anything is added across groups.
//
// Organisation as in the flat per-row kernel: one 16-wave workgroup per
// compute unit, waves 0..3 build the activation image (and the per-group
// sums of q) while waves 4..15 stream (tile, chunk) units of all planes.
// The image waves then copy the scales of the workgroup's tiles into LDS with
// contiguous loads, transposed to [tile][plane][group][row] so that a lane
// reads its four rows of one group with one 8-byte load (gathering them per
// unit from global memory, 64 scattered 8-byte pieces per load, cost more
// time than all the arithmetic).  Partial outputs of a tile from several
// waves go to separate LDS slots and are added in a fixed order, so the
// result is deterministic.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int GR_WAVES = 16;
constexpr int GR_THREADS = GR_WAVES * RBQ_WAVE;
constexpr int GR_PREP = 4;                             // waves that build the image
constexpr int GR_PREP_THREADS = GR_PREP * RBQ_WAVE;
constexpr int GR_STREAM = GR_WAVES - GR_PREP;          // waves that stream weights
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;                        // 512 columns = 4 groups
constexpr int GROUPS_PER_CHUNK = 4;
constexpr int NLIMB = 3;
constexpr int GR_MAX_K = 4;
constexpr int IMG_ENTRY_ROW = NLIMB * 16;              // one lane group, one bit position
constexpr int IMG_CHUNK = 8 * 4 * IMG_ENTRY_ROW + 64;  // padded: next chunk on other banks
constexpr int GR_MAX_XU = 4;                           // half-words per image thread
constexpr int GR_MAX_IN = GR_MAX_XU * GR_PREP_THREADS * 16;
constexpr int GR_MAX_TILES = GR_THREADS / TILE_ROWS;   // one finishing thread per row
constexpr int GR_SPIN_LIMIT = 1 << 22;                 // bound of each LDS wait (never reached;
                                                       // a wait that runs out makes the rows NaN)
constexpr int GR_RING = 2;

// LDS bytes: image, 16 zero bytes, per-group sums of q, the tiles' scales,
// per-(tile, wave) output slots.
size_t group_lds_bytes(int in, int K, int tiles_per_wg) {
    const size_t nchunks = (size_t)(in / 512), G = (size_t)(in / 128);
    return nchunks * IMG_CHUNK + 16 + G * 4 + (size_t)tiles_per_wg * K * G * TILE_ROWS * 2 +
           (size_t)tiles_per_wg * GR_STREAM * TILE_ROWS * 4;
}

// Waits until the LDS counter reaches `target`; a wait that runs out sets
// *failed, and the workgroup then writes fp16 NaN for its rows.
__device__ __forceinline__ void lds_wait_count(int *counter, int target, int *failed) {
    bool done = false;
    for (int i = 0; i < GR_SPIN_LIMIT; ++i) {
        if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) {
            done = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (!done)
        __hip_atomic_store(failed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp_row_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_row_add_i32(int x) {
    return x + __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

template <int K, int XU>
__global__ __launch_bounds__(GR_THREADS, 1) void gemm_group_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    const uint16_t *__restrict__ X, uint16_t *__restrict__ Y) {
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ uint32_t wmax[GR_PREP];
    __shared__ int shs;
    __shared__ int counters[3];       // image waves past the maximum, the image, the scales
    __shared__ int wait_failed;       // an LDS wait ran out: the rows are written as NaN

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int li = lane & 15, lg = lane >> 4;
    const int words = in >> 5;
    const int nchunks = words / CHUNK_WORDS;          // in % 512 == 0
    const int G = in >> 7;                            // groups per row
    const int pad = nchunks * IMG_CHUNK;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int NG = gridDim.x;
    const int t0 = (int)(((long)blockIdx.x * T) / NG);
    const int t1 = (int)(((long)(blockIdx.x + 1) * T) / NG);
    const int ntl = t1 - t0;

    int *gsum = reinterpret_cast<int *>(lds + pad + 16);                         // [G]
    uint16_t *scl = reinterpret_cast<uint16_t *>(lds + pad + 16 + G * 4);        // [ntl][K][G][16]
    float *red = reinterpret_cast<float *>(scl + (size_t)ntl * K * G * TILE_ROWS);   // [ntl][12][16]

    if (tid == 0) {
        counters[0] = counters[1] = counters[2] = 0;
        wait_failed = 0;
    }
    for (int i = tid; i < ntl * GR_STREAM * TILE_ROWS; i += GR_THREADS)
        red[i] = 0.0f;
    if (tid < 4)
        reinterpret_cast<uint32_t *>(lds + pad)[tid] = 0u;
    __syncthreads();

    if (wave < GR_PREP) {
        // ================= image waves =================
        // Thread t owns the half-words H = t + j * GR_PREP_THREADS (j < XU):
        // word w = H / 2, half e = H % 2, the 16 columns 32w + 16e + i.  Column
        // 32w + 8kk + s is byte kk of image entry (w, s), so a half-word holds
        // bytes 2e, 2e + 1 of the eight entries of its word.  Eight
        // consecutive half-words form one 128-column group.
        const int nh = words * 2;
        v4u xw[XU][2];
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int H = min(tid + j * GR_PREP_THREADS, nh - 1);
            const v4u *xp = reinterpret_cast<const v4u *>(X + 16 * H);
            xw[j][0] = xp[0];
            xw[j][1] = xp[1];
        }
        v2u16 mx2 = (v2u16){0, 0};
#pragma unroll
        for (int j = 0; j < XU; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, xw[j][h][c] & 0x7FFF7FFFu));
        const uint32_t mxw = wave_max_u32_dpp(max((uint32_t)mx2.x, (uint32_t)mx2.y));
        if (lane == 0) {
            wmax[wave] = mxw;
            __hip_atomic_fetch_add(&counters[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        lds_wait_count(&counters[0], GR_PREP, &wait_failed);
        uint32_t mx = 0;
#pragma unroll
        for (int v = 0; v < GR_PREP; ++v)
            mx = max(mx, wmax[v]);
        // |x| < 2^E; q = round(x * 2^sh), sh = 22 - E, |q| <= 2^22
        const int e = (int)(mx >> 10);
        const int sh = 22 - ((e == 0 ? 1 : e) - 14);
        const float scale = __builtin_ldexpf(1.0f, sh);
        // fma(x, 2^sh, 1.5*2^23) leaves 2^22 + q in the mantissa; v = q + 0x808080
        // lies in [0, 2^24), and its bytes xor 0x80 are the limbs
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int H = tid + j * GR_PREP_THREADS;
            const bool live = H < nh;
            int psum = 0;
            if (live) {
                const int w = H >> 1, eh = H & 1;
                unsigned char *dst = lds + (w / CHUNK_WORDS) * IMG_CHUNK +
                                     ((w >> 2) & 3) * IMG_ENTRY_ROW + (w & 3) * 4 + 2 * eh;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const uint32_t u0 = xw[j][0][s >> 1], u1 = xw[j][1][s >> 1];
                    const uint16_t h0 = (s & 1) ? (uint16_t)(u0 >> 16) : (uint16_t)u0;
                    const uint16_t h1 = (s & 1) ? (uint16_t)(u1 >> 16) : (uint16_t)u1;
                    const uint32_t v0 =
                        __builtin_bit_cast(uint32_t, __builtin_fmaf(h2f(h0), scale, 12582912.0f)) - 0x4ABF7F80u;
                    const uint32_t v1 =
                        __builtin_bit_cast(uint32_t, __builtin_fmaf(h2f(h1), scale, 12582912.0f)) - 0x4ABF7F80u;
                    psum += (int)(v0 + v1) - 2 * 0x808080;
                    const uint32_t l01 = __builtin_amdgcn_perm(v1, v0, 0x05010400u) ^ 0x80808080u;
                    const uint32_t l2 = __builtin_amdgcn_perm(v1, v0, 0x0C0C0602u) ^ 0x8080u;
                    unsigned char *d = dst + s * (4 * IMG_ENTRY_ROW);
                    *reinterpret_cast<uint16_t *>(d) = (uint16_t)l01;
                    *reinterpret_cast<uint16_t *>(d + 16) = (uint16_t)(l01 >> 16);
                    *reinterpret_cast<uint16_t *>(d + 32) = (uint16_t)l2;
                }
            }
            // the 8 half-words of a group sit in 8 consecutive lanes (live or
            // dead together, since nh is a multiple of 8); lane 8m + 7 adds them
            psum = dpp_row_add_i32<RBQ_DPP_ROW_SHR(1)>(psum);
            psum = dpp_row_add_i32<RBQ_DPP_ROW_SHR(2)>(psum);
            psum = dpp_row_add_i32<RBQ_DPP_ROW_SHR(4)>(psum);
            if (live && (lane & 7) == 7)
                gsum[H >> 3] = psum;
        }
        if (wave == 0 && lane == 0)
            shs = sh;
        if (lane == 0)
            __hip_atomic_fetch_add(&counters[1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

        // the tiles' scales: 8-byte pieces (4 groups of one row and plane),
        // contiguous in global memory, written to [tile][plane][group][row];
        // batches of SB loads are in flight together
        constexpr int SB = 8;
        const int pieces_row = G / GROUPS_PER_CHUNK;
        const int per_tk = TILE_ROWS * pieces_row;
        const int total = ntl * K * per_tk;
        for (int base = 0; base < total; base += GR_PREP_THREADS * SB) {
            v2u v[SB];
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int pc = min(base + b * GR_PREP_THREADS + tid, total - 1);
                const int tk = pc / per_tk, rem = pc - tk * per_tk;
                const int r = rem / pieces_row, g4 = (rem - r * pieces_row) * GROUPS_PER_CHUNK;
                const int tl = tk / K, k = tk - tl * K;
                const int row = min((t0 + tl) * TILE_ROWS + r, out - 1);
                v[b] = __builtin_nontemporal_load(
                    reinterpret_cast<const v2u *>(scales + ((size_t)k * out + row) * G + g4));
            }
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int pc = base + b * GR_PREP_THREADS + tid;
                if (pc < total) {
                    const int tk = pc / per_tk, rem = pc - tk * per_tk;
                    const int r = rem / pieces_row, g4 = (rem - r * pieces_row) * GROUPS_PER_CHUNK;
                    uint16_t *dst = scl + (size_t)tk * G * TILE_ROWS + r;
#pragma unroll
                    for (int t = 0; t < GROUPS_PER_CHUNK; ++t)
                        dst[(g4 + t) * TILE_ROWS] = (uint16_t)(v[b][t >> 1] >> (16 * (t & 1)));
                }
            }
        }
        if (lane == 0)
            __hip_atomic_fetch_add(&counters[2], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
        // ================= stream waves =================
        // Wave sw takes units sw, sw + 12, sw + 24, ... of the workgroup's
        // (tile, chunk) list: the 12 waves move through a tile's rows side by
        // side, so the rows are read front to back in long runs (each wave
        // owning one contiguous range instead reads 64-byte pieces of 16 rows
        // far apart, which HBM serves at about half the rate).
        const int sw = wave - GR_PREP;
        const int U = ntl * nchunks;
        const int n = U > sw ? (U - sw + GR_STREAM - 1) / GR_STREAM : 0;
        // loads past the wave's last unit repeat it: every load is
        // unconditional (a skipped load makes the compiler wait for all
        // outstanding loads where the paths meet)
        const int ulast = n > 0 ? sw + (n - 1) * GR_STREAM : min(sw, U - 1);
        const size_t plane_stride = (size_t)out * words;
        // u -> (tile u / nchunks, chunk u % nchunks): exact for u < 2^11 and
        // nchunks <= 32
        const uint32_t magic = ((1u << 21) + nchunks - 1) / nchunks;
        // Lane (li, lg) reads words 4lg .. 4lg+3 of the chunk in row li of the
        // tile (rows past the end read the last row, never stored).
        int lnext = sw;
        v4u wring[GR_RING][K];
        auto load_unit = [&](v4u (&wslot)[K]) {
            const int u = min(lnext, ulast);
            const int tq = (int)(((uint32_t)u * magic) >> 21);
            const int c = u - tq * nchunks;
            const int row = min((t0 + tq) * TILE_ROWS + li, out - 1);
            const uint32_t *p = planes + (size_t)row * words + c * CHUNK_WORDS + 4 * lg;
#pragma unroll
            for (int k = 0; k < K; ++k)
                wslot[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + k * plane_stride));
            lnext += GR_STREAM;
        };
#pragma unroll
        for (int d = 0; d < GR_RING; ++d)
            load_unit(wring[d]);
        lds_wait_count(&counters[1], GR_PREP, &wait_failed);

        // B: lane (li, lg) supplies MFMA column li from lane group lg, nonzero
        // only where column li's group li / 3 is this lane group's group
        const bool bl = li < 3 * GROUPS_PER_CHUNK && li / 3 == lg;
        const int b_off = bl ? lg * IMG_ENTRY_ROW + (li - 3 * lg) * 16 : pad;
        const int b_stride = bl ? 4 * IMG_ENTRY_ROW : 0;
        const int b_chunk = bl ? IMG_CHUNK : 0;
        // output column li = 3t + l: group t, limb l, weight 2^(8l) in S; the
        // limb-0 lanes also subtract sum q / 2 of the group: 2 S - sum q =
        // sum_l 2^(8l+1) (T_l - [l = 0] sum q / 2)
        const int gt = min(li / 3, GROUPS_PER_CHUNK - 1);
        const bool live_col = li < 3 * GROUPS_PER_CHUNK;
        const float zq = (live_col && li % 3 == 0) ? -0.5f : 0.0f;
        const float cl = live_col ? __builtin_ldexpf(1.0f, 8 * (li % 3) + 1) : 0.0f;
        float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        int pu = sw;                                      // the unit being consumed
        int ptile = t0 + (int)(((uint32_t)pu * magic) >> 21);
        int pchunk = pu - (ptile - t0) * nchunks;
        bool have_scales = false;
        auto unit = [&](const v4u (&wv)[K]) {
            v4i acc[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                acc[k] = (v4i){0, 0, 0, 0};
            const unsigned char *bp = lds + b_off + pchunk * b_chunk;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const v4i b = *reinterpret_cast<const v4i *>(bp + s * b_stride);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const v4i av = (v4i){(int)((wv[k].x >> s) & 0x01010101u), (int)((wv[k].y >> s) & 0x01010101u),
                                         (int)((wv[k].z >> s) & 0x01010101u), (int)((wv[k].w >> s) & 0x01010101u)};
                    acc[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, acc[k], 0, 0, 0);
                }
            }
            if (!have_scales) {   // uniform; only before the first unit's scales
                lds_wait_count(&counters[2], GR_PREP, &wait_failed);
                have_scales = true;
            }
            const float gq = (float)gsum[pchunk * GROUPS_PER_CHUNK + gt];
            const uint16_t *sp = scl + ((size_t)(ptile - t0) * K * G + pchunk * GROUPS_PER_CHUNK + gt) * TILE_ROWS +
                                 4 * lg;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const v2u a2 = *reinterpret_cast<const v2u *>(sp + (size_t)k * G * TILE_ROWS);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float a = h2f((uint16_t)(a2[v >> 1] >> (16 * (v & 1))));
                    yv[v] = __builtin_fmaf(a, __builtin_fmaf(zq, gq, (float)acc[k][v]), yv[v]);
                }
            }
        };
        // after unit i: at a tile's end or at the wave's last unit, add the
        // 16 columns of each row and store them in the (tile, wave) slot
        auto step = [&](int i) {
            pu += GR_STREAM;
            const int ntile = t0 + (int)(((uint32_t)pu * magic) >> 21);
            const bool tile_end = ntile != ptile;
            if (tile_end || i == n - 1) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float x = yv[v] * cl;
                    x = dpp_row_add<RBQ_DPP_ROW_SHR(1)>(x);
                    x = dpp_row_add<RBQ_DPP_ROW_SHR(2)>(x);
                    x = dpp_row_add<RBQ_DPP_ROW_SHR(4)>(x);
                    x = dpp_row_add<RBQ_DPP_ROW_SHR(8)>(x);
                    if (li == 15)
                        red[((ptile - t0) * GR_STREAM + sw) * TILE_ROWS + 4 * lg + v] = x;
                    yv[v] = 0.0f;
                }
            }
            ptile = ntile;
            pchunk = pu - (ptile - t0) * nchunks;
        };
        const int nbk = (n + GR_RING - 1) / GR_RING;
        for (int bi = 0; bi + 1 < nbk; ++bi) {
#pragma unroll
            for (int d = 0; d < GR_RING; ++d) {
                unit(wring[d]);
                load_unit(wring[d]);
                step(bi * GR_RING + d);
            }
        }
        if (nbk > 0) {
#pragma unroll
            for (int d = 0; d < GR_RING; ++d) {
                const int i = (nbk - 1) * GR_RING + d;
                if (i < n) {
                    unit(wring[d]);
                    step(i);
                }
            }
        }
    }
    __syncthreads();

    // ---- one thread per output row: the wave slots in a fixed order
    if (tid < ntl * TILE_ROWS && t0 * TILE_ROWS + tid < out) {
        const int tl = tid / TILE_ROWS, i = tid % TILE_ROWS;
        float y = 0.0f;
#pragma unroll
        for (int v = 0; v < GR_STREAM; ++v)
            y += red[(tl * GR_STREAM + v) * TILE_ROWS + i];
        const bool failed = __hip_atomic_load(&wait_failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
        Y[t0 * TILE_ROWS + tid] = failed ? (uint16_t)0x7E00u : f2h(__builtin_ldexpf(y, -shs));
    }
}

int group_num_cus() {
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

size_t group_lds_limit() {
    static size_t lim = 0;
    if (lim == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        lim = (size_t)v - 512;   // the kernel's static LDS comes on top
    }
    return lim;
}

int group_grid(int out) {
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    return T < group_num_cus() ? T : group_num_cus();
}

template <int K, int XU>
hipError_t launch_kx(const uint32_t *planes, const uint16_t *scales, int out, int in,
                     const uint16_t *X, uint16_t *Y, hipStream_t st) {
    const int G = group_grid(out);
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const size_t lds = group_lds_bytes(in, K, (T + G - 1) / G);
    hipLaunchKernelGGL((gemm_group_kernel<K, XU>), dim3(G), dim3(GR_THREADS), lds, st, planes, scales,
                       out, in, X, Y);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const uint32_t *planes, const uint16_t *scales, int out, int in,
                    const uint16_t *X, uint16_t *Y, hipStream_t st) {
    const int xu = (in / 16 + GR_PREP_THREADS - 1) / GR_PREP_THREADS;
    if (xu <= 1)
        return launch_kx<K, 1>(planes, scales, out, in, X, Y, st);
    if (xu <= 2)
        return launch_kx<K, 2>(planes, scales, out, in, X, Y, st);
    return launch_kx<K, 4>(planes, scales, out, in, X, Y, st);
}

}  // namespace

bool group_supports(int out, int in, int K, int group_size, int M) {
    if (group_size != 128 || K < 1 || K > GR_MAX_K || in <= 0 || in % 512 != 0 ||
        in > GR_MAX_IN || M != 1 || out < 1)
        return false;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int G = group_grid(out);
    const int tpw = (T + G - 1) / G;
    return tpw <= GR_MAX_TILES && group_lds_bytes(in, K, tpw) <= group_lds_limit();
}

hipError_t launch_gemm_group(const uint32_t *planes, const uint16_t *scales, int out, int in,
                             int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                             hipStream_t st) {
    if (!group_supports(out, in, K, group_size, M) || ((uintptr_t)scales & 7u) != 0)
        return hipErrorInvalidValue;
    switch (K) {
    case 1: return launch_k<1>(planes, scales, out, in, X, Y, st);
    case 2: return launch_k<2>(planes, scales, out, in, X, Y, st);
    case 3: return launch_k<3>(planes, scales, out, in, X, Y, st);
    default: return launch_k<4>(planes, scales, out, in, X, Y, st);
    }
}

}  // namespace rbq
