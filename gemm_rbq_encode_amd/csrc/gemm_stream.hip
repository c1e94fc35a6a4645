// gemm_stream.hip -- residual-binary GEMV for one or two tokens that streams
// whole weight rows through the int8 matrix cores of gfx950.
//
// Same arithmetic as the chunked decode kernel (gemm_decode.hip): y[m][r] =
// sum_k a_k[r] * (2 S_k - sum x), S_k = sum of x over set bits ("RaBiT"
// summary, paperlayer.ai, sections 4.1 and 4.2; D "GPU implementation"),
// each S_k an exact integer product on v_mfma_i32_16x16x64_i8 of masked
// weight bytes (w & (0x01010101 << s), one accumulator per bit position s)
// with activations split into three signed 8-bit limbs.  The organisation
// differs:
//   * the workgroup quantises the token's whole row of activations ONCE,
//     with one power-of-two scale per token for the whole row, into an LDS
//     image laid out as the MFMA B registers want it;
//   * each wave then owns a 16-row tile (or 1/P of its columns) and streams
//     its 512-column chunks with an RING-deep prefetch of weight words held
//     in registers, so HBM requests of later chunks are in flight while
//     earlier chunks are multiplied, and the accumulator epilogue is paid
//     once per tile instead of once per chunk.
// P waves of one workgroup share a tile when there are too few tiles to
// give every wave its own; their partial outputs are added in LDS in a
// fixed order.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int ST_WAVES = 4;
constexpr int ST_THREADS = ST_WAVES * RBQ_WAVE;
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;                   // 512 columns
constexpr int CHUNK_COLS = 32 * CHUNK_WORDS;
constexpr int IMG_PER_NC = 8 * 4 * 16;            // chunk image bytes per MFMA column
constexpr int ST_MAX_TOKENS = 2;
#ifndef RBQ_STREAM_PRE
#define RBQ_STREAM_PRE(RING) 1
#endif

// LDS budget of the activation image (bytes): in * 3 * tokens must fit.
constexpr int ST_IMG_MAX = 112 * 1024;
// rows of up to 2 words x 256 threads x 32 columns = 16384 columns, K <= 2

template <int K, int P, int MT, int RING, int XW, int PRE>
__global__ __launch_bounds__(ST_THREADS, 2) void gemm_stream_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y) {
    extern __shared__ __align__(16) unsigned char img[];   // [chunk][s][g][n][16] + 16 zero bytes
    __shared__ float red[ST_WAVES][MT][TILE_ROWS];
    __shared__ uint32_t wmax[ST_WAVES][MT];
    __shared__ float wsum[ST_WAVES][MT];

    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    // wave-uniform values live in scalar registers, so the branches on them
    // are scalar branches and loads under them carry no per-lane predicate
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE);
    const int m0 = blockIdx.y * MT;
    const int mt = min(M - m0, MT);
    const int NC = 3 * mt;
    const int words = in >> 5;
    const int nchunks = (words + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int img_chunk = IMG_PER_NC * NC;
    const int pad = nchunks * img_chunk;            // offset of the zero bytes

    // ---- this wave's work item: tile t, columns [c0, c0 + n) in chunks
    const int tiles = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int t = blockIdx.x * (ST_WAVES / P) + wave / P;
    const int part = wave % P;
    const int cpp = (nchunks + P - 1) / P;
    const int c0 = part * cpp;
    const int n = (t < tiles) ? max(0, min(nchunks, c0 + cpp) - c0) : 0;

    const int li = lane & 15, lg = lane >> 4;
    const int row0 = t * TILE_ROWS;
    // Rows past the end read the last row instead (their outputs are never
    // stored), so no load needs a per-lane guard; words past the end of a
    // row read a valid word and meet zeros in the activation image.
    const int row = min(row0 + li, out - 1);
    const uint32_t *prow = planes + (size_t)row * words;
    const size_t plane_stride = (size_t)out * words;

    // ---- activations first (they gate everything), then the first RING
    // chunks of weights, so the weights arrive while x is being quantised.
    // Thread i owns words i, i + 256, ... (XW of them; 32 columns each).
    uint4 xw[XW][MT][4];
#pragma unroll
    for (int j = 0; j < XW; ++j) {
        const int w = threadIdx.x + j * ST_THREADS;
        const int wc = min(w, words - 1);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mc = min(m, mt - 1);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xw[j][m][e] = reinterpret_cast<const uint4 *>(X + (size_t)(m0 + mc) * in + 32 * wc)[e];
        }
    }
    // Every weight load is unconditional (a chunk index past this wave's
    // range is clamped to its last chunk): a load skipped on some path makes
    // the compiler wait for all outstanding loads where the paths meet.
    const int clast = c0 + max(n, 1) - 1;
    v4u ring[RING][K];
    // PRE chunks of weights are requested before the activation work and
    // the rest of the ring after it: issuing the whole ring first stalls the
    // wave on a full memory queue before it can quantise x.
#pragma unroll
    for (int d = 0; d < PRE; ++d) {
        const int wi = min(min(c0 + d, clast) * CHUNK_WORDS + 4 * lg, words - 4);
#pragma unroll
        for (int k = 0; k < K; ++k)
            ring[d][k] = __builtin_nontemporal_load(
                reinterpret_cast<const v4u *>(prow + k * plane_stride + wi));
    }
    float a[K][4];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = min(row0 + 4 * lg + v, out - 1);
            a[k][v] = h2f(scales[(size_t)k * out + r]);
        }

    // ---- one power-of-two scale per token for the whole row: |x| < 2^E
    // (fp16 bit patterns without the sign compare like magnitudes)
    int sh[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        v2u16 mx2 = (v2u16){0, 0};
#pragma unroll
        for (int j = 0; j < XW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // duplicated (clamped) words only repeat real values: harmless for a max
                const uint4 u = xw[j][m][e];
                mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, u.x & 0x7FFF7FFFu));
                mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, u.y & 0x7FFF7FFFu));
                mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, u.z & 0x7FFF7FFFu));
                mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, u.w & 0x7FFF7FFFu));
            }
        const uint32_t mx = wave_max_u32_dpp(max((uint32_t)mx2.x, (uint32_t)mx2.y));
        if (lane == 0)
            wmax[wave][m] = mx;
    }
    if (threadIdx.x < 4)
        reinterpret_cast<uint32_t *>(img + pad)[threadIdx.x] = 0u;
    // the image of words past the row end (inside the last chunk) is zero
    for (int z = words * 8 * 3 * mt + threadIdx.x; z < nchunks * CHUNK_WORDS * 8 * 3 * mt;
         z += ST_THREADS) {
        // z enumerates 4-byte entries (word, s, limb) of missing words
        const int w = z / (8 * 3 * mt), rem = z % (8 * 3 * mt);
        const int ss = rem / (3 * mt), n_ = rem % (3 * mt);
        const int c = w / CHUNK_WORDS, g = (w >> 2) & 3, q = w & 3;
        *reinterpret_cast<uint32_t *>(img + (size_t)c * img_chunk + (size_t)g * NC * 16 + q * 4 +
                                      (size_t)ss * 4 * NC * 16 + n_ * 16) = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        uint32_t mx = wmax[0][m];
#pragma unroll
        for (int v = 1; v < ST_WAVES; ++v)
            mx = max(mx, wmax[v][m]);
        const int e = (int)(mx >> 10);
        sh[m] = 22 - ((e == 0 ? 1 : e) - 14);
    }
    // quantise: fma(x, 2^sh, 1.5*2^23) leaves q = round(x*2^sh) in the low
    // mantissa bits; v = q + 0x808080, and v ^ 0x808080 holds the signed
    // limbs (lo, mid, hi) of q in bytes 0..2
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int part_sum = 0;
        if (m < mt) {
            const float scale = __builtin_ldexpf(1.0f, sh[m]);
#pragma unroll
            for (int j = 0; j < XW; ++j) {
                const int w = threadIdx.x + j * ST_THREADS;
                if (w < words) {
                    uint32_t lb[32];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint4 u = xw[j][m][e];
                        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                        for (int h = 0; h < 8; ++h) {
                            const uint32_t hb = (h & 1) ? (uu[h >> 1] >> 16) : (uu[h >> 1] & 0xFFFFu);
                            const float f = __builtin_fmaf(h2f((uint16_t)hb), scale, 12582912.0f);
                            const uint32_t v = __builtin_bit_cast(uint32_t, f) + (0x808080u - 0x4B400000u);
                            part_sum += (int)v - 0x808080;   // q
                            lb[8 * e + h] = v ^ 0x808080u;
                        }
                    }
                    // word w: chunk w/16, MFMA lane group (w/4)%4, register w%4;
                    // byte kk of the 4-byte entry is column 8kk + s of the word
                    const int c = w / CHUNK_WORDS, g = (w >> 2) & 3, q = w & 3;
                    unsigned char *base = img + (size_t)c * img_chunk + (size_t)g * NC * 16 + q * 4;
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
#pragma unroll
                        for (int l = 0; l < 3; ++l) {
                            // l = 0: hi limb (byte 2), 1: mid (byte 1), 2: lo (byte 0)
                            const uint32_t sel = 0x0c0c0000u | ((uint32_t)(6 - l) << 8) | (uint32_t)(2 - l);
                            const uint32_t b01 = __builtin_amdgcn_perm(lb[8 + s], lb[s], sel);
                            const uint32_t b23 = __builtin_amdgcn_perm(lb[24 + s], lb[16 + s], sel);
                            *reinterpret_cast<uint32_t *>(base + (size_t)s * 4 * NC * 16 +
                                                          (3 * m + l) * 16) = b01 | (b23 << 16);
                        }
                    }
                }
            }
        }
        const float ws = wave_sum_f32_dpp((float)part_sum);   // sum of q over the row
        if (lane == 0)
            wsum[wave][m] = ws;
    }
    __syncthreads();
#pragma unroll
    for (int d = PRE; d < RING; ++d) {
        const int wi = min(min(c0 + d, clast) * CHUNK_WORDS + 4 * lg, words - 4);
#pragma unroll
        for (int k = 0; k < K; ++k)
            ring[d][k] = __builtin_nontemporal_load(
                reinterpret_cast<const v4u *>(prow + k * plane_stride + wi));
    }

    // ---- stream this wave's chunks
    v4i acc[K][8];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int s = 0; s < 8; ++s)
            acc[k][s] = (v4i){0, 0, 0, 0};
    const int b_off = (li < NC) ? (lg * NC + li) * 16 : pad;
    const int b_stride = (li < NC) ? 4 * NC * 16 : 0;
    const int b_chunk = (li < NC) ? img_chunk : 0;

    // blocks of RING chunks: all but the last consume the ring and refill it
    // with the next block (unconditionally); the last block only drains it
    const int nb = (n + RING - 1) / RING;
    auto chunk = [&](const v4u (&w)[K], int i) {
        const unsigned char *bp = img + b_off + (size_t)(c0 + i) * b_chunk;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const v4i b = *reinterpret_cast<const v4i *>(bp + s * b_stride);
            const uint32_t mask = 0x01010101u << s;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const v4i av = (v4i){(int)(w[k].x & mask), (int)(w[k].y & mask),
                                     (int)(w[k].z & mask), (int)(w[k].w & mask)};
                acc[k][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, acc[k][s], 0, 0, 0);
            }
        }
    };
    for (int bi = 0; bi + 1 < nb; ++bi) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            const int i = bi * RING + d;
            // consume the slot, then refill it: the refill may then reuse the
            // slot's registers, so no loop-carried copy of a pending load
            // (which would force a wait on every outstanding load) is needed
            chunk(ring[d], i);
            const int wi = min(min(c0 + i + RING, clast) * CHUNK_WORDS + 4 * lg, words - 4);
#pragma unroll
            for (int k = 0; k < K; ++k)
                ring[d][k] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u *>(prow + k * plane_stride + wi));
        }
    }
    if (nb > 0) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            const int i = (nb - 1) * RING + d;
            if (i < n)
                chunk(ring[d], i);
        }
    }

    // ---- epilogue: lane (li = 3m + limb, lg) holds rows 4*lg + v of MFMA column li
    const int my_m = li / 3;
    const bool owner = (li % 3 == 0) && li < NC;
    float sxm = 0.0f;
    int shm = sh[0];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (my_m == m) {
            float sx = wsum[0][m];
#pragma unroll
            for (int v = 1; v < ST_WAVES; ++v)
                sx += wsum[v][m];
            sxm = sx;
            shm = sh[m];
        }
    }
    // the term sum(x) belongs to the tile once, not once per part
    if (part != 0)
        sxm = 0.0f;
    float yv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float acc_y = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            int tt = -acc[k][7][v];
#pragma unroll
            for (int s = 0; s < 7; ++s)
                tt += acc[k][s][v] * (1 << (7 - s));
            const float tm = (float)row_shl_i32<1>(tt);
            const float tl = (float)row_shl_i32<2>(tt);
            const float T = (float)tt * 65536.0f + tm * 256.0f + tl;   // 2^7 * sum(bit * q)
            acc_y += a[k][v] * (T * (2.0f / 128.0f) - sxm);
        }
        yv[v] = __builtin_ldexpf(acc_y, -shm);
    }
    if (P == 1) {
        if (owner && t < tiles) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = row0 + 4 * lg + v;
                if (r < out)
                    Y[(size_t)(m0 + my_m) * out + r] = f2h(yv[v]);
            }
        }
    } else {
        if (owner) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wave][my_m][4 * lg + v] = yv[v];
        }
        __syncthreads();
        // one thread per (tile of this workgroup, token, row) adds the P parts
        const int per_wg = ST_WAVES / P;
        if (threadIdx.x < per_wg * mt * TILE_ROWS) {
            const int tl = threadIdx.x / (mt * TILE_ROWS);
            const int rem = threadIdx.x % (mt * TILE_ROWS);
            const int mm = rem / TILE_ROWS, i = rem % TILE_ROWS;
            const int tt = blockIdx.x * per_wg + tl;
            const int r = tt * TILE_ROWS + i;
            if (tt < tiles && r < out) {
                float y = 0.0f;
#pragma unroll
                for (int p = 0; p < P; ++p)
                    y += red[tl * P + p][mm][i];
                Y[(size_t)(m0 + mm) * out + r] = f2h(y);
            }
        }
    }
}

template <int K, int P, int MT, int RING>
hipError_t launch_kpr(const uint32_t *planes, const uint16_t *scales, int out, int in,
                      const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    const int tiles = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int per_wg = ST_WAVES / P;
    const int groups = (tiles + per_wg - 1) / per_wg;
    const int passes = (M + MT - 1) / MT;
    const int mt = M < MT ? M : MT;
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const size_t lds = (size_t)nchunks * IMG_PER_NC * 3 * mt + 16;
    if (in <= ST_THREADS * 32)
        hipLaunchKernelGGL((gemm_stream_kernel<K, P, MT, RING, 1, RBQ_STREAM_PRE(RING)>), dim3(groups, passes),
                           dim3(ST_THREADS), lds, st, planes, scales, out, in, X, M, Y);
    else
        hipLaunchKernelGGL((gemm_stream_kernel<K, P, MT, RING, 2, RBQ_STREAM_PRE(RING)>), dim3(groups, passes),
                           dim3(ST_THREADS), lds, st, planes, scales, out, in, X, M, Y);
    return hipGetLastError();
}

int num_cus() {
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

// Prefetch depth: deep enough to keep HBM busy, but the last block of a
// wave's chunks is padded to RING with repeated loads, so avoid depths
// that waste more than two loads per wave.
template <int K, int P, int MT>
hipError_t launch_kp(const uint32_t *planes, const uint16_t *scales, int out, int in,
                     const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int n = (nchunks + P - 1) / P;
    auto waste = [n](int r) { return (n + r - 1) / r * r - n; };
    if (K <= 2 && n >= 8 && waste(8) <= 2)
        return launch_kpr<K, P, MT, 8>(planes, scales, out, in, X, M, Y, st);
    if (n >= 4 && waste(4) <= 1)
        return launch_kpr<K, P, MT, 4>(planes, scales, out, in, X, M, Y, st);
    return launch_kpr<K, P, MT, 2>(planes, scales, out, in, X, M, Y, st);
}

template <int K, int MT>
hipError_t launch_km(const uint32_t *planes, const uint16_t *scales, int out, int in,
                     const uint16_t *X, int M, uint16_t *Y, hipStream_t st, int split) {
    const int tiles = (out + TILE_ROWS - 1) / TILE_ROWS;
    int P = split;
    if (P == 0)   // waves per tile: split tiles until there are about two waves per SIMD
        P = (tiles >= 8 * num_cus()) ? 1 : (tiles >= 2 * num_cus()) ? 2 : 4;
    switch (P) {
    case 1: return launch_kp<K, 1, MT>(planes, scales, out, in, X, M, Y, st);
    case 2: return launch_kp<K, 2, MT>(planes, scales, out, in, X, M, Y, st);
    default: return launch_kp<K, 4, MT>(planes, scales, out, in, X, M, Y, st);
    }
}

}  // namespace

bool stream_supports(int in, int K, int group_size, int M) {
    const int mt = M < ST_MAX_TOKENS ? M : ST_MAX_TOKENS;
    const long img = (long)((in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS) * IMG_PER_NC * 3 * mt;
    return group_size == 0 && K >= 1 && K <= 2 && in % 128 == 0 && in <= 2 * ST_THREADS * 32 &&
           M >= 1 && M <= ST_MAX_TOKENS && img <= ST_IMG_MAX;
}

hipError_t launch_gemm_stream(const uint32_t *planes, const uint16_t *scales, int out, int in,
                              int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                              hipStream_t st, int split) {
    if (!stream_supports(in, K, group_size, M))
        return hipErrorInvalidValue;
    if (M == 1)
        return K == 1 ? launch_km<1, 1>(planes, scales, out, in, X, M, Y, st, split)
                      : launch_km<2, 1>(planes, scales, out, in, X, M, Y, st, split);
    return K == 1 ? launch_km<1, 2>(planes, scales, out, in, X, M, Y, st, split)
                  : launch_km<2, 2>(planes, scales, out, in, X, M, Y, st, split);
    return hipErrorInvalidValue;
}

}  // namespace rbq
