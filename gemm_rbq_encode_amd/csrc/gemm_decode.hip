// gemm_decode.hip -- decode-batch (M <= 5 tokens per pass) residual-binary
// GEMV on the int8 matrix cores of gfx950.
//
// y[m][r] = sum_k a_k[r] * (B_k x_m)[r], with B_k x = 2 S_k - sum(x) and
// S_k = sum of x where the bit is set ("RaBiT" summary, paperlayer.ai,
// section 4.1: binary cores with per-channel scales, additions only;
// section 4.2: the K paths are independent at inference; D "GPU
// implementation": 32 columns packed per uint32).
//
// The decode GEMV streams 2 bits per weight from HBM; at 8 TB/s that is
// ~64 Tbit/s, more than the ~39 T lane-instructions/s of the vector ALUs,
// so a per-bit VALU loop cannot keep up.  Here each masked sum S_k is
// instead an integer matrix product on v_mfma_i32_16x16x64_i8:
//   A (16 rows x 64 k) = weight bits, unpacked with ONE v_and per 4 bits:
//       w & (0x01010101 << s) leaves bit 8j+s of word w in byte j, with the
//       value 2^s (s = 7 gives 0x80 = -128 as int8).  Each bit position s
//       gets its own accumulator, so the 2^s factor is removed exactly at
//       the end (shift left by 7-s, subtract for s = 7).
//   B (64 k x 16 n) = activations as signed 8-bit limbs: each token's x is
//       scaled by a power of two so that max|x| < 2^22, rounded to an
//       integer q (error <= 2^-23 of max|x|), and q = hi*2^16 + mid*2^8 + lo
//       with hi, mid, lo in [-128, 127]; column n = 3*token + limb.  One
//       MFMA therefore serves up to 5 tokens x 3 limbs.
// Integer accumulation is exact and order-free, so results do not depend
// on the schedule.  The MFMA pairs A and B by (lane/16, byte) and returns
// C[i][j] in lane j + 16*(i/4), register i%4.
//
// Work split: a workgroup (4 waves) owns 16 output rows; the row is cut
// into 1024-column chunks (32 words) and wave w takes chunks w, w+4, ...
// For each chunk a wave loads, per lane, 16 bytes x 2 of each plane (row
// lane%16, words 4*(lane/16) + {0..3} and +16) -- every load instruction
// reads 16 rows x 64 contiguous bytes -- quantises its 1024 activations
// into an LDS image laid out exactly as the B registers want them, and
// issues K*16 MFMAs.  Each wave converts its integer sums to float with
// its own activation scale; the 4 partial outputs are added in a fixed
// order, so the result is deterministic.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int DEC_WAVES = 8;
constexpr int DEC_THREADS = DEC_WAVES * RBQ_WAVE;
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;          // 512 columns per chunk
constexpr int CHUNK_COLS = 32 * CHUNK_WORDS;
constexpr int IMG_BYTES_PER_NC = 8 * 4 * 16;   // [s 8][g 4][16 bytes] per MFMA column
constexpr int MAX_TOKENS = 5;            // 3 limbs x 5 tokens <= 16 MFMA columns

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One batch = up to CPW chunks of this wave (chunks base, base+8, ...): all
// of its weight words and activations are requested before any of them is
// used, so a workgroup pays one memory round trip per batch (one batch
// covers rows of up to 4096*CPW columns).  Each batch has its own
// activation scale per token and is folded into a float partial output.
//
// DUAL: one token and per-plane input scales h_k [K][in] (row scales g_k in
// `scales`): y = sum_k g_k (.) (B_k (h_k (.) x)).  The K products h_k (.) x
// take the place of the tokens -- each is formed exactly in fp32 (two
// binary16 factors) and quantised with its own power of two -- and plane k
// keeps only its sums against copy k, so the MFMA count is that of one token.
template <int K, int CPW, int MT, bool DUAL>
__global__ __launch_bounds__(DEC_THREADS, 1) void gemm_decode_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y, const uint16_t *__restrict__ H) {
    static_assert(!DUAL || MT == K, "dual scales: one activation copy per plane");
    // LDS: per wave, the B image of one chunk, [s 8][g 4][n NC][16 bytes],
    // followed by 16 zero bytes read by the MFMA columns not in use
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ float red[DEC_WAVES][MT][TILE_ROWS];

    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE);
    const int row0 = blockIdx.x * TILE_ROWS;
    const int m0 = blockIdx.y * MT;
    const int mt = min(M - m0, MT);                 // tokens in this pass
    const int NC = 3 * mt;                          // MFMA columns in use
    const int words = in >> 5;
    const int nchunks = (words + CHUNK_WORDS - 1) / CHUNK_WORDS;
    unsigned char *img = lds + (size_t)wave * (IMG_BYTES_PER_NC * NC + 16);
    if (lane == 0)
        *reinterpret_cast<uint4 *>(img + IMG_BYTES_PER_NC * NC) = make_uint4(0, 0, 0, 0);

    const int li = lane & 15;        // A row / B column inside the MFMA
    const int lg = lane >> 4;        // lane group: k-slice of the MFMA
    // rows past the end read the last row (their outputs are never stored):
    // loads carry no per-lane guard, which would make the compiler wait for
    // every outstanding load where the guarded and unguarded paths meet
    const int row = min(row0 + li, out - 1);
    const int my_m = li / 3;         // token whose high limb this lane's column holds
    const bool owner = (li % 3 == 0) && li < NC;
    // B-register source of this lane: its column's image, or the zero pad
    const int b_off = (li < NC) ? (lg * NC + li) * 16 : IMG_BYTES_PER_NC * NC;
    const int b_stride = (li < NC) ? 4 * NC * 16 : 0;     // per bit position s

    // scales of the rows this lane's accumulators hold (rows 4*lg + v)
    float a[K][4];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = min(row0 + 4 * lg + v, out - 1);
            a[k][v] = h2f(scales[(size_t)k * out + r]);
        }
    float yacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // this lane's 8 activations of a chunk: columns 8*lane .. 8*lane+7, i.e.
    // word w = lane/4 (MFMA lane group w/4, register w%4), byte kk = lane%4,
    // bit position s = column % 8
    const int wq = lane >> 2;
    const int w_off = ((wq >> 2) * NC) * 16 + (wq & 3) * 4 + (lane & 3);

    for (int base = wave; base < nchunks; base += DEC_WAVES * CPW) {
        // ---- every load of the batch first
        v4u wv[CPW][K];
        uint4 xv[CPW][MT];      // DUAL: the h_k of this lane's columns
        uint4 x1[DUAL ? CPW : 1];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            // chunks past the row are never multiplied; words past the row
            // meet zero activations in the image
            const int c = min(base + DEC_WAVES * cc, nchunks - 1);
            const int wi = min(c * CHUNK_WORDS + 4 * lg, words - 4);
#pragma unroll
            for (int k = 0; k < K; ++k)
                wv[cc][k] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(
                    planes + ((size_t)k * out + row) * words + wi));
            const int col = c * CHUNK_COLS + 8 * lane;
            const int colc = min(col, in - 8);
            const bool ok = col < in;   // a select on the value, not a guarded load
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint16_t *src = DUAL ? H + (size_t)m * in + colc
                                           : X + (size_t)(m0 + min(m, mt - 1)) * in + colc;
                const uint4 u = *reinterpret_cast<const uint4 *>(src);
                xv[cc][m] = make_uint4(ok ? u.x : 0u, ok ? u.y : 0u, ok ? u.z : 0u, ok ? u.w : 0u);
            }
            if constexpr (DUAL) {
                const uint4 u = *reinterpret_cast<const uint4 *>(X + colc);
                x1[cc] = make_uint4(ok ? u.x : 0u, ok ? u.y : 0u, ok ? u.z : 0u, ok ? u.w : 0u);
            }
        }

        // ---- per-token scale of this batch: |x| < 2^E, integers below 2^22
        int sh[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if constexpr (DUAL) {
                // max |x h_k| in fp32 (non-negative floats order as integers);
                // a non-zero product is at least 2^-48
                uint32_t mb = 0;
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc) {
                    const uint32_t hh[4] = {xv[cc][m].x, xv[cc][m].y, xv[cc][m].z, xv[cc][m].w};
                    const uint32_t xx[4] = {x1[cc].x, x1[cc].y, x1[cc].z, x1[cc].w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float p = h2f((uint16_t)(xx[j >> 1] >> (16 * (j & 1)))) *
                                        h2f((uint16_t)(hh[j >> 1] >> (16 * (j & 1))));
                        mb = max(mb, __builtin_bit_cast(uint32_t, p) & 0x7FFFFFFFu);
                    }
                }
                const uint32_t mx = wave_max_u32_dpp(mb);
                sh[m] = mx == 0 ? 0 : 148 - (int)(mx >> 23);   // max < 2^(e - 126)
                continue;
            }
            v2u16 mx2 = (v2u16){0, 0};
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) {
                const uint4 u = xv[cc][m];
                const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, uu[e] & 0x7FFF7FFFu));
            }
            const uint32_t mx = wave_max_u32_dpp(max((uint32_t)mx2.x, (uint32_t)mx2.y));
            const int e = (int)(mx >> 10);
            sh[m] = 22 - ((e == 0 ? 1 : e) - 14);
        }

        v4i acc[K][8];
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int s = 0; s < 8; ++s)
                acc[k][s] = (v4i){0, 0, 0, 0};
        int sumq[MT];      // per lane: sum of (q + 0x808080) over its values
        int nq = 0;        // number of values summed per token and lane
#pragma unroll
        for (int m = 0; m < MT; ++m)
            sumq[m] = 0;

#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            if (base + DEC_WAVES * cc >= nchunks)
                break;
            // ---- quantise this chunk's activations into the B image.
            // fma(x, 2^sh, 1.5*2^23) rounds x*2^sh to the integer q in the low
            // mantissa bits (bits = 0x4B400000 + q); v = q + 0x808080 and
            // v ^ 0x808080 holds the signed limbs lo, mid, hi of q in bytes 0..2
            // (each byte read as int8 is V_l - 128, and the sum of those times
            // 2^(8l) is v - 0x808080 = q).
            nq += 8;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m >= mt)
                    break;
                const float scale = __builtin_ldexpf(1.0f, sh[m]);
                const uint4 u = xv[cc][m];
                const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
                const uint32_t xx[4] = {x1[DUAL ? cc : 0].x, x1[DUAL ? cc : 0].y, x1[DUAL ? cc : 0].z,
                                        x1[DUAL ? cc : 0].w};
                int part = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t hb = (j & 1) ? (uu[j >> 1] >> 16) : (uu[j >> 1] & 0xFFFFu);
                    float xf = h2f((uint16_t)hb);
                    if constexpr (DUAL)   // x_j h_kj, exact in fp32
                        xf = h2f((uint16_t)(xx[j >> 1] >> (16 * (j & 1)))) * xf;
                    const float f = __builtin_fmaf(xf, scale, 12582912.0f);
                    const uint32_t v = __builtin_bit_cast(uint32_t, f) + (0x808080u - 0x4B400000u);
                    part += (int)v;
                    const uint32_t lb = v ^ 0x808080u;
                    unsigned char *p = img + w_off + j * (4 * NC * 16) + 3 * m * 16;
                    p[0] = (unsigned char)(lb >> 16);    // hi limb  -> column 3m
                    p[16] = (unsigned char)(lb >> 8);    // mid limb -> column 3m+1
                    p[32] = (unsigned char)lb;           // lo limb  -> column 3m+2
                }
                sumq[m] += part;
            }
            wave_sync();

            // ---- MFMA over the chunk: A = masked weight bytes, B = limb image
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const v4i b = *reinterpret_cast<const v4i *>(img + b_off + s * b_stride);
                const uint32_t mask = 0x01010101u << s;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const v4u w = wv[cc][k];
                    const v4i av = (v4i){(int)(w.x & mask), (int)(w.y & mask),
                                         (int)(w.z & mask), (int)(w.w & mask)};
                    acc[k][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, acc[k][s], 0, 0, 0);
                }
            }
            wave_sync();   // the next chunk overwrites the image
        }

        // ---- fold the batch into float partial outputs
        int shm = sh[0];
        float sxm = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= mt)
                break;
            // sum of q over the wave = sum of (q + 0x808080) - count * 0x808080
            const float sx = wave_sum_f32_dpp((float)(sumq[m] - nq * 0x808080));
            if (my_m == m) {
                sxm = sx;
                shm = sh[m];
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float yv = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                int t = -acc[k][7][v];
#pragma unroll
                for (int s = 0; s < 7; ++s)
                    t += acc[k][s][v] * (1 << (7 - s));
                // t = 2^7 * sum over this lane's limb of (bit * limb); the mid and
                // lo limbs of the same token sit in the next two lanes
                const float tm = (float)row_shl_i32<1>(t);
                const float tl = (float)row_shl_i32<2>(t);
                const float T = (float)t * 65536.0f + tm * 256.0f + tl;   // 2^7 * sum(bit * q)
                const float contrib = a[k][v] * (T * (2.0f / 128.0f) - sxm);
                if constexpr (DUAL)
                    yv += (my_m == k) ? contrib : 0.0f;   // plane k against its own copy
                else
                    yv += contrib;
            }
            yacc[v] += __builtin_ldexpf(yv, -shm);
        }
    }

    if (owner) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[wave][my_m][4 * lg + v] = yacc[v];
    }
    __syncthreads();
    if constexpr (DUAL) {
        if (threadIdx.x < TILE_ROWS) {
            const int r = row0 + threadIdx.x;
            if (r < out) {
                float y = 0.0f;
#pragma unroll
                for (int w = 0; w < DEC_WAVES; ++w)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        y += red[w][m][threadIdx.x];
                Y[r] = f2h(y);
            }
        }
        return;
    }
    if (threadIdx.x < mt * TILE_ROWS) {
        const int mm = threadIdx.x / TILE_ROWS, i = threadIdx.x % TILE_ROWS;
        const int r = row0 + i;
        if (r < out) {
            float y = 0.0f;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w)
                y += red[w][mm][i];
            Y[(size_t)(m0 + mm) * out + r] = f2h(y);
        }
    }
}

template <int K, int CPW, int MT, bool DUAL = false>
hipError_t launch_kcm(const uint32_t *planes, const uint16_t *scales, int out, int in,
                      const uint16_t *X, int M, uint16_t *Y, hipStream_t st, const uint16_t *H = nullptr) {
    const int tiles = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int passes = (M + MT - 1) / MT;
    const int mt = M < MT ? M : MT;
    const size_t lds = (size_t)DEC_WAVES * (IMG_BYTES_PER_NC * 3 * mt + 16);
    hipLaunchKernelGGL((gemm_decode_kernel<K, CPW, MT, DUAL>), dim3(tiles, passes), dim3(DEC_THREADS),
                       lds, st, planes, scales, out, in, X, M, Y, H);
    return hipGetLastError();
}

template <int K>
hipError_t launch_dual_k(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                         const uint16_t *x, uint16_t *y, hipStream_t st) {
    // M = K "tokens" (the K scaled copies of x) in one pass
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int per_wave = (nchunks + DEC_WAVES - 1) / DEC_WAVES;
    if (per_wave <= 1)
        return launch_kcm<K, 1, K, true>(planes, g, out, in, x, K, y, st, h);
    if (per_wave <= 2)
        return launch_kcm<K, 2, K, true>(planes, g, out, in, x, K, y, st, h);
    return launch_kcm<K, 4, K, true>(planes, g, out, in, x, K, y, st, h);
}

template <int K>
hipError_t launch_k(const uint32_t *planes, const uint16_t *scales, int out, int in,
                    const uint16_t *X, int M, uint16_t *Y, hipStream_t st) {
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int per_wave = (nchunks + DEC_WAVES - 1) / DEC_WAVES;
    if (M == 1) {
        if (per_wave <= 1)
            return launch_kcm<K, 1, 1>(planes, scales, out, in, X, M, Y, st);
        if (per_wave <= 2)
            return launch_kcm<K, 2, 1>(planes, scales, out, in, X, M, Y, st);
        return launch_kcm<K, 4, 1>(planes, scales, out, in, X, M, Y, st);
    }
    if (per_wave <= 1)
        return launch_kcm<K, 1, MAX_TOKENS>(planes, scales, out, in, X, M, Y, st);
    if (per_wave <= 2)
        return launch_kcm<K, 2, MAX_TOKENS>(planes, scales, out, in, X, M, Y, st);
    return launch_kcm<K, 4, MAX_TOKENS>(planes, scales, out, in, X, M, Y, st);
}

}  // namespace

bool decode_supports(int in, int K, int group_size, int M) {
    return group_size == 0 && K >= 1 && K <= 4 && in % 128 == 0 && M >= 1 && M <= 65535 * 5;
}

bool dual_supports(int in, int K) {
    return K >= 1 && K <= 4 && in % 128 == 0;
}

hipError_t launch_gemv_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                            int K, const uint16_t *x, uint16_t *y, hipStream_t st) {
    if (!dual_supports(in, K))
        return hipErrorInvalidValue;
    switch (K) {
    case 1: return launch_dual_k<1>(planes, g, h, out, in, x, y, st);
    case 2: return launch_dual_k<2>(planes, g, h, out, in, x, y, st);
    case 3: return launch_dual_k<3>(planes, g, h, out, in, x, y, st);
    case 4: return launch_dual_k<4>(planes, g, h, out, in, x, y, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_decode(const uint32_t *planes, const uint16_t *scales, int out, int in,
                              int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                              hipStream_t st) {
    if (!decode_supports(in, K, group_size, M))
        return hipErrorInvalidValue;
    switch (K) {
    case 1: return launch_k<1>(planes, scales, out, in, X, M, Y, st);
    case 2: return launch_k<2>(planes, scales, out, in, X, M, Y, st);
    case 3: return launch_k<3>(planes, scales, out, in, X, M, Y, st);
    case 4: return launch_k<4>(planes, scales, out, in, X, M, Y, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rbq
