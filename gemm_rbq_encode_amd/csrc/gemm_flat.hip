// gemm_flat.hip -- residual-binary GEMV for a few tokens: one 16-wave
// workgroup per compute unit, with the activation image built by 4 waves
// while the other 12 already stream weights.
//
// y[m][r] = sum_k a_k[r] * (2 S_k - sum x), S_k = sum of x over the set bits
// of row r of plane k ("RaBiT" summary, paperlayer.ai, sections 4.1 and 4.2:
// binary cores with per-channel scales, the K paths side by side; D "GPU
// implementation": 32 columns per word).  S_k is an exact integer product on
// v_mfma_i32_16x16x64_i8:
//   * each token is quantised once, q = round(x * 2^sh) with one power of two
//     per token (|q| <= 2^22), and split into three signed bytes,
//     q = l_0 + 2^8 l_1 + 2^16 l_2, l_j in [-128, 127];
//   * the A operand is a masked weight word, w & (0x01010101 << s): byte kk
//     holds bit 8kk + s of the word times 2^s (bit 7 reads as -128);
//   * the B operand for bit position s holds the limbs of the matching
//     columns.  One accumulator per plane and bit position; the flush
//     T = sum_{s<7} 2^(7-s) acc_s - acc_7 = 2^7 sum(bit * limb).
//
// Organisation.  A GEMV reads each weight byte once, so its time is the HBM
// latency plus the bytes over the bandwidth -- if the memory is busy from
// the start and the arithmetic keeps pace with the arrivals:
//   * one workgroup per compute unit; workgroup b owns the 16-row tiles
//     [b T / G, (b+1) T / G), whose (tile, 512-column chunk) units are split
//     evenly, in order, over waves 4..15;
//   * those stream waves request their first RING units at entry and then
//     wait for the image; a wave whose loads exceed the memory queue stalls
//     at the issue of the next load, which is why the image is left to
//     waves 0..3, which request no weights: they load the activations with
//     16-byte loads, find the per-token maximum (meeting through an LDS
//     counter), write the image and count themselves done in LDS;
//   * a stream wave consumes a unit and requests the next one; the partial
//     sums of a tile from several waves meet in LDS as int32 additions
//     (exact, so the result does not depend on their order), and one
//     thread per output row applies the scales.
// The LDS waits are bounded; the waves they wait for belong to the same
// workgroup, run concurrently and wait for nothing themselves.
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int FL_WAVES = 16;
constexpr int FL_THREADS = FL_WAVES * RBQ_WAVE;
constexpr int FL_PREP = 4;                            // waves that build the image
constexpr int FL_PREP_THREADS = FL_PREP * RBQ_WAVE;
constexpr int FL_STREAM = FL_WAVES - FL_PREP;         // waves that stream weights
constexpr int TILE_ROWS = 16;
constexpr int CHUNK_WORDS = 16;                       // 512 columns
constexpr int IMG_PER_NC = 8 * 4 * 16;                // image bytes per chunk and MFMA column
constexpr int IMG_CHUNK_PAD = 64;                     // moves consecutive chunks to other LDS banks
constexpr int NLIMB = 3;
constexpr int FL_MAX_M = 16;                          // tokens per call (passes of up to 4)
constexpr int FL_MAX_TILES = FL_THREADS / TILE_ROWS;  // one finishing thread per row
constexpr int FL_MAX_XU = 4;                          // half-words per image thread and token
constexpr int FL_MAX_IN = FL_MAX_XU * FL_PREP_THREADS * 16;  // 16 columns per half-word
constexpr int FL_SPIN_LIMIT = 1 << 22;                // bound of each LDS wait (never reached;
                                                      // a wait that runs out makes the rows NaN)

// LDS bytes: activation image, 16 zero bytes, int32 partial sums.
size_t flat_lds_bytes(int in, int K, int mt, int tiles_per_wg) {
    const size_t nchunks = (size_t)((in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS);
    const size_t nc = (size_t)NLIMB * mt;
    return nchunks * (IMG_PER_NC * nc + IMG_CHUNK_PAD) + 16 +
           (size_t)tiles_per_wg * K * nc * TILE_ROWS * 4;
}

// Tokens per pass over the weights: 1, 2 or 4 (3 limbs x 4 tokens = 12 of
// the 16 MFMA columns).
int flat_tokens_per_pass(int M) { return M <= 2 ? M : 4; }

// Half-words (16 columns; padded words included) per image thread.
int flat_units_per_thread(int in) {
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    return (nchunks * CHUNK_WORDS * 2 + FL_PREP_THREADS - 1) / FL_PREP_THREADS;
}

// Waits until the LDS counter reaches `target` (relaxed reads: the writers
// release their LDS stores before counting, and LDS is coherent within the
// compute unit).  A wait that runs out sets *failed: the workgroup then
// writes fp16 NaN for its rows instead of a value built on missing data.
__device__ __forceinline__ void lds_wait_count(int *counter, int target, int *failed) {
    bool done = false;
    for (int i = 0; i < FL_SPIN_LIMIT; ++i) {
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

// DUAL: one token x and per-plane input scales H [K][in] (row scales in
// `scales`): y = sum_k a_k (.) (B_k (h_k (.) x)).  The K products h_k (.) x,
// exact in fp32, take the place of the tokens (MT = K, M = K), each with its
// own power of two, and plane k keeps only its sums against copy k.
template <int K, int MT, int XU, int RING, bool SILU, bool DUAL = false>
__global__ __launch_bounds__(FL_THREADS, 1) void gemm_flat_kernel(
    const uint32_t *__restrict__ planes, const uint16_t *__restrict__ scales, int out, int in,
    const uint16_t *__restrict__ X, int M, uint16_t *__restrict__ Y, const uint16_t *__restrict__ Hs = nullptr) {
    static_assert(!DUAL || (MT == K && !SILU), "dual scales: one activation copy per plane");
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ uint32_t wmax[MT][FL_PREP];
    __shared__ double wsum[MT][FL_PREP];   // exact: integer sums below 2^53
    __shared__ int shs[MT];
    __shared__ int counters[2];       // prep waves past the maximum, past the image
    __shared__ int wait_failed;       // an LDS wait ran out: the rows are written as NaN

    const int tid = threadIdx.x;
    const int lane = tid & (RBQ_WAVE - 1);
    // wave-uniform values in scalar registers: branches on them are scalar
    // and loads under them carry no per-lane predicate
    const int wave = __builtin_amdgcn_readfirstlane(tid / RBQ_WAVE);
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * MT;
    const int mt = min(M - m0, MT);
    const int NC = NLIMB * mt;
    const int words = in >> 5;
    const int nchunks = (words + CHUNK_WORDS - 1) / CHUNK_WORDS;
    const int img_chunk = IMG_PER_NC * NC + IMG_CHUNK_PAD;
    const int pad = nchunks * img_chunk;            // 16 zero bytes for unused MFMA columns

    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int G = gridDim.x;
    const int t0 = (int)(((long)blockIdx.x * T) / G);
    const int t1 = (int)(((long)(blockIdx.x + 1) * T) / G);
    const int ntl = t1 - t0;
    int *red = reinterpret_cast<int *>(lds + pad + 16);                         // [ntl][K][NC][16]

    // scales of the output row this thread finishes (requested after the
    // activations or the first weights, whose waits must not include them)
    const int frow = min(t0 * TILE_ROWS + tid, out - 1);
    uint16_t a_bits[K];
    auto load_scales = [&]() {
#pragma unroll
        for (int k = 0; k < K; ++k)
            a_bits[k] = scales[(size_t)k * out + frow];
    };

    // LDS set-up, then the entry barrier.  One token: before the branches
    // below.  Several tokens: the image waves first request their
    // activations, and the two kinds of waves reach a barrier that waits for
    // LDS only (so those loads stay in flight) in their own branches (each
    // wave passes one s_barrier).  (The same split for one token measured
    // slower.)
    auto lds_init = [&]() {
        if (tid == 0) {
            counters[0] = counters[1] = 0;
            wait_failed = 0;
        }
        for (int i = tid; i < ntl * K * NC * TILE_ROWS; i += FL_THREADS)
            red[i] = 0;
        if (tid < 4)
            reinterpret_cast<uint32_t *>(lds + pad)[tid] = 0u;
    };
    auto entry = [&]() {
        if constexpr (MT > 1) {
            lds_init();
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };
    if constexpr (MT == 1) {
        // (no load is outstanding here, so the barrier waits for nothing else)
        lds_init();
        __syncthreads();
    }

    if (wave < FL_PREP) {
        // ================= image waves =================
        // Thread t owns the half-words H = t + j * FL_PREP_THREADS (j < XU):
        // word w = H / 2, half e = H % 2, the 16 columns 32w + 16e + i, read
        // with two 16-byte loads.  Column 32w + 8kk + s is byte kk of image
        // entry (w, s), so a half-word holds bytes 2e and 2e + 1 of all eight
        // entries of its word.  Half-words past the row end load its last
        // one and are quantised with the scale 0 (limbs 0).
        const int nh = words * 2;                         // half-words of the row
        const int hpad = nchunks * CHUNK_WORDS * 2;       // with the padded words
        v4u xw[MT][XU][2];            // DUAL: the h_k of this thread's columns
        v4u x1[DUAL ? XU : 1][2];     // DUAL: x
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mc = min(m, mt - 1);
            const uint16_t *xrow = DUAL ? Hs + (size_t)m * in : X + (size_t)(m0 + mc) * in;
#pragma unroll
            for (int j = 0; j < XU; ++j) {
                const int Hh = min(tid + j * FL_PREP_THREADS, nh - 1);
                const v4u *xp = reinterpret_cast<const v4u *>(xrow + 16 * Hh);
                xw[m][j][0] = xp[0];
                xw[m][j][1] = xp[1];
            }
        }
        if constexpr (DUAL) {
#pragma unroll
            for (int j = 0; j < XU; ++j) {
                const int Hh = min(tid + j * FL_PREP_THREADS, nh - 1);
                const v4u *xp = reinterpret_cast<const v4u *>(X + 16 * Hh);
                x1[j][0] = xp[0];
                x1[j][1] = xp[1];
            }
        }
        entry();
        load_scales();
        // per-token maximum of |x| (fp16 bit patterns without the sign
        // compare like magnitudes; clamped repeats only repeat real values)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            uint32_t mloc;
            if constexpr (DUAL) {
                // max |x h_k| in fp32 (non-negative floats order as integers)
                mloc = 0;
#pragma unroll
                for (int j = 0; j < XU; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float p = h2f((uint16_t)(x1[j][h][c >> 1] >> (16 * (c & 1)))) *
                                            h2f((uint16_t)(xw[m][j][h][c >> 1] >> (16 * (c & 1))));
                            mloc = max(mloc, __builtin_bit_cast(uint32_t, p) & 0x7FFFFFFFu);
                        }
            } else {
                v2u16 mx2 = (v2u16){0, 0};
#pragma unroll
                for (int j = 0; j < XU; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            mx2 = __builtin_elementwise_max(
                                mx2, __builtin_bit_cast(v2u16, xw[m][j][h][c] & 0x7FFF7FFFu));
                mloc = max((uint32_t)mx2.x, (uint32_t)mx2.y);
            }
            const uint32_t mx = wave_max_u32_dpp(mloc);
            if (lane == 0)
                wmax[m][wave] = mx;
        }
        if (lane == 0)
            __hip_atomic_fetch_add(&counters[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        lds_wait_count(&counters[0], FL_PREP, &wait_failed);

        // |x| < 2^E per token; q = round(x * 2^sh), sh = 22 - E, |q| <= 2^22
        int sh[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            uint32_t mx = 0;
#pragma unroll
            for (int v = 0; v < FL_PREP; ++v)
                mx = max(mx, wmax[m][v]);
            if constexpr (DUAL) {   // fp32 maximum < 2^(e - 126); a non-zero product is >= 2^-48
                sh[m] = mx == 0 ? 0 : 148 - (int)(mx >> 23);
            } else {
                const int e = (int)(mx >> 10);
                sh[m] = 22 - ((e == 0 ? 1 : e) - 14);
            }
        }
        // Image entry (word w, bit s): the four columns 32w + 8kk + s, kk =
        // 0..3, one byte each, at [chunk w/16][s][lane group (w/4)%4][column
        // n][4 (w%4) + kk].  fma(x, 2^sh, 1.5*2^23) leaves 2^22 + q in the
        // mantissa; v = q + 0x808080 lies in [0, 2^24), and its bytes xor 0x80
        // are the limbs.  Each thread writes the two bytes of its half.
        int psum[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            psum[m] = 0;
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int H = tid + j * FL_PREP_THREADS;
            if (H < hpad) {
                const bool live = H < nh;
                const int w = H >> 1, e = H & 1;
                unsigned char *dst = lds + (w / CHUNK_WORDS) * img_chunk + ((w >> 2) & 3) * (NC * 16) +
                                     (w & 3) * 4 + 2 * e;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < mt) {
                        const float scale = live ? __builtin_ldexpf(1.0f, sh[m]) : 0.0f;
                        // DUAL: h_k read again (from L2) rather than kept in
                        // registers since the maximum
                        v4u hv[2];
                        if constexpr (DUAL) {
                            const v4u *hp = reinterpret_cast<const v4u *>(Hs + (size_t)m * in + 16 * min(H, nh - 1));
                            hv[0] = hp[0];
                            hv[1] = hp[1];
                        } else {
                            hv[0] = xw[m][j][0];
                            hv[1] = xw[m][j][1];
                        }
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            // columns 32w + 16e + s (byte 2e) and + 8 (byte 2e + 1)
                            const uint32_t u0 = hv[0][s >> 1], u1 = hv[1][s >> 1];
                            const uint16_t h0 = (s & 1) ? (uint16_t)(u0 >> 16) : (uint16_t)u0;
                            const uint16_t h1 = (s & 1) ? (uint16_t)(u1 >> 16) : (uint16_t)u1;
                            float f0 = h2f(h0), f1 = h2f(h1);
                            if constexpr (DUAL) {   // x_j h_kj, exact in fp32
                                const uint32_t w0 = x1[j][0][s >> 1], w1 = x1[j][1][s >> 1];
                                f0 = h2f((s & 1) ? (uint16_t)(w0 >> 16) : (uint16_t)w0) * f0;
                                f1 = h2f((s & 1) ? (uint16_t)(w1 >> 16) : (uint16_t)w1) * f1;
                            }
                            const uint32_t v0 =
                                __builtin_bit_cast(uint32_t, __builtin_fmaf(f0, scale, 12582912.0f)) -
                                0x4ABF7F80u;
                            const uint32_t v1 =
                                __builtin_bit_cast(uint32_t, __builtin_fmaf(f1, scale, 12582912.0f)) -
                                0x4ABF7F80u;
                            psum[m] += (int)(v0 + v1) - 2 * 0x808080;
                            // [v0.b0 v1.b0 v0.b1 v1.b1], [v0.b2 v1.b2 0 0]
                            const uint32_t l01 = __builtin_amdgcn_perm(v1, v0, 0x05010400u) ^ 0x80808080u;
                            const uint32_t l2 = __builtin_amdgcn_perm(v1, v0, 0x0C0C0602u) ^ 0x8080u;
                            unsigned char *d = dst + s * (4 * NC * 16) + (NLIMB * m) * 16;
                            *reinterpret_cast<uint16_t *>(d) = (uint16_t)l01;
                            *reinterpret_cast<uint16_t *>(d + 16) = (uint16_t)(l01 >> 16);
                            *reinterpret_cast<uint16_t *>(d + 32) = (uint16_t)l2;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const double ws = wave_sum_f64_dpp((double)psum[m]);   // sum of q over the wave's entries (exact)
            if (lane == 0)
                wsum[m][wave] = ws;
            if (wave == 0 && lane == 0)
                shs[m] = sh[m];
        }
        if (lane == 0)
            __hip_atomic_fetch_add(&counters[1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
        entry();
        // ================= stream waves =================
        const int sw = wave - FL_PREP;
        const int U = ntl * nchunks;
        const int u0 = (sw * U) / FL_STREAM;
        const int u1 = ((sw + 1) * U) / FL_STREAM;
        const int n = u1 - u0;
        // loads past the wave's last unit repeat it (a wave without units
        // repeats a neighbour's): every load is unconditional, since a load
        // skipped on some path makes the compiler wait for all outstanding
        // loads where the paths meet
        const int ulast = max(min(u0, U - 1), u1 - 1);
        const size_t plane_stride = (size_t)out * words;
        // unit u -> (tile u / nchunks, chunk u % nchunks) with u * magic >> 21:
        // exact for u < 2^11 and nchunks <= 32 (the error u * e / 2^21, e <
        // nchunks, stays below 1 / nchunks)
        const uint32_t magic = ((1u << 21) + nchunks - 1) / nchunks;
        // Lane (li, lg) reads words 4lg .. 4lg+3 of the chunk in row li of
        // the tile; rows past the end read the last row (never stored), words
        // past the end of a row read the last four words and meet zeros in
        // the image.  The address of load j comes from the clamped unit
        // min(u0 + j, ulast) alone, so no load depends on a branch.
        int lnext = u0;
        v4u ring[RING][K];
        auto load_unit = [&](v4u (&slot)[K]) {
            const int u = min(lnext, ulast);
            const int tq = (int)(((uint32_t)u * magic) >> 21);
            const int row = min((t0 + tq) * TILE_ROWS + li, out - 1);
            const int wi = min((u - tq * nchunks) * CHUNK_WORDS + 4 * lg, words - 4);
            const uint32_t *p = planes + (size_t)row * words + wi;
#pragma unroll
            for (int k = 0; k < K; ++k)
                slot[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + k * plane_stride));
            ++lnext;
        };
#pragma unroll
        for (int d = 0; d < RING; ++d)
            load_unit(ring[d]);
        load_scales();
        lds_wait_count(&counters[1], FL_PREP, &wait_failed);

        // acc[k][s] collects bit position s of plane k
        v4i acc[K][8];
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[k][j] = (v4i){0, 0, 0, 0};
        const int b_off = (li < NC) ? (lg * NC + li) * 16 : pad;
        const int b_stride = (li < NC) ? 4 * NC * 16 : 0;
        const int b_chunk = (li < NC) ? img_chunk : 0;

        int ptile = t0 + (int)(((uint32_t)u0 * magic) >> 21);
        int pchunk = u0 - (ptile - t0) * nchunks;
        auto chunk = [&](const v4u (&wv)[K]) {
            const unsigned char *bp = lds + b_off + pchunk * b_chunk;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const v4i b = *reinterpret_cast<const v4i *>(bp + s * b_stride);
                const uint32_t mask = 0x01010101u << s;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const v4i av = (v4i){(int)(wv[k].x & mask), (int)(wv[k].y & mask),
                                         (int)(wv[k].z & mask), (int)(wv[k].w & mask)};
                    acc[k][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, acc[k][s], 0, 0, 0);
                }
            }
        };
        // after unit i: move to the next chunk; at a tile's end or at the
        // wave's last unit, add T into LDS.  Lane (li, lg) holds rows 4lg + v
        // of MFMA column li.
        auto step = [&](int i) {
            const bool tile_end = ++pchunk == nchunks;
            if (tile_end || i == n - 1) {
                if (li < NC) {
                    int *rp = red + (ptile - t0) * K * NC * TILE_ROWS + li * TILE_ROWS + 4 * lg;
#pragma unroll
                    for (int k = 0; k < K; ++k)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            // modulo 2^32; the sum itself stays below 2^29
                            uint32_t t = 0u - (uint32_t)acc[k][7][v];
#pragma unroll
                            for (int q = 0; q < 7; ++q)
                                t += (uint32_t)acc[k][q][v] << (7 - q);
                            __hip_atomic_fetch_add(rp + k * NC * TILE_ROWS + v, (int)t, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                        }
                }
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[k][j] = (v4i){0, 0, 0, 0};
            }
            if (tile_end) {
                pchunk = 0;
                ++ptile;
            }
        };
        const int nbk = (n + RING - 1) / RING;
        for (int bi = 0; bi + 1 < nbk; ++bi) {
#pragma unroll
            for (int d = 0; d < RING; ++d) {
                // consume the slot, then refill it: the refill may reuse the
                // slot's registers, so no copy of a pending load is kept
                chunk(ring[d]);
                load_unit(ring[d]);
                step(bi * RING + d);
            }
        }
        if (nbk > 0) {
#pragma unroll
            for (int d = 0; d < RING; ++d) {
                const int i = (nbk - 1) * RING + d;
                if (i < n) {
                    chunk(ring[d]);
                    step(i);
                }
            }
        }
    }
    __syncthreads();

    // ---- one thread per output row.  Column 3m + l holds 2^7 sum(bit l_j);
    // 2^7 sum(bit q) = T_0 + 2^8 T_1 + 2^16 T_2 (exact in fp64), and
    // y = sum_k a_k (2 sum(bit q) - sum q) 2^-sh.  With the SiLU-mul epilogue
    // the rows come in (gate, up) pairs 2i, 2i + 1 -- neighbouring threads of
    // one wave, as tiles start at even rows -- and the even thread writes
    // silu(y_2i) * y_2i+1 to column i of a Y of out / 2 columns.
    auto row_sum = [&](int m) {
        const int tl = tid / TILE_ROWS, i = tid % TILE_ROWS;
        double sx = 0.0;
#pragma unroll
        for (int v = 0; v < FL_PREP; ++v)
            sx += wsum[m][v];
        float y = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int *rp = red + ((tl * K + k) * NC + NLIMB * m) * TILE_ROWS + i;
            const double t = (double)rp[0] + 256.0 * (double)rp[TILE_ROWS] +
                             65536.0 * (double)rp[2 * TILE_ROWS];
            // one explicit fma per plane, as in the program kernel
            y = __builtin_fmaf(h2f(a_bits[k]), (float)(t * (2.0 / 128.0) - sx), y);
        }
        return __builtin_ldexpf(y, -shs[m]);
    };
    const bool rowok = tid < ntl * TILE_ROWS && t0 * TILE_ROWS + tid < out;
    // fp16 NaN in place of every output of the workgroup after a wait ran out
    const bool failed = __hip_atomic_load(&wait_failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
    auto out16 = [&](uint16_t h) { return failed ? (uint16_t)0x7E00u : h; };
    if constexpr (DUAL) {
        // plane k against copy k, each copy with its own power of two
        if (rowok) {
            const int tl = tid / TILE_ROWS, i = tid % TILE_ROWS;
            float y = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                double sx = 0.0;
#pragma unroll
                for (int v = 0; v < FL_PREP; ++v)
                    sx += wsum[k][v];
                const int *rp = red + ((tl * K + k) * NC + NLIMB * k) * TILE_ROWS + i;
                const double t = (double)rp[0] + 256.0 * (double)rp[TILE_ROWS] +
                                 65536.0 * (double)rp[2 * TILE_ROWS];
                y += __builtin_ldexpf(h2f(a_bits[k]) * (float)(t * (2.0 / 128.0) - sx), -shs[k]);
            }
            Y[t0 * TILE_ROWS + tid] = out16(f2h(y));
        }
    } else if constexpr (!SILU) {
        if (rowok) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < mt)
                    Y[(size_t)(m0 + m) * out + t0 * TILE_ROWS + tid] = out16(f2h(row_sum(m)));
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mt) {
                const float y = rowok ? row_sum(m) : 0.0f;
                const float up = __shfl_down(y, 1, RBQ_WAVE);
                if (rowok && (tid & 1) == 0)
                    Y[(size_t)(m0 + m) * (out / 2) + (t0 * TILE_ROWS + tid) / 2] = out16(silu_mul_f16(y, up));
            }
        }
    }
}

int flat_num_cus() {
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

size_t flat_lds_limit() {
    static size_t lim = 0;
    if (lim == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        // the kernel's static LDS (maxima, sums, counters) comes on top
        lim = (size_t)v - 512;
    }
    return lim;
}

int flat_grid(int out) {
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    return T < flat_num_cus() ? T : flat_num_cus();
}

template <int K, int MT, int XU, int RING>
hipError_t launch_kmxr(const uint32_t *planes, const uint16_t *scales, int out, int in,
                       const uint16_t *X, int M, uint16_t *Y, int silu, hipStream_t st) {
    const int G = flat_grid(out);
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int tpw = (T + G - 1) / G;
    const int mt = M < MT ? M : MT;
    const size_t lds = flat_lds_bytes(in, K, mt, tpw);
    if (silu)
        hipLaunchKernelGGL((gemm_flat_kernel<K, MT, XU, RING, true>), dim3(G, (M + MT - 1) / MT),
                           dim3(FL_THREADS), lds, st, planes, scales, out, in, X, M, Y);
    else
        hipLaunchKernelGGL((gemm_flat_kernel<K, MT, XU, RING, false>), dim3(G, (M + MT - 1) / MT),
                           dim3(FL_THREADS), lds, st, planes, scales, out, in, X, M, Y);
    return hipGetLastError();
}

// Two units in flight per stream wave: deeper rings measured slower (their
// refills stall the issue of the wave's next loads for longer).
#ifndef RBQ_FLAT_RING
#define RBQ_FLAT_RING 2
#endif

template <int K, int MT, int XU>
hipError_t launch_kmx(const uint32_t *planes, const uint16_t *scales, int out, int in,
                      const uint16_t *X, int M, uint16_t *Y, int silu, hipStream_t st) {
    return launch_kmxr<K, MT, XU, RBQ_FLAT_RING>(planes, scales, out, in, X, M, Y, silu, st);
}

template <int K, int MT>
hipError_t launch_km(const uint32_t *planes, const uint16_t *scales, int out, int in,
                     const uint16_t *X, int M, uint16_t *Y, int silu, hipStream_t st) {
    const int xu = flat_units_per_thread(in);
    if (xu <= 1)
        return launch_kmx<K, MT, 1>(planes, scales, out, in, X, M, Y, silu, st);
    if (xu <= 2)
        return launch_kmx<K, MT, 2>(planes, scales, out, in, X, M, Y, silu, st);
    if (xu <= 3)
        return launch_kmx<K, MT, 3>(planes, scales, out, in, X, M, Y, silu, st);
    if constexpr (MT <= 2)   // four tokens hold at most 3 half-words each in registers
        return launch_kmx<K, MT, 4>(planes, scales, out, in, X, M, Y, silu, st);
    return hipErrorInvalidValue;
}

template <int K, int XU>
hipError_t launch_dual_x(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                         const uint16_t *x, uint16_t *y, hipStream_t st) {
    const int G = flat_grid(out);
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int tpw = (T + G - 1) / G;
    const size_t lds = flat_lds_bytes(in, K, K, tpw);
    hipLaunchKernelGGL((gemm_flat_kernel<K, K, XU, RBQ_FLAT_RING, false, true>), dim3(G, 1), dim3(FL_THREADS),
                       lds, st, planes, g, out, in, x, K, y, h);
    return hipGetLastError();
}

template <int K>
hipError_t launch_dual_k(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                         const uint16_t *x, uint16_t *y, hipStream_t st) {
    const int xu = flat_units_per_thread(in);
    if (xu <= 1)
        return launch_dual_x<K, 1>(planes, g, h, out, in, x, y, st);
    if (xu <= 2)
        return launch_dual_x<K, 2>(planes, g, h, out, in, x, y, st);
    if (xu <= 3)
        return launch_dual_x<K, 3>(planes, g, h, out, in, x, y, st);
    return launch_dual_x<K, 4>(planes, g, h, out, in, x, y, st);
}

}  // namespace

// The dual-scale layer on this kernel: the K scaled copies of x are its
// tokens (M = K).
bool flat_dual_supports(int out, int in, int K) { return flat_supports(out, in, K, 0, K); }
bool flat_dual_preferred(int out, int in, int K) { return flat_preferred(out, in, K, 0, K); }

hipError_t launch_gemv_dual_flat(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                                 int K, const uint16_t *x, uint16_t *y, hipStream_t st) {
    if (!flat_dual_supports(out, in, K))
        return hipErrorInvalidValue;
    return K == 1 ? launch_dual_k<1>(planes, g, h, out, in, x, y, st)
                  : launch_dual_k<2>(planes, g, h, out, in, x, y, st);
}

bool flat_supports(int out, int in, int K, int group_size, int M) {
    if (group_size != 0 || K < 1 || K > 2 || in % 128 != 0 || in <= 0 || in > FL_MAX_IN ||
        M < 1 || M > FL_MAX_M || out < 1 || (M > 2 && flat_units_per_thread(in) > 3))
        return false;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int G = flat_grid(out);
    const int tpw = (T + G - 1) / G;
    return tpw <= FL_MAX_TILES && flat_lds_bytes(in, K, flat_tokens_per_pass(M), tpw) <= flat_lds_limit();
}

// Measured on MI355X (fp16 in/out, K = 2, one and two tokens): ahead of
// the whole-row streaming kernel once every stream wave gets at least one
// (tile, chunk) unit; with fewer units per workgroup (4096 x 4096: 8) the
// streaming kernel, which spreads a tile over more workgroups, is faster.
bool flat_preferred(int out, int in, int K, int group_size, int M) {
    if (!flat_supports(out, in, K, group_size, M))
        return false;
    const int T = (out + TILE_ROWS - 1) / TILE_ROWS;
    const int G = flat_grid(out);
    const int nchunks = (in / 32 + CHUNK_WORDS - 1) / CHUNK_WORDS;
    return ((T + G - 1) / G) * nchunks >= FL_STREAM;
}

hipError_t launch_gemm_flat(const uint32_t *planes, const uint16_t *scales, int out, int in,
                            int K, int group_size, const uint16_t *X, int M, uint16_t *Y, int silu,
                            hipStream_t st) {
    if (!flat_supports(out, in, K, group_size, M) || (silu && out % 2 != 0))
        return hipErrorInvalidValue;
    const int mt = flat_tokens_per_pass(M);
    if (K == 1)
        return mt == 1 ? launch_km<1, 1>(planes, scales, out, in, X, M, Y, silu, st)
             : mt == 2 ? launch_km<1, 2>(planes, scales, out, in, X, M, Y, silu, st)
                       : launch_km<1, 4>(planes, scales, out, in, X, M, Y, silu, st);
    return mt == 1 ? launch_km<2, 1>(planes, scales, out, in, X, M, Y, silu, st)
         : mt == 2 ? launch_km<2, 2>(planes, scales, out, in, X, M, Y, silu, st)
                   : launch_km<2, 4>(planes, scales, out, in, X, M, Y, silu, st);
}

}  // namespace rbq
