// rebin.hip -- re-binarization of the K sign planes for fixed scales.
//
// The refinement in the QBB summary (atlas.scime.ai, "Approach") improves
// the binary bases after the analytical cascade.  Without data it can
// alternate two exact minimisations of ||W - sum_k a_k (.) B_k||^2: the K
// scales for fixed planes (refit.hip) and the planes for fixed scales, here.
// For fixed scales the objective is a sum over single weights, so each W_j
// takes the sign pattern s whose value c = sum_k s_k a_k is nearest to it.
// Pattern p has s_k = +1 where bit k of p is 1 (the plane bit).  Ties: a
// weight halfway between two values takes the larger value, and equal
// values go to the largest p (so sign(0) = +1, as in the encoder).  NaN is
// taken as -Inf.  A (row, group) whose scales are not all finite keeps its
// planes.
//
// Exact decisions with fp32 compares.  The 2^K values of a (row, group)
// are sums of K binary16 values, exact in fp64, and so is the midpoint m of
// two of them.  For an fp32 weight w and a real m, w >= m exactly when
// w >= RU(m), the smallest fp32 value not below m.  So each distinct value
// v_i (sorted, i >= 1) contributes one fp32 threshold RU((v_{i-1} + v_i)/2),
// and the rank of the nearest value, ties upward, is the number of
// thresholds at or below w.  Unused thresholds are NaN (never counted), and
// a NaN weight counts none (-Inf's rank).  Per plane a 32-bit mask maps rank
// to bit.  fp32 denormals are kept (the default mode on gfx950), so tiny
// weights compare exactly as well.
//
// Work: segments (row, group of n columns) are contiguous in W and their
// words contiguous in each plane, so a wave takes a run of consecutive
// segments.  Lane i computes segment i's thresholds and masks (O(4^K) fp64
// compares); the wave then streams the columns 64 at a time, one fp32 per
// lane (256 coalesced bytes), reading the current segment's thresholds with
// readlane, the next batch of loads in flight while one is decided.  The
// ballot of a chunk is two plane words; v_writelane gathers 64 words into
// one VGPR per plane, which is then stored coalesced.  The whole pass is a
// few dozen instructions per 64 weights, so it is bound by the read of W
// (4 bytes per weight against K/8 written).
#include "rbq.h"
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

// v_writelane_b32 (write one lane of a VGPR from a uniform value).
extern "C" __device__ int rbq_writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

namespace {

constexpr int RB_THREADS = 256;
constexpr int RB_WAVES = RB_THREADS / RBQ_WAVE;
constexpr int RB_UNROLL = 8;                  // chunk loads in flight per lane
constexpr int RB_FLAT_UNROLL = 16;            // the same for whole-chunk layouts
static_assert(32 % RB_FLAT_UNROLL == 0, "word flushes fall on batch ends");

__device__ __forceinline__ float ru_f32(double m) {
    float f = (float)m;                       // nearest
    if ((double)f < m) {                      // step up one fp32 unit
        const int b = __float_as_int(f);
        f = __int_as_float(f >= 0.0f ? b + 1 : b - 1);
    }
    return f;
}

// Thresholds and rank masks of one segment; `finite` is false when one of
// its scales is not.
// With `sorted` given, threshold p goes to sorted[rank - 1] instead of t[p]
// (rank order, as the K = 4 two-level count reads them).
template <int K>
__device__ void segment_setup(const uint16_t *__restrict__ scales, int out, int G, long seg, float (&t)[1 << K],
                              uint32_t (&mask)[K], bool &finite, float *sorted = nullptr) {
    constexpr int P = 1 << K;
    const long r = seg / G;
    const long g = seg - r * G;
    double a[K];
    finite = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        a[k] = (double)h2f(scales[((size_t)k * out + r) * G + g]);
        finite = finite && __builtin_isfinite(a[k]);
    }
    double c[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        double s = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k)
            s += ((p >> k) & 1) ? a[k] : -a[k];
        c[p] = s;
    }
    bool rep[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        bool top = true;                      // no larger pattern has this value
#pragma unroll
        for (int q = p + 1; q < P; ++q)
            top = top && c[q] != c[p];
        rep[p] = top;
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
        mask[k] = 0u;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        int rank = 0;
        double lower = -__builtin_inf();
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const bool below = c[q] < c[p];
            rank += (below && rep[q]) ? 1 : 0;
            lower = below ? fmax(lower, c[q]) : lower;
        }
        const float th = (rep[p] && rank > 0) ? ru_f32((lower + c[p]) * 0.5) : __builtin_nanf("");
        if (sorted == nullptr)
            t[p] = th;
        else if (rep[p] && rank > 0)
            sorted[rank - 1] = th;
#pragma unroll
        for (int k = 0; k < K; ++k)
            mask[k] |= (rep[p] && ((p >> k) & 1)) ? (1u << rank) : 0u;
    }
}

// Ragged layouts (n % 64 == 32: each segment ends in a half chunk, one
// word).  A wave takes SB whole segments and gathers words with a running
// cursor.
template <int K>
__global__ __launch_bounds__(RB_THREADS) void rebin_tail_kernel(const float *__restrict__ W, int out, int in, int n,
                                                           int sb, uint32_t *__restrict__ planes,
                                                           const uint16_t *__restrict__ scales,
                                                           int32_t *__restrict__ status) {
    constexpr int P = 1 << K;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int G = in / n;
    const long nseg = (long)out * G;
    // wave-uniform (readfirstlane tells the compiler so: the counters below
    // then live in scalar registers and the branches on them are scalar)
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / RBQ_WAVE));
    const long base = ((long)blockIdx.x * RB_WAVES + wave) * sb;
    if (base >= nseg)
        return;                               // whole wave; no barriers below
    const int nsb = (int)(nseg - base < sb ? nseg - base : sb);

    float t[P];
    uint32_t mask[K];
    bool fin = true;
    if (lane < nsb) {
        segment_setup<K>(scales, out, G, base + lane, t, mask, fin);
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p)
            t[p] = __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < K; ++k)
            mask[k] = 0u;
    }
    const int keep_lane = fin ? 0 : 1;
    const bool any_keep = __ballot(!fin) != 0;

    const int cps = (n + RBQ_WAVE - 1) / RBQ_WAVE;      // chunks per segment
    const int nchunks = nsb * cps;
    const float *wbase = W + (size_t)base * n;
    const size_t plane_stride = (size_t)out * (in >> 5);
    uint32_t *pbase = planes + (size_t)base * (n >> 5);

    uint32_t acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        acc[k] = 0u;
    uint32_t keepv = 0u;
    int cur = 0;                              // words emitted by this wave
    bool bad = false;                         // a non-finite weight seen

    float T[P];
    uint32_t M[K];
    int skip = 0;

    auto flush = [&](int first, int cnt) {
        if (lane < cnt && keepv == 0u) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                pbase[(size_t)k * plane_stride + first + lane] = acc[k];
        }
    };
    auto emit = [&](const uint64_t (&m)[K], bool high) {
        const int slot = cur & (RBQ_WAVE - 1);
#pragma unroll
        for (int k = 0; k < K; ++k)
            acc[k] = (uint32_t)rbq_writelane_i32((int)(uint32_t)(high ? m[k] >> 32 : m[k]), slot, (int)acc[k]);
        keepv = (uint32_t)rbq_writelane_i32(skip, slot, (int)keepv);
        ++cur;
        if ((cur & (RBQ_WAVE - 1)) == 0)
            flush(cur - RBQ_WAVE, RBQ_WAVE);
    };

    // loads of chunks q0 .. q0 + RB_UNROLL - 1 (segment lj, chunk lc of the first)
    int lj = 0, lc = 0;
    auto load = [&](float (&wv)[RB_UNROLL], int q0) {
#pragma unroll
        for (int u = 0; u < RB_UNROLL; ++u) {
            const int col = lc * RBQ_WAVE + lane;
            if (q0 + u < nchunks) {           // uniform
                wv[u] = col < n ? wbase[(size_t)lj * n + col] : 0.0f;
            } else {
                wv[u] = 0.0f;
            }
            if (++lc == cps) {
                lc = 0;
                ++lj;
            }
        }
    };

    int pj = 0, pc = 0;                       // segment, chunk of the next step
    float wcur[RB_UNROLL];
    load(wcur, 0);
    for (int q0 = 0; q0 < nchunks; q0 += RB_UNROLL) {
        float wnext[RB_UNROLL];
        if (q0 + RB_UNROLL < nchunks)
            load(wnext, q0 + RB_UNROLL);      // in flight while this batch is decided
#pragma unroll
        for (int u = 0; u < RB_UNROLL; ++u) {
            if (q0 + u >= nchunks)
                break;
            if (pc == 0 || u == 0) {
#pragma unroll
                for (int p = 0; p < P; ++p)
                    T[p] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t[p]), pj));
#pragma unroll
                for (int k = 0; k < K; ++k)
                    M[k] = (uint32_t)__builtin_amdgcn_readlane((int)mask[k], pj);
                skip = __builtin_amdgcn_readlane(keep_lane, pj);
            }
            const float w = wcur[u];
            const bool half = pc == cps - 1;
            bad = bad || ((!half || lane < 32) && !__builtin_isfinite(w));
            int rank = 0;
#pragma unroll
            for (int p = 0; p < P; ++p)
                rank += (w >= T[p]) ? 1 : 0;
            const uint32_t onehot = 1u << rank;
            uint64_t m[K];
#pragma unroll
            for (int k = 0; k < K; ++k)
                m[k] = __ballot((M[k] & onehot) != 0u);
            emit(m, false);
            if (!half)
                emit(m, true);
            if (++pc == cps) {
                pc = 0;
                ++pj;
            }
        }
#pragma unroll
        for (int u = 0; u < RB_UNROLL; ++u)
            wcur[u] = wnext[u];
    }
    const int rest = cur & (RBQ_WAVE - 1);
    if (rest != 0)
        flush(cur - rest, rest);

    if (status != nullptr) {
        const bool any_bad = __ballot(bad) != 0;
        if (lane == 0 && (any_bad || any_keep))
            atomicOr(status, (any_bad ? (int)RBQ_STATUS_NONFINITE_W : 0) |
                                 (any_keep ? (int)RBQ_STATUS_PLANES_KEPT : 0));
    }
}

// Whole-chunk layouts (n % 64 == 0): the matrix is one stream of 64-column
// chunks (chunk q = flat columns 64q .. 64q + 63, plane words 2q and 2q + 1;
// segment q / cps).  Wave w takes chunks [w cpw, (w + 1) cpw), cpw a
// multiple of 32, so every 32 chunks fill the 64 gathered words exactly.
// Its chunks touch at most 64 segments: lane i sets up segment seg0 + i.
template <int K>
__global__ __launch_bounds__(RB_THREADS) void rebin_flat_kernel(const float *__restrict__ W, int out, int in, int n,
                                                                int cpw, uint32_t *__restrict__ planes,
                                                                const uint16_t *__restrict__ scales,
                                                                int32_t *__restrict__ status) {
    constexpr int P = 1 << K;
    constexpr int U = RB_FLAT_UNROLL;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int G = in / n;
    const int cps = n / RBQ_WAVE;
    const long total = (long)out * G * cps;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / RBQ_WAVE));
    const long q_begin = ((long)blockIdx.x * RB_WAVES + wave) * cpw;
    if (q_begin >= total)
        return;                               // whole wave; no barriers below
    const int nq = (int)(total - q_begin < cpw ? total - q_begin : cpw);
    const long seg0 = q_begin / cps;
    const int nsb = (int)((q_begin + nq - 1) / cps - seg0 + 1);

    float t[P];
    uint32_t mask[K];
    bool fin = true;
    // K = 4: the 15 thresholds of segment i, sorted by rank (rank r at
    // index r - 1, NaN where a value repeats), at sorted[16 i ..] in this
    // wave's part of LDS.  They are non-decreasing, so w >= sorted[i] holds
    // for a prefix of i, and the rank -- that prefix's length -- is found
    // from indices 3, 7, 11 (which quarter) and then three of the quarter.
    // Only this wave reads what it wrote (in order, no barrier needed).
    __shared__ float4 sorted_lds[K == 4 ? RB_WAVES * RBQ_WAVE * 4 : 1];
    float *sorted = reinterpret_cast<float *>(sorted_lds) + (K == 4 ? wave * RBQ_WAVE * 16 : 0);
    if constexpr (K == 4) {
        const float nan = __builtin_nanf("");
        float4 *mine = reinterpret_cast<float4 *>(sorted + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mine[i] = make_float4(nan, nan, nan, nan);
    }
    if (lane < nsb) {
        segment_setup<K>(scales, out, G, seg0 + lane, t, mask, fin, K == 4 ? sorted + lane * 16 : nullptr);
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p)
            t[p] = __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < K; ++k)
            mask[k] = 0u;
    }
    if constexpr (K == 4) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the writes are done
        __builtin_amdgcn_wave_barrier();
    }
    const int keep_lane = fin ? 0 : 1;
    const bool any_keep = __ballot(!fin) != 0;

    float S3 = 0.0f, S7 = 0.0f, S11 = 0.0f;

    const float *wq = W + (size_t)q_begin * RBQ_WAVE + lane;
    const size_t plane_stride = (size_t)out * (in >> 5);
    uint32_t *pq = planes + (size_t)q_begin * 2;

    uint32_t acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        acc[k] = 0u;
    uint32_t keepv = 0u;
    bool bad = false;
    float T[P];
    uint32_t M[K];
    int skip = 0;

    auto load = [&](float (&wv)[U], int q0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            wv[u] = q0 + u < nq ? wq[(size_t)(q0 + u) * RBQ_WAVE] : 0.0f;   // uniform test
    };

    int pj = 0;                               // segment of chunk q, relative to seg0
    int pc = (int)(q_begin - seg0 * cps);     // chunk within it
    float wcur[U];
    load(wcur, 0);
    for (int q0 = 0; q0 < nq; q0 += U) {
        float wnext[U];
        if (q0 + U < nq)
            load(wnext, q0 + U);              // in flight while this batch is decided
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (q0 + u >= nq)
                break;
            if (pc == 0 || (q0 == 0 && u == 0)) {
                if constexpr (K == 4) {
                    S3 = sorted[pj * 16 + 3];
                    S7 = sorted[pj * 16 + 7];
                    S11 = sorted[pj * 16 + 11];
                } else {
#pragma unroll
                    for (int p = 0; p < P; ++p)
                        T[p] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t[p]), pj));
                }
#pragma unroll
                for (int k = 0; k < K; ++k)
                    M[k] = (uint32_t)__builtin_amdgcn_readlane((int)mask[k], pj);
                skip = __builtin_amdgcn_readlane(keep_lane, pj);
            }
            const float w = wcur[u];
            bad = bad || !__builtin_isfinite(w);
            int rank = 0;
            if constexpr (K == 4) {
                const int qt = (w >= S3 ? 1 : 0) + (w >= S7 ? 1 : 0) + (w >= S11 ? 1 : 0);
                const float4 v = *reinterpret_cast<const float4 *>(sorted + pj * 16 + 4 * qt);
                rank = 4 * qt + (w >= v.x ? 1 : 0) + (w >= v.y ? 1 : 0) + (w >= v.z ? 1 : 0);
            } else {
#pragma unroll
                for (int p = 0; p < P; ++p)
                    rank += (w >= T[p]) ? 1 : 0;
            }
            const uint32_t onehot = 1u << rank;
            const int slot = 2 * ((q0 + u) & 31);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint64_t m = __ballot((M[k] & onehot) != 0u);
                acc[k] = (uint32_t)rbq_writelane_i32((int)(uint32_t)m, slot, (int)acc[k]);
                acc[k] = (uint32_t)rbq_writelane_i32((int)(uint32_t)(m >> 32), slot + 1, (int)acc[k]);
            }
            if (any_keep) {
                keepv = (uint32_t)rbq_writelane_i32(skip, slot, (int)keepv);
                keepv = (uint32_t)rbq_writelane_i32(skip, slot + 1, (int)keepv);
            }
            if (++pc == cps) {
                pc = 0;
                ++pj;
            }
        }
        // 32 % U == 0 and the range starts 32-aligned, so the 64 gathered
        // words fill up only at the end of a batch
        const int qe = q0 + U < nq ? q0 + U : nq;
        if ((qe & 31) == 0 || qe == nq) {
            const int first = 2 * ((qe - 1) & ~31);
            const int cnt = 2 * qe - first;
            if (lane < cnt && keepv == 0u) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    pq[(size_t)k * plane_stride + first + lane] = acc[k];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            wcur[u] = wnext[u];
    }

    if (status != nullptr) {
        const bool any_bad = __ballot(bad) != 0;
        if (lane == 0 && (any_bad || any_keep))
            atomicOr(status, (any_bad ? (int)RBQ_STATUS_NONFINITE_W : 0) |
                                 (any_keep ? (int)RBQ_STATUS_PLANES_KEPT : 0));
    }
}

template <int K>
hipError_t launch_k(const float *W, int out, int in, int n, uint32_t *planes, const uint16_t *scales,
                    int32_t *status, hipStream_t st) {
    const long nseg = (long)out * (in / n);
    if (n % RBQ_WAVE == 0) {
        // about 8192 waves; a multiple of 32 chunks each, spanning at most
        // 64 segments
        const int cps = n / RBQ_WAVE;
        const long total = nseg * cps;
        long cpw = ((total + 8191) / 8192 + 31) / 32 * 32;
        const long cap = ((long)(RBQ_WAVE - 1) * cps) / 32 * 32;     // keeps nsb <= 64
        cpw = cpw > cap ? cap : cpw;
        cpw = cpw < 32 ? 32 : cpw;
        const long waves = (total + cpw - 1) / cpw;
        const long blocks = (waves + RB_WAVES - 1) / RB_WAVES;
        if (blocks > 0x7FFFFFFFL || total > 0x7FFFFFFFL * 32L)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((rebin_flat_kernel<K>), dim3((unsigned)blocks), dim3(RB_THREADS), 0, st, W, out, in, n,
                           (int)cpw, planes, scales, status);
        return hipGetLastError();
    }
    // a few thousand waves; at most 64 segments (one per lane) each
    long sb = (nseg + 4095) / 4096;
    sb = sb < 1 ? 1 : sb > RBQ_WAVE ? RBQ_WAVE : sb;
    const long waves = (nseg + sb - 1) / sb;
    const long blocks = (waves + RB_WAVES - 1) / RB_WAVES;
    if (blocks > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((rebin_tail_kernel<K>), dim3((unsigned)blocks), dim3(RB_THREADS), 0, st, W, out, in, n,
                       (int)sb, planes, scales, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rebinarize(const float *W, int out, int in, int K, int group_size, uint32_t *planes,
                             const uint16_t *scales, int32_t *status, hipStream_t st) {
    const int n = group_size ? group_size : in;
    if (out <= 0 || in <= 0 || n % 32 != 0 || in % n != 0)
        return hipErrorInvalidValue;
    switch (K) {
    case 1: return launch_k<1>(W, out, in, n, planes, scales, status, st);
    case 2: return launch_k<2>(W, out, in, n, planes, scales, status, st);
    case 3: return launch_k<3>(W, out, in, n, planes, scales, status, st);
    case 4: return launch_k<4>(W, out, in, n, planes, scales, status, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rbq
