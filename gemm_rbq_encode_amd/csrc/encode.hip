// encode.hip -- sequential residual binarization on gfx950.
//
// Computes, for every row r and group t (the whole row, or 128 columns),
// B_1 = sign(W), a_1 = mean|W|, R_1 = W - a_1 B_1, B_2 = sign(R_1), ...
// ("RaBiT" summary, paperlayer.ai, sections 4.2, B and G; "QBB" summary,
// atlas.scime.ai, "Approach": cascaded analytical residual binarization;
// the mean-|R| scale is the XNOR-Net closed form QBB builds on).
//
// Exactness.  The scale is defined as the serial fp64 sum of |R_j| in
// ascending column order, divided by n, rounded once to fp16.  A serial
// chain per row would leave most of the GPU idle, so each (row, group) is
// summed in parallel, first in fp32.  A summation tree of depth d over
// non-negative terms is within a relative d u/(1 - d u) of the exact sum
// (u = 2^-24 in fp32, 2^-53 in fp64), and the serial fp64 mean is within a
// relative ~n 2^-53 of the exact mean, so the serial mean lies within a known
// relative margin of the parallel mean m.  If every value in
// [m(1 - margin), m(1 + margin)] rounds to the same fp16 number, that number
// is the serial result (rounding is monotonic): the candidate h is the fp16
// rounding of m, accepted when the interval lies strictly between the
// midpoints of h and its two fp16 neighbours (exact in fp32).  The fp32 test
// leaves a few tenths of a percent of the means undecided.  Those take a
// second tier (whole rows: the parallel fp64 sum, margin (2n + 64) 2^-53,
// with the candidate rounded once from fp64 -- through fp32 it would round
// twice), and what is still undecided -- exact ties, or a mean within ~1e-11
// of an fp16 midpoint -- the serial sum itself: for a 128-column group from
// the residuals the wave holds (read lane by lane in column order), for a
// whole row by one lane that rebuilds each R_j from W and the scales already
// chosen.  Exact ties do occur at the later steps of 4-plane group encodings.
// Residuals are updated in fp32 with one rounding, exactly as the definition
// states.
//
#include "rbq_device.h"
#include "rbq_kernels.h"

#pragma clang fp contract(off)

namespace rbq {

namespace {

constexpr uint32_t UNDECIDED = 0xFFFFFFFFu;

// v_writelane_b32 (write one lane of a VGPR from a uniform value): this
// compiler has no builtin for it, so its LLVM intrinsic is named directly.
extern "C" __device__ int rbq_writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// fp16 bits of the mean S / n when the error bound decides it, else
// UNDECIDED.  S >= 0 (or NaN).
__device__ __forceinline__ uint32_t decide_scale(double S, int n) {
    const double nd = (double)n;
    const double m = S / nd;
    const double d = m * ((2.0 * nd + 64.0) * 0x1p-53);
    const uint32_t h = f64_to_f16_rne(m);
    if (!(h < 0x7BFFu))          // the largest finite value, infinity, NaN
        return UNDECIDED;
    const double v = (double)h2f((uint16_t)h);
    const double below = (h == 0u) ? -0x1p-24 : (double)h2f((uint16_t)(h - 1u));
    const double above = (double)h2f((uint16_t)(h + 1u));
    const bool inside = (m - d > 0.5 * (below + v)) && (m + d < 0.5 * (v + above));
    return inside ? h : UNDECIDED;
}

// The defining serial computation for columns [c0, c0+n) at step k: rebuild
// R_{k-1} of each column from W and the k earlier scales (hist[l*stride]),
// sum |R| in ascending order in fp64, divide (correctly rounded), round once.
__device__ __forceinline__ uint16_t serial_scale(const float *__restrict__ Wr, int c0,
                                                            int n, const float *hist, int stride,
                                                            int k) {
    double S = 0.0;
    for (int j = c0; j < c0 + n; ++j) {
        float R = Wr[j];
        for (int l = 0; l < k; ++l) {
            const float a = hist[l * stride];
            R = R - ((R >= 0.0f) ? a : -a);
        }
        S += (double)__builtin_fabsf(R);
    }
    return f64_to_f16_rne(div_rn(S, (double)n));
}

// fp16 bits of a mean m computed in fp32 when every value within a relative
// `margin` of m rounds to the same fp16 number (the interval lies strictly
// between the midpoints around the fp16 rounding of m), else UNDECIDED.  The
// margin covers the error of the fp32 sum and division plus two roundings of
// this test itself.  A mean below 2^-126 (inexact in fp32) rounds to 0
// either way.
__device__ __forceinline__ uint32_t decide_scale_f32(float m, float margin) {
    const uint32_t h = f2h(m);                   // one rounding, ties to even
    if (!(h < 0x7BFFu))                          // the largest finite value, infinity, NaN
        return UNDECIDED;
    const float v = h2f((uint16_t)h);
    const float below = (h == 0u) ? -0x1p-24f : h2f((uint16_t)(h - 1u));
    const float above = h2f((uint16_t)(h + 1u));
    const float d = m * margin;
    const bool inside = (m - d > 0.5f * (below + v)) && (m + d < 0.5f * (v + above));
    return inside ? h : UNDECIDED;
}

// Pairwise sum of N values (depth ceil(log2 N)), in a fixed order.
template <int N>
__device__ __forceinline__ float tree_sum(float (&t)[N]) {
#pragma unroll
    for (int w = 1; w < N; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w)
            t[i] = t[i] + t[i + w];
    return t[0];
}

constexpr int log2_ceil(int n) { return n <= 1 ? 0 : 1 + log2_ceil((n + 1) / 2); }

// Shared state of one workgroup while it encodes its rows.
template <int WAVES, int CPW>
struct EncodeLds {
    float part32[2][WAVES];         // per-wave fp32 row sums, alternating by exchange
    double part[2][WAVES];          // per-wave fp64 row sums (undecided steps)
    float hist_row[8];              // scales chosen so far (serial path)
    uint32_t decided_row;
};

// This wave's columns of row r: FULL, every chunk inside the row (one base
// address, the chunks at immediate offsets); otherwise columns past the row
// end are not read and hold 0.
template <int CPW, bool FULL>
__device__ __forceinline__ void load_row(float (&R)[CPW], const float *__restrict__ Wr, int in_row,
                                         int chunk0, int lane) {
    const float *p = Wr + chunk0 * RBQ_WAVE + lane;
    if constexpr (FULL) {
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            R[i] = p[i * RBQ_WAVE];
    } else {
        // the bounds are opaque here, so that per-chunk masks are not kept
        // in registers across rows
        int in = in_row, c0 = chunk0;
        asm volatile("" : "+s"(in), "+s"(c0));
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            R[i] = ((c0 + i) * RBQ_WAVE + lane < in) ? p[i * RBQ_WAVE] : 0.0f;
    }
}

// Step k of row r, whose columns this wave holds in R (columns past the row
// end hold 0 and keep it; FULL: this wave has none).  `phase` counts the
// workgroup's row-sum exchanges and picks the LDS buffer.  UPDATE: compute
// the next residual (not after the last step).
template <int WAVES, int CPW, bool FULL, bool UPDATE>
__device__ __forceinline__ void row_step(float (&R)[CPW], int r, int k, const float *__restrict__ Wr,
                                         int out, int in_row, uint32_t *__restrict__ planes,
                                         uint16_t *__restrict__ scales, int32_t *__restrict__ status,
                                         int force_serial, EncodeLds<WAVES, CPW> &sh, int &phase) {
    // fp32 sum: depth log2 CPW (lane) + 6 (wave) + log2 WAVES (workgroup),
    // division, test: within a relative 24 u for the shapes used here
    static_assert(log2_ceil(CPW) + 6 + log2_ceil(WAVES) <= 19, "fp32 margin");
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE);
    const int words = in_row >> 5;

    // the row sum: each wave's share, then the waves' shares in a fixed order
    float t[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i)               // columns past the row end hold 0
        t[i] = __builtin_fabsf(R[i]);
    const float sw = wave_sum_f32_dpp(tree_sum<CPW>(t));
    {
        const int b = phase & 1;
        ++phase;
        if (lane == 0)
            sh.part32[b][wave] = sw;
        lds_barrier();
        float p[WAVES];
#pragma unroll
        for (int v = 0; v < WAVES; ++v)
            p[v] = sh.part32[b][v];
        const float S32 = tree_sum<WAVES>(p);
        if (k == 0 && status != nullptr && !__builtin_isfinite(S32)) {
            // a non-finite sum: look for a non-finite element (a finite row
            // whose sum overflows is not flagged)
            bool bad = false;
#pragma unroll
            for (int i = 0; i < CPW; ++i)
                bad |= !__builtin_isfinite(R[i]);
            if (__ballot(bad) != 0 && lane == 0)
                atomicOr(status, (int32_t)1);
        }
        uint32_t h = force_serial ? UNDECIDED : decide_scale_f32(S32 / (float)in_row, 0x1.8p-20f);
        if (h == UNDECIDED) {   // the same in every wave: the same sum in the same order
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < CPW; ++i)
                s += (double)__builtin_fabsf(R[i]);
            s = wave_sum_f64_dpp(s);
            const int b2 = phase & 1;
            ++phase;
            if (lane == 0)
                sh.part[b2][wave] = s;
            lds_barrier();
            double S = sh.part[b2][0];
#pragma unroll
            for (int v = 1; v < WAVES; ++v)
                S += sh.part[b2][v];
            h = force_serial ? UNDECIDED : decide_scale(S, in_row);
            if (h == UNDECIDED) {
                if (threadIdx.x == 0)
                    sh.decided_row = serial_scale(Wr, 0, in_row, sh.hist_row, 1, k);
                lds_barrier();
                h = sh.decided_row;
            }
        }
        const float a = h2f((uint16_t)h);
        if (threadIdx.x == 0) {
            sh.hist_row[k] = a;
            scales[(size_t)k * out + r] = (uint16_t)h;
            if (status != nullptr && (h & 0x7FFFu) == 0x7C00u)
                atomicOr(status, (int32_t)2);
        }

        // signs, packed words (chunk i's ballot is words 2i and 2i + 1, put
        // in lanes 2i and 2i + 1) and the residual update R - (bit ? a : -a),
        // written as fma(sign, -a, R): the product is exact, so it rounds
        // once like the subtraction
        static_assert(2 * CPW <= RBQ_WAVE, "one packed word per lane");
        int in = in_row, chunk0 = wave * CPW;
        if constexpr (!FULL)   // masks derived from the bounds are not kept across steps
            asm volatile("" : "+s"(in), "+s"(chunk0));
        uint32_t wv = 0;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const bool plus = R[i] >= 0.0f;
            const uint64_t m = __ballot(plus);
            if constexpr (UPDATE) {
                const float upd = __builtin_fmaf(plus ? 1.0f : -1.0f, -a, R[i]);
                if constexpr (FULL) {
                    R[i] = upd;
                } else {
                    // chunk c = chunk0 + i is whole (c < in / 64), half (in % 64
                    // = 32: lanes < 32) or past the row end
                    const int c = chunk0 + i;
                    const bool valid = c < (in >> 6) || (c == (in >> 6) && lane < (in & 63));
                    R[i] = valid ? upd : R[i];
                }
            }
            wv = (uint32_t)rbq_writelane_i32((int)(uint32_t)m, 2 * i, (int)wv);
            wv = (uint32_t)rbq_writelane_i32((int)(uint32_t)(m >> 32), 2 * i + 1, (int)wv);
        }
        uint32_t *prow = planes + ((size_t)k * out + r) * words;
        const int idx = chunk0 * 2 + lane;
        if (lane < 2 * CPW && (FULL || idx < words))
            prow[idx] = wv;
    }
}

// All K steps of row r.
template <int WAVES, int CPW, bool FULL>
__device__ __forceinline__ void encode_row(int r, const float *__restrict__ W, int out, int in_row, int K,
                                           uint32_t *__restrict__ planes, uint16_t *__restrict__ scales,
                                           int32_t *__restrict__ status, int force_serial,
                                           EncodeLds<WAVES, CPW> &sh, int &phase) {
    const float *Wr = W + (size_t)r * in_row;
    float R[CPW];
    load_row<CPW, FULL>(R, Wr, in_row, __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE) * CPW,
                        threadIdx.x & (RBQ_WAVE - 1));
    for (int k = 0; k + 1 < K; ++k)
        row_step<WAVES, CPW, FULL, true>(R, r, k, Wr, out, in_row, planes, scales, status, force_serial, sh,
                                         phase);
    row_step<WAVES, CPW, FULL, false>(R, r, K - 1, Wr, out, in_row, planes, scales, status, force_serial, sh,
                                      phase);
}

// A workgroup encodes rows blockIdx.x, blockIdx.x + gridDim.x, ...  It does
// not prefetch its next row: further resident workgroups overlap their loads
// with this one's steps as well (4096 x 4096 with W in HBM: 18.2 us with a
// one-row prefetch, 18.4 us without; with W held in the last-level cache
// 17.0 and 14.8 us).
template <int WAVES, int CPW>
__global__ __launch_bounds__(WAVES * RBQ_WAVE) void encode_kernel(
    const float *__restrict__ W, int out, int in, int K, uint32_t *__restrict__ planes,
    uint16_t *__restrict__ scales, int32_t *__restrict__ status, int force_serial) {
    __shared__ EncodeLds<WAVES, CPW> sh;
    const int chunk0 = __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE) * CPW;
    const bool full = (chunk0 + CPW) * RBQ_WAVE <= in;   // no column past the row end
    int phase = 0;
    for (int r = blockIdx.x; r < out; r += gridDim.x) {
        if (full)
            encode_row<WAVES, CPW, true>(r, W, out, in, K, planes, scales, status, force_serial, sh, phase);
        else
            encode_row<WAVES, CPW, false>(r, W, out, in, K, planes, scales, status, force_serial, sh, phase);
    }
}

int encode_num_cus() {
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

template <int WAVES, int CPW>
hipError_t launch_cpw(const float *W, int out, int in, int K, uint32_t *planes, uint16_t *scales,
                      int32_t *status, int force_serial, hipStream_t st) {
    // as many resident workgroups as the compute units hold
    static int per_cu = 0;
    if (per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, encode_kernel<WAVES, CPW>,
                                                         WAVES * RBQ_WAVE, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        per_cu = n;
    }
    // Workgroups per compute unit: the most that fit whose rows divide
    // evenly enough.  A workgroup's rows run one after another, so a compute
    // unit finishes with its workgroup that has the most rows; p per unit
    // costs ceil(out / (cus p)) p row times against out / cus ideally
    // (11008 rows: 8 per unit give 6 x 8 = 48 against 43).
    const int cus = encode_num_cus();
    int p = per_cu;
    while (p > 1) {
        const long rows = ((long)out + (long)cus * p - 1) / ((long)cus * p);
        if (rows * p * cus <= (long)out * 105 / 100 + (long)cus)
            break;
        --p;
    }
    const long want = (long)cus * p;
    const int grid = (int)(want < out ? want : out);
    hipLaunchKernelGGL((encode_kernel<WAVES, CPW>), dim3(grid), dim3(WAVES * RBQ_WAVE), 0,
                       st, W, out, in, K, planes, scales, status, force_serial);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128-column groups
// ---------------------------------------------------------------------------

constexpr int GR_WAVES = 4;                     // waves per workgroup


// DPP lane permutations inside a row of 16 lanes: level L pairs each lane
// with the lane whose bit (3 - L) differs (row rotate by 8, half-row mirror,
// quad swaps by 2 and by 1).
template <int L>
__device__ __forceinline__ float row_partner(float x) {
    constexpr int ctrl = L == 0 ? 0x128 : L == 1 ? 0x141 : L == 2 ? 0x4E : 0xB1;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl,
                                                                 0xF, 0xF, false));
}

// One exchange level over N live values: with N > 1 value i (i < N/2) pairs
// with value i + N/2, the lane whose level bit is clear keeping i and its
// partner keeping i + N/2, each adding what the other sent; with N = 1 the
// two lanes simply add.  Every level is one rounded addition per lane.
template <int L, int N, int GPW>
__device__ __forceinline__ void fold_level(float (&v)[GPW], int lane) {
    if constexpr (N > 1) {
        const bool upper = (lane >> (3 - L)) & 1;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float send = upper ? v[i] : v[i + N / 2];
            const float keep = upper ? v[i + N / 2] : v[i];
            v[i] = keep + row_partner<L>(send);
        }
    } else {
        v[0] = v[0] + row_partner<L>(v[0]);
    }
    if constexpr (L < 3)
        fold_level<L + 1, (N > 1 ? N / 2 : 1), GPW>(v, lane);
}

// Step k of groups [q0, q0 + live) held by one wave: lane l holds element
// 128 q0 + 64 c + l in R[c].  After the reduction every lane of block g
// (lanes (16/GPW) g .. (16/GPW)(g + 1) - 1 of each 16-lane row) holds the
// sum of group g.  UPDATE: compute the next residual (not after the last
// step).
template <int GPW, bool UPDATE>
__device__ __forceinline__ void group_step(float (&R)[2 * GPW], int k, long ngroups, long q0, int live,
                                           int lane, uint32_t *__restrict__ planes,
                                           uint16_t *__restrict__ scales, int32_t *__restrict__ status,
                                           int force_serial) {
    constexpr int SPAN = 16 / GPW;               // lanes per group inside a row
    const int gl = (lane & 15) / SPAN;           // the group this lane's sum belongs to

    float v[GPW];
#pragma unroll
    for (int g = 0; g < GPW; ++g)
        v[g] = __builtin_fabsf(R[2 * g]) + __builtin_fabsf(R[2 * g + 1]);
    fold_level<0, GPW, GPW>(v, lane);
    float s = v[0];
    s = s + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, __builtin_bit_cast(int, s)));
    s = s + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, s)));

    if (k == 0 && status != nullptr && __ballot(!__builtin_isfinite(s)) != 0) {
        // a non-finite sum: look for a non-finite element (a finite W whose
        // sum overflows is not flagged)
        bool bad = false;
#pragma unroll
        for (int c = 0; c < 2 * GPW; ++c)
            bad |= !__builtin_isfinite(R[c]);
        if (__ballot(bad) != 0 && lane == 0)
            atomicOr(status, (int32_t)1);
    }

    // mean s / 128 (exact unless below 2^-126); margin 10 u
    uint32_t h = force_serial ? UNDECIDED : decide_scale_f32(s * 0x1p-7f, 0x1.4p-21f);
    const uint64_t undecided = __ballot(h == UNDECIDED);
    if (undecided != 0) {
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            if (((undecided >> (g * SPAN)) & 1u) && g < live) {   // uniform in the wave
                // the defining serial sum over the group's residuals in
                // column order: columns 64c + l sit in lane l of R[c]
                double S = 0.0;
#pragma unroll
                for (int c = 2 * g; c < 2 * g + 2; ++c)
#pragma nounroll
                    for (int l = 0; l < RBQ_WAVE; ++l)
                        S += (double)__builtin_fabsf(__builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, R[c]), l)));
                const uint32_t hs = f64_to_f16_rne(S * 0x1p-7);   // S / 128, exact
                h = (gl == g) ? hs : h;
                if (status != nullptr && (hs & 0x7FFFu) == 0x7C00u && lane == 0)
                    atomicOr(status, (int32_t)2);
            }
        }
    }

    // scales: the first lane of each group's block in row 0
    if (lane < 16 && lane % SPAN == 0 && gl < live)
        scales[(size_t)k * ngroups + q0 + gl] = (uint16_t)h;

    // signs, packed words (chunk c's ballot is words 2c and 2c + 1, put in
    // lanes 2c and 2c + 1) and the residual update R - (bit ? a : -a),
    // written as fma(sign, -a, R): the product is exact, so it rounds once
    // like the subtraction
    const float af = h2f((uint16_t)h);
    uint32_t wv = 0;
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, af), g * SPAN));
#pragma unroll
        for (int c = 2 * g; c < 2 * g + 2; ++c) {
            const bool plus = R[c] >= 0.0f;
            const uint64_t m = __ballot(plus);
            if constexpr (UPDATE)
                R[c] = __builtin_fmaf(plus ? 1.0f : -1.0f, -a, R[c]);
            wv = (uint32_t)rbq_writelane_i32((int)(uint32_t)m, 2 * c, (int)wv);
            wv = (uint32_t)rbq_writelane_i32((int)(uint32_t)(m >> 32), 2 * c + 1, (int)wv);
        }
    }
    if (lane < 4 * live)
        planes[(size_t)k * 4 * ngroups + (size_t)q0 * 4 + lane] = wv;
}

// Each wave encodes GPW consecutive groups, all K steps on registers.
template <int GPW>
__global__ __launch_bounds__(GR_WAVES * RBQ_WAVE) void encode_group_kernel(
    const float *__restrict__ W, long ngroups, int K, uint32_t *__restrict__ planes,
    uint16_t *__restrict__ scales, int32_t *__restrict__ status, int force_serial) {
    static_assert(GPW >= 1 && GPW <= 16 && (GPW & (GPW - 1)) == 0, "GPW: a power of two up to 16");
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const long q0 = ((long)blockIdx.x * GR_WAVES + threadIdx.x / RBQ_WAVE) * GPW;
    if (q0 >= ngroups)
        return;
    const int live = (int)(ngroups - q0 < GPW ? ngroups - q0 : GPW);   // groups to write

    float R[2 * GPW];
    const float *Wq = W + (size_t)q0 * 128 + lane;
#pragma unroll
    for (int c = 0; c < 2 * GPW; ++c)
        R[c] = (c / 2 < live) ? Wq[c * RBQ_WAVE] : 0.0f;

    for (int k = 0; k + 1 < K; ++k)
        group_step<GPW, true>(R, k, ngroups, q0, live, lane, planes, scales, status, force_serial);
    group_step<GPW, false>(R, K - 1, ngroups, q0, live, lane, planes, scales, status, force_serial);
}

template <int GPW>
hipError_t launch_gpw(const float *W, long ngroups, int K, uint32_t *planes, uint16_t *scales,
                      int32_t *status, int force_serial, hipStream_t st) {
    const long per_block = (long)GR_WAVES * GPW;
    const long blocks = (ngroups + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFL)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((encode_group_kernel<GPW>), dim3((unsigned)blocks), dim3(GR_WAVES * RBQ_WAVE), 0, st, W,
                       ngroups, K, planes, scales, status, force_serial);
    return hipGetLastError();
}

hipError_t launch_groups(const float *W, int out, int in, int K, uint32_t *planes, uint16_t *scales,
                         int32_t *status, int force_serial, hipStream_t st) {
    if (in % 128 != 0)
        return hipErrorInvalidValue;
    const long ngroups = (long)out * (in / 128);
    return launch_gpw<8>(W, ngroups, K, planes, scales, status, force_serial, st);
}

}  // namespace

hipError_t launch_encode(const float *W, int out, int in, int K, int group_size,
                         uint32_t *planes, uint16_t *scales, int32_t *status, int force_serial,
                         hipStream_t st) {
    if (group_size)
        return launch_groups(W, out, in, K, planes, scales, status, force_serial, st);
    // Rows of up to 4096 columns: 4 waves; up to 16384: 8 waves; longer: 16
    // waves.  Chunks per wave come in steps that keep the idle chunks of
    // the common widths few (11008 columns: 8 x 22 of 172 chunks; 8 x 24
    // would leave 20 idle).
    const int chunks = (in + RBQ_WAVE - 1) / RBQ_WAVE;
    const int waves = chunks <= 64 ? 4 : chunks <= 256 ? 8 : 16;
    const int need = (chunks + waves - 1) / waves;
#define RBQ_ENC_CASE(WV, C)                                                              \
    if (waves == WV && need <= C)                                                        \
        return launch_cpw<WV, C>(W, out, in, K, planes, scales, status, force_serial, st);
    RBQ_ENC_CASE(4, 2)
    RBQ_ENC_CASE(4, 4)
    RBQ_ENC_CASE(4, 8)
    RBQ_ENC_CASE(4, 16)
    RBQ_ENC_CASE(8, 12)
    RBQ_ENC_CASE(8, 16)
    RBQ_ENC_CASE(8, 20)
    RBQ_ENC_CASE(8, 22)
    RBQ_ENC_CASE(8, 24)
    RBQ_ENC_CASE(8, 28)
    RBQ_ENC_CASE(8, 32)
    RBQ_ENC_CASE(16, 24)
    RBQ_ENC_CASE(16, 32)
#undef RBQ_ENC_CASE
    return hipErrorInvalidValue;
}

}  // namespace rbq
