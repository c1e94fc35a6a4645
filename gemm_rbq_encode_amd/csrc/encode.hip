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
// summed in parallel in fp64 instead.  Any summation order of n
// non-negative terms is within a relative (n-1)u/(1-(n-1)u) of the exact
// sum (u = 2^-53), so the serial mean and the parallel mean differ by less
// than a relative (2n + 64)u (the 64u also covers both divisions).  If
// every value in that interval rounds to the same fp16 number, that number
// is the serial result (rounding is monotonic).  Otherwise -- an exact tie
// or a mean within ~1e-11 of an fp16 rounding boundary -- the serial sum is
// redone and divided with a correctly rounded division: for a 128-column
// group from the residuals the wave holds (read lane by lane in column
// order), for a whole row by one lane that rebuilds each R_j from W and the
// scales already chosen.  Exact ties do occur at the later steps of 4-plane
// group encodings (a few groups per 13824 x 5120 matrix).  Residuals are
// updated in fp32 with one rounding, exactly as the definition states.
//
// Deciding.  The candidate h is the fp16 rounding of m itself (one rounding
// from fp64: going through fp32 rounds twice and lands on the wrong side of
// an fp16 midpoint about once in 10^4 means, which sent a few rows of most
// matrices to the serial path); it is the answer for every value in
// [m - d, m + d] exactly when that interval lies strictly between the
// midpoints of h and its two fp16 neighbours (which fp64 holds exactly).
//
// Layout.  One workgroup (4 or 16 waves) per row; the row is cut into 64-column
// chunks and wave w keeps chunks [w*CPW, (w+1)*CPW) in registers, lane l
// holding column 64c + l of chunk c.  Loads are therefore coalesced 256-byte
// wave reads, a wave ballot of (R >= 0) is exactly the two packed words of a
// chunk, and a 128-column group is a chunk pair inside one wave.  W is read
// from HBM once; the K steps run on registers.  Sums are reduced with DPP;
// a row's waves meet at barriers that wait for LDS only, so the plane
// stores of earlier steps stay in flight.  A wave decides the scales of its
// 128-column groups together, lane g taking group g.
#include "rbq_device.h"
#include "rbq_kernels.h"

#pragma clang fp contract(off)

namespace rbq {

namespace {

constexpr uint32_t UNDECIDED = 0xFFFFFFFFu;

// Whole-wave fp64 sum (DPP row shifts and broadcasts, then lane 63), the
// same value in every lane.  Lanes a DPP move does not reach add +0.
template <int CTRL, int RMASK>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, RMASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, RMASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
    v += dpp_f64<RBQ_DPP_ROW_SHR(1), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_SHR(2), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_SHR(4), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_SHR(8), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_BCAST15, 0xA>(v);
    v += dpp_f64<RBQ_DPP_ROW_BCAST31, 0xC>(v);
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

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

// Shared state of one workgroup while it encodes its rows.
template <int WAVES, int CPW>
struct EncodeLds {
    double part[2][WAVES];          // per-wave row sums, alternating by step
    float hist_row[8];              // scales chosen so far (serial path)
    uint32_t decided_row;
    uint64_t bits[WAVES][CPW];      // each wave's chunk ballots of the current step
};

template <int WAVES, int CPW>
__device__ __forceinline__ void load_row(float (&R)[CPW], const float *__restrict__ Wr, int in,
                                         int chunk0, int lane) {
    // columns past the row end read its last column (never used: encode_row
    // replaces them by zeros)
#pragma unroll
    for (int i = 0; i < CPW; ++i)
        R[i] = Wr[min((chunk0 + i) * RBQ_WAVE + lane, in - 1)];
}

// All K steps of row r, whose columns this wave holds in R.  `phase` counts
// the workgroup's row-sum exchanges and picks the LDS buffer.
template <int WAVES, int CPW, bool GROUPED>
__device__ __forceinline__ void encode_row(float (&R)[CPW], int r, const float *__restrict__ W,
                                           int out, int in_row, int K,
                                           uint32_t *__restrict__ planes,
                                           uint16_t *__restrict__ scales,
                                           int32_t *__restrict__ status, int force_serial,
                                           EncodeLds<WAVES, CPW> &sh, int &phase) {
    constexpr int GPW = CPW / 2;  // 128-column groups per wave
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE);
    const int words = in_row >> 5;
    const int G = GROUPED ? in_row / 128 : 1;
    const float *Wr = W + (size_t)r * in_row;
    const int chunk0_row = wave * CPW;

    bool bad = false;
    {
        int in = in_row, chunk0 = chunk0_row;
        asm volatile("" : "+s"(in), "+s"(chunk0));
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            R[i] = ((chunk0 + i) * RBQ_WAVE + lane < in) ? R[i] : 0.0f;
            bad |= !__builtin_isfinite(R[i]);
        }
    }
    if (status != nullptr && __any(bad) && lane == 0)
        atomicOr(status, (int32_t)1);

    for (int k = 0; k < K; ++k) {
        // the bounds are re-read each step: masks derived from them are then
        // not kept in scalar registers across the whole loop
        int in = in_row, chunk0 = chunk0_row;
        asm volatile("" : "+s"(in), "+s"(chunk0));
        float a_row = 0.0f;
        float a_grp[GPW];
        if (!GROUPED) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < CPW; ++i)   // columns past the row end hold 0
                s += (double)__builtin_fabsf(R[i]);
            s = wave_sum_f64_dpp(s);
            const int b = phase & 1;
            ++phase;
            if (lane == 0)
                sh.part[b][wave] = s;
            lds_barrier();
            double S = sh.part[b][0];
#pragma unroll
            for (int v = 1; v < WAVES; ++v)
                S += sh.part[b][v];
            uint32_t h = force_serial ? UNDECIDED : decide_scale(S, in);
            if (h == UNDECIDED) {  // same decision in every thread of the block
                if (threadIdx.x == 0)
                    sh.decided_row = serial_scale(Wr, 0, in, sh.hist_row, 1, k);
                lds_barrier();
                h = sh.decided_row;
            }
            a_row = h2f((uint16_t)h);
            if (threadIdx.x == 0) {
                sh.hist_row[k] = a_row;
                scales[(size_t)k * out + r] = (uint16_t)h;
                if (status != nullptr && (h & 0x7FFFu) == 0x7C00u)
                    atomicOr(status, (int32_t)2);
            }
        } else {
            // the wave's group sums, then lane g decides group g
            double mine = 0.0;
#pragma unroll
            for (int g = 0; g < GPW; ++g) {
                const bool gvalid = (chunk0 + 2 * g) * RBQ_WAVE < in;
                double s = gvalid ? (double)__builtin_fabsf(R[2 * g]) +
                                        (double)__builtin_fabsf(R[2 * g + 1])
                                  : 0.0;
                s = wave_sum_f64_dpp(s);
                mine = (lane == g) ? s : mine;
            }
            const uint32_t hl = force_serial ? UNDECIDED : decide_scale(mine, 128);
#pragma unroll
            for (int g = 0; g < GPW; ++g) {
                const int col0 = (chunk0 + 2 * g) * RBQ_WAVE;  // group start (in % 128 == 0)
                const bool gvalid = col0 < in;
                uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)hl, g);
                if (h == UNDECIDED && gvalid) {  // uniform in the wave
                    // the defining serial sum, in column order, over the
                    // group's residuals: columns 128g' + l and 128g' + 64 + l
                    // sit in lane l of R[2g] and R[2g + 1]
                    double S = 0.0;
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        for (int l = 0; l < RBQ_WAVE; ++l)
                            S += (double)__builtin_fabsf(__builtin_bit_cast(
                                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, R[2 * g + c]), l)));
                    h = f64_to_f16_rne(div_rn(S, 128.0));
                }
                a_grp[g] = gvalid ? h2f((uint16_t)h) : 0.0f;
                if (lane == 0 && gvalid) {
                    scales[((size_t)k * out + r) * G + (col0 >> 7)] = (uint16_t)h;
                    if (status != nullptr && (h & 0x7FFFu) == 0x7C00u)
                        atomicOr(status, (int32_t)2);
                }
            }
        }

        // signs, packed words and the residual update.  Chunk i's ballot is
        // its two packed words; the ballots go through LDS so that lane 2i + h
        // picks up word h of chunk i with one read.
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            // chunk c = chunk0 + i is whole (c < in / 64), half (in % 64 = 32:
            // lanes < 32) or past the row end; columns past the end keep 0
            // and their bits are never stored
            const int c = chunk0 + i;
            const bool valid = c < (in >> 6) || (c == (in >> 6) && lane < (in & 63));
            const bool plus = R[i] >= 0.0f;
            const uint64_t m = __ballot(plus);
            const float a = GROUPED ? a_grp[i / 2] : a_row;
            if (valid)
                R[i] = R[i] - (plus ? a : -a);
            if (lane == 0)
                sh.bits[wave][i] = m;
        }
        static_assert(2 * CPW <= RBQ_WAVE, "one packed word per lane");
        const uint32_t wv = reinterpret_cast<const uint32_t *>(sh.bits[wave])[lane < 2 * CPW ? lane : 0];
        uint32_t *prow = planes + ((size_t)k * out + r) * words;
        const int idx = chunk0 * 2 + lane;
        if (lane < 2 * CPW && idx < words)
            prow[idx] = wv;
    }
}

// A workgroup encodes rows blockIdx.x, blockIdx.x + gridDim.x, ...; the
// loads of its next row are in flight while it encodes the current one.
template <int WAVES, int CPW, bool GROUPED>
__global__ __launch_bounds__(WAVES * RBQ_WAVE) void encode_kernel(
    const float *__restrict__ W, int out, int in, int K, uint32_t *__restrict__ planes,
    uint16_t *__restrict__ scales, int32_t *__restrict__ status, int force_serial) {
    static_assert(CPW % 2 == 0, "a 128-column group must be a chunk pair of one wave");
    __shared__ EncodeLds<WAVES, CPW> sh;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int chunk0 = __builtin_amdgcn_readfirstlane(threadIdx.x / RBQ_WAVE) * CPW;
    const int G = gridDim.x;
    int phase = 0;

    float R[CPW], Rn[CPW];
    load_row<WAVES, CPW>(R, W + (size_t)blockIdx.x * in, in, chunk0, lane);
    for (int r = blockIdx.x; r < out; r += G) {
        const bool more = r + G < out;
        if (more)
            load_row<WAVES, CPW>(Rn, W + (size_t)(r + G) * in, in, chunk0, lane);
        encode_row<WAVES, CPW, GROUPED>(R, r, W, out, in, K, planes, scales, status,
                                        force_serial, sh, phase);
        if (more) {
#pragma unroll
            for (int i = 0; i < CPW; ++i)
                R[i] = Rn[i];
        }
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

template <int WAVES, int CPW, bool GROUPED>
hipError_t launch_cpwg(const float *W, int out, int in, int K, uint32_t *planes, uint16_t *scales,
                       int32_t *status, int force_serial, hipStream_t st) {
    // as many resident workgroups as the compute units hold
    static int per_cu = 0;
    if (per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, encode_kernel<WAVES, CPW, GROUPED>,
                                                         WAVES * RBQ_WAVE, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        per_cu = n;
    }
    const long want = (long)encode_num_cus() * per_cu;
    const int grid = (int)(want < out ? want : out);
    hipLaunchKernelGGL((encode_kernel<WAVES, CPW, GROUPED>), dim3(grid), dim3(WAVES * RBQ_WAVE), 0,
                       st, W, out, in, K, planes, scales, status, force_serial);
    return hipGetLastError();
}

template <int WAVES, int CPW>
hipError_t launch_cpw(const float *W, int out, int in, int K, int group_size, uint32_t *planes,
                      uint16_t *scales, int32_t *status, int force_serial, hipStream_t st) {
    return group_size ? launch_cpwg<WAVES, CPW, true>(W, out, in, K, planes, scales, status,
                                                      force_serial, st)
                      : launch_cpwg<WAVES, CPW, false>(W, out, in, K, planes, scales, status,
                                                       force_serial, st);
}

}  // namespace

hipError_t launch_encode(const float *W, int out, int in, int K, int group_size,
                         uint32_t *planes, uint16_t *scales, int32_t *status, int force_serial,
                         hipStream_t st) {
    // Rows of up to 4096 columns: 4 waves; longer rows: 16 waves, so that each
    // lane keeps at most 2 x 32 values of two rows in registers.
    const int chunks = (in + RBQ_WAVE - 1) / RBQ_WAVE;
    const int waves = chunks <= 64 ? 4 : 16;
    const int need = (chunks + waves - 1) / waves;
#define RBQ_ENC_CASE(WV, C)                                                              \
    if (waves == WV && need <= C)                                                        \
        return launch_cpw<WV, C>(W, out, in, K, group_size, planes, scales, status,       \
                                 force_serial, st);
    RBQ_ENC_CASE(4, 2)
    RBQ_ENC_CASE(4, 4)
    RBQ_ENC_CASE(4, 8)
    RBQ_ENC_CASE(4, 16)
    RBQ_ENC_CASE(16, 6)
    RBQ_ENC_CASE(16, 8)
    RBQ_ENC_CASE(16, 12)
    RBQ_ENC_CASE(16, 16)
    RBQ_ENC_CASE(16, 24)
    RBQ_ENC_CASE(16, 32)
#undef RBQ_ENC_CASE
    return hipErrorInvalidValue;
}

}  // namespace rbq
