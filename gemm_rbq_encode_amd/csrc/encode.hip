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
// or a mean within ~1e-11 of an fp16 rounding boundary -- one lane redoes
// the serial sum, rebuilding each R_j from W and the scales already chosen,
// and divides with a correctly rounded division.  Residuals are updated in
// fp32 with one rounding, exactly as the definition states.
//
// Layout.  One workgroup (4 or 16 waves) per row; the row is cut into 64-column
// chunks and wave w keeps chunks [w*CPW, (w+1)*CPW) in registers, lane l
// holding column 64c + l of chunk c.  Loads are therefore coalesced 256-byte
// wave reads, a wave ballot of (R >= 0) is exactly the two packed words of a
// chunk, and a 128-column group is a chunk pair inside one wave.  W is read
// from HBM once; the K steps run on registers.
#include "rbq_device.h"
#include "rbq_kernels.h"

#pragma clang fp contract(off)

namespace rbq {

namespace {

constexpr uint32_t UNDECIDED = 0xFFFFFFFFu;

// fp16 bits of the mean when the error bound decides it, else UNDECIDED.
__device__ __forceinline__ uint32_t decide_scale(double S, int n) {
    const double nd = (double)n;
    const double m = S / nd;
    const double rel = (2.0 * nd + 64.0) * 0x1p-53;
    const double d = m * rel;
    const uint16_t hl = f64_to_f16_rne(m - d);
    const uint16_t hh = f64_to_f16_rne(m + d);
    return (hl == hh) ? (uint32_t)hl : UNDECIDED;
}

// The defining serial computation for columns [c0, c0+n) at step k: rebuild
// R_{k-1} of each column from W and the k earlier scales (hist[l*stride]),
// sum |R| in ascending order in fp64, divide (correctly rounded), round once.
__device__ __attribute__((noinline)) uint16_t serial_scale(const float *__restrict__ Wr, int c0,
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

template <int WAVES, int CPW>
__global__ __launch_bounds__(WAVES * RBQ_WAVE) void encode_kernel(
    const float *__restrict__ W, int out, int in, int K, int group_size,
    uint32_t *__restrict__ planes, uint16_t *__restrict__ scales, int32_t *__restrict__ status,
    int force_serial) {
    static_assert(CPW % 2 == 0, "a 128-column group must be a chunk pair of one wave");
    constexpr int GPW = CPW / 2;  // 128-column groups per wave

    __shared__ double part[2][WAVES];
    __shared__ float hist_row[8];
    __shared__ uint32_t decided_row;
    __shared__ float hist_grp[WAVES][8][GPW];

    const int r = blockIdx.x;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const int wave = threadIdx.x / RBQ_WAVE;
    const int words = in >> 5;
    const int G = group_size ? in / group_size : 1;
    const float *Wr = W + (size_t)r * in;
    const int chunk0 = wave * CPW;

    float R[CPW];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int col = (chunk0 + i) * RBQ_WAVE + lane;
        R[i] = (col < in) ? Wr[col] : 0.0f;
        bad |= !__builtin_isfinite(R[i]);
    }
    if (status != nullptr && __any(bad) && lane == 0)
        atomicOr(status, (int32_t)1);

    for (int k = 0; k < K; ++k) {
        float a_row = 0.0f;
        float a_grp[GPW];
        if (group_size == 0) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int col = (chunk0 + i) * RBQ_WAVE + lane;
                if (col < in)
                    s += (double)__builtin_fabsf(R[i]);
            }
            s = wave_sum_f64(s);
            if (lane == 0)
                part[k & 1][wave] = s;
            __syncthreads();
            double S = part[k & 1][0];
#pragma unroll
            for (int v = 1; v < WAVES; ++v)
                S += part[k & 1][v];
            uint32_t h = force_serial ? UNDECIDED : decide_scale(S, in);
            if (h == UNDECIDED) {  // same decision in every thread of the block
                if (threadIdx.x == 0)
                    decided_row = serial_scale(Wr, 0, in, hist_row, 1, k);
                __syncthreads();
                h = decided_row;
            }
            a_row = h2f((uint16_t)h);
            if (threadIdx.x == 0) {
                hist_row[k] = a_row;
                scales[(size_t)k * out + r] = (uint16_t)h;
                if (status != nullptr && (h & 0x7FFFu) == 0x7C00u)
                    atomicOr(status, (int32_t)2);
            }
        } else {
#pragma unroll
            for (int g = 0; g < GPW; ++g) {
                const int col0 = (chunk0 + 2 * g) * RBQ_WAVE;  // group start (in % 128 == 0)
                const bool gvalid = col0 < in;
                double s = gvalid ? (double)__builtin_fabsf(R[2 * g]) +
                                        (double)__builtin_fabsf(R[2 * g + 1])
                                  : 0.0;
                s = wave_sum_f64(s);
                s = __shfl(s, 0, RBQ_WAVE);  // one value for the whole wave
                uint32_t h = force_serial ? UNDECIDED : decide_scale(s, 128);
                if (h == UNDECIDED && gvalid) {  // uniform in the wave
                    uint32_t hs = 0;
                    if (lane == 0)
                        hs = serial_scale(Wr, col0, 128, &hist_grp[wave][0][g], GPW, k);
                    h = __shfl(hs, 0, RBQ_WAVE);
                }
                a_grp[g] = gvalid ? h2f((uint16_t)h) : 0.0f;
                if (lane == 0 && gvalid) {
                    hist_grp[wave][k][g] = a_grp[g];
                    scales[((size_t)k * out + r) * G + (col0 >> 7)] = (uint16_t)h;
                    if (status != nullptr && (h & 0x7FFFu) == 0x7C00u)
                        atomicOr(status, (int32_t)2);
                }
            }
        }

        // signs, packed words and the residual update
        uint32_t wv[(2 * CPW + RBQ_WAVE - 1) / RBQ_WAVE];
#pragma unroll
        for (int q = 0; q < (2 * CPW + RBQ_WAVE - 1) / RBQ_WAVE; ++q)
            wv[q] = 0;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int col = (chunk0 + i) * RBQ_WAVE + lane;
            const bool valid = col < in;
            const bool plus = valid && (R[i] >= 0.0f);
            const uint64_t m = __ballot(plus);
            const float a = (group_size == 0) ? a_row : a_grp[i / 2];
            if (valid)
                R[i] = R[i] - (plus ? a : -a);
            const int w0 = (2 * i) % RBQ_WAVE, q = (2 * i) / RBQ_WAVE;
            if (lane == w0)
                wv[q] = (uint32_t)m;
            if (lane == w0 + 1)
                wv[q] = (uint32_t)(m >> 32);
        }
        uint32_t *prow = planes + ((size_t)k * out + r) * words;
#pragma unroll
        for (int q = 0; q < (2 * CPW + RBQ_WAVE - 1) / RBQ_WAVE; ++q) {
            const int idx = chunk0 * 2 + q * RBQ_WAVE + lane;
            if (q * RBQ_WAVE + lane < 2 * CPW && idx < words)
                prow[idx] = wv[q];
        }
    }
}

template <int WAVES, int CPW>
hipError_t launch_cpw(const float *W, int out, int in, int K, int group_size, uint32_t *planes,
                      uint16_t *scales, int32_t *status, int force_serial, hipStream_t st) {
    hipLaunchKernelGGL((encode_kernel<WAVES, CPW>), dim3(out), dim3(WAVES * RBQ_WAVE), 0, st, W,
                       out, in, K, group_size, planes, scales, status, force_serial);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const float *W, int out, int in, int K, int group_size,
                         uint32_t *planes, uint16_t *scales, int32_t *status, int force_serial,
                         hipStream_t st) {
    // Rows of up to 4096 columns: 4 waves; longer rows: 16 waves, so that each
    // lane keeps at most 32 values of the row in registers.
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
