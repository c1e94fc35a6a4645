// rbq_device.h -- device helpers shared by the librbq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define RBQ_WAVE 64

namespace rbq {

// binary16 bits -> float (exact).
__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// SiLU (sigmoid-weighted linear unit) v / (1 + e^-v) in fp32, for the
// gate of a gated MLP: the gate/up epilogue writes silu(gate) * up.
__device__ __forceinline__ float silu_f32(float v) {
    return v / (1.0f + expf(-v));
}

// float -> binary16 bits, rounded to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// double -> binary16 bits with ONE rounding to nearest, ties to even,
// computed on the integer bit pattern (never through fp32).  Subnormal
// results are kept; values at or beyond 65520 become infinity.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double v) {
    uint64_t b = (uint64_t)__double_as_longlong(v);
    uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
    int e = (int)(mag >> 52);
    uint64_t frac = mag & 0x000FFFFFFFFFFFFFull;
    if (e == 0x7FF)
        return (uint16_t)(sign | (frac ? 0x7E00u : 0x7C00u));
    int E = e - 1023;                      // unbiased exponent (normal doubles)
    if (E >= 16)
        return (uint16_t)(sign | 0x7C00u);
    if (E < -25)                           // below 2^-25: rounds to zero
        return (uint16_t)sign;
    uint64_t sig = frac | (1ull << 52);    // value = sig * 2^(E-52)
    int qexp = (E < -14) ? -24 : E - 10;   // fp16 quantum in this binade
    int shift = 52 + qexp - E;             // 42 .. 53 bits dropped
    uint64_t n = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (n & 1)))
        ++n;
    uint32_t bits = (E < -14) ? (uint32_t)n
                              : ((uint32_t)(E + 15) << 10) + (uint32_t)n - 1024u;
    if (bits >= 0x7C00u)
        bits = 0x7C00u;
    return (uint16_t)(sign | bits);
}

// silu(gate) * up as binary16 bits, rounded once: the product of two fp32
// values is exact in fp64.  Every kernel with the gate/up epilogue writes
// through this, so none depends on whether the compiler fuses the product
// and the conversion into one mixed-precision fma (one rounding) or rounds
// to fp32 first (two).
__device__ __forceinline__ uint16_t silu_mul_f16(float gate, float up) {
    return f64_to_f16_rne((double)silu_f32(gate) * (double)up);
}

// Correctly rounded S / n in fp64 (n a positive integer), whatever the
// accuracy of the compiler's division sequence: the quotient is corrected by
// the exact remainder S - q n (an FMA) to the nearer neighbour, ties to even.
__device__ __forceinline__ double div_rn(double S, double n) {
    double q = S / n;
    double r0 = __fma_rn(-q, n, S);
    if (r0 == 0.0)
        return q;
    // q >= 0 here (S >= 0, n > 0); its neighbours are the adjacent bit patterns
    uint64_t bq0 = (uint64_t)__double_as_longlong(q);
    double q1 = __longlong_as_double((long long)((r0 > 0.0) ? bq0 + 1 : bq0 - 1));
    double r1 = __fma_rn(-q1, n, S);
    double a0 = __builtin_fabs(r0), a1 = __builtin_fabs(r1);
    if (a1 < a0)
        return q1;
    if (a1 == a0) {
        uint64_t bq = (uint64_t)__double_as_longlong(q);
        return (bq & 1) ? q1 : q;
    }
    return q;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, RBQ_WAVE);
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, RBQ_WAVE);
    return v;
}

}  // namespace rbq

namespace rbq {

// DPP controls (GFX9): row_shr:n, row_shl:n, row_bcast:15, row_bcast:31.
#define RBQ_DPP_ROW_SHR(n) (0x110 + (n))
#define RBQ_DPP_ROW_SHL(n) (0x100 + (n))
#define RBQ_DPP_ROW_BCAST15 0x142
#define RBQ_DPP_ROW_BCAST31 0x143

// Value of lane (lane + n) inside the same row of 16 lanes (n = 1 or 2);
// lanes whose source falls outside the row get 0.
template <int N>
__device__ __forceinline__ int row_shl_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_SHL(N), 0xF, 0xF, false);
}

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

// Sum of each row of 16 lanes, in lane 15 of that row (DPP row shifts; the
// same order in every row).
__device__ __forceinline__ double row16_sum_f64_dpp(double v) {
    v += dpp_f64<RBQ_DPP_ROW_SHR(1), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_SHR(2), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_SHR(4), 0xF>(v);
    v += dpp_f64<RBQ_DPP_ROW_SHR(8), 0xF>(v);
    return v;
}

// Whole-wave sum of an int, returned to every lane (DPP row shifts, row
// broadcasts, then lane 63).
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_SHR(1), 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_SHR(2), 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_SHR(4), 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_SHR(8), 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_BCAST15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, RBQ_DPP_ROW_BCAST31, 0xC, 0xF, false);
    return __builtin_amdgcn_readlane(v, 63);
}

template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_add_f32(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, x), CTRL, RMASK, 0xF, false));
}

// Whole-wave sum of a float, returned to every lane.
__device__ __forceinline__ float wave_sum_f32_dpp(float v) {
    v = dpp_add_f32<RBQ_DPP_ROW_SHR(1), 0xF>(v);
    v = dpp_add_f32<RBQ_DPP_ROW_SHR(2), 0xF>(v);
    v = dpp_add_f32<RBQ_DPP_ROW_SHR(4), 0xF>(v);
    v = dpp_add_f32<RBQ_DPP_ROW_SHR(8), 0xF>(v);
    v = dpp_add_f32<RBQ_DPP_ROW_BCAST15, 0xA>(v);
    v = dpp_add_f32<RBQ_DPP_ROW_BCAST31, 0xC>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Whole-wave maximum of an unsigned int, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
    int x = (int)v;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, RBQ_DPP_ROW_SHR(1), 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, RBQ_DPP_ROW_SHR(2), 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, RBQ_DPP_ROW_SHR(4), 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, RBQ_DPP_ROW_SHR(8), 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, RBQ_DPP_ROW_BCAST15, 0xA, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, RBQ_DPP_ROW_BCAST31, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

}  // namespace rbq
