// encode_dual.hip -- residual binarization with two scale vectors per path.
//
// Path k is diag(g_k) B_k diag(h_k) ("RaBiT" summary, paperlayer.ai,
// section 4.1: binary cores with per-channel scaling vectors).  Its scales
// come from a residual SVID (section 4.3 and "RaBiT initialization";
// Tmax = 20 SVID iterations in "Training configuration"), without the
// calibration-data preconditioning:
//   B_k = sign(R_{k-1})   (R_0 = W; sign(0) = +1, also for -0.0)
//   |R_{k-1}| ~ u v^T by 20 alternating least-squares steps from v = 1:
//       u = |R| v / (v.v),  v = |R|^T u / (u.u)
//   c = sqrt(||u|| / ||v||), g_k = fp16(u / c), h_k = fp16(v c)  (one rounding)
//   R_k = R_{k-1} - (bit ? 1 : -1) g_k[r] h_k[j]   in fp32 (the product of two
//       binary16 values is exact in fp32, so this rounds once)
//
// Kernels per path: `svid_pass` (u for every row and per-workgroup partial
// sums of |R|^T u and of u.u), `svid_reduce` (v from the partials, one
// workgroup per 64 columns), 20 times; then
// `svid_finish` (balance and round) and `svid_update` (signs into plane
// words, next residual).  All sums are fp64 in a fixed order, so the result
// is deterministic for a given device; it differs from other summation
// orders only in the last bits of fp64, which survive the fp16 rounding
// only for a value within ~1e-13 of an fp16 rounding boundary.
//
// Workspace (rbq_encode_dual_workspace_bytes): R fp32 [out][in], u [out],
// v [in], column partials [in/64][SV_G][64] (each workgroup writes 64
// consecutive columns per wave store) and u.u partials [SV_G], all fp64 but
// R, each at a 256-byte boundary.
#include "rbq.h"
#include "rbq_device.h"
#include "rbq_kernels.h"

namespace rbq {

namespace {

constexpr int SVID_ITERS = 20;
constexpr int SV_THREADS = 1024;                 // pass kernel: 16 waves
constexpr int SV_WAVES = SV_THREADS / RBQ_WAVE;
constexpr int SV_G = 256;                        // pass workgroups (fixed: the partials' count)
constexpr int SV_RB = 256;                       // reduce / finish / update block

struct Ws {
    float *R;
    double *u, *v, *vpart, *upart;
};

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

inline Ws carve(void *base, int out, int in) {
    char *p = (char *)base;
    Ws w;
    w.R = (float *)p;          p += align256((size_t)out * in * 4);
    w.u = (double *)p;         p += align256((size_t)out * 8);
    w.v = (double *)p;         p += align256((size_t)in * 8);
    w.vpart = (double *)p;     p += align256((size_t)SV_G * in * 8);
    w.upart = (double *)p;
    return w;
}

// Sum over the wave, the same value in every lane (each butterfly step adds
// the same two values in both lanes of a pair).
__device__ __forceinline__ double wave_sum_f64_shfl(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, RBQ_WAVE);
    return v;
}

// Sum over a workgroup of NW waves in wave order, returned to every thread.
template <int NW>
__device__ __forceinline__ double block_sum_f64(double v, double *red) {
    v = wave_sum_f64_shfl(v);
    if ((threadIdx.x & (RBQ_WAVE - 1)) == 0)
        red[threadIdx.x / RBQ_WAVE] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        s += red[w];
    return s;
}

// v = 1 before the first pass.
__global__ __launch_bounds__(SV_RB) void svid_init(double *__restrict__ v, int in) {
    const int j = blockIdx.x * SV_RB + threadIdx.x;
    if (j < in)
        v[j] = 1.0;
}

// u_r = sum_j |R_rj| v_j / (v.v) for the rows of workgroup b, RPI at a
// time (rows b RPI .. b RPI + RPI - 1, then SV_G RPI further on): their
// loads are in flight together and one barrier serves all of them.
// Workgroup b also sums |R_rj| u_r over its rows per column, and u_r^2, in
// row order.
template <int CPT, int RPI>
__global__ __launch_bounds__(SV_THREADS) void svid_pass(const float *__restrict__ R, int out, int in,
                                                        const double *__restrict__ v, double *__restrict__ u,
                                                        double *__restrict__ vpart, double *__restrict__ upart) {
    __shared__ double red[2][RPI][SV_WAVES];
    __shared__ double red_vv[SV_WAVES];
    __shared__ double vsh[CPT * SV_THREADS];    // v, read once per row from LDS
    const int t = threadIdx.x;
    const int lane = t & (RBQ_WAVE - 1), wave = t / RBQ_WAVE;
    double acc[CPT];
    double vv = 0.0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = t + SV_THREADS * i;
        const double vj = (j < in) ? v[j] : 0.0;
        vsh[j] = vj;
        vv += vj * vj;
        acc[i] = 0.0;
    }
    vv = block_sum_f64<SV_WAVES>(vv, red_vv);    // also makes vsh visible
    double uu = 0.0;
    int phase = 0;
    for (int r0 = blockIdx.x * RPI; r0 < out; r0 += SV_G * RPI) {
        float a[RPI][CPT];
#pragma unroll
        for (int q = 0; q < RPI; ++q) {
            // a uniform row address plus 32-bit column offsets: no 64-bit
            // address per load kept in registers
            const float *rowp = R + (size_t)min(r0 + q, out - 1) * in;
            const bool live = r0 + q < out;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const unsigned j = (unsigned)t + SV_THREADS * i;
                const float x = rowp[min(j, (unsigned)in - 1u)];
                a[q][i] = (live && j < (unsigned)in) ? __builtin_fabsf(x) : 0.0f;
            }
        }
        const int b = phase & 1;
        ++phase;
#pragma unroll
        for (int q = 0; q < RPI; ++q) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                s += (double)a[q][i] * vsh[t + SV_THREADS * i];
            s = wave_sum_f64_dpp(s);
            if (lane == 0)
                red[b][q][wave] = s;
        }
        __syncthreads();
        // row q's sum over the 16 waves: lane 16q' + w reads wave w's share
        // of row qq + q', each row of 16 lanes adds them in wave order, and
        // lane 16q' + 15 holds the total (the same in every wave)
        double S[RPI];
#pragma unroll
        for (int qq = 0; qq < RPI; qq += 4) {
            const int q = qq + (lane >> 4);
            const double p = (q < RPI) ? red[b][q < RPI ? q : 0][lane & 15] : 0.0;
            const double rs = row16_sum_f64_dpp(p);
#pragma unroll
            for (int d = 0; d < 4 && qq + d < RPI; ++d)
                S[qq + d] = __longlong_as_double((long long)(
                    ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                         (int)(uint32_t)((uint64_t)__double_as_longlong(rs) >> 32), 16 * d + 15) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(rs), 16 * d + 15)));
        }
        // keep the loaded values as fp32 across the barrier (their fp64
        // conversions are not shared between the two sums: twice the
        // registers)
#pragma unroll
        for (int q = 0; q < RPI; ++q)
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                asm volatile("" : "+v"(a[q][i]));
#pragma unroll
        for (int q = 0; q < RPI; ++q) {
            const double ur = (vv > 0.0) ? S[q] / vv : 0.0;   // rows past the end: 0
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                acc[i] += (double)a[q][i] * ur;
            if (t == 0 && r0 + q < out) {
                u[r0 + q] = ur;
                uu += ur * ur;
            }
        }
    }
    // partials [in/64][SV_G][64]: a wave stores 64 consecutive columns
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = t + SV_THREADS * i;
        if (j < in)
            vpart[((size_t)(j >> 6) * SV_G + blockIdx.x) * 64 + (j & 63)] = acc[i];
    }
    if (t == 0)
        upart[blockIdx.x] = uu;
}

// v_j = (sum over workgroups of the partials, in workgroup order) / (u.u):
// one workgroup per 64 columns, wave w adding workgroups [64w, 64w + 64)
// for lane j, then wave 0 adding the four waves' sums in order.
__global__ __launch_bounds__(SV_RB) void svid_reduce(const double *__restrict__ vpart,
                                                      const double *__restrict__ upart, int groups, int in,
                                                      double *__restrict__ v) {
    static_assert(SV_G == 4 * RBQ_WAVE && SV_RB == 4 * RBQ_WAVE, "four waves of 64 workgroups");
    __shared__ double part[4][RBQ_WAVE];
    const int lane = threadIdx.x & (RBQ_WAVE - 1), wave = threadIdx.x / RBQ_WAVE;
    const double *p = vpart + (size_t)blockIdx.x * SV_G * 64 + lane;
    double s = 0.0;
    const int b0 = wave * RBQ_WAVE;
    const int nb = min(RBQ_WAVE, groups - b0);          // may be <= 0
#pragma unroll 16
    for (int b = 0; b < nb; ++b)
        s += p[(size_t)(b0 + b) * 64];
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0) {
        // u.u: lane l adds workgroups l, l + 64, l + 128, l + 192, then the wave
        double uu = 0.0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int b = lane + RBQ_WAVE * m;
            uu += (b < groups) ? upart[b] : 0.0;
        }
        uu = wave_sum_f64_shfl(uu);
        const double t = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        const int j = blockIdx.x * 64 + lane;
        if (j < in)
            v[j] = (uu > 0.0) ? t / uu : 0.0;
    }
}

// Balanced scales, one rounding each: g = fp16(u / c), h = fp16(v c),
// c = sqrt(||u|| / ||v||); zero when either vector is zero.
__global__ __launch_bounds__(SV_RB) void svid_finish(const double *__restrict__ u, const double *__restrict__ v,
                                                      const double *__restrict__ upart, int groups, int out,
                                                      int in, uint16_t *__restrict__ g, uint16_t *__restrict__ h,
                                                      int32_t *__restrict__ status) {
    __shared__ double red_u[SV_RB / RBQ_WAVE], red_v[SV_RB / RBQ_WAVE];
    const double uu = block_sum_f64<SV_RB / RBQ_WAVE>(
        (int)threadIdx.x < groups ? upart[threadIdx.x] : 0.0, red_u);
    double vs = 0.0;
    for (int j = threadIdx.x; j < in; j += SV_RB)
        vs += v[j] * v[j];
    const double vv = block_sum_f64<SV_RB / RBQ_WAVE>(vs, red_v);
    const double nu = sqrt(uu), nv = sqrt(vv);
    const bool zero = !(nu > 0.0) || !(nv > 0.0);
    const double c = zero ? 1.0 : sqrt(nu / nv);
    const int i = blockIdx.x * SV_RB + threadIdx.x;
    bool inf = false;
    if (i < out) {
        const uint16_t b = zero ? (uint16_t)0 : f64_to_f16_rne(u[i] / c);
        g[i] = b;
        inf |= (b & 0x7FFFu) == 0x7C00u;
    }
    if (i < in) {
        const uint16_t b = zero ? (uint16_t)0 : f64_to_f16_rne(v[i] * c);
        h[i] = b;
        inf |= (b & 0x7FFFu) == 0x7C00u;
    }
    if (status != nullptr && __any(inf) && (threadIdx.x & (RBQ_WAVE - 1)) == 0)
        atomicOr(status, (int32_t)RBQ_STATUS_SCALE_OVERFLOW);
}

// Signs of R into plane words (a wave covers 64 consecutive columns of one
// row: its ballot is two words) and, unless LAST, the next residual.
template <bool LAST>
__global__ __launch_bounds__(SV_RB) void svid_update(const float *__restrict__ Rin, float *__restrict__ Rout,
                                                      int out, int in, const uint16_t *__restrict__ g,
                                                      const uint16_t *__restrict__ h, uint32_t *__restrict__ plane,
                                                      int32_t *__restrict__ status, int check) {
    const size_t e = (size_t)blockIdx.x * SV_RB + threadIdx.x;
    const size_t total = (size_t)out * in;
    const int lane = threadIdx.x & (RBQ_WAVE - 1);
    const bool live = e < total;              // whole waves: total % 64 == 0
    const int r = live ? (int)(e / in) : 0;
    const int j = live ? (int)(e - (size_t)r * in) : 0;
    const float x = live ? Rin[e] : 0.0f;
    const bool plus = x >= 0.0f;
    const uint64_t m = __ballot(plus);
    if (live && lane < 2)   // lane l: word 2q + l of the wave's 64 columns [64q, 64q + 64)
        plane[(e - lane) / 32 + lane] = (uint32_t)(m >> (32 * lane));
    if (check && status != nullptr && __any(live && !__builtin_isfinite(x)) && lane == 0)
        atomicOr(status, (int32_t)RBQ_STATUS_NONFINITE_W);
    if constexpr (!LAST) {
        if (live) {
            const float a = h2f(g[r]) * h2f(h[j]);   // exact
            Rout[e] = x - (plus ? a : -a);
        }
    }
}

}  // namespace

size_t encode_dual_workspace_bytes(int out, int in) {
    if (out <= 0 || in <= 0)
        return 0;
    return align256((size_t)out * in * 4) + align256((size_t)out * 8) + align256((size_t)in * 8) +
           align256((size_t)SV_G * in * 8) + align256((size_t)SV_G * 8);
}

hipError_t launch_encode_dual(const float *W, int out, int in, int K, uint32_t *planes, uint16_t *g, uint16_t *h,
                              void *workspace, int32_t *status, hipStream_t st) {
    if (out <= 0 || in <= 0 || in % 128 != 0 || in > RBQ_DUAL_MAX_IN || K < 1 || K > 8)
        return hipErrorInvalidValue;
    const Ws w = carve(workspace, out, in);
    const int nvb = (in + SV_RB - 1) / SV_RB;
    // columns per thread (4, 8, 12 or 16) and rows per barrier (8, 4, 3, 2)
    const int cpt = (in + SV_THREADS - 1) / SV_THREADS;
    const int rpi = cpt <= 4 ? 8 : cpt <= 8 ? 4 : cpt <= 12 ? 3 : 2;
    auto pass = cpt <= 4 ? svid_pass<4, 8> : cpt <= 8 ? svid_pass<8, 4> : cpt <= 12 ? svid_pass<12, 3>
                                                                              : svid_pass<16, 2>;
    const int row_blocks = (out + rpi - 1) / rpi;
    const int groups = row_blocks < SV_G ? row_blocks : SV_G;
    const size_t words = (size_t)out * (in / 32);
    const size_t total = (size_t)out * in;
    const unsigned upd_blocks = (unsigned)((total + SV_RB - 1) / SV_RB);
    const unsigned fin_blocks = (unsigned)(((out > in ? out : in) + SV_RB - 1) / SV_RB);
    for (int k = 0; k < K; ++k) {
        const float *Rk = (k == 0) ? W : w.R;
        hipLaunchKernelGGL(svid_init, dim3(nvb), dim3(SV_RB), 0, st, w.v, in);
        for (int it = 0; it < SVID_ITERS; ++it) {
            hipLaunchKernelGGL(pass, dim3(groups), dim3(SV_THREADS), 0, st, Rk, out, in, (const double *)w.v,
                               w.u, w.vpart, w.upart);
            hipLaunchKernelGGL(svid_reduce, dim3(in / 64), dim3(SV_RB), 0, st, (const double *)w.vpart,
                               (const double *)w.upart, groups, in, w.v);
        }
        uint16_t *gk = g + (size_t)k * out, *hk = h + (size_t)k * in;
        hipLaunchKernelGGL(svid_finish, dim3(fin_blocks), dim3(SV_RB), 0, st, (const double *)w.u,
                           (const double *)w.v, (const double *)w.upart, groups, out, in, gk, hk, status);
        uint32_t *pk = planes + (size_t)k * words;
        if (k + 1 < K)
            hipLaunchKernelGGL(svid_update<false>, dim3(upd_blocks), dim3(SV_RB), 0, st, Rk, w.R, out, in,
                               (const uint16_t *)gk, (const uint16_t *)hk, pk, status, k == 0 ? 1 : 0);
        else
            hipLaunchKernelGGL(svid_update<true>, dim3(upd_blocks), dim3(SV_RB), 0, st, Rk, w.R, out, in,
                               (const uint16_t *)gk, (const uint16_t *)hk, pk, status, k == 0 ? 1 : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace rbq
