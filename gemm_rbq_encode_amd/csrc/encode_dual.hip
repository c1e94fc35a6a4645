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
// sums of |R|^T u and of u.u), `svid_reduce` (v from the partials, added in
// workgroup order, and per-block partial sums of v.v), 20 times; then
// `svid_finish` (balance and round) and `svid_update` (signs into plane
// words, next residual).  All sums are fp64 in a fixed order, so the result
// is deterministic for a given device; it differs from other summation
// orders only in the last bits of fp64, which survive the fp16 rounding
// only for a value within ~1e-13 of an fp16 rounding boundary.
//
// Workspace (rbq_encode_dual_workspace_bytes): R fp32 [out][in], u [out],
// v [in], column partials [SV_G][in], u.u partials [SV_G], v.v partials
// [ceil(in / 256)], all fp64 but R, each at a 256-byte boundary.
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
    double *u, *v, *vpart, *upart, *vvpart;
};

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

inline Ws carve(void *base, int out, int in) {
    char *p = (char *)base;
    Ws w;
    w.R = (float *)p;          p += align256((size_t)out * in * 4);
    w.u = (double *)p;         p += align256((size_t)out * 8);
    w.v = (double *)p;         p += align256((size_t)in * 8);
    w.vpart = (double *)p;     p += align256((size_t)SV_G * in * 8);
    w.upart = (double *)p;     p += align256((size_t)SV_G * 8);
    w.vvpart = (double *)p;
    return w;
}

__device__ __forceinline__ double wave_sum_f64_shfl(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, RBQ_WAVE);
    return v;
}

// v = 1 (and v.v = in) before the first pass.
__global__ __launch_bounds__(SV_RB) void svid_init(double *__restrict__ v, double *__restrict__ vvpart, int in,
                                                    int nvb) {
    const int j = blockIdx.x * SV_RB + threadIdx.x;
    if (j < in)
        v[j] = 1.0;
    if (j < nvb)
        vvpart[j] = (j == 0) ? (double)in : 0.0;
}

// u_r = sum_j |R_rj| v_j / (v.v) for rows r = b, b + SV_G, ...; workgroup b
// also sums |R_rj| u_r over its rows per column, and u_r^2.
template <int CPT>
__global__ __launch_bounds__(SV_THREADS) void svid_pass(const float *__restrict__ R, int out, int in,
                                                        const double *__restrict__ v,
                                                        const double *__restrict__ vvpart, int nvb,
                                                        double *__restrict__ u, double *__restrict__ vpart,
                                                        double *__restrict__ upart) {
    __shared__ double red[2][SV_WAVES];
    const int t = threadIdx.x;
    const int lane = t & (RBQ_WAVE - 1), wave = t / RBQ_WAVE;
    double vv = 0.0;
    for (int i = 0; i < nvb; ++i)
        vv += vvpart[i];
    double vj[CPT], acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = t + SV_THREADS * i;
        vj[i] = (j < in) ? v[j] : 0.0;
        acc[i] = 0.0;
    }
    double uu = 0.0;
    float a[CPT], an[CPT];
    auto load = [&](float(&dst)[CPT], int r) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int j = t + SV_THREADS * i;
            dst[i] = (j < in) ? __builtin_fabsf(R[(size_t)r * in + j]) : 0.0f;
        }
    };
    int phase = 0;
    if (blockIdx.x < out)
        load(a, blockIdx.x);
    for (int r = blockIdx.x; r < out; r += SV_G) {
        const bool more = r + SV_G < out;
        if (more)
            load(an, r + SV_G);
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            s += (double)a[i] * vj[i];
        s = wave_sum_f64_shfl(s);
        const int b = phase & 1;
        ++phase;
        if (lane == 0)
            red[b][wave] = s;
        __syncthreads();
        double S = 0.0;
#pragma unroll
        for (int w = 0; w < SV_WAVES; ++w)
            S += red[b][w];
        const double ur = (vv > 0.0) ? S / vv : 0.0;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            acc[i] += (double)a[i] * ur;
        if (t == 0) {
            u[r] = ur;
            uu += ur * ur;
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                a[i] = an[i];
        }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = t + SV_THREADS * i;
        if (j < in)
            vpart[(size_t)blockIdx.x * in + j] = acc[i];
    }
    if (t == 0)
        upart[blockIdx.x] = uu;
}

// v_j = (sum over workgroups of the partials, in order) / (u.u); per block
// of columns, the sum of v_j^2.
__global__ __launch_bounds__(SV_RB) void svid_reduce(const double *__restrict__ vpart,
                                                      const double *__restrict__ upart, int groups, int in,
                                                      double *__restrict__ v, double *__restrict__ vvpart) {
    __shared__ double red[SV_RB / RBQ_WAVE];
    const int j = blockIdx.x * SV_RB + threadIdx.x;
    double uu = 0.0;
    for (int b = 0; b < groups; ++b)
        uu += upart[b];
    double vj = 0.0;
    if (j < in) {
        double s = 0.0;
        for (int b = 0; b < groups; ++b)
            s += vpart[(size_t)b * in + j];
        vj = (uu > 0.0) ? s / uu : 0.0;
        v[j] = vj;
    }
    const double w = wave_sum_f64_shfl(vj * vj);
    if ((threadIdx.x & (RBQ_WAVE - 1)) == 0)
        red[threadIdx.x / RBQ_WAVE] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < SV_RB / RBQ_WAVE; ++i)
            s += red[i];
        vvpart[blockIdx.x] = s;
    }
}

// Balanced scales, one rounding each: g = fp16(u / c), h = fp16(v c),
// c = sqrt(||u|| / ||v||); zero when either vector is zero.
__global__ __launch_bounds__(SV_RB) void svid_finish(const double *__restrict__ u, const double *__restrict__ v,
                                                      const double *__restrict__ upart, int groups,
                                                      const double *__restrict__ vvpart, int nvb, int out,
                                                      int in, uint16_t *__restrict__ g, uint16_t *__restrict__ h) {
    double uu = 0.0, vv = 0.0;
    for (int b = 0; b < groups; ++b)
        uu += upart[b];
    for (int b = 0; b < nvb; ++b)
        vv += vvpart[b];
    const double nu = sqrt(uu), nv = sqrt(vv);
    const bool zero = !(nu > 0.0) || !(nv > 0.0);
    const double c = zero ? 1.0 : sqrt(nu / nv);
    const int i = blockIdx.x * SV_RB + threadIdx.x;
    if (i < out)
        g[i] = zero ? (uint16_t)0 : f64_to_f16_rne(u[i] / c);
    if (i < in)
        h[i] = zero ? (uint16_t)0 : f64_to_f16_rne(v[i] * c);
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
    const int nvb = (in + SV_RB - 1) / SV_RB;
    return align256((size_t)out * in * 4) + align256((size_t)out * 8) + align256((size_t)in * 8) +
           align256((size_t)SV_G * in * 8) + align256((size_t)SV_G * 8) + align256((size_t)nvb * 8);
}

hipError_t launch_encode_dual(const float *W, int out, int in, int K, uint32_t *planes, uint16_t *g, uint16_t *h,
                              void *workspace, int32_t *status, hipStream_t st) {
    if (out <= 0 || in <= 0 || in % 128 != 0 || in > RBQ_DUAL_MAX_IN || K < 1 || K > 8)
        return hipErrorInvalidValue;
    const Ws w = carve(workspace, out, in);
    const int nvb = (in + SV_RB - 1) / SV_RB;
    const int groups = out < SV_G ? out : SV_G;
    const size_t words = (size_t)out * (in / 32);
    const size_t total = (size_t)out * in;
    const unsigned upd_blocks = (unsigned)((total + SV_RB - 1) / SV_RB);
    const unsigned fin_blocks = (unsigned)(((out > in ? out : in) + SV_RB - 1) / SV_RB);
    for (int k = 0; k < K; ++k) {
        const float *Rk = (k == 0) ? W : w.R;
        hipLaunchKernelGGL(svid_init, dim3(nvb), dim3(SV_RB), 0, st, w.v, w.vvpart, in, nvb);
        for (int it = 0; it < SVID_ITERS; ++it) {
            // columns per thread: 4, 8, 12 or 16
            const int cpt = (in + SV_THREADS - 1) / SV_THREADS;
            auto pass = cpt <= 4 ? svid_pass<4> : cpt <= 8 ? svid_pass<8> : cpt <= 12 ? svid_pass<12> : svid_pass<16>;
            hipLaunchKernelGGL(pass, dim3(groups), dim3(SV_THREADS), 0, st, Rk, out, in,
                               (const double *)w.v, (const double *)w.vvpart, nvb, w.u, w.vpart, w.upart);
            hipLaunchKernelGGL(svid_reduce, dim3(nvb), dim3(SV_RB), 0, st, (const double *)w.vpart,
                               (const double *)w.upart, groups, in, w.v, w.vvpart);
        }
        uint16_t *gk = g + (size_t)k * out, *hk = h + (size_t)k * in;
        hipLaunchKernelGGL(svid_finish, dim3(fin_blocks), dim3(SV_RB), 0, st, (const double *)w.u,
                           (const double *)w.v, (const double *)w.upart, groups, (const double *)w.vvpart, nvb,
                           out, in, gk, hk);
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
