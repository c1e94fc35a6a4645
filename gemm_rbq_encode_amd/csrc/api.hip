// api.hip -- the C ABI of librbq (include/rbq.h): argument checks, kernel
// selection and launches on the caller's stream.  No allocation happens
// here; every buffer belongs to the caller.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "rbq.h"
#include "rbq_kernels.h"

namespace {

thread_local int32_t g_last_hip_error = 0;
std::atomic<int> g_forced_path{RBQ_PATH_AUTO};
std::atomic<int> g_stream_split{0};

rbq_status hip_fail(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return RBQ_ERR_HIP;
}

rbq_status device_present() {
    static std::once_flag once;
    static int count = 0;
    std::call_once(once, [] {
        if (hipGetDeviceCount(&count) != hipSuccess)
            count = 0;
        (void)hipGetLastError();
    });
    return count > 0 ? RBQ_OK : RBQ_ERR_NO_DEVICE;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int groups_of(const rbq_shape &s) {
    return s.group_size ? s.in_features / s.group_size : 1;
}

}  // namespace

extern "C" {

rbq_status rbq_check_shape(rbq_shape s) {
    if (s.out_features < 0 || s.in_features < 0 || s.in_features % 32 != 0)
        return RBQ_ERR_INVALID_ARG;
    if (s.num_planes < 1 || s.num_planes > 8)
        return RBQ_ERR_INVALID_ARG;
    if (s.group_size != 0 && s.group_size != 128)
        return RBQ_ERR_INVALID_ARG;
    if (s.group_size == 128 && s.in_features % 128 != 0)
        return RBQ_ERR_INVALID_ARG;
    return RBQ_OK;
}

size_t rbq_planes_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK)
        return 0;
    return (size_t)s.num_planes * (size_t)s.out_features * (size_t)(s.in_features / 32) * 4u;
}

size_t rbq_scales_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK)
        return 0;
    if (s.in_features == 0)
        return 0;
    return (size_t)s.num_planes * (size_t)s.out_features * (size_t)groups_of(s) * 2u;
}

rbq_status rbq_encode_ex(const float *W, rbq_shape s, uint32_t *planes, uint16_t *scales,
                         int32_t *status_dev, uint32_t flags, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (flags & ~(uint32_t)RBQ_ENCODE_FORCE_SERIAL)
        return RBQ_ERR_INVALID_ARG;
    if (s.out_features == 0 || s.in_features == 0)
        return RBQ_OK;
    if (W == nullptr || planes == nullptr || scales == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(W, 4) || !aligned(planes, 4) || !aligned(scales, 2) ||
        (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    if (s.in_features > RBQ_ENCODE_MAX_IN)
        return RBQ_ERR_UNSUPPORTED;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_encode(W, s.out_features, s.in_features, s.num_planes,
                                      s.group_size, planes, scales, status_dev,
                                      (flags & RBQ_ENCODE_FORCE_SERIAL) ? 1 : 0,
                                      (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_encode(const float *W, rbq_shape s, uint32_t *planes, uint16_t *scales,
                      int32_t *status_dev, void *stream) {
    return rbq_encode_ex(W, s, planes, scales, status_dev, 0u, stream);
}

rbq_status rbq_refit(const float *W, rbq_shape s, const uint32_t *planes, uint16_t *scales,
                     int32_t *status_dev, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (s.out_features == 0 || s.in_features == 0)
        return RBQ_OK;
    if (W == nullptr || planes == nullptr || scales == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(W, 16) || !aligned(planes, 4) || !aligned(scales, 2) ||
        (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    if (s.in_features > RBQ_ENCODE_MAX_IN)
        return RBQ_ERR_UNSUPPORTED;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_refit(W, s.out_features, s.in_features, s.num_planes, s.group_size, planes,
                                     scales, status_dev, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_rebinarize(const float *W, rbq_shape s, uint32_t *planes, const uint16_t *scales,
                          int32_t *status_dev, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (s.out_features == 0 || s.in_features == 0)
        return RBQ_OK;
    if (W == nullptr || planes == nullptr || scales == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(W, 4) || !aligned(planes, 4) || !aligned(scales, 2) ||
        (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    if (s.num_planes > RBQ_REBIN_MAX_PLANES)
        return RBQ_ERR_UNSUPPORTED;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_rebinarize(W, s.out_features, s.in_features, s.num_planes, s.group_size, planes,
                                          scales, status_dev, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

size_t rbq_gemm_workspace_bytes(rbq_shape s, int32_t M) {
    if (rbq_check_shape(s) != RBQ_OK || M < 2)
        return 0;
    return rbq::split_workspace_bytes(s.out_features, s.in_features, s.num_planes, s.group_size, M);
}

rbq_path rbq_set_path(rbq_path p) {
    return (rbq_path)g_forced_path.exchange((int)p);
}

int32_t rbq_set_stream_split(int32_t waves_per_tile) {
    if (waves_per_tile != 0 && waves_per_tile != 1 && waves_per_tile != 2 && waves_per_tile != 4)
        return -1;
    return g_stream_split.exchange(waves_per_tile);
}

// The choice among the families that need no workspace.
static rbq_path select_path_no_workspace(rbq_shape s, int32_t M) {
    if (rbq::group_supports(s.out_features, s.in_features, s.num_planes, s.group_size, M))
        return RBQ_PATH_GROUP;
    if (rbq::flat_preferred(s.out_features, s.in_features, s.num_planes, s.group_size, M))
        return RBQ_PATH_FLAT;
    if (rbq::stream_supports(s.in_features, s.num_planes, s.group_size, M))
        return RBQ_PATH_STREAM;
    if (M <= 16 && rbq::decode_supports(s.in_features, s.num_planes, s.group_size, M))
        return RBQ_PATH_DECODE;
    if (M > 16 && rbq::prefill_supports(s.in_features, s.num_planes, s.group_size, M))
        return RBQ_PATH_PREFILL;
    return RBQ_PATH_VALU;
}

rbq_path rbq_select_path(rbq_shape s, int32_t M) {
    if (rbq::split_preferred(s.out_features, s.in_features, s.num_planes, s.group_size, M))
        return RBQ_PATH_SPLIT;
    return select_path_no_workspace(s, M);
}

}  // extern "C"

// rbq_gemm_ex and rbq_gemm_noalloc: argument checks, the kernel family, the
// launch.  `workspace` / `ws_bytes` is the caller's buffer or the static one.
static rbq_status gemm_impl(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                            const uint16_t *X, int32_t M, uint16_t *Y, void *workspace,
                            size_t ws_bytes, uint32_t epilogue, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (M < 0)
        return RBQ_ERR_INVALID_ARG;
    if (epilogue != RBQ_EPILOGUE_NONE && epilogue != RBQ_EPILOGUE_SILU_MUL)
        return RBQ_ERR_INVALID_ARG;
    const int silu = epilogue == RBQ_EPILOGUE_SILU_MUL;
    if (silu && s.out_features % 2 != 0)
        return RBQ_ERR_INVALID_ARG;
    const int64_t ycols = silu ? s.out_features / 2 : s.out_features;
    if (ws_bytes > 0 && workspace == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (M == 0 || s.out_features == 0)
        return RBQ_OK;
    if (Y == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(Y, 2))
        return RBQ_ERR_ALIGNMENT;
    hipStream_t hs = (hipStream_t)stream;
    if (s.in_features == 0) {  // empty sums: Y = 0
        if ((st = device_present()) != RBQ_OK)
            return st;
        hipError_t e = rbq::launch_fill_zero_u16(Y, (int64_t)M * ycols, hs);   // silu(0) * 0 = 0
        return e == hipSuccess ? RBQ_OK : hip_fail(e);
    }
    if (planes == nullptr || scales == nullptr || X == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(planes, 16) || !aligned(scales, 2) || !aligned(X, 16))
        return RBQ_ERR_ALIGNMENT;
    rbq_path path = (rbq_path)g_forced_path.load();
    const size_t ws_need = rbq_gemm_workspace_bytes(s, M);
    if (path == RBQ_PATH_AUTO) {
        path = rbq_select_path(s, M);
        if (path == RBQ_PATH_SPLIT && (ws_bytes < ws_need || !aligned(workspace, 4)))
            path = select_path_no_workspace(s, M);
        if (path == RBQ_PATH_GROUP && !aligned(scales, 8))   // the group kernel reads 4 scales at once
            path = RBQ_PATH_VALU;
        if (silu)   // the epilogue is built into the flat and VALU kernels
            path = rbq::flat_supports(s.out_features, s.in_features, s.num_planes, s.group_size, M)
                       ? RBQ_PATH_FLAT : RBQ_PATH_VALU;
    }
    if (silu && path != RBQ_PATH_FLAT && path != RBQ_PATH_VALU)
        return RBQ_ERR_UNSUPPORTED;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e;
    switch (path) {
    case RBQ_PATH_VALU:
        e = rbq::launch_gemm_valu(planes, scales, s.out_features, s.in_features, s.num_planes,
                                  s.group_size, X, M, Y, silu, hs);
        break;
    case RBQ_PATH_DECODE:
        if (!rbq::decode_supports(s.in_features, s.num_planes, s.group_size, M))
            return RBQ_ERR_UNSUPPORTED;
        e = rbq::launch_gemm_decode(planes, scales, s.out_features, s.in_features, s.num_planes,
                                    s.group_size, X, M, Y, hs);
        break;
    case RBQ_PATH_PREFILL:
        if (!rbq::prefill_supports(s.in_features, s.num_planes, s.group_size, M))
            return RBQ_ERR_UNSUPPORTED;
        e = rbq::launch_gemm_prefill(planes, scales, s.out_features, s.in_features, s.num_planes,
                                     s.group_size, X, M, Y, hs);
        break;
    case RBQ_PATH_STREAM:
        if (!rbq::stream_supports(s.in_features, s.num_planes, s.group_size, M))
            return RBQ_ERR_UNSUPPORTED;
        e = rbq::launch_gemm_stream(planes, scales, s.out_features, s.in_features, s.num_planes,
                                    s.group_size, X, M, Y, hs, g_stream_split.load());
        break;
    case RBQ_PATH_FLAT:
        if (!rbq::flat_supports(s.out_features, s.in_features, s.num_planes, s.group_size, M))
            return RBQ_ERR_UNSUPPORTED;
        e = rbq::launch_gemm_flat(planes, scales, s.out_features, s.in_features, s.num_planes,
                                  s.group_size, X, M, Y, silu, hs);
        break;
    case RBQ_PATH_SPLIT:
        if (!rbq::split_supports(s.out_features, s.in_features, s.num_planes, s.group_size, M))
            return RBQ_ERR_UNSUPPORTED;
        if (ws_bytes < ws_need)
            return RBQ_ERR_INVALID_ARG;
        if (!aligned(workspace, 4))
            return RBQ_ERR_ALIGNMENT;
        e = rbq::launch_gemm_split(planes, scales, s.out_features, s.in_features, s.num_planes,
                                   s.group_size, X, M, Y, workspace, ws_bytes, hs);
        break;
    case RBQ_PATH_GROUP:
        if (!rbq::group_supports(s.out_features, s.in_features, s.num_planes, s.group_size, M))
            return RBQ_ERR_UNSUPPORTED;
        if (!aligned(scales, 8))
            return RBQ_ERR_ALIGNMENT;
        e = rbq::launch_gemm_group(planes, scales, s.out_features, s.in_features, s.num_planes,
                                   s.group_size, X, M, Y, hs);
        break;
    default:
        return RBQ_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

// ---- the static scratch of rbq_gemm_noalloc ----------------------------------
// One copy per GPU, held until the process ends.  In host code `scratch` names
// a host-side stand-in, not the device array: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is passed to kernels.  Calls on one GPU share the array.
static __device__ __align__(256) unsigned char scratch[RBQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of `scratch` on the current device (nullptr and the
// HIP error on failure).
void *scratch_on_current_device(hipError_t *err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = r;
        g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
    });
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

rbq_status rbq_gemm_ex(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                       const uint16_t *X, int32_t M, uint16_t *Y, void *workspace,
                       size_t ws_bytes, uint32_t epilogue, void *stream) {
    return gemm_impl(planes, scales, s, X, M, Y, workspace, ws_bytes, epilogue, stream);
}

rbq_status rbq_gemm_noalloc(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                            const uint16_t *X, int32_t M, uint16_t *Y, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (M < 0)
        return RBQ_ERR_INVALID_ARG;
    // the same choice as rbq_gemm given a large enough workspace; more scratch
    // than the static array holds is refused before anything is enqueued
    const rbq_path forced = (rbq_path)g_forced_path.load();
    const bool may_split = forced == RBQ_PATH_SPLIT ||
                           (forced == RBQ_PATH_AUTO && rbq_select_path(s, M) == RBQ_PATH_SPLIT);
    const size_t need = may_split ? rbq_gemm_workspace_bytes(s, M) : 0;
    if (need > RBQ_NOALLOC_SCRATCH_BYTES)
        return RBQ_ERR_SCRATCH_LIMIT;
    if (need == 0 || M == 0 || s.out_features == 0 || s.in_features == 0)
        return gemm_impl(planes, scales, s, X, M, Y, nullptr, 0, RBQ_EPILOGUE_NONE, stream);
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = hipSuccess;
    void *ws = scratch_on_current_device(&e);
    if (ws == nullptr)
        return hip_fail(e == hipSuccess ? hipErrorInvalidSymbol : e);
    return gemm_impl(planes, scales, s, X, M, Y, ws, RBQ_NOALLOC_SCRATCH_BYTES, RBQ_EPILOGUE_NONE, stream);
}

rbq_status rbq_gemm(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                    const uint16_t *X, int32_t M, uint16_t *Y, void *workspace,
                    size_t ws_bytes, void *stream) {
    return rbq_gemm_ex(planes, scales, s, X, M, Y, workspace, ws_bytes, RBQ_EPILOGUE_NONE, stream);
}

rbq_status rbq_gemv(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                    const uint16_t *x, uint16_t *y, void *stream) {
    return rbq_gemm(planes, scales, s, x, 1, y, nullptr, 0, stream);
}

size_t rbq_dual_g_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK || s.group_size != 0)
        return 0;
    return (size_t)s.num_planes * (size_t)s.out_features * 2u;
}

size_t rbq_dual_h_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK || s.group_size != 0)
        return 0;
    return (size_t)s.num_planes * (size_t)s.in_features * 2u;
}

size_t rbq_encode_dual_workspace_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK || s.group_size != 0)
        return 0;
    return rbq::encode_dual_workspace_bytes(s.out_features, s.in_features);
}

rbq_status rbq_encode_dual(const float *W, rbq_shape s, uint32_t *planes, uint16_t *g, uint16_t *h,
                           void *workspace, size_t workspace_bytes, int32_t *status_dev, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (s.group_size != 0)
        return RBQ_ERR_INVALID_ARG;
    if (s.out_features == 0 || s.in_features == 0)
        return RBQ_OK;
    if (s.in_features % 128 != 0 || s.in_features > RBQ_DUAL_MAX_IN)
        return RBQ_ERR_UNSUPPORTED;
    if (W == nullptr || planes == nullptr || g == nullptr || h == nullptr || workspace == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (workspace_bytes < rbq_encode_dual_workspace_bytes(s))
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(W, 4) || !aligned(planes, 4) || !aligned(g, 2) || !aligned(h, 2) ||
        !aligned(workspace, 256) || (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_encode_dual(W, s.out_features, s.in_features, s.num_planes, planes, g, h,
                                           workspace, status_dev, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_gemv_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, rbq_shape s,
                         const uint16_t *x, uint16_t *y, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (s.group_size != 0)
        return RBQ_ERR_INVALID_ARG;
    if (s.out_features == 0)
        return RBQ_OK;
    if (y == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(y, 2))
        return RBQ_ERR_ALIGNMENT;
    hipStream_t hs = (hipStream_t)stream;
    if (s.in_features == 0) {  // empty sums: y = 0
        if ((st = device_present()) != RBQ_OK)
            return st;
        hipError_t e = rbq::launch_fill_zero_u16(y, s.out_features, hs);
        return e == hipSuccess ? RBQ_OK : hip_fail(e);
    }
    // the flat kernel on tall layers of up to 8192 columns, else the decode
    // kernel; rbq_set_path can force either of the two.  (Measured, K = 2:
    // 22016 x 4096 10.7 us flat against 14.9 decode; 4096 x 11008 10.5 flat
    // against 8.4 decode, where the flat kernel's image waves quantise two
    // copies of three half-words per thread.)
    rbq_path path = (rbq_path)g_forced_path.load();
    if (path == RBQ_PATH_AUTO)
        path = rbq::flat_dual_preferred(s.out_features, s.in_features, s.num_planes) && s.in_features <= 8192
                   ? RBQ_PATH_FLAT
                   : RBQ_PATH_DECODE;
    if (path == RBQ_PATH_FLAT ? !rbq::flat_dual_supports(s.out_features, s.in_features, s.num_planes)
                              : (path != RBQ_PATH_DECODE || !rbq::dual_supports(s.in_features, s.num_planes)))
        return RBQ_ERR_UNSUPPORTED;
    if (planes == nullptr || g == nullptr || h == nullptr || x == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(planes, 16) || !aligned(g, 2) || !aligned(h, 16) || !aligned(x, 16))
        return RBQ_ERR_ALIGNMENT;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = path == RBQ_PATH_FLAT
                       ? rbq::launch_gemv_dual_flat(planes, g, h, s.out_features, s.in_features, s.num_planes, x,
                                                    y, hs)
                       : rbq::launch_gemv_dual(planes, g, h, s.out_features, s.in_features, s.num_planes, x, y,
                                               hs);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_gemm_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, rbq_shape s,
                         const uint16_t *X, int32_t M, uint16_t *Y, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (s.group_size != 0 || M < 0)
        return RBQ_ERR_INVALID_ARG;
    if (M == 0 || s.out_features == 0)
        return RBQ_OK;
    // one token: the matrix-core kernels of rbq_gemv_dual where they take the
    // shape (and no plain-kernel run is forced)
    if (M == 1 && (rbq_path)g_forced_path.load() != RBQ_PATH_VALU && rbq::dual_supports(s.in_features, s.num_planes))
        return rbq_gemv_dual(planes, g, h, s, X, Y, stream);
    if (Y == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(Y, 2))
        return RBQ_ERR_ALIGNMENT;
    hipStream_t hs = (hipStream_t)stream;
    if (s.in_features == 0) {  // empty sums: Y = 0
        if ((st = device_present()) != RBQ_OK)
            return st;
        hipError_t e = rbq::launch_fill_zero_u16(Y, (int64_t)M * s.out_features, hs);
        return e == hipSuccess ? RBQ_OK : hip_fail(e);
    }
    if (planes == nullptr || g == nullptr || h == nullptr || X == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(planes, 16) || !aligned(g, 2) || !aligned(h, 16) || !aligned(X, 16))
        return RBQ_ERR_ALIGNMENT;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_gemm_valu_dual(planes, g, h, s.out_features, s.in_features, s.num_planes, X, M, Y,
                                              hs);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

size_t rbq_program_bytes(int32_t n_ops) { return rbq::program_bytes(n_ops); }

size_t rbq_program_counters_bytes(int32_t n_ops) {
    if (n_ops < 1 || n_ops > RBQ_PROGRAM_MAX_OPS)
        return 0;
    return rbq::program_counters_bytes(n_ops);
}

// Host only: the checks and the image need no device (the image is laid out
// for the current device's compute units, or 256 when none is visible).
rbq_status rbq_program_build(const rbq_program_op *ops, int32_t n_ops, int32_t num_planes, void *image,
                             size_t image_bytes) {
    return rbq::program_build(ops, n_ops, num_planes, image, image_bytes);
}

rbq_status rbq_program_run(const void *image, const void *image_dev, int32_t *counters_dev,
                           int32_t *status_dev, void *stream) {
    if (image == nullptr || image_dev == nullptr || counters_dev == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(image_dev, 16) || !aligned(counters_dev, 4) || (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    rbq_status st = device_present();
    if (st != RBQ_OK)
        return st;
    if ((st = rbq::program_check(image)) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_program(image, image_dev, counters_dev, status_dev, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_qat_encode(const float *W, rbq_shape s, const uint16_t *scales, uint32_t *planes,
                          int32_t *status_dev, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (!rbq::qat_supports(s.num_planes))
        return RBQ_ERR_UNSUPPORTED;
    if (s.out_features == 0 || s.in_features == 0)
        return RBQ_OK;
    if (W == nullptr || planes == nullptr || scales == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(W, 4) || !aligned(planes, 4) || !aligned(scales, 2) ||
        (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_qat_encode(W, s.out_features, s.in_features, s.num_planes, s.group_size, scales,
                                          planes, status_dev, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_qat_forward(const float *W, const uint16_t *scales, rbq_shape s, const uint16_t *X, int32_t M,
                           uint32_t *planes, uint16_t *Y, void *workspace, size_t ws_bytes, int32_t *status_dev,
                           void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (M < 0)
        return RBQ_ERR_INVALID_ARG;
    if ((st = rbq_qat_encode(W, s, scales, planes, status_dev, stream)) != RBQ_OK)
        return st;
    return gemm_impl(planes, scales, s, X, M, Y, workspace, ws_bytes, RBQ_EPILOGUE_NONE, stream);
}

size_t rbq_qat_backward_workspace_bytes(rbq_shape s, int32_t M) {
    if (rbq_check_shape(s) != RBQ_OK || M < 1)
        return 0;
    return rbq::qat_backward_workspace_bytes(M, s.out_features, s.in_features);
}

rbq_status rbq_qat_backward(const uint32_t *planes, const uint16_t *scales, rbq_shape s, const uint16_t *X,
                            const uint16_t *dY, int32_t M, float *dX, float *dW, float *dscales, void *workspace,
                            size_t ws_bytes, int32_t *status_dev, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (!rbq::qat_supports(s.num_planes))
        return RBQ_ERR_UNSUPPORTED;
    if (M < 0 || (dscales != nullptr && dW == nullptr) || (ws_bytes > 0 && workspace == nullptr))
        return RBQ_ERR_INVALID_ARG;
    const bool want_dx = dX != nullptr && M > 0 && s.in_features > 0;
    const bool want_dw = dW != nullptr && s.out_features > 0 && s.in_features > 0;
    if (!want_dx && !want_dw)
        return RBQ_OK;
    if (M > 0 && dY == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (want_dw && M > 0 && X == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if ((want_dx || dscales != nullptr) && s.out_features > 0 && (planes == nullptr || scales == nullptr))
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(planes, 4) || !aligned(scales, 2) || !aligned(X, 2) || !aligned(dY, 2) || !aligned(dX, 4) ||
        !aligned(dW, 4) || !aligned(dscales, 4) || !aligned(workspace, 4) ||
        (status_dev != nullptr && !aligned(status_dev, 4)))
        return RBQ_ERR_ALIGNMENT;
    if ((st = device_present()) != RBQ_OK)
        return st;
    hipError_t e = rbq::launch_qat_backward(planes, scales, s.out_features, s.in_features, s.num_planes,
                                            s.group_size, X, dY, M, want_dx ? dX : nullptr,
                                            want_dw ? dW : nullptr, want_dw ? dscales : nullptr, workspace,
                                            ws_bytes, status_dev, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

rbq_status rbq_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (buf == nullptr || sink == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return RBQ_ERR_ALIGNMENT;
    rbq_status st = device_present();
    if (st != RBQ_OK || bytes == 0)
        return st;
    hipError_t e = rbq::launch_probe_read(buf, bytes, sink, (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

size_t rbq_tiles_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK)
        return 0;
    return rbq::tiles_bytes(s.num_planes, s.out_features, s.in_features);
}

rbq_status rbq_pack_tiles(const uint32_t *planes, rbq_shape s, uint32_t *tiles, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (planes == nullptr || tiles == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (s.in_features % 128 != 0)
        return RBQ_ERR_UNSUPPORTED;
    if (!aligned(planes, 16) || !aligned(tiles, 16))
        return RBQ_ERR_ALIGNMENT;
    const uintptr_t p0 = (uintptr_t)planes, p1 = p0 + rbq_planes_bytes(s);
    const uintptr_t t0 = (uintptr_t)tiles, t1 = t0 + rbq_tiles_bytes(s);
    if (p0 < t1 && t0 < p1)
        return RBQ_ERR_INVALID_ARG;
    st = device_present();
    if (st != RBQ_OK || s.out_features == 0 || s.in_features == 0)
        return st;
    hipError_t e = rbq::launch_pack_tiles(planes, s.num_planes, s.out_features, s.in_features, tiles,
                                          (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

size_t rbq_scale_tiles_bytes(rbq_shape s) {
    if (rbq_check_shape(s) != RBQ_OK || s.group_size != 128 || s.num_planes % 2 != 0)
        return 0;
    return rbq::scale_tiles_bytes(s.num_planes, s.out_features, s.in_features);
}

rbq_status rbq_pack_scale_tiles(const uint16_t *scales, rbq_shape s, uint16_t *tiles, void *stream) {
    rbq_status st = rbq_check_shape(s);
    if (st != RBQ_OK)
        return st;
    if (scales == nullptr || tiles == nullptr)
        return RBQ_ERR_INVALID_ARG;
    if (s.group_size != 128 || s.num_planes % 2 != 0)
        return RBQ_ERR_UNSUPPORTED;
    if (!aligned(scales, 2) || !aligned(tiles, 16))
        return RBQ_ERR_ALIGNMENT;
    const uintptr_t p0 = (uintptr_t)scales, p1 = p0 + rbq_scales_bytes(s);
    const uintptr_t t0 = (uintptr_t)tiles, t1 = t0 + rbq_scale_tiles_bytes(s);
    if (p0 < t1 && t0 < p1)
        return RBQ_ERR_INVALID_ARG;
    st = device_present();
    if (st != RBQ_OK || s.out_features == 0 || s.in_features == 0)
        return st;
    hipError_t e = rbq::launch_pack_scale_tiles(scales, s.num_planes, s.out_features, s.in_features, tiles,
                                                (hipStream_t)stream);
    return e == hipSuccess ? RBQ_OK : hip_fail(e);
}

int32_t rbq_last_hip_error(void) { return g_last_hip_error; }

const char *rbq_status_string(rbq_status st) {
    switch (st) {
    case RBQ_OK: return "RBQ_OK";
    case RBQ_ERR_INVALID_ARG: return "RBQ_ERR_INVALID_ARG: invalid argument";
    case RBQ_ERR_ALIGNMENT: return "RBQ_ERR_ALIGNMENT: misaligned pointer";
    case RBQ_ERR_UNSUPPORTED: return "RBQ_ERR_UNSUPPORTED: not supported by this build";
    case RBQ_ERR_NO_DEVICE: return "RBQ_ERR_NO_DEVICE: no HIP device";
    case RBQ_ERR_HIP: return "RBQ_ERR_HIP: HIP runtime error";
    case RBQ_ERR_SCRATCH_LIMIT:
        return "RBQ_ERR_SCRATCH_LIMIT: the call needs more scratch than rbq_gemm_noalloc's static buffer "
               "(RBQ_NOALLOC_SCRATCH_BYTES) holds";
    }
    return "unknown rbq_status";
}

const char *rbq_version(void) { return "rbq 0.1.0 (gfx950)"; }

}  // extern "C"
