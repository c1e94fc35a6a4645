// Streaming-read probe: the HBM read rate one launch reaches on a buffer of
// a given size.  A measurement aid for the GEMV kernels, which read their
// packed planes once per launch: a probe of the same byte count, run the
// same way (one launch per matrix, matrices larger than the caches together),
// is the rate those launches could reach if they did nothing but read.
//
// 16-byte non-temporal loads, four in flight per lane, over a grid of 256-lane
// workgroups sized to the buffer (at least 16 KiB per workgroup, at most 8 per
// compute unit).  The loaded words are folded into one value per lane; a lane
// writes it only in the never-seen case that it equals a magic constant, so
// the loads stay live and the probe writes nothing in practice (one word,
// shared by every lane, is the only place it could write).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rbq_kernels.h"

namespace rbq {

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

constexpr int PROBE_THREADS = 256;
constexpr uint32_t PROBE_MAGIC = 0x9e3779b9u;

__global__ __launch_bounds__(PROBE_THREADS) void probe_read_kernel(const v4u *buf, size_t n16,
                                                                   const uint8_t *tail, uint32_t n_tail,
                                                                   uint32_t *sink) {
    const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
    size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
    GLOBAL const v4u *p = (GLOBAL const v4u *)buf;
    v4u acc = (v4u){0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u a = __builtin_nontemporal_load(p + i);
        const v4u b = __builtin_nontemporal_load(p + i + stride);
        const v4u c = __builtin_nontemporal_load(p + i + 2 * stride);
        const v4u d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= (a + b) ^ (c + d);
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (blockIdx.x == 0 && threadIdx.x < n_tail) v ^= tail[threadIdx.x];
    if (v == PROBE_MAGIC) *sink = v;
}

}  // namespace

static int probe_grid(size_t bytes) {
    const size_t per_wg = 16u << 10;
    size_t g = (bytes + per_wg - 1) / per_wg;
    const size_t cap = 8 * 256;
    if (g > cap) g = cap;
    return g < 1 ? 1 : (int)g;
}

hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const uint32_t n_tail = (uint32_t)(bytes % 16);
    const uint8_t *tail = (const uint8_t *)buf + n16 * 16;
    hipLaunchKernelGGL(probe_read_kernel, dim3(probe_grid(bytes)), dim3(PROBE_THREADS), 0, stream,
                       (const v4u *)buf, n16, tail, n_tail, sink);
    return hipGetLastError();
}

}  // namespace rbq
