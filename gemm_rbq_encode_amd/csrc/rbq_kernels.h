// rbq_kernels.h -- host-side launchers of the librbq kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rbq.h"

namespace rbq {

// Encoder: one workgroup of 256 threads per output row.
hipError_t launch_encode(const float *W, int out, int in, int K, int group_size,
                         uint32_t *planes, uint16_t *scales, int32_t *status,
                         int force_serial, hipStream_t st);

// Joint least-squares refit of the K scales for fixed planes (in place).
hipError_t launch_refit(const float *W, int out, int in, int K, int group_size, const uint32_t *planes,
                        uint16_t *scales, int32_t *status, hipStream_t st);
hipError_t launch_rebinarize(const float *W, int out, int in, int K, int group_size, uint32_t *planes,
                             const uint16_t *scales, int32_t *status, hipStream_t st);

// fp32 VALU bit loop, any M (correctness baseline and fallback).
// silu != 0: rows come in (gate, up) pairs 2i, 2i+1 and Y[m][i] =
// silu(y_2i) * y_2i+1 (Y has out / 2 columns; out even).
hipError_t launch_gemm_valu(const uint32_t *planes, const uint16_t *scales, int out, int in,
                            int K, int group_size, const uint16_t *X, int M, uint16_t *Y, int silu,
                            hipStream_t st);

// int8-MFMA decode kernel (per-row scales, K <= 4, in % 128 == 0); M is
// processed in passes of 5 tokens.
bool decode_supports(int in, int K, int group_size, int M);
hipError_t launch_gemm_decode(const uint32_t *planes, const uint16_t *scales, int out, int in,
                              int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                              hipStream_t st);

// Dual-scale GEMV on the decode kernel: y = sum_k g_k (.) (B_k (h_k (.) x)),
// g [K][out], h [K][in] binary16, one token (K <= 4, in % 128 == 0).
bool dual_supports(int in, int K);
hipError_t launch_gemm_valu_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                                 int K, const uint16_t *X, int M, uint16_t *Y, hipStream_t st);
hipError_t launch_gemv_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                            int K, const uint16_t *x, uint16_t *y, hipStream_t st);

// The same on the flat kernel (K <= 2; the layers it serves for two tokens).
bool flat_dual_supports(int out, int in, int K);
bool flat_dual_preferred(int out, int in, int K);
hipError_t launch_gemv_dual_flat(const uint32_t *planes, const uint16_t *g, const uint16_t *h, int out, int in,
                                 int K, const uint16_t *x, uint16_t *y, hipStream_t st);

// Residual SVID encoder (dual scales); workspace layout in encode_dual.hip.
size_t encode_dual_workspace_bytes(int out, int in);
hipError_t launch_encode_dual(const float *W, int out, int in, int K, uint32_t *planes, uint16_t *g,
                              uint16_t *h, void *workspace, int32_t *status, hipStream_t st);

// Whole-row streaming int8-MFMA kernel for 1-2 tokens (per-row scales,
// K <= 4, in % 128 == 0, activation image of in*3*M bytes in LDS).  split =
// waves per 16-row tile (1, 2 or 4), 0 = chosen from the tile count.
bool stream_supports(int in, int K, int group_size, int M);
hipError_t launch_gemm_stream(const uint32_t *planes, const uint16_t *scales, int out, int in,
                              int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                              hipStream_t st, int split);

// One-workgroup-per-CU int8-MFMA GEMV for 1-2 tokens (per-row scales,
// K <= 2, in % 128 == 0): 12 waves stream weight units while 4 build the
// activation image; tile partial sums combined as int32 in LDS.
bool flat_supports(int out, int in, int K, int group_size, int M);
// Whether the flat kernel is the faster choice (many 16-row tiles per CU).
bool flat_preferred(int out, int in, int K, int group_size, int M);
hipError_t launch_gemm_flat(const uint32_t *planes, const uint16_t *scales, int out, int in,
                            int K, int group_size, const uint16_t *X, int M, uint16_t *Y, int silu,
                            hipStream_t st);

// One-workgroup-per-compute-unit int8-MFMA GEMV for one token with a scale
// per (row, 128-column group), K <= 4, in % 512 == 0; scales 8-byte aligned.
bool group_supports(int out, int in, int K, int group_size, int M);
hipError_t launch_gemm_group(const uint32_t *planes, const uint16_t *scales, int out, int in,
                             int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                             hipStream_t st);

// Few-token GEMM (2 <= M <= 16, per-row scales, K <= 2) on the fp16 matrix
// cores with the input columns split over workgroups: with several slices,
// fp32 partial outputs in a workspace of split_workspace_bytes (0 for one
// slice), added in slice order by a second kernel.
bool split_supports(int out, int in, int K, int group_size, int M);
bool split_preferred(int out, int in, int K, int group_size, int M);
size_t split_workspace_bytes(int out, int in, int K, int group_size, int M);
hipError_t launch_gemm_split(const uint32_t *planes, const uint16_t *scales, int out, int in, int K,
                             int group_size, const uint16_t *X, int M, uint16_t *Y, void *workspace,
                             size_t ws_bytes, hipStream_t st);

// fp16-MFMA prefill GEMM over LDS-unpacked What (in % 64 == 0, K <= 4).
bool prefill_supports(int in, int K, int group_size, int M);
hipError_t launch_gemm_prefill(const uint32_t *planes, const uint16_t *scales, int out, int in,
                               int K, int group_size, const uint16_t *X, int M, uint16_t *Y,
                               hipStream_t st);

// Programs of one-token GEMVs in one persistent launch (gemv_program.hip).
size_t program_bytes(int n_ops);
rbq_status program_build(const rbq_program_op *ops, int n_ops, int K, void *image, size_t bytes);
rbq_status program_check(const void *image);   // a valid image for the current device
int program_num_ops(const void *image);
size_t program_counters_bytes(int n_ops);
hipError_t launch_program(const void *image, const void *image_dev, int32_t *counters, int32_t *status,
                          hipStream_t st);

// Coupled forward and straight-through backward (qat.hip), K <= 4.
bool qat_supports(int K);
hipError_t launch_qat_encode(const float *W, int out, int in, int K, int group_size, const uint16_t *scales,
                             uint32_t *planes, int32_t *status, hipStream_t st);
size_t qat_backward_workspace_bytes(int M, int out, int in);
hipError_t launch_qat_backward(const uint32_t *planes, const uint16_t *scales, int out, int in, int K,
                               int group_size, const uint16_t *X, const uint16_t *dY, int M, float *dX,
                               float *dW, float *dscales, void *workspace, size_t ws_bytes, int32_t *status,
                               hipStream_t st);

// Streaming-read probe (probe.hip): one launch reading `bytes` bytes.
hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);

// Tile layout of the planes (tiles.hip): 16 rows x 512 columns of a plane per
// contiguous 1 KB block; in % 128 == 0.
size_t tiles_bytes(int K, int out, int in);
hipError_t launch_pack_tiles(const uint32_t *planes, int K, int out, int in, uint32_t *tiles, hipStream_t st);
// ... and of g128 scales (K even): K * 128 bytes per 16-row, 512-column unit.
size_t scale_tiles_bytes(int K, int out, int in);
hipError_t launch_pack_scale_tiles(const uint16_t *scales, int K, int out, int in, uint16_t *stiles,
                                   hipStream_t st);

// Y = 0 for in_features == 0 (an empty sum).
hipError_t launch_fill_zero_u16(uint16_t *Y, int64_t n, hipStream_t st);

}  // namespace rbq
