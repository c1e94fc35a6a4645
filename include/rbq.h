/*
 * rbq.h -- C ABI of librbq, residual-binarized linear layers on AMD MI355X
 * (gfx950).
 *
 * The layer is y = sum_{k=1..K} a_k (.) (B_k x): K binary (+-1) cores with
 * scale vectors, computed with additions and subtractions only ("RaBiT:
 * Residual-Aware Binarization Training for Accurate and Efficient LLMs",
 * paperlayer.ai summary, section 4.1; "QBB: Quantization with Binary Bases
 * for LLMs", atlas.scime.ai summary, "Approach").  The cores come from
 * sequential residual binarization of one full-precision weight:
 * B_1 = sign(W), R_1 = W - a_1 B_1, B_2 = sign(R_1), ... (RaBiT sections 4.2,
 * A and B).
 *
 * Storage format (every entry point reads and writes this format):
 *   planes  uint32 [K][out][in/32], row-major.  Word w of row r of plane k
 *           holds columns 32w .. 32w+31, bit b (least significant first) is
 *           column 32w + b, and a set bit means +1, a clear bit -1 (RaBiT D
 *           "GPU implementation": 32 columns per uint32).
 *   scales  IEEE binary16 bit patterns, uint16 [K][out][G], where G = 1 for
 *           one scale per output row (group_size 0, RaBiT) or in/128 for one
 *           scale per row per group of 128 consecutive input columns
 *           (group_size 128, QBB "W(4x1)A16g128").
 *   g, h    (dual-scale entry points only: rbq_encode_dual, rbq_gemv_dual)
 *           binary16 row scales g [K][out] and input-column scales h
 *           [K][in] of y = sum_k g_k (.) (B_k (h_k (.) x)) (RaBiT section 4.1:
 *           scaling vectors on both sides of each binary core).
 *   x, y    IEEE binary16 bit patterns, row-major [M][in] and [M][out].
 *   W       fp32, row-major [out][in].
 *
 * Memory and streams.  Every pointer argument is a DEVICE pointer owned by
 * the caller (allocated with hipMalloc, or by PyTorch); the library never
 * allocates, frees or keeps a pointer after a call returns.  `stream` is a
 * hipStream_t (NULL = the null stream); each call only enqueues work on it
 * and returns, so results are ready when the stream reaches that point.
 * Calls are stateless and may be made from several host threads.
 *
 * Errors.  Argument errors are found on the host before anything is
 * enqueued, and then nothing is written.  RBQ_ERR_HIP means a HIP call
 * failed; rbq_last_hip_error() returns its hipError_t on the calling thread.
 * Errors found in the data on the device are reported through `status_dev`.
 */
#ifndef RBQ_H
#define RBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rbq_status {
    RBQ_OK = 0,
    RBQ_ERR_INVALID_ARG = 1,   /* null pointer, bad size, K or group size */
    RBQ_ERR_ALIGNMENT = 2,     /* a pointer is not aligned as required */
    RBQ_ERR_UNSUPPORTED = 3,   /* valid, but beyond what this build handles */
    RBQ_ERR_NO_DEVICE = 4,     /* no HIP device is visible */
    RBQ_ERR_HIP = 5,           /* a HIP runtime call or launch failed */
    RBQ_ERR_SCRATCH_LIMIT = 6  /* rbq_gemm_noalloc: the call needs more scratch
                                  than RBQ_NOALLOC_SCRATCH_BYTES */
} rbq_status;

/* Shape of one encoded linear layer.
 *   out_features  rows of W (outputs), >= 0
 *   in_features   columns of W (inputs), >= 0 and a multiple of 32
 *   num_planes    K, 1..8
 *   group_size    0 (one scale per row) or 128 (in_features % 128 == 0) */
typedef struct rbq_shape {
    int32_t out_features;
    int32_t in_features;
    int32_t num_planes;
    int32_t group_size;
} rbq_shape;

/* Bits of the device status word written by rbq_encode, rbq_refit,
 * rbq_rebinarize and rbq_encode_dual. */
#define RBQ_STATUS_NONFINITE_W     1u   /* some entry of W was NaN or +-Inf */
#define RBQ_STATUS_SCALE_OVERFLOW  2u   /* some scale rounded to +-Inf in fp16 */
#define RBQ_STATUS_REFIT_KEPT      4u   /* rbq_refit kept the given scales of some
                                           (row, group): singular normal
                                           equations, non-finite W, or a
                                           solution outside binary16 */
#define RBQ_STATUS_PLANES_KEPT     8u   /* rbq_rebinarize kept the planes of some
                                           (row, group) whose scales are not all
                                           finite */

/* Flags for rbq_encode_ex. */
#define RBQ_ENCODE_FORCE_SERIAL    1u   /* take the serial summation for every
                                           (row, group): slow, same results */

/* Largest in_features the encoder handles in this build. */
#define RBQ_ENCODE_MAX_IN          32768

/* Returns RBQ_OK if `s` is a valid shape, else RBQ_ERR_INVALID_ARG. */
rbq_status rbq_check_shape(rbq_shape s);

/* Bytes of the planes array: K * out * (in/32) * 4.  0 for an invalid shape. */
size_t rbq_planes_bytes(rbq_shape s);

/* Bytes of the scales array: K * out * G * 2.  0 for an invalid shape. */
size_t rbq_scales_bytes(rbq_shape s);

/*
 * rbq_encode -- sequential residual binarization (RaBiT sections 4.2, B and
 * G "RaBiT training"; QBB "Approach": cascaded analytical residual
 * binarization; scale = mean absolute residual, the closed form of XNOR-Net,
 * which QBB lists under "Builds on").
 *
 * For each row r and each group t of n columns (n = in, or 128), with
 * R = W[r, group t] in fp32, for k = 1..K:
 *   bit_j   = (R_j >= 0)             sign(0) = +1, also for -0.0
 *   a_k     = mean_j |R_j|, where the sum is the serial fp64 sum in
 *             ascending column order, divided by n in fp64 (correctly
 *             rounded), then rounded ONCE to binary16 (nearest, ties even)
 *   R_j     = R_j - (bit_j ? a_k : -a_k)   in fp32, against the stored a_k
 * and writes bit_j to planes[k][r] and a_k to scales[k][r][t].
 * Results are bit-identical to that definition (the kernel sums in parallel
 * with a proven error bound and falls back to the serial sum whenever the
 * bound cannot decide the fp16 rounding).
 *
 *   W           device, fp32 [out][in], 4-byte aligned, read only
 *   planes      device, uint32 [K][out][in/32], 4-byte aligned, written
 *   scales      device, uint16 [K][out][G], 2-byte aligned, written
 *   status_dev  device int32 or NULL.  If given, the kernel ORs
 *               RBQ_STATUS_* bits into it (the caller clears it first).
 *               Non-finite W is outside the method; its planes and scales
 *               are then unspecified.
 * Errors: RBQ_ERR_INVALID_ARG (shape, null pointer), RBQ_ERR_ALIGNMENT,
 * RBQ_ERR_UNSUPPORTED (in > RBQ_ENCODE_MAX_IN), RBQ_ERR_NO_DEVICE,
 * RBQ_ERR_HIP.  An empty shape (out == 0 or in == 0) enqueues nothing.
 */
rbq_status rbq_encode(const float *W, rbq_shape s, uint32_t *planes, uint16_t *scales,
                      int32_t *status_dev, void *stream);

/* rbq_encode with flags (RBQ_ENCODE_*); flags = 0 is rbq_encode. */
rbq_status rbq_encode_ex(const float *W, rbq_shape s, uint32_t *planes, uint16_t *scales,
                         int32_t *status_dev, uint32_t flags, void *stream);

/*
 * rbq_refit -- joint least-squares refit of the K scales of every (row,
 * group) for fixed planes: the data-free part of the refinement of the
 * binary bases in the QBB summary ("Approach"; the cascade of rbq_encode
 * fits each scale for its own step only).  For each row r and group t of n
 * columns, with the planes B_k held fixed:
 *   minimise sum_j (W_j - sum_k a_k B_kj)^2,
 *   normal equations G a = b, G_kl = sum_j B_kj B_lj (exact integers),
 *   b_k = sum_j B_kj W_j in fp64; G = L D L^T in fp64 in a fixed order;
 *   each a_k rounded once to binary16 (nearest, ties to even).
 * A (row, group) whose pivot D_i <= n 2^-30 (dependent planes), whose W has a
 * non-finite entry, or whose solution is not finite in binary16 keeps its
 * given scales.  With K = 1 the result equals rbq_encode's scale.
 *
 *   W            device, fp32 [out][in] row-major, 16-byte aligned
 *   planes       device, the planes of W (format above), 4-byte aligned
 *   scales       device, fp16 bits [K][out][G], 2-byte aligned: read (the
 *                scales kept where no refit is made, normally rbq_encode's)
 *                and overwritten with the refit
 *   status_dev   device int32 or NULL; RBQ_STATUS_NONFINITE_W and
 *                RBQ_STATUS_REFIT_KEPT are OR-ed in (never cleared)
 * The fp64 sums b_k are added in parallel, so a refit scale can differ by
 * one binary16 unit from one computed with another summation order.
 * Errors: RBQ_ERR_INVALID_ARG, RBQ_ERR_ALIGNMENT, RBQ_ERR_UNSUPPORTED
 * (in_features > RBQ_ENCODE_MAX_IN), RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP.  An empty
 * shape enqueues nothing.
 */
rbq_status rbq_refit(const float *W, rbq_shape s, const uint32_t *planes, uint16_t *scales,
                     int32_t *status_dev, void *stream);

/* Largest K rbq_rebinarize handles (2^K candidate values per weight). */
#define RBQ_REBIN_MAX_PLANES       4

/*
 * rbq_rebinarize -- the planes for fixed scales: the other half of the
 * data-free refinement of the binary bases in the QBB summary ("Approach"),
 * alternated with rbq_refit.  With the scales of every (row, group) fixed,
 * sum_j (W_j - sum_k a_k B_kj)^2 is minimised weight by weight: W_j takes
 * the sign pattern s (s_k = +-1) whose value sum_k s_k a_k is nearest to
 * it, decided exactly (no rounding in the comparison).  Ties: a weight
 * halfway between two values takes the larger value; among patterns of
 * equal value the one with the most +1 bits in the highest planes (the
 * largest p = sum_k [s_k = +1] 2^k) wins, which keeps sign(0) = +1: with
 * K = 1 the planes are sign(W), and with K = 2 and a_1 > a_2 they are
 * rbq_encode's.  A NaN weight takes the smallest value's pattern, +-Inf the
 * largest or smallest.
 *
 *   W            device, fp32 [out][in] row-major, 4-byte aligned, read only
 *   planes       device, uint32 [K][out][in/32], 4-byte aligned: overwritten,
 *                except the words of a (row, group) whose scales are not all
 *                finite, which are kept
 *   scales       device, fp16 bits [K][out][G], 2-byte aligned, read only
 *   status_dev   device int32 or NULL; RBQ_STATUS_NONFINITE_W and
 *                RBQ_STATUS_PLANES_KEPT are OR-ed in (never cleared)
 * The result does not depend on the launch or on the summation order.
 * Errors: RBQ_ERR_INVALID_ARG, RBQ_ERR_ALIGNMENT, RBQ_ERR_UNSUPPORTED
 * (num_planes > RBQ_REBIN_MAX_PLANES), RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP.  An
 * empty shape enqueues nothing.
 */
rbq_status rbq_rebinarize(const float *W, rbq_shape s, uint32_t *planes, const uint16_t *scales,
                          int32_t *status_dev, void *stream);

/*
 * rbq_gemm -- Y[m] = sum_k a_k (.) (B_k X[m]) for M tokens (RaBiT section
 * 4.1: binary cores with per-channel scales, additions and subtractions
 * only; section 4.2: the K paths run in parallel at inference; QBB "Key
 * results": per-group scales).  Equivalently Y = X What^T with
 * What[r][j] = sum_k a_k[r][t(j)] (bit ? +1 : -1).  Accumulation is fp32 or
 * wider; each output is rounded once to binary16.
 *
 *   planes, scales  device, encoded layer (format above); planes 16-byte
 *                   aligned, scales 2-byte aligned; any finite fp16 scales
 *   X               device, fp16 [M][in], 16-byte aligned
 *   M               tokens, >= 0 (0 enqueues nothing)
 *   Y               device, fp16 [M][out], 2-byte aligned, written
 *   workspace       device scratch of ws_bytes >= rbq_gemm_workspace_bytes
 *                   (may be NULL when that is 0); contents on return are
 *                   unspecified
 * Errors: RBQ_ERR_INVALID_ARG, RBQ_ERR_ALIGNMENT, RBQ_ERR_NO_DEVICE,
 * RBQ_ERR_HIP.  The one- and few-token kernels coordinate their waves
 * through bounded waits on LDS counters (the bound is never reached in a
 * correct launch); should one run out, the workgroup writes fp16 NaN for
 * all of its outputs instead of a value built on missing data.
 */
rbq_status rbq_gemm(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                    const uint16_t *X, int32_t M, uint16_t *Y,
                    void *workspace, size_t ws_bytes, void *stream);

/* Epilogues of rbq_gemm_ex. */
#define RBQ_EPILOGUE_NONE          0u
#define RBQ_EPILOGUE_SILU_MUL      1u   /* gated-MLP gate/up: see rbq_gemm_ex */

/*
 * rbq_gemm_ex -- rbq_gemm with an epilogue on the outputs (RaBiT section 5
 * and QBB "Key results" measure whole decoder layers, whose MLP multiplies
 * SiLU of the gate projection into the up projection).
 *   RBQ_EPILOGUE_NONE      rbq_gemm.
 *   RBQ_EPILOGUE_SILU_MUL  the layer's rows come in (gate, up) pairs: row 2i
 *                          is gate row i, row 2i+1 up row i (out even).  Y is
 *                          fp16 [M][out/2] with
 *                          Y[m][i] = silu(y[m][2i]) * y[m][2i+1],
 *                          silu(v) = v / (1 + e^-v), from the fp32 sums,
 *                          rounded once to binary16.  Served by the
 *                          RBQ_PATH_FLAT and RBQ_PATH_VALU families (another
 *                          forced family returns RBQ_ERR_UNSUPPORTED).
 * Other arguments and errors as rbq_gemm; an unknown epilogue or an odd out
 * with RBQ_EPILOGUE_SILU_MUL is RBQ_ERR_INVALID_ARG.
 */
rbq_status rbq_gemm_ex(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                       const uint16_t *X, int32_t M, uint16_t *Y,
                       void *workspace, size_t ws_bytes, uint32_t epilogue, void *stream);

/* Workspace bytes the split-column kernel family (RBQ_PATH_SPLIT) needs for
 * this shape and M: S * M * out fp32 partial outputs when the input columns
 * are split into S > 1 slices (in > 4096); 0 when one slice takes the whole
 * row or when that family cannot take the call (M < 2 or > 16, group
 * scales, K > 2).  With less workspace than this (or none) rbq_gemm chooses
 * another family; a forced RBQ_PATH_SPLIT then returns RBQ_ERR_INVALID_ARG.
 * The workspace must be 4-byte aligned; its contents need no
 * initialisation. */
size_t rbq_gemm_workspace_bytes(rbq_shape s, int32_t M);

/* Size of the static device buffer rbq_gemm_noalloc takes its scratch from
 * (one per GPU the library runs on, held until the process ends). */
#define RBQ_NOALLOC_SCRATCH_BYTES  (8u << 20)

/*
 * rbq_gemm_noalloc -- rbq_gemm for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results and
 * kernel choice as rbq_gemm given a workspace of rbq_gemm_workspace_bytes;
 * the scratch the split-column kernels need (S * M * out fp32 partial
 * outputs) comes from a static device array of RBQ_NOALLOC_SCRATCH_BYTES
 * per GPU instead.  It never calls hipMalloc, hipFree or any allocating
 * routine.  Every call on one GPU shares that GPU's array, so calls that
 * may overlap on one GPU (different streams, different host threads without
 * ordering) race and give unspecified results; calls ordered on one stream
 * are safe.  The array needs no initialisation and keeps the last call's
 * partial sums.
 * Errors: as rbq_gemm, and RBQ_ERR_SCRATCH_LIMIT (before anything is
 * enqueued) when the call would need more than RBQ_NOALLOC_SCRATCH_BYTES.
 */
rbq_status rbq_gemm_noalloc(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                            const uint16_t *X, int32_t M, uint16_t *Y, void *stream);

/* rbq_gemv -- rbq_gemm with M = 1 (one decode token):
 * y = sum_k a_k (.) (B_k x), x fp16 [in], y fp16 [out]. */
rbq_status rbq_gemv(const uint32_t *planes, const uint16_t *scales, rbq_shape s,
                    const uint16_t *x, uint16_t *y, void *stream);

/*
 * Dual-scale paths (RaBiT section 4.1: each binary core carries per-channel
 * scaling vectors on its output and its input side):
 *   y = sum_k g_k (.) (B_k (h_k (.) x))
 * with planes B_k as above (group_size must be 0), g_k binary16 [K][out] and
 * h_k binary16 [K][in].
 */

/* Largest in_features rbq_encode_dual handles in this build. */
#define RBQ_DUAL_MAX_IN            16384

/* Bytes of g (K * out * 2) and of h (K * in * 2); 0 for an invalid shape or
 * group_size != 0. */
size_t rbq_dual_g_bytes(rbq_shape s);
size_t rbq_dual_h_bytes(rbq_shape s);

/* Device workspace rbq_encode_dual needs: the fp32 residual (out * in * 4)
 * plus fp64 vectors and per-workgroup partial sums (about 2 KB per input
 * column); 0 for an invalid shape. */
size_t rbq_encode_dual_workspace_bytes(rbq_shape s);

/*
 * rbq_encode_dual -- residual binarization whose scales come from a residual
 * SVID (RaBiT section 4.3 and "RaBiT initialization", Tmax = 20 SVID
 * iterations in "Training configuration"; the calibration-data
 * preconditioning is left out).  With R_0 = W (fp32), for k = 1..K:
 *   B_k = (R_{k-1} >= 0)              sign(0) = +1, also for -0.0
 *   |R_{k-1}| ~ u v^T by 20 alternating least-squares steps from v = 1:
 *       u = |R| v / (v.v),  then  v = |R|^T u / (u.u)   (fp64)
 *   c = sqrt(||u|| / ||v||);  g_k = fp16(u / c), h_k = fp16(v c), each
 *       rounded once to nearest even (zero scales for an all-zero |R|)
 *   R_k = R_{k-1} - (bit ? 1 : -1) g_k[r] h_k[j]   in fp32
 *
 *   W          device fp32 [out][in], finite, 4-byte aligned, read only
 *   planes     device uint32 [K][out][in/32], 4-byte aligned, written
 *   g, h       device binary16 [K][out] and [K][in], 2-byte aligned, written
 *   workspace  device, rbq_encode_dual_workspace_bytes(s) bytes, 256-byte
 *              aligned, any contents; calls that share one overlap on the
 *              stream order only
 *   status_dev device int32 or NULL: RBQ_STATUS_NONFINITE_W and
 *              RBQ_STATUS_SCALE_OVERFLOW (a g or h entry rounded to +-Inf)
 *              are OR-ed in
 * The sums are fp64 in a fixed order (deterministic on a given device); a
 * different order changes a stored scale only when its value lies within
 * ~1e-13 of an fp16 rounding boundary.
 * Errors: RBQ_ERR_INVALID_ARG (shape, group_size != 0, null pointer,
 * workspace too small), RBQ_ERR_ALIGNMENT, RBQ_ERR_UNSUPPORTED
 * (in % 128 != 0 or in > RBQ_DUAL_MAX_IN), RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP.
 * An empty shape enqueues nothing.
 */
rbq_status rbq_encode_dual(const float *W, rbq_shape s, uint32_t *planes, uint16_t *g, uint16_t *h,
                           void *workspace, size_t workspace_bytes, int32_t *status_dev, void *stream);

/*
 * rbq_gemm_dual -- Y[m] = sum_k g_k (.) (B_k (h_k (.) X[m])) for M tokens
 * (RaBiT section 4.1: scaling vectors on both sides of each binary core).
 * One token takes rbq_gemv_dual's matrix-core kernels where they serve the
 * shape (K <= 4, in % 128 == 0) and RBQ_PATH_VALU is not forced; otherwise
 * a plain fp32 kernel runs (each product h_k[j] X[m][j] exact in fp32, fp32
 * sums, one binary16 rounding of each output), not tuned for speed.
 *   planes  device uint32 [K][out][in/32], 16-byte aligned
 *   g       device binary16 [K][out], 2-byte aligned
 *   h       device binary16 [K][in], 16-byte aligned
 *   X       device fp16 [M][in], 16-byte aligned;  Y device fp16 [M][out], written
 *   M       tokens, >= 0 (0 enqueues nothing)
 * group_size must be 0 (RBQ_ERR_INVALID_ARG).  Errors: RBQ_ERR_INVALID_ARG,
 * RBQ_ERR_ALIGNMENT, RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP (and rbq_gemv_dual's for
 * one token).
 */
rbq_status rbq_gemm_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, rbq_shape s,
                         const uint16_t *X, int32_t M, uint16_t *Y, void *stream);

/*
 * rbq_gemv_dual -- y = sum_k g_k (.) (B_k (h_k (.) x)) for one token, on the
 * int8 matrix cores: the K products h_k (.) x (exact in fp32) take the place
 * of tokens, each quantised to three 8-bit limbs with its own power of two.
 *   planes  device uint32 [K][out][in/32], 16-byte aligned
 *   g       device binary16 [K][out], 2-byte aligned
 *   h       device binary16 [K][in], 16-byte aligned
 *   x       device fp16 [in], 16-byte aligned;  y device fp16 [out], written
 * K <= 4 and in % 128 == 0 (else RBQ_ERR_UNSUPPORTED); group_size must be 0
 * (RBQ_ERR_INVALID_ARG).  out == 0 enqueues nothing; in == 0 writes y = 0.
 * Kernel family: RBQ_PATH_FLAT where rbq_gemm would take it for two tokens
 * (K <= 2, tall layers) and in <= 8192, else RBQ_PATH_DECODE; rbq_set_path
 * may force either (any other forced family gives RBQ_ERR_UNSUPPORTED).
 * Errors as rbq_gemm.
 */
rbq_status rbq_gemv_dual(const uint32_t *planes, const uint16_t *g, const uint16_t *h, rbq_shape s,
                         const uint16_t *x, uint16_t *y, void *stream);

/*
 * Programs: a list of one-token GEMVs run by ONE persistent launch.
 *
 * A decode step is a chain of GEMVs whose weights do not depend on the
 * activations (RaBiT summary section 4.2: at inference the binary paths run
 * side by side with additions only; section 5 and QBB "Key results" time
 * whole decoder layers).  Launched one by one, each GEMV pays the launch and
 * the ramp of its first memory requests; a program streams the weights of
 * every op back to back on all compute units, and an op that reads an
 * earlier op's output waits for it on the device (its weights are fetched
 * meanwhile).  Each op computes exactly what rbq_gemv computes (per-row
 * scales, one token), or rbq_gemm_ex with RBQ_EPILOGUE_SILU_MUL.
 */
#define RBQ_PROGRAM_MAX_OPS        512

/* Status bits written by rbq_program_run. */
#define RBQ_STATUS_PROGRAM_TIMEOUT  16u  /* a bounded wait of rbq_program_run ran
                                            out (not every workgroup was resident:
                                            the device was shared); the outputs
                                            are then unspecified */
#define RBQ_STATUS_PROGRAM_MISMATCH 32u  /* image_dev does not hold the image
                                            passed on the host; nothing was run */

/*
 * Plane layouts an op of a program may read.
 *
 * RBQ_LAYOUT_ROWS is the layout every other call takes: uint32 [K][out][in/32],
 * row r of plane k holds columns 32w .. 32w+31 in word w (RaBiT summary,
 * section D "GPU implementation": 32 columns per 32-bit word).
 *
 * RBQ_LAYOUT_TILES holds the same bits reordered so that each unit of work
 * of the one-token kernels -- 16 rows by 512 columns of one plane -- is one
 * contiguous 1 KB block, read by one 64-lane load of 16 bytes per lane:
 *   uint32 [K][T][C][4][16][4],  T = ceil(out / 16),  C = ceil(in / 512);
 *   element [k][t][c][g][i][j] = word 16c + 4g + j of row 16t + i of plane k,
 *   zero where that row (>= out) or word (>= in / 32) does not exist.
 * A row-major 16-row unit is 16 runs of 64 bytes, half a 128-byte line each;
 * the contiguous block is 8 whole lines.  rbq_pack_tiles writes this layout
 * from the row layout once, when the weights are loaded.
 */
#define RBQ_LAYOUT_ROWS  0u
#define RBQ_LAYOUT_TILES 1u

/* Bytes of the tile layout of shape s (0 for an invalid shape). */
size_t rbq_tiles_bytes(rbq_shape s);

/*
 * rbq_pack_tiles -- write the RBQ_LAYOUT_TILES copy of row-layout planes.
 *   planes  device uint32 [K][out][in/32], 16-byte aligned (read only)
 *   tiles   device, rbq_tiles_bytes(s) bytes, 16-byte aligned; every byte
 *           is written, padding with zeros
 * s.in_features % 128 == 0 (else RBQ_ERR_UNSUPPORTED); s.group_size does
 * not change the planes and is only checked for validity.  out == 0 or
 * in == 0 enqueues nothing.  Errors: RBQ_ERR_INVALID_ARG (null pointer, bad
 * shape, tiles overlapping planes), RBQ_ERR_ALIGNMENT, RBQ_ERR_NO_DEVICE,
 * RBQ_ERR_HIP.
 */
rbq_status rbq_pack_tiles(const uint32_t *planes, rbq_shape s, uint32_t *tiles, void *stream);

/*
 * Scale tiles: the scales of a layer with one scale per row and 128-column
 * group (QBB summary, "Approach" and the W(4x1)A16g128 rows of "Key
 * results"), reordered so that a one-token kernel loads the scales of a
 * 16-row, 512-column unit (4 groups) together with its planes, K * 128 bytes
 * per unit:
 *   fp16 [T][C][K/2][4][4][2][4],  T = ceil(out / 16),  C = ceil(in / 512);
 *   element [t][c][p][g][q][kk][v] = scales[2p + kk][16t + 4q + v][4c + g],
 *   zero where the row (>= out) or the group (>= in / 128) does not exist.
 * Needs s.group_size == 128 and an even K; rbq_scale_tiles_bytes is 0
 * otherwise.
 */
size_t rbq_scale_tiles_bytes(rbq_shape s);

/*
 * rbq_pack_scale_tiles -- write the scale tiles of g128 scales.
 *   scales  device fp16 [K][out][in/128], 2-byte aligned (read only)
 *   tiles   device, rbq_scale_tiles_bytes(s) bytes, 16-byte aligned; every
 *           byte is written
 * s.group_size must be 128 and K even (else RBQ_ERR_UNSUPPORTED).  out == 0
 * or in == 0 enqueues nothing.  Errors as rbq_pack_tiles.
 */
rbq_status rbq_pack_scale_tiles(const uint16_t *scales, rbq_shape s, uint16_t *tiles, void *stream);

/* One op of a program. */
typedef struct rbq_program_op {
    const uint32_t *planes;   /* device, 16-byte aligned: [K][out][in/32], or the
                                 RBQ_LAYOUT_TILES copy (planes_layout) */
    const uint16_t *scales;   /* device, fp16 [K][out] (one scale per row), 2-byte aligned */
    const uint16_t *x;        /* device, fp16 [in], 16-byte aligned */
    uint16_t *y;              /* device, fp16 [out] ([out/2] with SILU_MUL), 2-byte aligned */
    int32_t out_features;     /* 1 .. 256 * number of compute units */
    int32_t in_features;      /* multiple of 128, at most 16384 */
    uint32_t epilogue;        /* RBQ_EPILOGUE_NONE or RBQ_EPILOGUE_SILU_MUL (out even) */
    int32_t wait_for;         /* -1, or an earlier op: this op reads x only after
                                 every op up to and including that one has
                                 written all of its y */
    uint32_t planes_layout;   /* RBQ_LAYOUT_ROWS or RBQ_LAYOUT_TILES; the
                                 results are the same bits in either */
    int32_t group_size;       /* 0: scales fp16 [K][out], one per row.
                                 128: one scale per row and 128-column group;
                                 planes in RBQ_LAYOUT_TILES and `scales` the
                                 scale tiles of rbq_pack_scale_tiles (16-byte
                                 aligned); K = 2 or 4.  The ops of one program
                                 are all of one kind. */
    int32_t tokens;           /* tokens T the op carries: 0 or 1 (x fp16 [in], y
                                 as above), 2 or 4 (x fp16 [T][in], y [T][out] or
                                 [T][out/2]; each token is quantised on its own,
                                 so token m's y equals that of a one-token op on
                                 row m of x).  Ops of several tokens take K = 2,
                                 per-row scales, RBQ_LAYOUT_TILES, no waits and
                                 in <= 12288 (T = 2) or in <= 4096 (T = 4);
                                 every op of a program has the same count. */
} rbq_program_op;

/* Bytes of the program image for n_ops ops on the current device (0 when
 * n_ops is outside 1 .. RBQ_PROGRAM_MAX_OPS). */
size_t rbq_program_bytes(int32_t n_ops);

/* Bytes of the counters a program run uses (int32 words: per op, one on
 * each of 8 separate 128-byte lines, and one for the run). */
size_t rbq_program_counters_bytes(int32_t n_ops);

/*
 * rbq_program_build -- check a list of ops and write its program image into
 * host memory (`image`, image_bytes >= rbq_program_bytes(n_ops)).  Host only;
 * enqueues nothing and needs no device.  The image is for the current device
 * (it depends on the number of compute units; 256 when no device is
 * visible), and rbq_program_run refuses it on another.  The caller copies it to device memory
 * (16-byte aligned) and passes both copies to rbq_program_run.
 *
 * Ordering rules, checked here: every workgroup runs the ops in list order on
 * its own rows, so two ops j < i that touch one buffer (i reads what j
 * wrote, i writes what j read, or both write it) must be ordered by a wait:
 * some op in j+1 .. i must have wait_for >= j.  An op's y may not overlap its
 * own x, or any op's planes or scales.
 * Errors: RBQ_ERR_INVALID_ARG (null pointer, bad shape, epilogue or
 * planes_layout, wait_for not an earlier op, an unordered overlap, image too
 * small),
 * RBQ_ERR_ALIGNMENT, RBQ_ERR_UNSUPPORTED (num_planes > 2 for per-row ops or
 * not 2 or 4 for g128 ops, g128 ops mixed with per-row ops or on the row
 * layout, in_features % 128 != 0 or > 16384, out_features too large, too
 * many ops).
 */
rbq_status rbq_program_build(const rbq_program_op *ops, int32_t n_ops, int32_t num_planes, void *image,
                             size_t image_bytes);

/*
 * rbq_program_run -- run a program on `stream`: one launch of one 16-wave
 * workgroup per compute unit.
 *   image        the host image written by rbq_program_build
 *   image_dev    device copy of the same bytes, 16-byte aligned (read only)
 *   counters_dev device int32, rbq_program_counters_bytes(n_ops) bytes, all
 *                zero before the first run;
 *                every run that completes leaves them zero again.  One set
 *                per program that may run concurrently with another.
 *   status_dev   device int32 or NULL: RBQ_STATUS_PROGRAM_* bits are OR-ed in
 * Needs the whole device: the waits between ops assume that every workgroup
 * of the launch is resident (they are bounded, and report
 * RBQ_STATUS_PROGRAM_TIMEOUT instead of hanging).
 * Errors: RBQ_ERR_INVALID_ARG (null pointer, an image that is not a valid
 * program for this device), RBQ_ERR_ALIGNMENT, RBQ_ERR_NO_DEVICE,
 * RBQ_ERR_HIP.
 */
rbq_status rbq_program_run(const void *image, const void *image_dev, int32_t *counters_dev,
                           int32_t *status_dev, void *stream);

/* ---------------------------------------------------------------------------
 * Coupled (QAT-style) forward and straight-through backward.
 *
 * RaBiT summary (paperlayer.ai), section 4.2 "Coupled Training" and the
 * "RaBiT training" procedure (section G): training keeps one shared fp32
 * weight W and learnable scales; each forward pass derives the binary cores
 * again from W, path by path, B_1 = sign(W), R_1 = W - a_1 B_1,
 * B_2 = sign(R_1), ...; the shared weight takes the whole gradient.  Here the
 * scales are given (the learnable ones), sign(0) = +1, every residual step is
 * one fp32 operation against the binary16 scale, and the backward is the
 * straight-through estimator: sign() passes gradients unchanged.
 * num_planes 1..4 (RBQ_ERR_UNSUPPORTED above), group_size 0 or 128.
 * ------------------------------------------------------------------------- */

/*
 * rbq_qat_encode -- binary cores of W for the given scales (the cascade
 * above; planes bit-identical to it).
 *   W       device fp32 [out][in], row-major (read only)
 *   scales  device binary16 [K][out][G] (read only)
 *   planes  device uint32 [K][out][in/32], written
 *   status  device int32 or NULL: RBQ_STATUS_NONFINITE_W is OR-ed in when W
 *           holds NaN or Inf (NaN takes -1 on every plane)
 * Errors: RBQ_ERR_INVALID_ARG (shape, null pointer), RBQ_ERR_ALIGNMENT,
 * RBQ_ERR_UNSUPPORTED (K > 4), RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP.
 */
rbq_status rbq_qat_encode(const float *W, rbq_shape s, const uint16_t *scales, uint32_t *planes,
                          int32_t *status, void *stream);

/*
 * rbq_qat_forward -- the coupled forward: planes = rbq_qat_encode(W, scales),
 * then Y = rbq_gemm(planes, scales, X) (the same kernels, tolerance and
 * workspace rules as rbq_gemm).  The planes are kept for the backward.
 *   X [M][in] fp16, Y [M][out] fp16, device; workspace as for rbq_gemm.
 * Errors: those of rbq_qat_encode and rbq_gemm.
 */
rbq_status rbq_qat_forward(const float *W, const uint16_t *scales, rbq_shape s, const uint16_t *X, int32_t M,
                           uint32_t *planes, uint16_t *Y, void *workspace, size_t ws_bytes, int32_t *status,
                           void *stream);

/*
 * rbq_qat_backward -- straight-through gradients of Y = X What^T,
 * What = sum_k a_k B_k, given dY:
 *   dW[r][j]       = sum_m dY[m][r] X[m][j]           fp32 [out][in]
 *   dscales[k][r][t] = sum over columns j of group t of B_k[r][j] dW[r][j]
 *                                                      fp32 [K][out][G]
 *   dX[m][j]       = sum_r dY[m][r] What[r][j]        fp32 [M][in]
 * Any of dX, dW may be NULL (not computed); dscales needs dW.  X, dY fp16
 * [M][in], [M][out]; planes and scales as written by the forward.  dW is
 * exact products with fp32 accumulation; dscales sums the fp32 dW in fp64;
 * dX forms What in fp32 and multiplies its two fp16 parts (relative 2^-22,
 * absolute 2^-25 where the lower part is subnormal) with fp32 accumulation.
 *   status  device int32 or NULL: RBQ_STATUS_SCALE_OVERFLOW is OR-ed in when
 *           a formed weight of What is not below 65520 in magnitude (or not
 *           finite); dX is then not meaningful
 *   workspace  device memory of rbq_qat_backward_workspace_bytes(s, M) bytes
 *           (0 for many tokens): with few tokens dX is computed in slices of
 *           the contraction whose fp32 partial sums it holds, added in slice
 *           order (deterministic); a smaller workspace (or NULL with
 *           ws_bytes 0) gives the same result from one slice, more slowly.
 *           Calls that share a workspace must be ordered on one stream.
 * Errors: RBQ_ERR_INVALID_ARG (shape, M < 0, a needed pointer NULL, dscales
 * without dW, ws_bytes > 0 with a NULL workspace), RBQ_ERR_ALIGNMENT,
 * RBQ_ERR_UNSUPPORTED (K > 4), RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP.
 */
size_t rbq_qat_backward_workspace_bytes(rbq_shape s, int32_t M);
rbq_status rbq_qat_backward(const uint32_t *planes, const uint16_t *scales, rbq_shape s, const uint16_t *X,
                            const uint16_t *dY, int32_t M, float *dX, float *dW, float *dscales, void *workspace,
                            size_t ws_bytes, int32_t *status, void *stream);

/*
 * rbq_probe_read -- measurement aid, not a step of the method: one launch that
 * reads `bytes` bytes at `buf` from device memory with 16-byte non-temporal
 * loads and discards them, so that a GEMV launch can be compared with a plain
 * read of the same size run the same way (the roofline of a kernel that reads
 * its packed planes once).
 *   buf   device memory, 16-byte aligned, `bytes` readable bytes (read only)
 *   sink  device uint32: written only if the folded loads hit a fixed magic
 *         value (practically never); keeps the loads from being dropped
 * Errors: RBQ_ERR_INVALID_ARG (null pointer), RBQ_ERR_ALIGNMENT,
 * RBQ_ERR_NO_DEVICE, RBQ_ERR_HIP.  bytes == 0 launches nothing.
 */
rbq_status rbq_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Kernel families rbq_gemm can use; RBQ_PATH_AUTO picks by shape and M. */
typedef enum rbq_path {
    RBQ_PATH_AUTO = 0,
    RBQ_PATH_VALU = 1,      /* plain fp32 VALU bit loop, any M */
    RBQ_PATH_DECODE = 2,    /* int8 MFMA on masked bits, 512-column chunks split over
                               8 waves, 5 tokens per pass */
    RBQ_PATH_PREFILL = 3,   /* fp16 MFMA, large M: What formed in registers by table
                               lookup (K <= 2) or unpacked into LDS (K = 3, 4) */
    RBQ_PATH_STREAM = 4,    /* int8 MFMA, whole rows streamed per wave: M <= 2, K <= 2,
                               in <= 16384 */
    RBQ_PATH_FLAT = 5,      /* int8 MFMA, one 16-wave workgroup per compute unit whose
                               (tile, chunk) units are split evenly over 12 waves while
                               4 build the activation image: M <= 2, K <= 2,
                               in <= 16384; taken for layers of many rows */
    RBQ_PATH_GROUP = 6,     /* int8 MFMA for one token with 128-column group scales
                               (group_size 128, K <= 4, in % 512 == 0, in <= 16384,
                               scales 8-byte aligned); the lanes that hold a group's
                               MFMA sums apply its scales.  Layout as RBQ_PATH_FLAT */
    RBQ_PATH_SPLIT = 7      /* fp16 MFMA for 2..16 tokens (per-row scales, K <= 2), What
                               formed in registers from the sign words, the input columns
                               split over workgroups; with several slices fp32 partial
                               outputs in the workspace, added in slice order by a
                               second kernel */
} rbq_path;

/* Forces rbq_gemm/rbq_gemv to one kernel family for the whole process (for
 * tests and A/B measurement).  A forced path that cannot take a call makes
 * that call return RBQ_ERR_UNSUPPORTED.  Returns the previous setting. */
rbq_path rbq_set_path(rbq_path p);

/* Waves that share one 16-row tile in RBQ_PATH_STREAM (1, 2 or 4; 0 = chosen
 * from the number of tiles, the default).  For tuning and A/B measurement;
 * results do not depend on it beyond fp32 rounding.  Returns the previous
 * setting, or -1 (and changes nothing) for any other value. */
int32_t rbq_set_stream_split(int32_t waves_per_tile);

/* The kernel family rbq_gemm would take for this shape and M. */
rbq_path rbq_select_path(rbq_shape s, int32_t M);

/* hipError_t of the last RBQ_ERR_HIP on the calling thread (0 if none). */
int32_t rbq_last_hip_error(void);

/* Static text for a status code. */
const char *rbq_status_string(rbq_status st);

/* Library version string. */
const char *rbq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RBQ_H */
