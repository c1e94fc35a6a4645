"""rbq: residual-binarized linear layers on AMD MI355X (gfx950).

y = sum_k a_k (.) (B_k x) with K packed +-1 sign planes and fp16 scales per
row or per row per group of 128 columns, encoded by sequential residual
binarization (RaBiT summary, paperlayer.ai, sections 4.1 and 4.2; QBB
summary, atlas.scime.ai, "Approach").  The work runs in HIP kernels of
librbq.so behind the C ABI in include/rbq.h; this package only marshals
torch tensors into those calls.
"""
from ._binding import (  # noqa: F401
    PATH_AUTO, PATH_DECODE, PATH_FLAT, PATH_GROUP, PATH_PREFILL, PATH_SPLIT, PATH_STREAM, PATH_VALU,
    RBQ_ENCODE_FORCE_SERIAL, RBQ_EPILOGUE_NONE, RBQ_EPILOGUE_SILU_MUL, RBQ_ERR_ALIGNMENT, RBQ_ERR_HIP, RBQ_ERR_INVALID_ARG,
    RBQ_ERR_NO_DEVICE, RBQ_ERR_SCRATCH_LIMIT, RBQ_LAYOUT_ROWS, RBQ_LAYOUT_TILES, RBQ_ERR_UNSUPPORTED, RBQ_NOALLOC_SCRATCH_BYTES, RBQ_OK, RBQ_PROGRAM_MAX_OPS, RBQ_STATUS_NONFINITE_W,
    RBQ_STATUS_PLANES_KEPT, RBQ_STATUS_PROGRAM_MISMATCH, RBQ_STATUS_PROGRAM_TIMEOUT, RBQ_STATUS_REFIT_KEPT, RBQ_STATUS_SCALE_OVERFLOW, LIB_PATH, Program, ProgramOp, RbqError, RbqLibraryMissing, Shape, check,
    encode, encode_dual, encode_dual_workspace_bytes, gemm, gemm_dual, gemm_noalloc, gemv, gemv_dual, groups_per_row, last_hip_error, lib, pack_scale_tiles, pack_tiles, planes_bytes, probe_read, qat_backward, qat_encode, qat_forward, rebinarize, refit,
    scale_tiles_bytes, scales_bytes, tiles_bytes,
    select_path, set_path, set_stream_split, shape, status_string, version,
)
