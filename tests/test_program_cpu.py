"""Host checks of rbq_program_build (no GPU): shapes, alignment, waits that
point forward, and the ordering rule for ops that share a buffer.  The
pointers are fake device addresses; the build only compares them."""
import ctypes

import pytest

import gemm_rbq_encode_amd as rbq

MiB = 1 << 20


def op(planes, scales, x, y, out=256, inf=512, epilogue=0, wait_for=-1, layout=0, group=0, tokens=0):
    return rbq.ProgramOp(planes, scales, x, y, out, inf, epilogue, wait_for, layout, group, tokens)


def build(ops, K=2, nbytes=None):
    L = rbq.lib()
    arr = (rbq.ProgramOp * len(ops))(*ops)
    n = int(L.rbq_program_bytes(len(ops)))
    assert n > 0
    buf = (ctypes.c_ubyte * (n if nbytes is None else nbytes))()
    return L.rbq_program_build(ctypes.cast(arr, ctypes.c_void_p), len(ops), K, ctypes.cast(buf, ctypes.c_void_p),
                               n if nbytes is None else nbytes)


# distinct fake buffers: weights at 1 GiB + k MiB, activations at 2 GiB + k MiB
def W(k):
    return (1 << 30) + k * MiB


def A(k):
    return (2 << 30) + k * MiB


def independent(n):
    return [op(W(2 * i), W(2 * i + 1), A(0), A(1 + i)) for i in range(n)]


def test_valid_programs_build():
    assert build(independent(1)) == rbq.RBQ_OK
    assert build(independent(128)) == rbq.RBQ_OK
    chain = [op(W(0), W(1), A(0), A(1)),
             op(W(2), W(3), A(1), A(2), wait_for=0),
             op(W(4), W(5), A(2), A(3), epilogue=rbq.RBQ_EPILOGUE_SILU_MUL, wait_for=1),
             op(W(6), W(7), A(3), A(0), out=512, inf=128, wait_for=2)]    # writes the first op's x
    assert build(chain) == rbq.RBQ_OK
    assert build(chain, K=1) == rbq.RBQ_OK


def test_bad_arguments():
    L = rbq.lib()
    assert L.rbq_program_build(None, 1, 2, None, 0) == rbq.RBQ_ERR_INVALID_ARG
    assert build([op(0, W(1), A(0), A(1))]) == rbq.RBQ_ERR_INVALID_ARG               # null planes
    assert build([op(W(0), W(1), A(0), A(1), out=0)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build([op(W(0), W(1), A(0), A(1), inf=100)]) == rbq.RBQ_ERR_INVALID_ARG   # not a multiple of 32
    assert build([op(W(0), W(1), A(0), A(1), inf=96)]) == rbq.RBQ_ERR_UNSUPPORTED    # not a multiple of 128
    assert build([op(W(0), W(1), A(0), A(1), inf=16512)]) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([op(W(0), W(1), A(0), A(1), epilogue=7)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build([op(W(0), W(1), A(0), A(1), out=255, epilogue=1)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build([op(W(0), W(1), A(0), A(1), wait_for=0)]) == rbq.RBQ_ERR_INVALID_ARG    # not earlier
    assert build(independent(2)[:1] + [op(W(2), W(3), A(0), A(5), wait_for=3)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build(independent(1), K=3) == rbq.RBQ_ERR_UNSUPPORTED
    assert build(independent(1), nbytes=16) == rbq.RBQ_ERR_INVALID_ARG
    assert int(rbq.lib().rbq_program_bytes(0)) == 0
    assert int(rbq.lib().rbq_program_bytes(rbq.RBQ_PROGRAM_MAX_OPS + 1)) == 0


def test_alignment():
    assert build([op(W(0) + 8, W(1), A(0), A(1))]) == rbq.RBQ_ERR_ALIGNMENT   # planes 16-byte
    assert build([op(W(0), W(1), A(0) + 8, A(1))]) == rbq.RBQ_ERR_ALIGNMENT   # x 16-byte
    assert build([op(W(0), W(1) + 1, A(0), A(1))]) == rbq.RBQ_ERR_ALIGNMENT
    assert build([op(W(0), W(1), A(0), A(1) + 1)]) == rbq.RBQ_ERR_ALIGNMENT


def test_unordered_sharing_is_refused():
    # op 1 reads op 0's y without waiting (read after write)
    raw = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(1), A(2))]
    assert build(raw) == rbq.RBQ_ERR_INVALID_ARG
    raw[1].wait_for = 0
    assert build(raw) == rbq.RBQ_OK
    # op 1 overwrites op 0's x (write after read)
    war = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(2), A(0) + 256, out=64)]
    assert build(war) == rbq.RBQ_ERR_INVALID_ARG
    war[1].wait_for = 0
    assert build(war) == rbq.RBQ_OK
    # both write one buffer (write after write)
    waw = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), A(1) + 64, out=64)]
    assert build(waw) == rbq.RBQ_ERR_INVALID_ARG
    # a wait on an op after the writer orders it too (every workgroup runs the ops in order)
    mid = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), A(2)), op(W(4), W(5), A(2), A(3), wait_for=1),
           op(W(6), W(7), A(1), A(4))]
    assert build(mid) == rbq.RBQ_OK
    # ... but a wait on an op before the writer does not
    early = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), A(2)), op(W(4), W(5), A(1), A(3), wait_for=0),
             op(W(6), W(7), A(2), A(4))]
    assert build(early) == rbq.RBQ_ERR_INVALID_ARG


def test_outputs_may_not_overlap_inputs_or_weights():
    assert build([op(W(0), W(1), A(0), A(0) + 128)]) == rbq.RBQ_ERR_INVALID_ARG     # y inside its own x
    assert build([op(W(0), W(1), A(0), W(0) + 4096)]) == rbq.RBQ_ERR_INVALID_ARG    # y inside the planes
    two = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), W(1))]                   # y on another op's scales
    assert build(two) == rbq.RBQ_ERR_INVALID_ARG


def test_planes_layout():
    assert build([op(W(0), W(1), A(0), A(1), layout=rbq.RBQ_LAYOUT_TILES)]) == rbq.RBQ_OK
    mixed = [op(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), A(2), layout=rbq.RBQ_LAYOUT_TILES)]
    assert build(mixed) == rbq.RBQ_OK
    assert build([op(W(0), W(1), A(0), A(1), layout=2)]) == rbq.RBQ_ERR_INVALID_ARG
    # 250 x 640, K = 2: the row layout takes 2*250*20*4 = 40000 bytes, the
    # tile layout 2 * 16 tiles * 2 chunks * 1 KB = 65536; a y between the two
    # ends overlaps only the tiled planes
    y = W(0) + 50000
    assert build([op(W(0), W(1), A(0), y, out=250, inf=640)]) == rbq.RBQ_OK
    assert build([op(W(0), W(1), A(0), y, out=250, inf=640, layout=rbq.RBQ_LAYOUT_TILES)]) == \
        rbq.RBQ_ERR_INVALID_ARG


def test_tiles_bytes_and_pack_arguments():
    L = rbq.lib()
    assert int(L.rbq_tiles_bytes(rbq.shape(250, 640, 2))) == 2 * 16 * 2 * 1024
    assert int(L.rbq_tiles_bytes(rbq.shape(4096, 11008, 2))) == 2 * 256 * 22 * 1024
    assert int(L.rbq_tiles_bytes(rbq.shape(16, 512, 1))) == 1024
    assert int(L.rbq_tiles_bytes(rbq.shape(0, 512, 1))) == 0
    assert int(L.rbq_tiles_bytes(rbq.shape(16, 100, 1))) == 0          # not a shape
    s = rbq.shape(250, 640, 2)
    assert L.rbq_pack_tiles(None, s, W(4), None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_pack_tiles(W(0), s, None, None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_pack_tiles(W(0), rbq.shape(250, 96, 2), W(4), None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_pack_tiles(W(0) + 4, s, W(4), None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_pack_tiles(W(0), s, W(4) + 8, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_pack_tiles(W(0), s, W(0) + 39984, None) == rbq.RBQ_ERR_INVALID_ARG   # overlap
    # (no call here passes every check: on a machine with a device it would
    # launch on these fake addresses)


def gop(planes, scales, x, y, out=256, inf=512, **kw):
    return op(planes, scales, x, y, out, inf, layout=rbq.RBQ_LAYOUT_TILES, group=128, **kw)


def test_group_programs():
    """Programs of g128 ops: K = 2 or 4, tiled planes, scale tiles 16-byte
    aligned, no per-row ops beside them."""
    for K in (2, 4):
        assert build([gop(W(0), W(1), A(0), A(1)), gop(W(2), W(3), A(1), A(2), wait_for=0)], K=K) == rbq.RBQ_OK
    assert build([gop(W(0), W(1), A(0), A(1))], K=1) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([gop(W(0), W(1), A(0), A(1))], K=3) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([op(W(0), W(1), A(0), A(1), group=128)], K=4) == rbq.RBQ_ERR_UNSUPPORTED      # row layout
    assert build([op(W(0), W(1), A(0), A(1), group=64)], K=2) == rbq.RBQ_ERR_INVALID_ARG
    assert build([gop(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), A(2))], K=2) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([op(W(0), W(1), A(0), A(1)), gop(W(2), W(3), A(0), A(2))], K=2) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([gop(W(0), W(1) + 8, A(0), A(1))], K=4) == rbq.RBQ_ERR_ALIGNMENT             # scale tiles
    # per-row programs stay at K <= 2
    assert build([op(W(0), W(1), A(0), A(1), layout=rbq.RBQ_LAYOUT_TILES)], K=4) == rbq.RBQ_ERR_UNSUPPORTED
    # 250 x 640, K = 4: scale tiles 16 tiles * 2 chunks * 512 bytes = 16384; a y
    # 10000 bytes into them overlaps (the [K][out][G] scales would end at 10000)
    assert build([gop(W(0), W(1), A(0), W(1) + 12000, out=250, inf=640)], K=4) == rbq.RBQ_ERR_INVALID_ARG
    assert build([gop(W(0), W(1), A(0), W(1) + 16384, out=250, inf=640)], K=4) == rbq.RBQ_OK


def test_scale_tiles_bytes_and_pack_arguments():
    L = rbq.lib()
    assert int(L.rbq_scale_tiles_bytes(rbq.shape(5120, 13824, 4, 128))) == 320 * 27 * 512
    assert int(L.rbq_scale_tiles_bytes(rbq.shape(250, 640, 2, 128))) == 16 * 2 * 256
    assert int(L.rbq_scale_tiles_bytes(rbq.shape(250, 640, 2, 0))) == 0       # per-row scales
    assert int(L.rbq_scale_tiles_bytes(rbq.shape(250, 640, 3, 128))) == 0     # odd K
    s = rbq.shape(250, 640, 4, 128)
    assert L.rbq_pack_scale_tiles(None, s, W(4), None) == rbq.RBQ_ERR_INVALID_ARG
    assert L.rbq_pack_scale_tiles(W(0), rbq.shape(250, 640, 4, 0), W(4), None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_pack_scale_tiles(W(0), rbq.shape(250, 640, 3, 128), W(4), None) == rbq.RBQ_ERR_UNSUPPORTED
    assert L.rbq_pack_scale_tiles(W(0) + 1, s, W(4), None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_pack_scale_tiles(W(0), s, W(4) + 8, None) == rbq.RBQ_ERR_ALIGNMENT
    assert L.rbq_pack_scale_tiles(W(0), s, W(0) + 16, None) == rbq.RBQ_ERR_INVALID_ARG        # overlap


def pop(planes, scales, x, y, out=256, inf=512, **kw):
    """a two-token op on the tile layout"""
    kw.setdefault("tokens", 2)
    return op(planes, scales, x, y, out, inf, layout=rbq.RBQ_LAYOUT_TILES, **kw)


def test_two_token_programs():
    """Two-token ops: K = 2, per-row scales, tile layout, no waits, in <=
    12288, every op of the program with two tokens; x and y hold two rows,
    which the overlap checks count."""
    many = [pop(W(2 * i), W(2 * i + 1), A(0), A(1 + i), out=4096 + 16 * i, inf=4096) for i in range(64)]
    assert build(many) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(1), out=4096, inf=11008)]) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(1), out=4096, inf=12288)]) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(1), out=4096, inf=12416)]) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([pop(W(0), W(1), A(0), A(1), epilogue=rbq.RBQ_EPILOGUE_SILU_MUL)]) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(1))], K=1) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([op(W(0), W(1), A(0), A(1), tokens=2)]) == rbq.RBQ_ERR_UNSUPPORTED            # row layout
    assert build([pop(W(0), W(1), A(0), A(1)), pop(W(2), W(3), A(1), A(2), wait_for=0)]) == \
        rbq.RBQ_ERR_UNSUPPORTED                                                                   # a wait
    assert build([pop(W(0), W(1), A(0), A(1)), op(W(2), W(3), A(0), A(2), layout=rbq.RBQ_LAYOUT_TILES)]) == \
        rbq.RBQ_ERR_INVALID_ARG                                                                   # mixed counts
    assert build([pop(W(0), W(1), A(0), A(1), tokens=3)]) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([pop(W(0), W(1), A(0), A(1), tokens=8)]) == rbq.RBQ_ERR_UNSUPPORTED
    # four-token ops: inputs of at most 4096 columns
    four = [pop(W(2 * i), W(2 * i + 1), A(0), A(1 + i), out=22016 if i % 2 else 4096, inf=4096, tokens=4)
            for i in range(96)]
    assert build(four) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(1), inf=4224, tokens=4)]) == rbq.RBQ_ERR_UNSUPPORTED
    assert build([pop(W(0), W(1), A(0), A(1), tokens=4), pop(W(2), W(3), A(0), A(2))]) == rbq.RBQ_ERR_INVALID_ARG
    # x of 4 x 512 fp16 = 4096 bytes
    assert build([pop(W(0), W(1), A(0), A(0) + 3072, tokens=4)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build([pop(W(0), W(1), A(0), A(0) + 4096, tokens=4)]) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(1), tokens=-1)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build([op(W(0), W(1), A(0), A(1), layout=rbq.RBQ_LAYOUT_TILES, tokens=1),
                  op(W(2), W(3), A(0), A(2), layout=rbq.RBQ_LAYOUT_TILES, tokens=0)]) == rbq.RBQ_OK
    assert build([gop(W(0), W(1), A(0), A(1), tokens=2)], K=4) == rbq.RBQ_ERR_UNSUPPORTED
    # x of 2 x 512 fp16 = 2048 bytes: a y 1024 bytes in overlaps only the second token's row
    assert build([op(W(0), W(1), A(0), A(0) + 1024, layout=rbq.RBQ_LAYOUT_TILES)]) == rbq.RBQ_OK
    assert build([pop(W(0), W(1), A(0), A(0) + 1024)]) == rbq.RBQ_ERR_INVALID_ARG
    # y of 2 x 256 fp16 = 1024 bytes: a second op's y 600 bytes on overlaps it
    assert build([pop(W(0), W(1), A(0), A(1)), pop(W(2), W(3), A(0), A(1) + 600)]) == rbq.RBQ_ERR_INVALID_ARG
    assert build([pop(W(0), W(1), A(0), A(1)), pop(W(2), W(3), A(0), A(1) + 1024)]) == rbq.RBQ_OK
