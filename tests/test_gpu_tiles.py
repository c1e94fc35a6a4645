"""GPU checks of the tile layout (RBQ_LAYOUT_TILES) through the C ABI.

rbq_pack_tiles is a permutation of 16-byte pieces with zero padding: its
output must equal, byte for byte, the same permutation written here with
numpy reshapes.  A program reading tiled planes must give exactly the bits
of the same program on the row layout (the sums are exact integers, so the
order of the weight bytes in memory cannot change them), and the row-layout
program is itself held to the oracle and to the per-call kernels in
test_gpu_program.py; one op per shape is also checked against the oracle here.
"""
import numpy as np
import pytest
import torch

import gemm_rbq_encode_amd as rbq
import oracle
import workloads

pytestmark = pytest.mark.gpu
REL_L2 = 1e-3
MAX_ABS_RMS = 1e-2


def dev():
    return torch.device("cuda:0")


def tiles_reference(p):
    """numpy: [K][out][words] -> [K][T][C][g][i][j] = p[k][16t+i][16c+4g+j], zero padded."""
    K, out, words = p.shape
    T, C = -(-out // 16), -(-words // 16)
    P = np.zeros((K, T * 16, C * 16), dtype=np.uint32)
    P[:, :out, :words] = p
    return P.reshape(K, T, 16, C, 4, 4).transpose(0, 1, 3, 4, 2, 5).reshape(K, T, C, 256)


def layer(out, inf, K, seed):
    p = workloads.random_planes(K, out, inf, seed=seed)
    rng = np.random.default_rng(seed + 1)
    a = rng.uniform(0.5, 1.5, (K, out, 1)) / np.sqrt(K * inf)
    s = (a * rng.choice([-1.0, 1.0], (K, out, 1))).astype(np.float16).view(np.uint16)
    return p, s


def to_dev(p, s):
    return (torch.from_numpy(np.ascontiguousarray(p).view(np.int32)).to(dev()),
            torch.from_numpy(np.ascontiguousarray(s).reshape(s.shape[0], -1).view(np.float16)).to(dev()))


def assert_close(y, yref, what):
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    yref = np.asarray(yref, dtype=np.float64).reshape(-1)
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(yref ** 2))
    assert np.linalg.norm(y - yref) <= REL_L2 * np.linalg.norm(yref), what
    assert np.abs(y - yref).max() <= MAX_ABS_RMS * rms, what


@pytest.mark.parametrize("K,out,inf", [(1, 16, 512), (2, 17, 128), (2, 4100, 640), (3, 300, 1152),
                                       (4, 33, 16384), (2, 4096, 11008), (8, 48, 1024)])
def test_pack_tiles_matches_the_permutation(K, out, inf):
    p = workloads.random_planes(K, out, inf, seed=out + inf + K)
    pt = torch.from_numpy(p.view(np.int32)).to(dev())
    ref = tiles_reference(p)
    assert int(rbq.tiles_bytes(rbq.shape(out, inf, K))) == ref.nbytes
    tiles = torch.full(ref.shape, -1, dtype=torch.int32, device=dev())   # every byte must be written
    print(f"pack_tiles K={K} {out}x{inf}", flush=True)
    rbq.pack_tiles(pt, tiles=tiles)
    torch.cuda.synchronize()
    assert np.array_equal(tiles.cpu().numpy().view(np.uint32), ref)
    assert torch.equal(rbq.pack_tiles(pt), tiles)


def test_pack_tiles_empty_shapes_enqueue_nothing():
    L = rbq.lib()
    buf = torch.full((64,), 7, dtype=torch.int32, device=dev())
    stream = torch.cuda.current_stream().cuda_stream
    assert L.rbq_pack_tiles(buf.data_ptr(), rbq.shape(0, 512, 2), buf[32:].data_ptr(), stream) == rbq.RBQ_OK
    assert L.rbq_pack_tiles(buf.data_ptr(), rbq.shape(16, 0, 2), buf[32:].data_ptr(), stream) == rbq.RBQ_OK
    torch.cuda.synchronize()
    assert (buf == 7).all()


def run_program(ops, K):
    prog = rbq.Program(ops, num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert not prog.counters.any()
    return prog


@pytest.mark.parametrize("K", [1, 2])
def test_program_on_tiles_equals_rows(K):
    """The fused Llama-2-7B decode shapes and ragged ones (rows not a
    multiple of 16, inputs not a multiple of 512, gate/up pairs), each op
    once on each layout, in one program with both layouts mixed (the kernel
    that chooses the addressing per op), and again in a program of tiled
    ops only (the kernel built for that layout alone)."""
    shapes = [(12288, 4096, 0), (4096, 4096, 0), (22016, 4096, 1), (4096, 11008, 0), (17, 384, 0),
              (4100, 640, 0), (300, 16384, 0), (34, 512, 1), (1, 128, 0)]
    ops, host = [], []
    for i, (o, n, epi) in enumerate(shapes):
        p, s = layer(o, n, K, seed=500 + i)
        pt, st = to_dev(p, s)
        x = torch.from_numpy(workloads.gaussian_activations(1, n, seed=50 + i)[0].view(np.float16)).to(dev())
        ny = o // 2 if epi else o
        y_rows = torch.full((ny,), float("nan"), dtype=torch.float16, device=dev())
        y_tiles = torch.full((ny,), float("nan"), dtype=torch.float16, device=dev())
        tiles = rbq.pack_tiles(pt)
        ops.append({"planes": pt, "scales": st, "x": x, "y": y_rows, "epilogue": epi})
        ops.append({"planes": tiles, "scales": st, "x": x, "y": y_tiles, "epilogue": epi})
        host.append((p, s, x.cpu().numpy().view(np.uint16), epi, y_rows, y_tiles))
    print(f"program rows+tiles K={K} ({len(ops)} ops)", flush=True)
    run_program(ops, K)
    only = [dict(o, y=torch.full_like(o["y"], float("nan"))) for o in ops[1::2]]
    print(f"program tiles only K={K} ({len(only)} ops)", flush=True)
    run_program(only, K)
    for i, (p, s, xb, epi, y_rows, y_tiles) in enumerate(host):
        assert torch.equal(y_rows.view(torch.int16), y_tiles.view(torch.int16)), f"op {shapes[i]}"
        assert torch.equal(y_rows.view(torch.int16), only[i]["y"].view(torch.int16)), f"op {shapes[i]}, tiles only"
        yr = oracle.gemm(p, s, xb)
        if epi:
            yr = oracle.silu_mul(yr)
        assert_close(y_tiles.cpu().numpy(), yr[0], f"op {shapes[i]} against the oracle")


def test_chain_on_tiles_equals_rows():
    """A two-layer decoder chain with waits (qkv -> o -> gate/up with
    silu * up -> down -> next qkv) on tiled planes, against the same chain on
    the row layout, bit for bit."""
    x0 = workloads.gaussian_activations(1, 4096, seed=21)[0]
    specs = [("qkv", 12288, 4096, 0), ("o", 4096, 4096, 0), ("gu", 22016, 4096, 1), ("down", 4096, 11008, 0)]
    results = {}
    weights = []
    for L in range(2):
        for j, (name, o, n, epi) in enumerate(specs):
            p, s = layer(o, n, 2, seed=9000 + 10 * L + j)
            weights.append(to_dev(p, s))
    for layout in ("rows", "tiles"):
        cur = torch.from_numpy(x0.view(np.float16).copy()).to(dev())
        ops, outs = [], []
        for L in range(2):
            for j, (name, o, n, epi) in enumerate(specs):
                pt, st = weights[4 * L + j]
                y = torch.full((o // 2 if epi else o,), float("nan"), dtype=torch.float16, device=dev())
                ops.append({"planes": pt if layout == "rows" else rbq.pack_tiles(pt), "scales": st,
                            "x": cur[:n] if name == "o" else cur, "y": y, "epilogue": epi,
                            "wait_for": len(ops) - 1})
                outs.append(y)
                cur = y
        print(f"chain on {layout}", flush=True)
        run_program(ops, 2)
        results[layout] = outs
    for i, (a, b) in enumerate(zip(results["rows"], results["tiles"])):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"chain op {i}"
