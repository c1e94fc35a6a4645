"""GPU parity of programs of g128 ops (one scale per row and 128-column
group, K = 2 or 4), through the C ABI.

rbq_pack_scale_tiles is a permutation of the scales with zero padding: its
output must equal, byte for byte, the same permutation written here with
numpy reshapes.  Every op of a program must meet the single-call bar against
the fp64 oracle (relative L2 error <= 1e-3, max abs error <= 1e-2 rms(y_ref));
the fp32 sums of a program are added in a fixed order, so two runs give the
same bits.
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


def assert_close(y, yref, what):
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    yref = np.asarray(yref, dtype=np.float64).reshape(-1)
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(yref ** 2))
    rel = np.linalg.norm(y - yref) / max(np.linalg.norm(yref), 1e-300)
    mx = np.abs(y - yref).max()
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e}"
    assert mx <= MAX_ABS_RMS * rms, f"{what}: max-abs {mx:.3e} vs rms {rms:.3e}"


def scale_tiles_reference(s, inf):
    """numpy: fp16 bits [K][out][G] -> [T][C][K/2][4 groups][4 quads][2][4 rows], zero padded."""
    K, out, G = s.shape
    T, C = -(-out // 16), -(-inf // 512)
    S = np.zeros((K, T * 16, C * 4), dtype=np.uint16)
    S[:, :out, :G] = s
    S = S.reshape(K // 2, 2, T, 4, 4, C, 4)            # [pp][kk][t][q][v][c][g]
    return S.transpose(2, 5, 0, 6, 3, 1, 4).reshape(T, C, K * 64)


def g128_layer(out, inf, K, seed):
    """Random planes; scales a ~ 1/sqrt(K in) per (row, group) with random signs."""
    p = workloads.random_planes(K, out, inf, seed=seed)
    rng = np.random.default_rng(seed + 1)
    G = inf // 128
    a = rng.uniform(0.5, 1.5, (K, out, G)) / np.sqrt(K * inf)
    s = (a * rng.choice([-1.0, 1.0], (K, out, G))).astype(np.float16).view(np.uint16)
    return p, s


def device_op(p, s, inf, x, y, **kw):
    pt = torch.from_numpy(np.ascontiguousarray(p).view(np.int32)).to(dev())
    st = torch.from_numpy(np.ascontiguousarray(s).view(np.float16)).to(dev())
    return dict({"planes": rbq.pack_tiles(pt), "scales": rbq.pack_scale_tiles(st, inf), "x": x, "y": y,
                 "group_size": 128, "out_features": p.shape[1]}, **kw)


def run_program(ops, K):
    prog = rbq.Program(ops, num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert not prog.counters.any()
    return prog


@pytest.mark.parametrize("K,out,inf", [(2, 16, 512), (4, 17, 128), (4, 300, 640), (2, 4100, 1152),
                                       (4, 5120, 13824), (8, 33, 1024)])
def test_pack_scale_tiles_matches_the_permutation(K, out, inf):
    _, s = g128_layer(out, inf, K, seed=out + inf)
    st = torch.from_numpy(s.view(np.float16)).to(dev())
    ref = scale_tiles_reference(s, inf)
    assert rbq.scale_tiles_bytes(rbq.shape(out, inf, K, 128)) == ref.nbytes
    tiles = torch.full(ref.shape, float("nan"), dtype=torch.float16, device=dev())   # every byte is written
    print(f"pack_scale_tiles K={K} {out}x{inf}", flush=True)
    rbq.pack_scale_tiles(st, inf, tiles=tiles)
    torch.cuda.synchronize()
    assert np.array_equal(tiles.cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("K", [2, 4])
def test_group_program_matches_oracle(K):
    """The Llama-2-13B shapes and ragged ones (rows not a multiple of 16,
    one group, inputs not a multiple of 512, a gate/up pair epilogue), in one
    program; run twice, the second run giving the same bits."""
    shapes = [(5120, 5120, 0), (13824, 5120, 0), (5120, 13824, 0), (300, 640, 0), (17, 128, 0),
              (4100, 1152, 0), (34, 512, 1)]
    ops, host = [], []
    for i, (o, n, epi) in enumerate(shapes):
        p, s = g128_layer(o, n, K, seed=700 + 10 * K + i)
        x = torch.from_numpy(workloads.gaussian_activations(1, n, seed=70 + i)[0].view(np.float16)).to(dev())
        y = torch.full((o // 2 if epi else o,), float("nan"), dtype=torch.float16, device=dev())
        ops.append(device_op(p, s, n, x, y, epilogue=epi))
        host.append((p, s, x.cpu().numpy().view(np.uint16), epi))
    print(f"group program K={K} ({len(ops)} ops)", flush=True)
    prog = run_program(ops, K)
    first = [o["y"].clone() for o in ops]
    for i, ((p, s, xb, epi), op) in enumerate(zip(host, ops)):
        yr = oracle.gemm(p, s, xb, 128)
        if epi:
            yr = oracle.silu_mul(yr)
        assert_close(op["y"].cpu().numpy(), yr[0], f"op {shapes[i]}")
    for o in ops:
        o["y"].fill_(float("nan"))
    prog.run()
    torch.cuda.synchronize()
    for i, (a, o) in enumerate(zip(first, ops)):
        assert torch.equal(a.view(torch.int16), o["y"].view(torch.int16)), f"op {shapes[i]}: second run differs"


def test_group_program_chain_with_waits():
    """Two decoder layers (q/k/v on x, o on q, gate/up with silu * up, down;
    the next layer on down's output), each op waiting for the one before it.
    Each op is checked against the oracle on the input the program gave it,
    which the op may only have read after its producer had written all of it."""
    K, d, ff = 4, 1024, 2816
    specs = [("qkv", 3 * d, d, 0), ("o", d, d, 0), ("gu", 2 * ff, d, 1), ("down", d, ff, 0)]
    x0 = torch.from_numpy(workloads.gaussian_activations(1, d, seed=31)[0].view(np.float16)).to(dev())
    ops, host = [], []
    cur = x0
    for L in range(2):
        for j, (name, o, n, epi) in enumerate(specs):
            p, s = g128_layer(o, n, K, seed=8000 + 10 * L + j)
            y = torch.full((o // 2 if epi else o,), float("nan"), dtype=torch.float16, device=dev())
            xin = cur[:n] if name == "o" else cur
            ops.append(device_op(p, s, n, xin, y, epilogue=epi, wait_for=len(ops) - 1))
            host.append((name, p, s, epi, xin))
            cur = y
    ops[0]["wait_for"] = -1
    print("group chain", flush=True)
    prog = run_program(ops, K)
    for i, ((name, p, s, epi, xin), op) in enumerate(zip(host, ops)):
        yr = oracle.gemm(p, s, xin.cpu().numpy().view(np.uint16)[None, :], 128)
        if epi:
            yr = oracle.silu_mul(yr)
        assert_close(op["y"].cpu().numpy(), yr[0], f"chain op {i} ({name})")
    ref = [o["y"].clone() for o in ops]
    for rep in range(2):
        for o in ops:
            o["y"].fill_(float("nan"))
        prog.run()
        torch.cuda.synchronize()
        assert not prog.counters.any()
        for i, (a, o) in enumerate(zip(ref, ops)):
            assert torch.equal(a.view(torch.int16), o["y"].view(torch.int16)), (rep, i)


def test_many_independent_g128_ops():
    """Thirty independent g128 ops (K = 4) of random ragged shapes, spread
    over op groups, against the oracle; two runs give the same bits."""
    rng = np.random.default_rng(17)
    ops, host = [], []
    for i in range(30):
        o = int(rng.integers(1, 3000))
        n = int(rng.integers(1, 65)) * 128
        p, s = g128_layer(o, n, 4, seed=9000 + i)
        x = torch.from_numpy(workloads.gaussian_activations(1, n, seed=900 + i)[0].view(np.float16)).to(dev())
        y = torch.full((o,), float("nan"), dtype=torch.float16, device=dev())
        ops.append(device_op(p, s, n, x, y))
        host.append((p, s, x.cpu().numpy().view(np.uint16)))
    print("many g128 ops", flush=True)
    prog = run_program(ops, 4)
    first = [o["y"].clone() for o in ops]
    for i, ((p, s, xb), op) in enumerate(zip(host, ops)):
        assert_close(op["y"].cpu().numpy(), oracle.gemm(p, s, xb, 128)[0], f"op {i} {p.shape[1]}x{xb.shape[0]}")
    prog.run()
    torch.cuda.synchronize()
    for i, (a, o) in enumerate(zip(first, ops)):
        assert torch.equal(a.view(torch.int16), o["y"].view(torch.int16)), f"op {i}: second run differs"
