"""GPU parity of programs (rbq_program_build / rbq_program_run): lists of
one-token GEMVs in one persistent launch, through the C ABI.

Every op must meet the single-call bar against the fp64 oracle (relative
L2 error <= 1e-3, max abs error <= 1e-2 rms(y_ref)).  The program's kernel
does the flat kernel's arithmetic (same quantisation, exact int32 sums, same
fp32 epilogue), so each op must also equal rbq_gemv / rbq_gemm_ex forced to
the flat family bit for bit -- for chains too, where that shows that every
op read its input only after the op it waits for had written all of it.
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


def assert_close(y, yref, what, rel_l2=REL_L2, max_abs_rms=MAX_ABS_RMS):
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    yref = np.asarray(yref, dtype=np.float64).reshape(-1)
    assert np.isfinite(y).all(), what
    rms = np.sqrt(np.mean(yref ** 2))
    rel = np.linalg.norm(y - yref) / max(np.linalg.norm(yref), 1e-300)
    mx = np.abs(y - yref).max()
    assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e}"
    assert mx <= max_abs_rms * rms, f"{what}: max-abs {mx:.3e} vs rms {rms:.3e}"


def layer(out, inf, K, seed, norm=True):
    """Random planes; scales a_k ~ 1/sqrt(K in) so that y ~ N(0, 1) for x ~ N(0, 1)."""
    p = workloads.random_planes(K, out, inf, seed=seed)
    rng = np.random.default_rng(seed + 1)
    a = rng.uniform(0.5, 1.5, (K, out, 1)) / np.sqrt(K * inf) if norm else rng.uniform(0.001, 0.05, (K, out, 1))
    s = (a * rng.choice([-1.0, 1.0], (K, out, 1))).astype(np.float16).view(np.uint16)
    return p, s


def to_dev(p, s):
    return (torch.from_numpy(np.ascontiguousarray(p).view(np.int32)).to(dev()),
            torch.from_numpy(np.ascontiguousarray(s).reshape(s.shape[0], -1).view(np.float16)).to(dev()))


def eager_flat(pt, st, x, epilogue=0):
    old = rbq.set_path(rbq.PATH_FLAT)
    try:
        y = rbq.gemm(pt, st, x.reshape(1, -1), 0, epilogue=epilogue)
    finally:
        rbq.set_path(old)
    return y.reshape(-1)


def interleave_gate_up(p, s):
    """rows (gate i, up i) -> 2i, 2i+1"""
    n = p.shape[1] // 2
    perm = np.stack([np.arange(n), np.arange(n) + n], axis=1).reshape(-1)
    return np.ascontiguousarray(p[:, perm]), np.ascontiguousarray(s[:, perm])


@pytest.mark.parametrize("K", [1, 2])
def test_independent_llama2_7b_shapes(K):
    """The fused Llama-2-7B decode shapes, two layers' worth, all on one x
    (and down on its own x): no op waits."""
    shapes = [(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008)] * 2
    xs = {n: torch.from_numpy(workloads.gaussian_activations(1, n, seed=n)[0].view(np.float16)).to(dev())
          for n in (4096, 11008)}
    host, ops, ys = [], [], []
    for i, (o, n) in enumerate(shapes):
        p, s = layer(o, n, K, seed=100 + i, norm=False)
        pt, st = to_dev(p, s)
        y = torch.full((o,), float("nan"), dtype=torch.float16, device=dev())
        host.append((p, s))
        ops.append({"planes": pt, "scales": st, "x": xs[n], "y": y})
        ys.append(y)
    prog = rbq.Program(ops, num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert not prog.counters.any()
    for i, ((o, n), (p, s), op) in enumerate(zip(shapes, host, ops)):
        xb = xs[n].cpu().numpy().view(np.uint16)
        assert_close(ys[i].cpu().numpy(), oracle.gemm(p, s, xb)[0], f"op {i} {o}x{n}")
        ref = eager_flat(op["planes"], op["scales"], xs[n])
        assert torch.equal(ys[i].view(torch.int16), ref.view(torch.int16)), f"op {i} differs from rbq_gemv"


def build_chain(layers, K=2, seed=7):
    """Decoder-layer chain on distinct buffers: qkv on x; o on q (the first
    4096 qkv outputs); gate/up (rows interleaved) with silu * up on o's
    output; down on h; the next layer's qkv on down's output.  Each op waits
    for the one before it."""
    x0 = workloads.gaussian_activations(1, 4096, seed=seed)[0]
    host, ops, outs = [], [], []
    x_dev = torch.from_numpy(x0.view(np.float16).copy()).to(dev())
    cur = x_dev
    for L in range(layers):
        specs = [("qkv", 12288, 4096, 0), ("o", 4096, 4096, 0), ("gu", 22016, 4096, 1), ("down", 4096, 11008, 0)]
        for j, (name, o, n, epi) in enumerate(specs):
            p, s = layer(o, n, K, seed=seed * 1000 + 10 * L + j)
            if epi:
                p, s = interleave_gate_up(p, s)
            pt, st = to_dev(p, s)
            ny = o // 2 if epi else o
            y = torch.full((ny,), float("nan"), dtype=torch.float16, device=dev())
            xin = cur[:n] if name == "o" else cur
            ops.append({"planes": pt, "scales": st, "x": xin, "y": y, "epilogue": epi,
                        "wait_for": len(ops) - 1})
            host.append((name, p, s, epi))
            outs.append(y)
            cur = y
    ops[0]["wait_for"] = -1
    return x0, host, ops, outs


@pytest.mark.parametrize("layers", [1, 3])
def test_chain_with_waits(layers):
    x0, host, ops, outs = build_chain(layers)
    prog = rbq.Program(ops, num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert not prog.counters.any()
    # eager: the same calls one by one (flat kernel), bit for bit
    for i, op in enumerate(ops):
        ref = eager_flat(op["planes"], op["scales"], op["x"], op.get("epilogue", 0))
        assert torch.equal(outs[i].view(torch.int16), ref.view(torch.int16)), f"op {i} ({host[i][0]})"
    # the oracle, run down the same chain from x0 with each output rounded to
    # fp16 as the library stores it.  Both sides round differently at every
    # op and the differences travel down the chain (the layers keep y ~ N(0,1),
    # so they are not amplified on average): op d of the chain is held to
    # sqrt(d + 1) times the single-op bar.
    x = x0.view(np.uint16)[None, :]
    for d, ((name, p, s, epi), y) in enumerate(zip(host, outs)):
        xin = x[:, :4096] if name == "o" else x
        yr = oracle.gemm(p, s, np.ascontiguousarray(xin))
        if epi:
            yr = oracle.silu_mul(yr)
        f = np.sqrt(d + 1.0)
        assert_close(y.cpu().numpy(), yr[0], f"chain op {d} ({name})", REL_L2 * f, MAX_ABS_RMS * f)
        x = yr.astype(np.float16).view(np.uint16)


def test_repeated_runs_and_graph_replays():
    """Counters return to zero after every run, so runs can repeat; the run
    captured in a HIP graph replays bit for bit, with eager work between."""
    x0, host, ops, outs = build_chain(2, seed=11)
    prog = rbq.Program(ops, num_planes=2)
    prog.run()
    torch.cuda.synchronize()
    ref = [y.clone() for y in outs]
    for _ in range(2):
        for y in outs:
            y.fill_(float("nan"))
        prog.run()
        torch.cuda.synchronize()
        assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(outs, ref))
        assert not prog.counters.any()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        prog.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, j)
        assert not prog.counters.any()
        _ = eager_flat(ops[0]["planes"], ops[0]["scales"], ops[0]["x"])


@pytest.mark.parametrize("K", [1, 2])
def test_ragged_and_small_ops(K):
    """Rows not a multiple of 16, fewer tiles than workgroups (idle
    workgroups and waves), the widest and narrowest inputs, the most rows,
    an odd number of gate/up pairs, and a run of waits."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shapes = [(1, 128, 0), (17, 384, 0), (300, 16384, 0), (4100, 640, 0), (16 * 16 * cus, 128, 0),
              (34, 512, 1), (4098, 2048, 1), (23, 1024, 0)]
    host, ops, outs = [], [], []
    for i, (o, n, epi) in enumerate(shapes):
        p, s = layer(o, n, K, seed=300 + i)
        pt, st = to_dev(p, s)
        x = torch.from_numpy(workloads.gaussian_activations(1, n, seed=i)[0].view(np.float16)).to(dev())
        y = torch.full((o // 2 if epi else o,), float("nan"), dtype=torch.float16, device=dev())
        ops.append({"planes": pt, "scales": st, "x": x, "y": y, "epilogue": epi,
                    "wait_for": i - 1 if i % 3 == 2 else -1})
        host.append((p, s, x.cpu().numpy().view(np.uint16), epi))
        outs.append(y)
    prog = rbq.Program(ops, num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i, ((p, s, xb, epi), y) in enumerate(zip(host, outs)):
        yr = oracle.gemm(p, s, xb)
        if epi:
            yr = oracle.silu_mul(yr)
        assert_close(y.cpu().numpy(), yr[0], f"op {i} {shapes[i]}")


def test_many_small_ops():
    """300 ops of 64 x 256 (most workgroups idle in each), chained in runs of
    ten through distinct buffers."""
    n_ops = 300
    ops, host, outs = [], [], []
    x = torch.from_numpy(workloads.gaussian_activations(1, 256, seed=5)[0].view(np.float16)).to(dev())
    xs_host = [x.cpu().numpy().view(np.uint16)]
    cur = x
    for i in range(n_ops):
        p, s = layer(256, 256, 2, seed=1000 + i)
        pt, st = to_dev(p, s)
        y = torch.empty(256, dtype=torch.float16, device=dev())
        chained = i % 10 != 0
        ops.append({"planes": pt, "scales": st, "x": cur if chained else x, "y": y,
                    "wait_for": i - 1 if chained else -1})
        host.append((p, s, chained))
        outs.append(y)
        cur = y
    prog = rbq.Program(ops, num_planes=2)
    prog.run()
    torch.cuda.synchronize()
    for i, op in enumerate(ops):
        ref = eager_flat(op["planes"], op["scales"], op["x"])
        assert torch.equal(outs[i].view(torch.int16), ref.view(torch.int16)), f"op {i}"
    p, s, _ = host[0]
    assert_close(outs[0].cpu().numpy(), oracle.gemm(p, s, xs_host[0])[0], "op 0")


def test_mismatched_device_image_runs_nothing():
    a_ops, b_ops = [], []
    for ops, seed in ((a_ops, 1), (b_ops, 2)):
        p, s = layer(64, 128, 2, seed=seed)
        pt, st = to_dev(p, s)
        x = torch.zeros(128, dtype=torch.float16, device=dev())
        ops.append({"planes": pt, "scales": st, "x": x, "y": torch.full((64,), 5.0, dtype=torch.float16,
                                                                       device=dev())})
    pa, pb = rbq.Program(a_ops), rbq.Program(b_ops + b_ops[:0])
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    L = rbq.lib()
    import ctypes
    st = L.rbq_program_run(ctypes.cast(pa._host, ctypes.c_void_p), pb.image_dev.data_ptr(), pa.counters.data_ptr(),
                           status.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == rbq.RBQ_OK
    assert int(status.item()) & rbq.RBQ_STATUS_PROGRAM_MISMATCH
    assert bool((a_ops[0]["y"] == 5.0).all()) and bool((b_ops[0]["y"] == 5.0).all())
    # a corrupted host image is refused before launch
    bad = (ctypes.c_ubyte * len(pa._host)).from_buffer_copy(bytes(pa._host))
    bad[40] ^= 1
    assert L.rbq_program_run(ctypes.cast(bad, ctypes.c_void_p), pa.image_dev.data_ptr(), pa.counters.data_ptr(),
                             None, None) == rbq.RBQ_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", [1, 2])
def test_many_independent_ragged_ops(seed):
    """Sixty independent ops of random ragged shapes (rows 1..6000, inputs
    128..16384 columns), half on the tile layout, some sharing x with the op
    before them (the image is reused when both fall in one op group): the
    program splits them over op groups, each group planning its own slots
    and images.  Every op must equal rbq_gemv's flat kernel bit for bit, on
    two runs in a row."""
    rng = np.random.default_rng(seed)
    ops, outs = [], []
    prev_x = None
    for i in range(60):
        o = int(rng.integers(1, 6001))
        n = int(rng.integers(1, 129)) * 128
        if prev_x is not None and rng.random() < 0.3 and prev_x.numel() == n:
            x = prev_x
        else:
            x = torch.from_numpy(workloads.gaussian_activations(1, n, seed=seed * 1000 + i)[0].view(np.float16)).to(dev())
        p, s = layer(o, n, 2, seed=seed * 5000 + i)
        pt, st = to_dev(p, s)
        epi = int(o % 2 == 0 and rng.random() < 0.2)
        y = torch.full((o // 2 if epi else o,), float("nan"), dtype=torch.float16, device=dev())
        planes = rbq.pack_tiles(pt) if i % 2 else pt
        ops.append({"planes": planes, "scales": st, "x": x, "y": y, "epilogue": epi, "rows_planes": pt})
        outs.append(y)
        prev_x = x
    prog = rbq.Program([{k: v for k, v in op.items() if k != "rows_planes"} for op in ops], num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    for run in range(2):
        for y in outs:
            y.fill_(float("nan"))
        print(f"many ragged ops seed={seed} run {run}", flush=True)
        prog.run(status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert not prog.counters.any()
        for i, op in enumerate(ops):
            ref = eager_flat(op["rows_planes"], op["scales"], op["x"], op["epilogue"])
            assert torch.equal(outs[i].view(torch.int16), ref.view(torch.int16)), f"run {run} op {i}"


@pytest.mark.parametrize("M", [4, 16])
def test_batch_tokens_as_ops_on_shared_planes(M):
    """A batch of M tokens through one linear as M one-token ops on the same
    planes (tile layout), one after another, as a decode step for a batch
    runs them: every token's output meets the oracle's bar, equals rbq_gemv
    on the flat kernel bit for bit, and the batch agrees with rbq_gemm at M
    tokens within the same bar."""
    shapes = [(12288, 4096), (4096, 11008)]
    ops, checks = [], []
    for i, (o, n) in enumerate(shapes):
        p, s = layer(o, n, 2, seed=300 + i)
        pt, st = to_dev(p, s)
        tiles = rbq.pack_tiles(pt)
        X = workloads.gaussian_activations(M, n, seed=310 + i)
        xd = torch.from_numpy(X.view(np.float16)).to(dev())
        Y = torch.full((M, o), float("nan"), dtype=torch.float16, device=dev())
        for m in range(M):
            ops.append({"planes": tiles, "scales": st, "x": xd[m], "y": Y[m]})
        checks.append((p, s, pt, st, X, xd, Y))
    prog = rbq.Program(ops, num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i, (p, s, pt, st, X, xd, Y) in enumerate(checks):
        yref = oracle.gemm(p, s, X)
        for m in range(M):
            assert_close(Y[m].cpu().numpy(), yref[m], f"linear {i} token {m}")
            ref = eager_flat(pt, st, xd[m])
            assert torch.equal(Y[m].view(torch.int16), ref.view(torch.int16)), f"linear {i} token {m}"
        yb = rbq.gemm(pt, st, xd, 0)
        assert_close(Y.cpu().numpy(), yb.cpu().numpy(), f"linear {i} against rbq_gemm at {M} tokens")


def two_token_program(shapes, seed, T=2):
    """Ops of T tokens (x [T][in], y [T][out] or [T][out / 2]) on tiled planes."""
    host, ops, outs = [], [], []
    for i, (o, n, epi) in enumerate(shapes):
        p, s = layer(o, n, 2, seed=seed + i)
        if epi:
            p, s = interleave_gate_up(p, s)
        pt, st = to_dev(p, s)
        X = workloads.gaussian_activations(T, n, seed=seed + 50 + i)
        xd = torch.from_numpy(X.view(np.float16)).to(dev())
        y = torch.full((T, o // 2 if epi else o), float("nan"), dtype=torch.float16, device=dev())
        ops.append({"planes": rbq.pack_tiles(pt), "scales": st, "x": xd, "y": y, "epilogue": epi, "tokens": T})
        host.append((p, s, pt, st, X, xd, epi))
        outs.append(y)
    return host, ops, outs


def one_token_program(pt, st, x, epi):
    """the same op on one token, as a one-op program on the tile layout"""
    y = torch.full((pt.shape[1] // 2 if epi else pt.shape[1],), float("nan"), dtype=torch.float16, device=dev())
    rbq.Program([{"planes": rbq.pack_tiles(pt), "scales": st, "x": x, "y": y, "epilogue": epi}], num_planes=2).run()
    torch.cuda.synchronize()
    return y


def check_two_token_outputs(host, outs, shapes, against_flat=False):
    for i, ((p, s, pt, st, X, xd, epi), y) in enumerate(zip(host, outs)):
        yr = oracle.gemm(p, s, X)
        if epi:
            yr = oracle.silu_mul(yr)
        for m in range(X.shape[0]):
            what = f"op {i} {shapes[i]} token {m}"
            assert_close(y[m].cpu().numpy(), yr[m], what)
            ref = eager_flat(pt, st, xd[m], epilogue=epi) if against_flat else one_token_program(pt, st, xd[m], epi)
            assert torch.equal(y[m].view(torch.int16), ref.view(torch.int16)), f"{what}: not the one-token result"


def test_two_token_ops_llama2_7b_shapes():
    """The fused Llama-2-7B decode shapes with two tokens per op (gate/up with
    the SiLU-mul epilogue): each token's output equals rbq_gemv's on that
    token bit for bit, and the run leaves the counters clear for the next."""
    shapes = [(12288, 4096, 0), (4096, 4096, 0), (22016, 4096, 1), (4096, 11008, 0)] * 2
    host, ops, outs = two_token_program(shapes, seed=500)
    prog = rbq.Program(ops, num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert not prog.counters.any()
    check_two_token_outputs(host, outs, shapes, against_flat=True)
    first = [y.clone() for y in outs]
    for y in outs:
        y.fill_(float("nan"))
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for a, b in zip(first, outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_two_token_ops_ragged():
    """Rows not a multiple of 16, inputs not a multiple of 512 (padded tile
    units), the widest two-token input (12288 columns), few tiles, and
    consecutive ops on the same x (the image is built once)."""
    shapes = [(1, 128, 0), (17, 384, 0), (300, 12288, 0), (4100, 640, 0), (34, 512, 1), (4098, 2048, 1),
              (23, 1152, 0), (999, 1152, 0)]
    host, ops, outs = two_token_program(shapes, seed=700)
    # op 7 reads op 6's x
    ops[7]["x"] = ops[6]["x"]
    host[7] = host[7][:4] + host[6][4:6] + host[7][6:]
    prog = rbq.Program(ops, num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_two_token_outputs(host, outs, shapes)


def test_four_token_ops_llama2_7b_shapes():
    """The fused Llama-2-7B decode shapes of 4096 inputs with four tokens per
    op (12 of the 16 MFMA columns), gate/up with the SiLU-mul epilogue: each
    token's output equals rbq_gemv's bit for bit; a second run repeats it."""
    shapes = [(12288, 4096, 0), (4096, 4096, 0), (22016, 4096, 1)] * 2
    host, ops, outs = two_token_program(shapes, seed=900, T=4)
    prog = rbq.Program(ops, num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert not prog.counters.any()
    check_two_token_outputs(host, outs, shapes, against_flat=True)
    first = [y.clone() for y in outs]
    for y in outs:
        y.fill_(float("nan"))
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for a, b in zip(first, outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_four_token_ops_ragged():
    """Four-token ops on ragged shapes up to the widest input they take (4096
    columns), an odd number of gate/up pairs, and two ops on one x."""
    shapes = [(1, 128, 0), (17, 384, 0), (300, 4096, 0), (4100, 640, 0), (34, 512, 1), (4098, 2048, 1),
              (23, 1152, 0), (999, 1152, 0)]
    host, ops, outs = two_token_program(shapes, seed=1100, T=4)
    ops[7]["x"] = ops[6]["x"]
    host[7] = host[7][:4] + host[6][4:6] + host[7][6:]
    prog = rbq.Program(ops, num_planes=2)
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    prog.run(status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check_two_token_outputs(host, outs, shapes)
