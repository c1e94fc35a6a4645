"""Benchmark: K=2 batch-1 GEMV on the Llama-2-7B decoder linears.

One step is one decode token through the seven linears (q, k, v, o 4096x4096;
gate, up 11008x4096; down 4096x11008) of each of 32 layers.  By default q, k,
v are stacked row-wise into one 12288x4096 matrix and gate, up into one
22016x4096 matrix, as decode engines lay them out (4 GEMVs per layer, 128 per
step; every row is encoded on its own, so the stacked encoding is exactly the
separate ones); --layout separate runs the 7 linears as 224 GEMVs.  Each
layer has its own copy of the encoded planes and scales (1.63 GB in total,
far more than the L2 and Infinity Cache), so every step streams the weights
from HBM.  Each GEMV reads the token of its decoder-layer input (one per
layer for the attention input, o_proj, the MLP input and down_proj; q/k/v
and gate/up share theirs) and writes its own output.  The weights are seeded
synthetic N(0, 0.02^2) matrices with 0.1 % outliers x20, encoded on the GPU
by rbq_encode; activations are N(0, 1) fp16.

The step runs as ONE persistent launch (rbq_program_run over the step's
GEMVs); the same step as one rbq_gemv launch per GEMV in a HIP graph is
reported beside it.

Reported (one JSON line):
  value      whole-job GB/s = algorithmic bytes per step / wall time per step
             (bytes = K*out*in/8 planes + 2*K*out scales + 2*in x + 2*out y)
  roofline   the program kernel: algorithmic bytes per launch / its mean
             device duration (HIP events around back-to-back launches on its
             stream), against MI355X's 8 TB/s HBM peak; traffic from
             FETCH_SIZE + WRITE_SIZE counters when recorded for this source
  cpu_baseline  the CPU oracle on the host cores on a bounded sample, and on
             one thread
  launches   the step as per-GEMV launches; per launch group its mean launch
             time and a streaming read of the same plane bytes (rbq_probe_read)
  read_probe the step's plane bytes read as per-matrix launches and as one
  decode_layer_chain  the 32 layers chained (each GEMV reads the previous
             one's output; gate/up with the SiLU-mul epilogue), as one
             program launch and as per-GEMV launches
  other_layout  the same step in the other layout (separate: 224 GEMVs) as
             one program launch
  encode / refit / encode_refit_per_shape / gemv_dual_per_shape  the other
             entry points on the same shapes
  other_workloads  skinny M=4 and M=16 per call, the batch-4 and batch-16
             decode steps as program launches (several-token ops),
             Llama-2-13B K=4 g128 per call and its decode step as one
             program, and the Llama-3-8B prefill set with K = 3 and 4 beside
             it (--no-extra skips them; --workload runs one of them on its
             own line)
  qat        the coupled forward (cores re-derived from W, then the layer)
             and the straight-through backward on the Llama-2-7B shapes

Every timing starts after about 0.3 s of untimed back-to-back runs of the
same work (clocks settle under load) and the --warmup steps.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "K=2 batch-1 GEMV effective GB/s and % HBM peak on Llama-2-7B layers"
DTYPE_INT8_LIMBS = ("i8x3: x as three int8 limbs of a 22-bit fixed-point value, sign bits as int8 0/1, "
                    "exact int32 accumulation")


def dtype_of(path_name):
    if path_name in ("prefill", "split"):
        return "f16 MFMA, f32 accumulation"
    return "f32" if path_name == "valu" else DTYPE_INT8_LIMBS


def gemv_bytes(out_f, in_f, K, G, M=1):
    return K * out_f * in_f // 8 + 2 * K * out_f * G + 2 * M * in_f + 2 * M * out_f


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--kernel-reps", type=int, default=3,
                    help="passes over all layers for the per-launch kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--path", choices=["auto", "valu", "decode", "stream", "flat", "group", "split"],
                    default="auto")
    ap.add_argument("--split", type=int, default=0,
                    help="waves per 16-row tile in the streaming kernel (0 = automatic)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--layout", choices=["fused", "separate"], default="fused",
                    help="fused: q/k/v stacked into one 12288x4096 matrix and gate/up into one "
                         "22016x4096 matrix (4 launches per layer); separate: 7 launches per layer")
    ap.add_argument("--planes-layout", choices=["tiles", "rows"], default="tiles",
                    help="plane layout the decode program reads: tiles (RBQ_LAYOUT_TILES, packed once "
                         "from the row layout by rbq_pack_tiles) or rows ([K][out][in/32])")
    ap.add_argument("--workload", default="llama2_7b",
                    choices=["llama2_7b", "llama2_7b_skinny", "llama2_7b_skinny_program", "llama2_13b_g128",
                             "llama2_13b_g128_program", "llama3_8b_prefill"],
                    help="the default is the headline decode GEMV; the others print their own line")
    ap.add_argument("--tokens", type=int, default=0, help="token count for llama2_7b_skinny (4 or 16)")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave the skinny, 13B g128 and prefill sets out of the decode line")
    ap.add_argument("--encode-counter-pass", action="store_true",
                    help="for hardware-counter runs: encoder launches on the Llama-2-7B (K=2) and "
                         "Llama-2-13B g128 (K=4) shapes, each after a cache-flushing copy, then exit")
    ap.add_argument("--counter-pass", action="store_true",
                    help="for hardware-counter runs: a few eager launches of each decode shape "
                         "(no graph, no timing), then a plain copy of known size")
    return ap.parse_args()


def path_names(rbq):
    return {rbq.PATH_VALU: "valu", rbq.PATH_DECODE: "decode", rbq.PATH_PREFILL: "prefill",
            rbq.PATH_STREAM: "stream", rbq.PATH_FLAT: "flat", rbq.PATH_GROUP: "group",
            rbq.PATH_SPLIT: "split"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU path is not built.", file=sys.stderr)
        sys.exit(2)
    if args.encode_counter_pass:
        encode_counter_pass(args)
        return
    if args.counter_pass:
        counter_pass(args)
    elif args.workload == "llama2_7b":
        bench_decode(args)
    elif args.workload == "llama2_13b_g128_program":
        import torch

        import gemm_rbq_encode_amd as rbq
        import workloads
        torch.cuda.set_device(0)
        print(json.dumps(group_program_step(args, torch, rbq, workloads, torch.device("cuda:0"),
                                            cpu_seconds=args.cpu_seconds)), flush=True)
    elif args.workload == "llama2_7b_skinny_program":
        import torch

        import gemm_rbq_encode_amd as rbq
        import workloads
        torch.cuda.set_device(0)
        print(json.dumps(skinny_program_step(args, torch, rbq, workloads, torch.device("cuda:0"), args.tokens or 4,
                                             cpu_seconds=args.cpu_seconds, layout=args.layout)), flush=True)
    else:
        bench_layer_set(args)


COPY_PROBE_BYTES = 256 << 20
TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "gemv_llama2_7b_decode_hbm_traffic.json")
TRAFFIC_PROFILE_13B = os.path.join(ROOT, "profiles", "gemv_llama2_13b_g128_program_hbm_traffic.json")
TRAFFIC_PROFILE_BATCH = os.path.join(ROOT, "profiles", "gemv_llama2_7b_batch_program_hbm_traffic.json")


def profile_entry(shape_key, kernel_prefix, path=None):
    """The recorded counter entry for this launch (shape key and kernel name
    prefix), or None when there is none or the kernel's source has changed
    since it was taken."""
    import hashlib
    try:
        with open(path or TRAFFIC_PROFILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    for e in doc.get("entries", []):
        if e["shape"] != shape_key or not e["kernel"].startswith(kernel_prefix):
            continue
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_rbq_encode_amd", "csrc",
                           e["source"])
        try:
            with open(src, "rb") as f:
                digest = hashlib.sha256(f.read()).hexdigest()
        except OSError:
            return None
        return e if digest == e["source_sha256"] else None
    return None


def measured_traffic(shape_key, kernel_prefix, path=None):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated against a copy
    of known size) recorded for this launch, or None."""
    e = profile_entry(shape_key, kernel_prefix, path)
    return None if e is None else e.get("traffic_bytes")


def rocprof_mean_us(shape_key, kernel_prefix="gemv_program_kernel", path=None):
    """Mean kernel duration (us) in the recorded rocprofv3 kernel trace of the
    benchmark run, or None."""
    e = profile_entry(shape_key, kernel_prefix, path)
    return None if e is None else e.get("rocprof_mean_us")


def counter_pass(args):
    """Launches for `rocprofv3 --pmc`: the decode step's program (as the
    benchmark builds it) three times, then each fused decode shape 8 times
    through rbq_gemv (rotating the layers' copies, so no launch finds its
    planes in a cache), then torch copies of a 256 MiB buffer, whose read and
    write bytes calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    import gemm_rbq_encode_amd as rbq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "llama2_7b_skinny_program":
        skinny_counter_pass(args, torch, rbq, workloads, dev, args.tokens or 4)
        return
    wl = workloads.WORKLOADS["llama2_7b"]
    K, group = wl.num_planes, wl.group_size
    groups, layers, shapes, widths, Ws, _, _ = decode_sets(torch, rbq, workloads, wl, dev, args.layout,
                                                           args.layers)
    del Ws
    xs = decode_activations(torch, workloads, wl, dev, args.layout, widths, args.layers)
    ys = [[torch.empty(sh.out_features, dtype=torch.float16, device=dev) for sh in shapes]
          for _ in range(args.layers)]
    ops = [{"planes": program_planes(rbq, args, layers[l][i][0]), "scales": layers[l][i][1], "x": xs[l][i],
            "y": ys[l][i]} for l in range(args.layers) for i in range(len(groups))]
    prog = rbq.Program(ops, num_planes=K)
    nbytes = sum(gemv_bytes(sh.out_features, sh.in_features, K, 1) for sh in shapes) * args.layers
    for _ in range(3):
        prog.run()
    torch.cuda.synchronize()
    print(f"counter pass: {program_key(args)} x3 ({len(ops)} ops, "
          f"{nbytes} algorithmic bytes per launch)", flush=True)
    del prog
    for op in ops:
        op["planes"] = None
    for i, sh in enumerate(shapes):
        for l in range(min(8, args.layers)):
            rbq.gemv(layers[l][i][0], layers[l][i][1], xs[l][i], group, y=ys[l][i])
        torch.cuda.synchronize()
        print(f"counter pass: {sh.out_features}x{sh.in_features} x{min(8, args.layers)} "
              f"({gemv_bytes(sh.out_features, sh.in_features, K, 1)} algorithmic bytes per launch)", flush=True)
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"counter pass: copy of {COPY_PROBE_BYTES} bytes x4", flush=True)


def skinny_counter_pass(args, torch, rbq, workloads, dev, M):
    """Launches for `rocprofv3 --pmc` (with --workload llama2_7b_skinny_program):
    the batch-M decode step as the benchmark's per-linear programs (four-token
    ops for the 4096-column inputs, two-token ops for down), each run three
    times in step order, then torch copies of a 256 MiB buffer for the
    calibration."""
    wl = workloads.WORKLOADS["llama2_7b_skinny"]
    K = wl.num_planes
    groups, layers, shapes, widths, Ws, _, _ = decode_sets(torch, rbq, workloads, wl, dev, "fused", args.layers)
    del Ws
    tiles = [[rbq.pack_tiles(p) for p, _ in layer] for layer in layers]
    slots = X_SLOTS["fused"]
    xs = {sl: torch.from_numpy(workloads.layer_activations(wl, widths[i], args.layers * M, sl).view(
        np.float16)).to(dev).reshape(args.layers, M, widths[i]) for i, sl in enumerate(slots)}
    progs = []
    for i, sh in enumerate(shapes):
        tok = 4 if sh.in_features <= 4096 else 2
        ys = [torch.empty((M, sh.out_features), dtype=torch.float16, device=dev) for _ in range(args.layers)]
        progs.append((sh, tok, rbq.Program([{"planes": tiles[l][i], "scales": layers[l][i][1],
                                              "x": xs[slots[i]][l][m:m + tok], "y": ys[l][m:m + tok], "tokens": tok}
                                             for l in range(args.layers) for m in range(0, M, tok)], num_planes=K),
                      ys))
    for _ in range(3):
        for sh, tok, pr, _ in progs:
            pr.run()
    torch.cuda.synchronize()
    for sh, tok, pr, _ in progs:
        nb = gemv_bytes(sh.out_features, sh.in_features, K, 1, M) * args.layers
        print(f"skinny counter pass: {sh.out_features}x{sh.in_features}, {args.layers} layers, {M} tokens in ops "
              f"of {tok}: {pr.n_ops} ops x3 ({nb} algorithmic bytes per launch)", flush=True)
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"skinny counter pass: copy of {COPY_PROBE_BYTES} bytes x4", flush=True)


def encode_counter_pass(args):
    """Launches for `rocprofv3 --pmc`: rbq_encode, then rbq_rebinarize,
    three times each on each Llama-2-7B shape (per-row scales, K=2) and
    Llama-2-13B shape (g128, K=4), each launch after a copy of a 256 MiB
    buffer that evicts W from the caches; the copies' read and write bytes
    calibrate the counters."""
    import torch

    import gemm_rbq_encode_amd as rbq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for out_f, in_f, K, group in ((4096, 4096, 2, 0), (11008, 4096, 2, 0), (4096, 11008, 2, 0),
                                  (5120, 5120, 4, 128), (13824, 5120, 4, 128), (5120, 13824, 4, 128)):
        g = torch.Generator(device="cpu").manual_seed(out_f * 31 + in_f + K)
        W = (torch.randn((out_f, in_f), generator=g) * 0.02).to(dev)
        p, sc = rbq.encode(W, K, group)
        for _ in range(3):
            dst.copy_(src)
            rbq.encode(W, K, group, planes=p, scales=sc)
        # then rbq_rebinarize with those scales (W read, planes rewritten)
        for _ in range(3):
            dst.copy_(src)
            rbq.rebinarize(W, p, sc, group)
        torch.cuda.synchronize()
        nbytes = 4 * W.numel() + 4 * p.numel() + 2 * sc.numel()
        print(f"encode counter pass: {out_f}x{in_f} K={K} g={group} x3 encode, x3 rebinarize "
              f"({nbytes} algorithmic bytes each)", flush=True)
        del W, p, sc


def graph_launch_us(torch, dev, fns, reps):
    """Mean device time per launch (us) of the launches `fns`: they are
    captured once in a HIP graph on a side stream and the graph is replayed
    `reps` times between two HIP events recorded on that same stream, so the
    host never sits between two launches."""
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        graph.replay()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(side)
        for _ in range(reps):
            graph.replay()
        b.record(side)
    b.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * len(fns))


def rotation_copies(W, total_bytes=640 * 2 ** 20):
    """Copies of W whose combined size exceeds the caches (32 MB L2 + 256 MB
    MALL) about twice, so that a launch cycling over them reads W from HBM."""
    n = max(1, -(-total_bytes // (4 * W.numel())))
    return [W] + [W.clone() for _ in range(n - 1)]


def graph_ms(torch, dev, fns, reps):
    """Milliseconds per replay of one HIP graph holding the calls `fns`
    (captured on a side stream, replayed back to back `reps` times)."""
    stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def group_program_step(args, torch, rbq, workloads, dev, n_layers=40, cpu_seconds=4.0):
    """The Llama-2-13B decode step with K = 4 and one scale per 128-column
    group (QBB "Key results", W(4x1)A16g128), fused layout, n_layers layers,
    each with its own copy of the weights (planes and scales in their tile
    layouts, packed once), as ONE program launch: 4 GEMVs per layer, each
    reading its own activations.  Reports whole-job GB/s of algorithmic
    bytes, the kernel's mean launch time from HIP events, and the layer-0
    outputs against rbq_gemv (the per-call g128 kernel) run on the same
    inputs.  Returns the JSON object."""
    wl = workloads.WORKLOADS["llama2_13b_g128"]
    K, group = wl.num_planes, wl.group_size
    groups, layers1, shapes, widths, Ws, p_enc, s_enc = decode_sets(torch, rbq, workloads, wl, dev, "fused", 1)
    del Ws, p_enc, s_enc
    base = layers1[0]
    tiles = [[(rbq.pack_tiles(p), rbq.pack_scale_tiles(sc, sh.in_features)) for (p, sc), sh in zip(base, shapes)]
             for _ in range(n_layers)]
    xs = decode_activations(torch, workloads, wl, dev, "fused", widths, n_layers)
    ys = [[torch.empty(sh.out_features, dtype=torch.float16, device=dev) for sh in shapes] for _ in range(n_layers)]
    ops = [{"planes": tiles[l][i][0], "scales": tiles[l][i][1], "x": xs[l][i], "y": ys[l][i], "group_size": group,
            "out_features": shapes[i].out_features} for l in range(n_layers) for i in range(len(groups))]
    per_op = [gemv_bytes(sh.out_features, sh.in_features, K, sh.in_features // group) for sh in shapes]
    nbytes = sum(per_op) * n_layers
    prog = rbq.Program(ops, num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    run = (lambda: prog.run(status))
    settle(torch, run)
    us = event_launch_us(torch, run, stream, max(args.steps, 20))
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    if int(status.item()) != 0:
        raise rbq.RbqError(rbq.RBQ_ERR_HIP, f"program status {int(status.item()):#x}")
    # layer 0 against the per-call kernel on the row layouts (both are held
    # to the oracle's bound in the tests; they add their fp32 sums in
    # different orders)
    diff = 0.0
    for i, (p, sc) in enumerate(base):
        ref = rbq.gemv(p, sc, xs[0][i], group)
        diff = max(diff, float((ys[0][i].float() - ref.float()).abs().max() / ref.float().abs().max().clamp_min(1e-30)))
    line = {"metric": f"K={K} g128 batch-1 GEMV effective GB/s on Llama-2-13B layers, decode step as one program",
            "value": round(nbytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "ms_per_step": round(ms, 4),
            "dtype": DTYPE_INT8_LIMBS,
            "config": {"workload": "llama2_13b_g128_decode_program", "layers": n_layers, "layout": "fused",
                       "ops_per_layer": {name: f"{sh.out_features}x{sh.in_features}"
                                         for (name, _), sh in zip(groups, shapes)},
                       "num_planes": K, "group_size": group, "tokens": 1, "bytes_per_step": nbytes,
                       "planes_layout": "tiles (rbq_pack_tiles), scales as scale tiles (rbq_pack_scale_tiles)"},
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "traffic": measured_traffic(f"program_fused_{n_layers}layers_g128", "gemv_program_kernel",
                                                     TRAFFIC_PROFILE_13B),
                         "kernel": f"gemv_program_kernel<{K}> g128 ({len(ops)} ops)",
                         "bytes_per_launch": nbytes, "mean_launch_us": round(us, 2),
                         "rocprof_mean_launch_us": rocprof_mean_us(f"program_fused_{n_layers}layers_g128",
                                                                   path=TRAFFIC_PROFILE_13B)},
            "layer0_max_rel_diff_vs_rbq_gemv": diff, "cpu_baseline": None}
    if cpu_seconds > 0:
        samples = [(p.cpu().numpy().view(np.uint32), sc.cpu().numpy().view(np.uint16),
                    xs[0][i].cpu().numpy().view(np.uint16)[None, :], group, per_op[i])
                   for i, (p, sc) in enumerate(base)]
        line["cpu_baseline"] = oracle_baseline(samples, cpu_seconds, max_reps=20)
        line["cpu_baseline"]["sample"] = "layer 0 at M=1: " + line["cpu_baseline"]["sample"]
    del prog, tiles, xs, ys, base, layers1
    torch.cuda.empty_cache()
    return line


def skinny_program_step(args, torch, rbq, workloads, dev, M, cpu_seconds=4.0, layout="fused"):
    """The Llama-2-7B decode step for a batch of M tokens (K = 2, fused
    layout, args.layers layers with their own weights, planes in the tile
    layout) as program launches, in three forms of the same arithmetic (each
    token quantised on its own, as in rbq_gemm):
      * four- and two-token ops (M a multiple of 4): q/k/v, o and gate/up
        (4096 inputs) as ops of four tokens, whose limbs fill 12 of the 16
        MFMA columns, so a unit of planes feeds four tokens for the same
        MFMAs; down (11008 inputs, too wide for a four-token image) as ops of
        two tokens; one launch per linear (the reported value), or one
        launch for the four-token ops and one for the two-token ones;
      * two-token ops (M even), one launch;
      * one-token ops on shared planes, one launch.
    The ops of a linear run one after another, so its planes come from HBM
    once and from the caches otherwise.  A form whose launches would exceed
    RBQ_PROGRAM_MAX_OPS ops is left out.  Reports whole-job GB/s of
    algorithmic bytes (planes and scales once, M tokens of x and y), the
    step's launch time from HIP events, and layer 0 against rbq_gemm at M
    tokens.  Returns the JSON object, or None when no form fits."""
    wl = workloads.WORKLOADS["llama2_7b_skinny"]
    K, group = wl.num_planes, wl.group_size
    n_layers = args.layers
    groups, layers, shapes, widths, Ws, _, _ = decode_sets(torch, rbq, workloads, wl, dev, layout, n_layers)
    del Ws
    tiles = [[rbq.pack_tiles(p) for p, _ in layer] for layer in layers]
    slots = X_SLOTS[layout]
    per_slot = {sl: torch.from_numpy(workloads.layer_activations(wl, widths[i], n_layers * M, sl).view(
        np.float16)).to(dev).reshape(n_layers, M, widths[i]) for i, sl in enumerate(slots)}
    xs = [[per_slot[sl][l] for sl in slots] for l in range(n_layers)]
    # algorithmic bytes per linear: planes and scales once, M tokens of its x and y
    per_lin = [gemv_bytes(sh.out_features, sh.in_features, K, 1, M) for sh in shapes]
    nbytes = sum(per_lin) * n_layers
    stream = torch.cuda.current_stream(dev)
    narrow = [i for i, sh in enumerate(shapes) if sh.in_features <= 4096]
    wide = [i for i in range(len(shapes)) if i not in narrow]
    candidates = []
    if M % 4 == 0:
        # one launch per linear: each program's op groups and LDS layout fit
        # its own shape (mixed in one launch, the 22016-row gate/up ops leave
        # room for one op group only, which the 4096-row ops run poorly)
        candidates.append(("4_and_2_token_ops_per_linear", [([i], 4 if i in narrow else 2)
                                                            for i in range(len(shapes))]))
        candidates.append(("4_and_2_token_ops", [(narrow, 4), (wide, 2)]))
    if M % 2 == 0:
        candidates.append(("2_token_ops", [(list(range(len(shapes))), 2)]))
    candidates.append(("1_token_ops", [(list(range(len(shapes))), 1)]))
    forms = {}
    for name, parts in candidates:
        if any(n_layers * len(lins) * (M // tok) > rbq.RBQ_PROGRAM_MAX_OPS for lins, tok in parts if lins):
            continue
        ys = [[torch.empty((M, sh.out_features), dtype=torch.float16, device=dev) for sh in shapes]
              for _ in range(n_layers)]
        progs = []
        for lins, tok in parts:
            if lins:
                progs.append(rbq.Program([{"planes": tiles[l][i], "scales": layers[l][i][1], "x": xs[l][i][m:m + tok],
                                           "y": ys[l][i][m:m + tok], "tokens": tok}
                                          for l in range(n_layers) for i in lins for m in range(0, M, tok)],
                                         num_planes=K))
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def run(progs=progs, status=status):
            for pr in progs:
                pr.run(status)
        settle(torch, run)
        us = event_launch_us(torch, run, stream, max(args.steps, 20))
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
        if int(status.item()) != 0:
            raise rbq.RbqError(rbq.RBQ_ERR_HIP, f"program status {int(status.item()):#x}")
        diff = 0.0
        for i, (p, sc) in enumerate(layers[0]):
            ref = rbq.gemm(p, sc, xs[0][i], group)
            diff = max(diff, float((ys[0][i].float() - ref.float()).abs().max() /
                                   ref.float().abs().max().clamp_min(1e-30)))
        forms[name] = {"launches": len(progs), "ops": [pr.n_ops for pr in progs],
                       "tokens_per_op": {shapes[i].in_features: tok for lins, tok in parts for i in lins},
                       "ms_per_step": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "mean_step_launch_us": round(us, 2), "layer0_max_rel_diff_vs_rbq_gemm": diff}
        del progs, ys
    if not forms:
        return None
    name = next(n for n, _ in candidates if n in forms)
    f = forms[name]
    line = {"metric": f"K={K} batch-{M} GEMM effective GB/s on Llama-2-7B layers, decode step as program launches",
            "value": round(nbytes / (f["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": f["ms_per_step"], "dtype": DTYPE_INT8_LIMBS,
            "config": {"workload": f"llama2_7b_skinny_m{M}_decode_program", "layers": n_layers, "layout": layout,
                       "ops_per_layer": {name_: f"{sh.out_features}x{sh.in_features}"
                                         for (name_, _), sh in zip(groups, shapes)},
                       "num_planes": K, "group_size": group, "tokens": M, "form": name,
                       "launches_per_step": f["launches"], "ops": f["ops"], "bytes_per_step": nbytes,
                       "planes_layout": "tiles (rbq_pack_tiles)"},
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (f["mean_step_launch_us"] * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(nbytes / (f["mean_step_launch_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "traffic": (measured_traffic(f"batch{M}_per_linear", "gemv_program_kernel", TRAFFIC_PROFILE_BATCH)
                                     if name == "4_and_2_token_ops_per_linear" and layout == "fused" else None),
                         "kernel": f"gemv_program_kernel<{K}> ({name})",
                         "bytes_per_launch": nbytes, "mean_launch_us": f["mean_step_launch_us"]},
            "layer0_max_rel_diff_vs_rbq_gemm": f["layer0_max_rel_diff_vs_rbq_gemm"],
            "forms": forms, "cpu_baseline": None}
    if cpu_seconds > 0:
        samples = [(p.cpu().numpy().view(np.uint32), sc.cpu().numpy().view(np.uint16),
                    xs[0][i].cpu().numpy().view(np.uint16), group, per_lin[i])
                   for i, (p, sc) in enumerate(layers[0])]
        line["cpu_baseline"] = oracle_baseline(samples, cpu_seconds, max_reps=20)
        line["cpu_baseline"]["sample"] = f"layer 0 at M={M}: " + line["cpu_baseline"]["sample"]
    del tiles, xs, layers, per_slot
    torch.cuda.empty_cache()
    return line


def prefill_more_planes(args, torch, rbq, workloads, dev, M=2048, shapes=((14336, 4096), (4096, 14336))):
    """The prefill contraction at K = 3 and K = 4 (per-row scales, and K = 4
    with 128-column groups as in QBB), which run the kernel that unpacks
    What into LDS: random planes and scales (the time does not depend on the
    values), M fp16 tokens; per-launch device time from HIP events around
    graph replays, dense-equivalent TFLOP/s (2 M out in / t)."""
    res = {}
    X = torch.from_numpy(workloads.gaussian_activations(M, max(i for _, i in shapes), seed=77).view(np.float16)).to(dev)
    for K, group in ((3, 0), (4, 0), (4, 128)):
        per = {}
        for out_f, in_f in shapes:
            p = torch.from_numpy(workloads.random_planes(K, out_f, in_f, seed=out_f + in_f + K).view(np.int32)).to(dev)
            G = in_f // group if group else 1
            sc = torch.from_numpy((np.random.default_rng(K).uniform(0.001, 0.01, (K, out_f, G))).astype(
                np.float16)).to(dev).reshape(K, -1)
            Xs = X[:, :in_f].contiguous()
            Y = torch.empty((M, out_f), dtype=torch.float16, device=dev)
            fn = (lambda p=p, sc=sc, Xs=Xs, Y=Y: rbq.gemm(p, sc, Xs, group, Y=Y))
            fn()
            torch.cuda.synchronize()
            us = graph_launch_us(torch, dev, [fn], max(args.kernel_reps, 3))
            per[f"{out_f}x{in_f}"] = {"mean_us": round(us, 2),
                                      "TFLOPs_dense_eq": round(2.0 * M * out_f * in_f / (us * 1e-6) / 1e12, 1)}
            del p, sc, Xs, Y
        res[f"K{K}" + ("_g128" if group else "")] = per
    del X
    torch.cuda.empty_cache()
    return res


def bench_layer_set(args):
    import torch

    import gemm_rbq_encode_amd as rbq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(json.dumps(measure_layer_set(args, args.workload, args.tokens, torch, rbq, workloads, dev)), flush=True)


def measure_layer_set(args, workload, tokens, torch, rbq, workloads, dev, with_prep=True, cpu_seconds=None):
    """Skinny, grouped-scale and prefill workloads: each linear of the set is
    run back to back (one launch each) over a rotation of encoded copies;
    reports algorithmic GB/s (decode-like sets) or dense-equivalent TFLOP/s
    (prefill), the per-launch device time from HIP events, and the CPU
    oracle on a bounded sample.  Returns the JSON line as a dict."""
    wl = workloads.WORKLOADS[workload]
    K, group = wl.num_planes, wl.group_size
    M = tokens or max(wl.tokens)
    stream = torch.cuda.current_stream(dev)
    # distinct shapes only (q/k/v/o and gate/up share shapes)
    uniq = []
    for i, lin in enumerate(wl.linears):
        if all((lin.out_features, lin.in_features) != (l.out_features, l.in_features) for _, l in uniq):
            uniq.append((i, lin))
    prefill = workload == "llama3_8b_prefill"
    rot = 2 if prefill else max(2, int(2.0e9 // sum(
        K * l.out_features * l.in_features // 8 for _, l in uniq)))
    sets, prep = [], {}
    for i, lin in uniq:
        W = torch.from_numpy(workloads.workload_weight(wl, i)).to(dev)
        p, sc = rbq.encode(W, K, group)
        X = torch.from_numpy(workloads.workload_activations(wl, lin.in_features, M).view(np.float16)).to(dev)
        Y = torch.empty((M, lin.out_features), dtype=torch.float16, device=dev)
        copies = [(p.clone(), sc.clone()) for _ in range(rot)]
        sets.append((lin, copies, X, Y))
        if not with_prep:
            del W
            continue
        # encoder and refit time of this shape (outputs rewritten in place)
        key = f"{lin.out_features}x{lin.in_features}"
        pe, se, sr = torch.empty_like(p), torch.empty_like(sc), sc.clone()
        # one call per copy of W (copies exceed the caches), three replays
        Wc = rotation_copies(W)
        enc_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.encode(Wi, K, group, planes=pe, scales=se))
                                       for Wi in Wc], 3) / len(Wc)
        ref_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.refit(Wi, p, sr, group)) for Wi in Wc], 3) / len(Wc)
        pr = p.clone()
        rb_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.rebinarize(Wi, pr, sc, group)) for Wi in Wc], 3) / len(Wc)
        del Wc
        wb, pb, sb = 4 * W.numel(), 4 * p.numel(), 2 * sc.numel()
        prep[key] = {"encode_us": round(enc_ms * 1e3, 1),
                     "encode_GBps": round((wb + pb + sb) / (enc_ms * 1e-3) / 1e9, 1),
                     "refit_us": round(ref_ms * 1e3, 1),
                     "refit_GBps": round((wb + pb + 2 * sb) / (ref_ms * 1e-3) / 1e9, 1),
                     "rebinarize_us": round(rb_ms * 1e3, 1),
                     "rebinarize_GBps": round((wb + pb + sb) / (rb_ms * 1e-3) / 1e9, 1)}
        del pe, se, sr, pr
        del W
    torch.cuda.synchronize()
    forced = {"auto": rbq.PATH_AUTO, "valu": rbq.PATH_VALU, "decode": rbq.PATH_DECODE,
              "stream": rbq.PATH_STREAM, "flat": rbq.PATH_FLAT, "group": rbq.PATH_GROUP,
              "split": rbq.PATH_SPLIT}[args.path]
    rbq.set_path(forced)
    path = forced if forced != rbq.PATH_AUTO else rbq.select_path(
        rbq.shape(uniq[0][1].out_features, uniq[0][1].in_features, K, group), M)
    names = path_names(rbq)
    launches = []
    for r in range(rot):   # one pass over every shape and rotation copy
        for lin, copies, X, Y in sets:
            p, sc = copies[r % rot]
            launches.append((f"{lin.out_features}x{lin.in_features}",
                             (lambda p=p, sc=sc, X=X, Y=Y: rbq.gemm(p, sc, X, group, Y=Y))))
    for _, fn in launches[:len(sets) * 2]:
        fn()
    torch.cuda.synchronize()
    # whole-set wall time: one pass over every shape and rotation copy,
    # captured in a HIP graph and replayed (launch cost off the host)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _, fn in launches:
            fn()
    torch.cuda.synchronize()
    settle(torch, graph.replay)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / (args.steps * rot)   # one pass over the shapes
    mean_us = {}
    for lin, copies, X, Y in sets:
        key = f"{lin.out_features}x{lin.in_features}"
        fns = [(lambda p=p, sc=sc, X=X, Y=Y: rbq.gemm(p, sc, X, group, Y=Y)) for p, sc in copies]
        mean_us[key] = graph_launch_us(torch, dev, fns, max(args.kernel_reps, 1))
    per_shape = {}
    tot_bytes = tot_flop = tot_us = 0.0
    for lin, _, _, _ in sets:
        key = f"{lin.out_features}x{lin.in_features}"
        G = lin.in_features // group if group else 1
        nbytes = gemv_bytes(lin.out_features, lin.in_features, K, G, M)
        flop = 2.0 * M * lin.out_features * lin.in_features
        us = mean_us[key]
        per_shape[key] = {"bytes": nbytes, "mean_us": round(us, 3),
                          "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "TFLOPs_dense_eq": round(flop / (us * 1e-6) / 1e12, 2)}
        tot_bytes += nbytes
        tot_flop += flop
        tot_us += us
    if prefill:
        metric = "prefill dense-equivalent TFLOP/s (2*M*out*in / t), fp16 MFMA"
        value = tot_flop / wall / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(tot_flop / (tot_us * 1e-6) / 1e12, 2),
                "peak": 2500.0, "unit": "TFLOP/s"}
    else:
        metric = f"K={K} batch-{M} GEMM effective GB/s on {wl.name} layers"
        value = tot_bytes / wall / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": round(tot_bytes / (tot_us * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = f"rbq gemm ({names[path]})"
    roof["per_shape"] = per_shape
    line = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype_of(names[path]),
            "data": "synthetic",
            "config": {"workload": wl.name, "linears": [f"{l.out_features}x{l.in_features}" for _, l in uniq],
                       "num_planes": K, "group_size": group, "tokens": M, "rotation": rot,
                       "path": names[path],
                       "path_per_shape": {f"{l.out_features}x{l.in_features}": names[
                           forced if forced != rbq.PATH_AUTO else
                           rbq.select_path(rbq.shape(l.out_features, l.in_features, K, group), M)]
                           for _, l in uniq}},
            "roofline": roof, "cpu_baseline": None}
    if prep:
        line["encode_refit_per_shape"] = prep
    budget = args.cpu_seconds if cpu_seconds is None else cpu_seconds
    if budget > 0:
        # the oracle on the first copy of each shape; prefill on 16 of the tokens
        m_cpu = min(M, 16)
        samples = []
        for lin, copies, X, _ in sets:
            G = lin.in_features // group if group else 1
            work = 2.0 * m_cpu * lin.out_features * lin.in_features if prefill else \
                gemv_bytes(lin.out_features, lin.in_features, K, G, m_cpu)
            samples.append((copies[0][0].cpu().numpy().view(np.uint32), copies[0][1].cpu().numpy().view(np.uint16),
                            X[:m_cpu].cpu().numpy().view(np.uint16), group, work))
        line["cpu_baseline"] = oracle_baseline(samples, budget, unit="TFLOP/s" if prefill else "GB/s",
                                               max_reps=20)
        line["cpu_baseline"]["sample"] = (f"one copy of each shape at {m_cpu} token(s): "
                                          + line["cpu_baseline"]["sample"])
    for _, copies, X, Y in sets:
        del copies[:]
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return line


X_SLOTS = {"fused": (0, 1, 2, 3), "separate": (0, 0, 0, 1, 2, 2, 3)}


def settle(torch, fn, seconds=0.3):
    """Untimed: run `fn` back to back for about `seconds`, so that the GPU's
    clocks reach their level under this load before a timing starts (right
    after idle gaps the first tens of launches run at other clocks)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def event_launch_us(torch, fn, stream, reps):
    """Mean device time (us) of one launch of `fn`: `reps` launches back to
    back between two HIP events recorded on `stream`, the stream it
    launches on."""
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def oracle_baseline(samples, seconds, unit="GB/s", max_reps=50):
    """The CPU oracle (fp64 dequantize-and-multiply) over `samples`, a list of
    (planes, scales, X, group_size, work) with work in algorithmic bytes
    (unit GB/s) or dense-equivalent flops (unit TFLOP/s), repeated for about
    `seconds`, with all its threads and then with one thread for a third of
    that time.  Returns the cpu_baseline object."""
    import oracle

    def run(budget):
        t0 = time.perf_counter()
        done, reps = 0, 0
        while True:
            for p, s, X, g, nb in samples:
                oracle.gemm(p, s, X, g)
                done += nb
            reps += 1
            if time.perf_counter() - t0 >= budget or reps >= max_reps:
                return done, reps, time.perf_counter() - t0

    cores = oracle.num_threads()
    done, reps, el = run(seconds)
    oracle.set_num_threads(1)
    try:
        done1, reps1, el1 = run(seconds / 3)
    finally:
        oracle.set_num_threads(cores)
    div = 1e12 if unit == "TFLOP/s" else 1e9
    return {"value": round(done / el / div, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "single_thread_value": round(done1 / el1 / div, 6),
            "sample": f"{reps} pass(es) over {len(samples)} linear(s) in {el:.1f} s on {cores} threads, "
                      f"{reps1} in {el1:.1f} s on 1 thread (fp64 dequantize-and-multiply)"}


def decode_sets(torch, rbq, workloads, wl, dev, layout, n_layers):
    """The decode step's weights: the seven Llama-2-7B linears drawn from the
    seeded generator and encoded on the GPU, grouped by layout ("fused"
    stacks q/k/v and gate/up row-wise; rows are encoded independently, so the
    stacked planes and scales are exactly the separate ones placed one after
    another), and one copy per layer.  Returns (groups, layers, shapes,
    widths, Ws, planes, scales) with layers[l][i] = (planes, scales)."""
    K, group = wl.num_planes, wl.group_size
    Ws, enc_planes, enc_scales = [], [], []
    for i, _ in enumerate(wl.linears):
        W = torch.from_numpy(workloads.workload_weight(wl, i)).to(dev)
        p, s = rbq.encode(W, K, group)
        Ws.append(W)
        enc_planes.append(p)
        enc_scales.append(s)
    if layout == "fused":
        groups = [("qkv_proj", [0, 1, 2]), ("o_proj", [3]), ("gate_up_proj", [4, 5]), ("down_proj", [6])]
    else:
        groups = [(lin.name, [i]) for i, lin in enumerate(wl.linears)]
    g_planes, g_scales, shapes, widths = [], [], [], []
    for _, idx in groups:
        p = torch.cat([enc_planes[i] for i in idx], dim=1).contiguous()
        s = torch.cat([enc_scales[i] for i in idx], dim=1).contiguous()
        g_planes.append(p)
        g_scales.append(s)
        shapes.append(rbq.shape(p.shape[1], p.shape[2] * 32, K, group))
        widths.append(p.shape[2] * 32)
    layers = [[(p.clone(), s.clone()) for p, s in zip(g_planes, g_scales)] for _ in range(n_layers)]
    torch.cuda.synchronize()
    return groups, layers, shapes, widths, Ws, enc_planes, enc_scales


def decode_activations(torch, workloads, wl, dev, layout, widths, n_layers):
    """xs[l][i]: the fp16 token that launch group i of layer l reads (one
    buffer per decoder-layer input, shared only by q/k/v and by gate/up as in
    a decoder)."""
    slots = X_SLOTS[layout]
    width_of = {}
    for i, sl in enumerate(slots):
        width_of[sl] = widths[i]
    per_slot = {sl: torch.from_numpy(workloads.layer_activations(wl, n, n_layers, sl).view(np.float16)).to(dev)
                for sl, n in width_of.items()}
    return [[per_slot[sl][l] for sl in slots] for l in range(n_layers)]


def chain_buffers(torch, dev, layers, shapes, x):
    """Interleaved (gate, up) row pairs for the SiLU-mul epilogue, and the
    activation buffers of a chained decoder step."""
    n_ff = shapes[2].out_features // 2
    perm = torch.stack([torch.arange(n_ff), torch.arange(n_ff) + n_ff], dim=1).reshape(-1).to(dev)
    gu = [(p.index_select(1, perm).contiguous(), s.index_select(1, perm).contiguous())
          for p, s in (layer[2] for layer in layers)]
    bufs = {"x": x,
            "qkv": torch.empty(shapes[0].out_features, dtype=torch.float16, device=dev),
            "o": torch.empty(shapes[1].out_features, dtype=torch.float16, device=dev),
            "h": torch.empty(n_ff, dtype=torch.float16, device=dev),
            "y": torch.empty(shapes[3].out_features, dtype=torch.float16, device=dev)}
    return gu, bufs, n_ff


def program_planes(rbq, args, planes):
    """The planes a decode program reads: the tile-layout copy (packed once,
    as when the weights are loaded) or the row-layout tensor itself."""
    return rbq.pack_tiles(planes) if args.planes_layout == "tiles" else planes


def program_key(args, layout=None):
    key = f"program_{layout or args.layout}_{args.layers}layers"
    return key + "_tiles" if args.planes_layout == "tiles" else key


def chain_program_ops(rbq, layers, gu, bufs, n_q, tiles=None):
    """A chained decoder step as program ops: q/k/v on the layer input (x,
    then the previous layer's down output), o on q (the attention between
    them is outside this library), gate/up with the SiLU-mul epilogue on o's
    output, down on h; each op waits for the one before it."""
    def pl(p):
        return tiles(p) if tiles else p
    ops = []
    for l, layer in enumerate(layers):
        ops.append({"planes": pl(layer[0][0]), "scales": layer[0][1], "x": bufs["x"] if l == 0 else bufs["y"],
                    "y": bufs["qkv"], "wait_for": len(ops) - 1})
        ops.append({"planes": pl(layer[1][0]), "scales": layer[1][1], "x": bufs["qkv"][:n_q], "y": bufs["o"],
                    "wait_for": len(ops) - 1})
        ops.append({"planes": pl(gu[l][0]), "scales": gu[l][1], "x": bufs["o"], "y": bufs["h"],
                    "epilogue": rbq.RBQ_EPILOGUE_SILU_MUL, "wait_for": len(ops) - 1})
        ops.append({"planes": pl(layer[3][0]), "scales": layer[3][1], "x": bufs["h"], "y": bufs["y"],
                    "wait_for": len(ops) - 1})
    return ops


def decode_layer_chain(args, torch, rbq, L, dev, layers, shapes, x, K):
    """The 32 layers as a chained decoder step (chain_program_ops' order and
    dependencies), once as one program launch and once as 4 launches per
    layer in a HIP graph.  Reports ms and GB/s over the same algorithmic
    bytes (h is written once at half the gate/up rows).  The program reads
    the planes in args.planes_layout, the launches the row layout."""
    gu, bufs, n_ff = chain_buffers(torch, dev, layers, shapes, x)
    n_q = shapes[1].in_features
    per_layer = sum(gemv_bytes(sh.out_features, sh.in_features, K, 1) for sh in shapes) - 2 * n_ff
    total = per_layer * len(layers)
    stream = torch.cuda.current_stream(dev)

    def launches(st):
        for l, (layer, (gp, gs)) in enumerate(zip(layers, gu)):
            xin = bufs["x"] if l == 0 else bufs["y"]
            rcs = (L.rbq_gemv(layer[0][0].data_ptr(), layer[0][1].data_ptr(), shapes[0], xin.data_ptr(),
                              bufs["qkv"].data_ptr(), st),
                   L.rbq_gemv(layer[1][0].data_ptr(), layer[1][1].data_ptr(), shapes[1], bufs["qkv"].data_ptr(),
                              bufs["o"].data_ptr(), st),
                   L.rbq_gemm_ex(gp.data_ptr(), gs.data_ptr(), shapes[2], bufs["o"].data_ptr(), 1,
                                 bufs["h"].data_ptr(), None, 0, rbq.RBQ_EPILOGUE_SILU_MUL, st),
                   L.rbq_gemv(layer[3][0].data_ptr(), layer[3][1].data_ptr(), shapes[3], bufs["h"].data_ptr(),
                              bufs["y"].data_ptr(), st))
            if any(rcs):
                raise rbq.RbqError(max(rcs), "decode layer chain")

    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launches(side.cuda_stream)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        launches(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()

    def wall_ms(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)

    settle(torch, graph.replay)
    ms_launch = wall_ms(graph.replay)
    y_launch = bufs["y"].clone()
    del graph
    prog = rbq.Program(chain_program_ops(rbq, layers, gu, bufs, n_q,
                                         (lambda p: program_planes(rbq, args, p))), num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    settle(torch, lambda: prog.run(status))
    ms_prog = wall_ms(lambda: prog.run(status))
    torch.cuda.synchronize()
    st = int(status.item())
    if st:
        raise rbq.RbqError(rbq.RBQ_ERR_HIP, f"decode chain program status {st:#x}")
    same = bool(torch.equal(bufs["y"], y_launch))
    del prog, gu
    return {"layers": len(layers), "ops_per_layer": 4, "bytes_per_step": total,
            "program": {"ms_per_step": round(ms_prog, 4), "GBps": round(total / (ms_prog * 1e-3) / 1e9, 1)},
            "launches": {"ms_per_step": round(ms_launch, 4), "GBps": round(total / (ms_launch * 1e-3) / 1e9, 1),
                         "graph": True},
            "program_output_equals_launches": same, "program_planes_layout": args.planes_layout,
            "epilogue": "silu(gate)*up in the gate/up op"}


def bench_qat(torch, rbq, workloads, dev, shapes=((4096, 4096), (11008, 4096), (4096, 11008)), K=2,
              tokens=(16, 2048)):
    """The coupled forward and the straight-through backward on the
    Llama-2-7B linear shapes: the cores for given scales (GB/s over W read
    and planes written), the forward (cores + layer) and the backward (dW,
    scale gradients, dX) per token count, as mean ms of graph replays and
    dense-equivalent TFLOP/s (2*M*out*in per product: one for the forward,
    two for the backward)."""
    res = {}
    for out_f, in_f in shapes:
        W = torch.from_numpy(workloads.gaussian_weight(out_f, in_f, 4000 + out_f, outliers=True)).to(dev)
        _, sc = rbq.encode(W, K, 0)
        planes = torch.empty((K, out_f, in_f // 32), dtype=torch.int32, device=dev)
        Wc = rotation_copies(W)
        enc_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.qat_encode(Wi, sc, 0, planes=planes)) for Wi in Wc],
                          3) / len(Wc)
        del Wc
        entry = {"encode_us": round(enc_ms * 1e3, 1),
                 "encode_GBps": round((4 * W.numel() + 4 * planes.numel()) / (enc_ms * 1e-3) / 1e9, 1)}
        for M in tokens:
            X = torch.from_numpy(workloads.gaussian_activations(M, in_f, 4100).view(np.float16)).to(dev)
            dY = torch.from_numpy(workloads.gaussian_activations(M, out_f, 4101).view(np.float16)).to(dev)
            Y = torch.empty((M, out_f), dtype=torch.float16, device=dev)
            need = int(rbq.lib().rbq_gemm_workspace_bytes(rbq.shape(out_f, in_f, K, 0), M))
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            dX = torch.empty((M, in_f), dtype=torch.float32, device=dev)
            dW = torch.empty((out_f, in_f), dtype=torch.float32, device=dev)
            ds = torch.empty((K, out_f, 1), dtype=torch.float32, device=dev)
            L = rbq.lib()
            s = rbq.shape(out_f, in_f, K, 0)

            def fwd():
                rbq.check(L.rbq_qat_forward(W.data_ptr(), sc.data_ptr(), s, X.data_ptr(), M, planes.data_ptr(),
                                            Y.data_ptr(), ws.data_ptr(), need, None,
                                            torch.cuda.current_stream(dev).cuda_stream), "rbq_qat_forward")

            bneed = int(L.rbq_qat_backward_workspace_bytes(s, M))
            bws = torch.empty(max(bneed, 4), dtype=torch.uint8, device=dev)

            def bwd():
                rbq.check(L.rbq_qat_backward(planes.data_ptr(), sc.data_ptr(), s, X.data_ptr(), dY.data_ptr(), M,
                                             dX.data_ptr(), dW.data_ptr(), ds.data_ptr(), bws.data_ptr(), bneed,
                                             None, torch.cuda.current_stream(dev).cuda_stream), "rbq_qat_backward")

            f_ms = graph_ms(torch, dev, [fwd], 5)
            b_ms = graph_ms(torch, dev, [bwd], 5)
            flop = 2.0 * M * out_f * in_f
            entry[f"m{M}"] = {"forward_ms": round(f_ms, 4), "forward_TFLOPs": round(flop / (f_ms * 1e-3) / 1e12, 1),
                              "backward_ms": round(b_ms, 4),
                              "backward_TFLOPs": round(2 * flop / (b_ms * 1e-3) / 1e12, 1)}
            del X, dY, Y, ws, dX, dW, ds, bws
        res[f"{out_f}x{in_f}"] = entry
        del W, sc, planes
    torch.cuda.empty_cache()
    return {"num_planes": K, "scales": "per row", "per_shape": res}


def other_layout_program(args, torch, rbq, workloads, wl, dev, layout):
    """The same decode step in the other layout, as one program launch:
    whole-job ms and GB/s, and the kernel's mean launch time from HIP events
    on its stream."""
    K = wl.num_planes
    groups, layers, shapes, widths, Ws, p_enc, s_enc = decode_sets(torch, rbq, workloads, wl, dev, layout,
                                                                   args.layers)
    del Ws, p_enc, s_enc
    xs = decode_activations(torch, workloads, wl, dev, layout, widths, args.layers)
    ys = [[torch.empty(sh.out_features, dtype=torch.float16, device=dev) for sh in shapes]
          for _ in range(args.layers)]
    nbytes = sum(gemv_bytes(sh.out_features, sh.in_features, K, 1) for sh in shapes) * args.layers
    prog = rbq.Program([{"planes": program_planes(rbq, args, layers[l][i][0]), "scales": layers[l][i][1],
                         "x": xs[l][i], "y": ys[l][i]}
                        for l in range(args.layers) for i in range(len(groups))], num_planes=K)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    run = (lambda: prog.run(status))
    settle(torch, run)
    us = event_launch_us(torch, run, stream, max(args.steps, 20))
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    if int(status.item()) != 0:
        raise rbq.RbqError(rbq.RBQ_ERR_HIP, f"program status {int(status.item()):#x}")
    del prog, layers, xs, ys
    torch.cuda.empty_cache()
    return {"layout": layout, "planes_layout": args.planes_layout, "ops": len(groups) * args.layers,
            "bytes_per_step": nbytes,
            "ms_per_step": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "mean_launch_us": round(us, 2), "kernel_GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def bench_decode(args):
    import torch

    import gemm_rbq_encode_amd as rbq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS["llama2_7b"]
    K, group = wl.num_planes, wl.group_size
    L = rbq.lib()
    path = {"auto": rbq.PATH_AUTO, "valu": rbq.PATH_VALU, "decode": rbq.PATH_DECODE,
            "stream": rbq.PATH_STREAM, "flat": rbq.PATH_FLAT,
            "group": rbq.PATH_GROUP, "split": rbq.PATH_SPLIT}[args.path]
    rbq.set_path(path)
    rbq.set_stream_split(args.split)
    stream = torch.cuda.current_stream(dev)

    groups, layers, shapes, widths, Ws, enc_planes, enc_scales = decode_sets(
        torch, rbq, workloads, wl, dev, args.layout, args.layers)

    # ---- encoder, refit and re-binarization per distinct shape, dual encoder
    enc_bytes = sum(4 * W.numel() + 4 * p.numel() + 2 * s.numel() for W, p, s in zip(Ws, enc_planes, enc_scales))
    enc_ms = graph_ms(torch, dev, [(lambda W=W, p=p, s=s: rbq.encode(W, K, group, planes=p, scales=s))
                                   for W, p, s in zip(Ws, enc_planes, enc_scales)], 5)
    ref_scales = [s.clone() for s in enc_scales]
    ref_bytes = sum(4 * W.numel() + p.numel() * 4 + 4 * s.numel() for W, p, s in zip(Ws, enc_planes, ref_scales))
    ref_ms = graph_ms(torch, dev, [(lambda W=W, p=p, s=s: rbq.refit(W, p, s, group))
                                   for W, p, s in zip(Ws, enc_planes, ref_scales)], 5)
    prep = {}
    for W, p, s in zip(Ws, enc_planes, enc_scales):
        key = f"{W.shape[0]}x{W.shape[1]}"
        if key in prep:
            continue
        pe, se, sr = torch.empty_like(p), torch.empty_like(s), s.clone()
        Wc = rotation_copies(W)
        e_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.encode(Wi, K, group, planes=pe, scales=se))
                                     for Wi in Wc], 3) / len(Wc)
        r_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.refit(Wi, p, sr, group)) for Wi in Wc], 3) / len(Wc)
        pr = p.clone()
        rb_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.rebinarize(Wi, pr, s, group)) for Wi in Wc], 3) / len(Wc)
        del Wc
        wb, pb, sb = 4 * W.numel(), 4 * p.numel(), 2 * s.numel()
        shp = rbq.shape(W.shape[0], W.shape[1], K, 0)
        wsd = torch.empty(rbq.encode_dual_workspace_bytes(shp), dtype=torch.uint8, device=dev)
        pd = torch.empty_like(p)
        gd = torch.empty((K, W.shape[0]), dtype=torch.float16, device=dev)
        hd = torch.empty((K, W.shape[1]), dtype=torch.float16, device=dev)
        d_ms = graph_ms(torch, dev, [lambda: rbq.encode_dual(W, K, workspace=wsd, planes=pd, g=gd, h=hd)], 3)
        prep[key] = {"encode_us": round(e_ms * 1e3, 1),
                     "encode_GBps": round((wb + pb + sb) / (e_ms * 1e-3) / 1e9, 1),
                     "refit_us": round(r_ms * 1e3, 1),
                     "refit_GBps": round((wb + pb + 2 * sb) / (r_ms * 1e-3) / 1e9, 1),
                     "rebinarize_us": round(rb_ms * 1e3, 1),
                     "rebinarize_GBps": round((wb + pb + sb) / (rb_ms * 1e-3) / 1e9, 1),
                     "encode_dual_us": round(d_ms * 1e3, 1)}
        del pe, se, sr, pr, wsd, pd, gd, hd
    del Ws, ref_scales, enc_planes, enc_scales

    # ---- the step: every launch group of every layer, each reading its own
    # activations and writing its own output
    xs = decode_activations(torch, workloads, wl, dev, args.layout, widths, args.layers)
    ys = [[torch.empty(sh.out_features, dtype=torch.float16, device=dev) for sh in shapes]
          for _ in range(args.layers)]
    per_call = [gemv_bytes(sh.out_features, sh.in_features, K, 1) for sh in shapes]
    bytes_per_step = sum(per_call) * args.layers
    ops = [{"planes": layers[l][i][0], "scales": layers[l][i][1], "x": xs[l][i], "y": ys[l][i]}
           for l in range(args.layers) for i in range(len(groups))]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    # the program reads the tile layout by default: packed once, as when the
    # weights are loaded (the pack's own rate is reported, outside the step)
    pack = None
    if args.planes_layout == "tiles":
        pk = [(lambda p=op["planes"], t=torch.empty_like(rbq.pack_tiles(op["planes"])):
               rbq.pack_tiles(p, tiles=t)) for op in ops[:len(groups)]]
        pk_ms = graph_ms(torch, dev, pk, 3)
        pk_bytes = sum(2 * op["planes"].numel() * 4 for op in ops[:len(groups)])
        pack = {"what": "rbq_pack_tiles of one layer's planes (row layout read, tile layout written)",
                "ms": round(pk_ms, 4), "GBps": round(pk_bytes / (pk_ms * 1e-3) / 1e9, 1)}
        del pk
    prog_ops = [dict(op, planes=program_planes(rbq, args, op["planes"])) for op in ops]
    prog = rbq.Program(prog_ops, num_planes=K)

    def run_step():
        prog.run(status)

    # the kernel's own duration first (HIP events around back-to-back
    # launches on its stream), then the whole-job timing
    settle(torch, run_step)
    prog_us = event_launch_us(torch, run_step, stream, max(args.steps, 20))
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    if int(status.item()) != 0:
        raise rbq.RbqError(rbq.RBQ_ERR_HIP, f"program status {int(status.item()):#x}")
    prog_out = [y.clone() for y in ys[-1]]
    rows_program = None
    if args.planes_layout == "tiles":
        # the same program on the row layout, for comparison
        del prog, prog_ops
        torch.cuda.empty_cache()
        prog_r = rbq.Program(ops, num_planes=K)
        run_r = (lambda: prog_r.run(status))
        settle(torch, run_r)
        r_us = event_launch_us(torch, run_r, stream, max(args.steps, 20))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run_r()
        torch.cuda.synchronize()
        r_ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
        if int(status.item()) != 0:
            raise rbq.RbqError(rbq.RBQ_ERR_HIP, f"program status {int(status.item()):#x}")
        rows_program = {"planes_layout": "rows", "ms_per_step": round(r_ms, 4),
                        "GBps": round(bytes_per_step / (r_ms * 1e-3) / 1e9, 1), "mean_launch_us": round(r_us, 2),
                        "kernel_GBps": round(bytes_per_step / (r_us * 1e-6) / 1e9, 1),
                        "output_equals_tiles": all(bool(torch.equal(a, b)) for a, b in zip(prog_out, ys[-1]))}
        del prog_r

    # ---- the same step as one rbq_gemv launch per op, in a HIP graph
    def launch_step(st):
        for op in ops:
            rc = L.rbq_gemv(op["planes"].data_ptr(), op["scales"].data_ptr(),
                            rbq.shape(op["planes"].shape[1], op["planes"].shape[2] * 32, K, group),
                            op["x"].data_ptr(), op["y"].data_ptr(), st)
            if rc != 0:
                raise rbq.RbqError(rc, "rbq_gemv")

    names = path_names(rbq)
    shape_paths = {f"{sh.out_features}x{sh.in_features}":
                   names[rbq.select_path(sh, 1) if path == rbq.PATH_AUTO else path] for sh in shapes}
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launch_step(side.cuda_stream)
    side.synchronize()
    # the two runs may take different kernel families for a shape, so they
    # agree to the decode bound rather than bit for bit
    launch_diff = max(float((a.float() - b.float()).abs().max() / b.float().abs().max().clamp_min(1e-30))
                      for a, b in zip(prog_out, ys[-1]))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        launch_step(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    settle(torch, graph.replay)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_launches = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    del graph

    # ---- per launch group: rbq_gemv launch time and a read of the same bytes
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    reps = max(args.kernel_reps, 1) * 4
    per_shape = {}
    for i, (name, _) in enumerate(groups):
        fns = [(lambda op=ops[l * len(groups) + i]: rbq.gemv(op["planes"], op["scales"], op["x"], group,
                                                            y=op["y"]))
               for l in range(args.layers)]
        us = graph_launch_us(torch, dev, fns, reps)
        pbufs = [layers[l][i][0] for l in range(args.layers)]
        pus = graph_launch_us(torch, dev, [(lambda b=b: rbq.probe_read(b, sink)) for b in pbufs], reps)
        pbytes = pbufs[0].numel() * 4
        per_shape[name] = {"shape": f"{shapes[i].out_features}x{shapes[i].in_features}",
                           "bytes": per_call[i], "gemv_us": round(us, 3),
                           "gemv_GBps": round(per_call[i] / (us * 1e-6) / 1e9, 1),
                           "read_probe_bytes": pbytes, "read_probe_us": round(pus, 3),
                           "read_probe_GBps": round(pbytes / (pus * 1e-6) / 1e9, 1),
                           "gemv_time_over_probe": round(us / pus, 3)}
    # the whole step's planes read back to back as separate launches, and
    # the same byte count read by one launch
    step_bufs = [op["planes"] for op in ops]
    step_probe_us = graph_launch_us(torch, dev, [(lambda b=b: rbq.probe_read(b, sink)) for b in step_bufs], 2)
    step_probe_ms = step_probe_us * len(step_bufs) * 1e-3
    plane_bytes = sum(b.numel() * 4 for b in step_bufs)
    big = torch.empty(plane_bytes, dtype=torch.uint8, device=dev)
    big.fill_(1)
    one_us = event_launch_us(torch, lambda: rbq.probe_read(big, sink), stream, 5)
    del big
    read_probe = {"step_plane_bytes": plane_bytes,
                  "per_matrix_launches_GBps": round(plane_bytes / (step_probe_ms * 1e-3) / 1e9, 1),
                  "one_launch_GBps": round(plane_bytes / (one_us * 1e-6) / 1e9, 1),
                  "program_time_over_one_launch_read": round(prog_us / one_us, 3)}

    # ---- dual-scale layer y = sum_k g_k (B_k (h_k x)) on the same planes
    dual_shape = {}
    hvec = {}
    for i, (name, _) in enumerate(groups):
        n_in = widths[i]
        if n_in not in hvec:
            hvec[n_in] = torch.ones((K, n_in), dtype=torch.float16, device=dev)
        fns = [(lambda op=ops[l * len(groups) + i], h=hvec[n_in]:
                rbq.gemv_dual(op["planes"], op["scales"], h, op["x"], y=op["y"]))
               for l in range(args.layers)]
        us = graph_launch_us(torch, dev, fns, reps)
        nb = per_call[i] + 2 * K * n_in
        dual_shape[name] = {"shape": f"{shapes[i].out_features}x{n_in}", "bytes": nb,
                            "mean_us": round(us, 3), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}

    layer_chain = None
    if args.layout == "fused" and path in (rbq.PATH_AUTO, rbq.PATH_FLAT, rbq.PATH_VALU):
        layer_chain = decode_layer_chain(args, torch, rbq, L, dev, layers, shapes, xs[0][0], K)
    other_layout = None if args.no_extra else other_layout_program(
        args, torch, rbq, workloads, wl, dev, "separate" if args.layout == "fused" else "fused")

    cpu = None
    if args.cpu_seconds > 0:
        samples = [(layers[0][i][0].cpu().numpy().view(np.uint32), layers[0][i][1].cpu().numpy().view(np.uint16),
                    xs[0][i].cpu().numpy().view(np.uint16)[None, :], group, per_call[i])
                   for i in range(len(groups))]
        cpu = oracle_baseline(samples, args.cpu_seconds)
        cpu["sample"] = "layer 0 at M=1: " + cpu["sample"]

    others = {}
    if not args.no_extra:
        for name, tokens in (("llama2_7b_skinny", 4), ("llama2_7b_skinny", 16), ("llama2_13b_g128", 1),
                             ("llama3_8b_prefill", 2048)):
            sub = measure_layer_set(args, name, tokens, torch, rbq, workloads, dev,
                                    with_prep=name != "llama2_7b_skinny", cpu_seconds=min(args.cpu_seconds, 4.0))
            others[f"{name}_m{tokens}"] = {k: sub[k] for k in ("metric", "value", "unit", "ms_per_step", "dtype",
                                                               "config", "roofline", "cpu_baseline")
                                           if k in sub}
            if "encode_refit_per_shape" in sub:
                others[f"{name}_m{tokens}"]["encode_refit_per_shape"] = sub["encode_refit_per_shape"]
        others["llama3_8b_prefill_m2048"]["more_planes_unpack_kernel"] = prefill_more_planes(
            args, torch, rbq, workloads, dev)

    if not args.no_extra:
        others["llama2_13b_g128_program"] = group_program_step(args, torch, rbq, workloads, dev,
                                                               cpu_seconds=min(args.cpu_seconds, 4.0))
        for mb in (4, 16):
            sk = skinny_program_step(args, torch, rbq, workloads, dev, mb, cpu_seconds=min(args.cpu_seconds, 4.0))
            if sk is not None:
                others[f"llama2_7b_skinny_m{mb}_program"] = sk

    qat = None if args.no_extra else bench_qat(torch, rbq, workloads, dev)

    prog_key = program_key(args)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_INT8_LIMBS,
        "data": "synthetic",
        "config": {"workload": "llama2_7b_decode_gemv", "layers": args.layers,
                   "linears": [f"{l.name} {l.out_features}x{l.in_features}" for l in wl.linears],
                   "layout": args.layout,
                   "ops_per_layer": {name: f"{sh.out_features}x{sh.in_features}"
                                     for (name, _), sh in zip(groups, shapes)},
                   "num_planes": K, "group_size": group, "tokens": 1,
                   "bytes_per_step": bytes_per_step, "launches_per_step": 1,
                   "kernel": "rbq_program_run (one persistent launch over every op of the step)",
                   "planes_layout": ("tiles: RBQ_LAYOUT_TILES, 1 KB per 16-row x 512-column unit, packed once "
                                     "from the row layout by rbq_pack_tiles" if args.planes_layout == "tiles"
                                     else "rows: [K][out][in/32]"),
                   "activations": "one token per decoder-layer input (q/k/v and gate/up share theirs)",
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(bytes_per_step / (prog_us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(bytes_per_step / (prog_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(prog_key, "gemv_program_kernel"),
                     "kernel": f"gemv_program_kernel<{K}> ({len(ops)} ops)",
                     "bytes_per_launch": bytes_per_step, "mean_launch_us": round(prog_us, 2),
                     "rocprof_mean_launch_us": rocprof_mean_us(prog_key)},
        "cpu_baseline": cpu,
        "rows_layout_program": rows_program,
        "pack_tiles": pack,
        "launches": {"ms_per_step": round(ms_launches, 4),
                     "GBps": round(bytes_per_step / (ms_launches * 1e-3) / 1e9, 1),
                     "launches_per_step": len(ops), "graph": True, "path_per_shape": shape_paths,
                     "last_layer_max_rel_diff_vs_program": launch_diff, "per_shape": per_shape},
        "read_probe": read_probe,
        "encode": {"linears": len(wl.linears), "ms": round(enc_ms, 4),
                   "GBps": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 1)},
        "refit": {"linears": len(wl.linears), "ms": round(ref_ms, 4),
                  "GBps": round(ref_bytes / (ref_ms * 1e-3) / 1e9, 1)},
        "encode_refit_per_shape": prep,
        "gemv_dual_per_shape": dual_shape,
        "decode_layer_chain": layer_chain,
        "other_layout": other_layout,
        "other_workloads": others or None,
        "qat": qat,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
