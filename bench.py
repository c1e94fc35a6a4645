"""Benchmark: K=2 batch-1 GEMV on the Llama-2-7B decoder linears.

One step is one decode token through the seven linears (q, k, v, o 4096x4096;
gate, up 11008x4096; down 4096x11008) of each of 32 layers, captured once in
a HIP graph and replayed.  By default q, k, v are stacked row-wise into one
12288x4096 matrix and gate, up into one 22016x4096 matrix, as decode engines
lay them out (4 rbq_gemv launches per layer, 128 per step; every row is
encoded on its own, so the stacked encoding is exactly the separate ones);
--layout separate runs the 7 linears as 224 launches.  Each layer has its own
copy of the encoded planes and scales (1.63 GB in total, far more than the
L2 and Infinity Cache), so every step streams the weights from HBM.  The
weights are seeded synthetic N(0, 0.02^2) matrices with 0.1 % outliers x20,
encoded on the GPU by rbq_encode; activations are N(0, 1) fp16.

Reported (one JSON line):
  value      whole-job GB/s = algorithmic bytes per step / wall time per step
             (bytes = K*out*in/8 planes + 2*K*out scales + 2*in x + 2*out y)
  roofline   the GEMV kernel alone: algorithmic bytes per launch / its mean
             device duration, from HIP events around each launch on the
             library's stream, against MI355X's 8 TB/s HBM peak
  cpu_baseline  the CPU oracle on the host cores on a bounded sample
  encode     rbq_encode of the seven linears (GB/s over W read + planes and
             scales written)
  refit      rbq_refit of the seven linears (GB/s over W and planes read,
             scales read and written); on the 13B g128 set both are timed
             per distinct shape
  encode_refit_per_shape  per distinct shape, one matrix at a time (W
             rotated over copies larger than the caches): encoder, refit,
             re-binarization (GB/s over W and scales read, planes written)
             and, on the decode workload, the dual-scale encoder

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
    ap.add_argument("--workload", default="llama2_7b",
                    choices=["llama2_7b", "llama2_7b_skinny", "llama2_13b_g128", "llama3_8b_prefill"],
                    help="the default is the headline decode GEMV; the others print their own line")
    ap.add_argument("--tokens", type=int, default=0, help="token count for llama2_7b_skinny (4 or 16)")
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
    else:
        bench_layer_set(args)


COPY_PROBE_BYTES = 256 << 20
TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "gemv_llama2_7b_decode_hbm_traffic.json")


def measured_traffic(shape_key, path_name):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated against a copy
    of known size) recorded for this shape, or None when there is no record or
    the kernel's source has changed since the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_PROFILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    for e in doc.get("entries", []):
        if e["shape"] != shape_key or not e["kernel"].startswith(f"gemm_{path_name}_kernel"):
            continue
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_rbq_encode_amd", "csrc",
                           e["source"])
        try:
            with open(src, "rb") as f:
                digest = hashlib.sha256(f.read()).hexdigest()
        except OSError:
            return None
        return e["traffic_bytes"] if digest == e["source_sha256"] else None
    return None


def counter_pass(args):
    """Launches for `rocprofv3 --pmc`: each fused decode shape of the
    Llama-2-7B layer 8 times through rbq_gemv (rotating 8 encoded copies, so
    no launch finds its planes in a cache), then torch copies of a 256 MiB
    buffer, whose read bytes calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    import gemm_rbq_encode_amd as rbq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS["llama2_7b"]
    K = wl.num_planes
    for out_f, in_f in ((12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008)):
        g = torch.Generator(device="cpu").manual_seed(out_f * 31 + in_f)
        W = (torch.randn((out_f, in_f), generator=g) * 0.02).to(dev)
        p, sc = rbq.encode(W, K, 0)
        del W
        copies = [(p.clone(), sc.clone()) for _ in range(8)]
        x = torch.from_numpy(workloads.workload_activations(wl, in_f, 1).view(np.float16)).to(dev)[0]
        for pp, ss in copies:
            rbq.gemv(pp, ss, x)
        torch.cuda.synchronize()
        print(f"counter pass: {out_f}x{in_f} x8 "
              f"({gemv_bytes(out_f, in_f, K, 1)} algorithmic bytes per launch)", flush=True)
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"counter pass: copy of {COPY_PROBE_BYTES} bytes x4", flush=True)


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


def decode_layer_chain(args, torch, rbq, L, dev, layers, shapes, xs, K, group):
    """The same 32 layers as a chained decoder step: q/k/v on x, o on q
    (the attention between them is outside this library), gate/up with the
    silu(gate) * up epilogue on rows interleaved as (gate, up) pairs, down on
    its output h.  Each launch reads what the one before it wrote, as in
    decoding.  One HIP graph per step; reports ms and GB/s over the same
    algorithmic bytes (h is written once at half the gate/up rows)."""
    n_ff = shapes[2].out_features // 2
    perm = torch.stack([torch.arange(n_ff), torch.arange(n_ff) + n_ff], dim=1).reshape(-1).to(dev)
    gu = [(p.index_select(1, perm).contiguous(), s.index_select(1, perm).contiguous())
          for p, s in (layer[2] for layer in layers)]
    x = xs[shapes[0].in_features]
    qkv = torch.empty(shapes[0].out_features, dtype=torch.float16, device=dev)
    o = torch.empty(shapes[1].out_features, dtype=torch.float16, device=dev)
    h = torch.empty(n_ff, dtype=torch.float16, device=dev)
    y = torch.empty(shapes[3].out_features, dtype=torch.float16, device=dev)

    def step(st):
        for layer, (gp, gs) in zip(layers, gu):
            rcs = (L.rbq_gemv(layer[0][0].data_ptr(), layer[0][1].data_ptr(), shapes[0], x.data_ptr(),
                              qkv.data_ptr(), st),
                   L.rbq_gemv(layer[1][0].data_ptr(), layer[1][1].data_ptr(), shapes[1], qkv.data_ptr(),
                              o.data_ptr(), st),
                   L.rbq_gemm_ex(gp.data_ptr(), gs.data_ptr(), shapes[2], x.data_ptr(), 1, h.data_ptr(),
                                 None, 0, rbq.RBQ_EPILOGUE_SILU_MUL, st),
                   L.rbq_gemv(layer[3][0].data_ptr(), layer[3][1].data_ptr(), shapes[3], h.data_ptr(),
                              y.data_ptr(), st))
            if any(rcs):
                raise rbq.RbqError(max(rcs), "decode layer chain")

    stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(side.cuda_stream)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    per_layer = sum(gemv_bytes(sh.out_features, sh.in_features, K, 1) for sh in shapes) - 2 * n_ff
    del graph, gu
    return {"layers": len(layers), "ms_per_step": round(ms, 4),
            "GBps": round(per_layer * len(layers) / (ms * 1e-3) / 1e9, 1),
            "launches_per_layer": 4, "epilogue": "silu(gate)*up in the gate/up launch"}


def bench_layer_set(args):
    """Skinny, grouped-scale and prefill workloads: each linear of the set is
    run back to back (one launch each) over a rotation of encoded copies;
    reports algorithmic GB/s (decode-like sets) or dense-equivalent TFLOP/s
    (prefill), and the per-launch device time from HIP events."""
    import torch

    import gemm_rbq_encode_amd as rbq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    K, group = wl.num_planes, wl.group_size
    M = args.tokens or max(wl.tokens)
    stream = torch.cuda.current_stream(dev)
    # distinct shapes only (q/k/v/o and gate/up share shapes)
    uniq = []
    for i, lin in enumerate(wl.linears):
        if all((lin.out_features, lin.in_features) != (l.out_features, l.in_features) for _, l in uniq):
            uniq.append((i, lin))
    prefill = args.workload == "llama3_8b_prefill"
    rot = 2 if prefill else max(2, int(2.0e9 // sum(
        K * l.out_features * l.in_features // 8 for _, l in uniq)))
    sets, prep = [], {}
    for i, lin in uniq:
        W = torch.from_numpy(workloads.workload_weight(wl, i)).to(dev)
        p, sc = rbq.encode(W, K, group)
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
        X = torch.from_numpy(workloads.workload_activations(wl, lin.in_features, M).view(np.float16)).to(dev)
        Y = torch.empty((M, lin.out_features), dtype=torch.float16, device=dev)
        copies = [(p.clone(), sc.clone()) for _ in range(rot)]
        sets.append((lin, copies, X, Y))
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
            "dtype": "f16" if names[path] in ("prefill", "split") else ("i8" if names[path] != "valu" else "f32"),
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
    print(json.dumps(line), flush=True)


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

    # ---- weights: layer 0 from the seeded generator, encoded on the GPU
    stream = torch.cuda.current_stream(dev)
    enc_planes, enc_scales, enc_bytes, Ws = [], [], 0, []
    for i, lin in enumerate(wl.linears):
        W = torch.from_numpy(workloads.workload_weight(wl, i)).to(dev)
        p, s = rbq.encode(W, K, group)
        Ws.append(W)
        enc_planes.append(p)
        enc_scales.append(s)
        enc_bytes += 4 * W.numel() + p.numel() * 4 + s.numel() * 2
    torch.cuda.synchronize()
    # encoder time: the seven encodes (outputs rewritten in place) captured in
    # one HIP graph, replayed back to back
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    enc_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(enc_graph, stream=side):
        for W, p, s in zip(Ws, enc_planes, enc_scales):
            rbq.encode(W, K, group, planes=p, scales=s)
    torch.cuda.synchronize()
    enc_graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    enc_reps = 5
    e0.record(stream)
    for _ in range(enc_reps):
        enc_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1) / enc_reps
    del enc_graph
    # refit time: the seven refits (into copies of the scales) in one graph
    ref_scales = [s.clone() for s in enc_scales]
    ref_bytes = sum(4 * W.numel() + p.numel() * 4 + 4 * s.numel()
                    for W, p, s in zip(Ws, enc_planes, ref_scales))
    ref_ms = graph_ms(torch, dev, [(lambda W=W, p=p, s=s: rbq.refit(W, p, s, group))
                                   for W, p, s in zip(Ws, enc_planes, ref_scales)], 5)
    # per distinct shape: encoder and refit time of one matrix
    prep = {}
    for W, p, s in zip(Ws, enc_planes, enc_scales):
        key = f"{W.shape[0]}x{W.shape[1]}"
        if key in prep:
            continue
        pe, se, sr = torch.empty_like(p), torch.empty_like(s), s.clone()
        # one call per copy of W (copies exceed the caches), three replays
        Wc = rotation_copies(W)
        e_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.encode(Wi, K, group, planes=pe, scales=se))
                                     for Wi in Wc], 3) / len(Wc)
        r_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.refit(Wi, p, sr, group)) for Wi in Wc], 3) / len(Wc)
        pr = p.clone()
        rb_ms = graph_ms(torch, dev, [(lambda Wi=Wi: rbq.rebinarize(Wi, pr, s, group)) for Wi in Wc], 3) / len(Wc)
        del Wc
        wb, pb, sb = 4 * W.numel(), 4 * p.numel(), 2 * s.numel()
        # dual-scale encoder (residual SVID, 20 alternating steps per plane)
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
    del Ws, ref_scales

    # ---- launch groups.  "fused" stacks the rows of q, k, v (and of gate, up)
    # into one matrix: rows are encoded independently, so the stacked planes
    # and scales are exactly the separate ones placed one after another.
    if args.layout == "fused":
        groups = [("qkv_proj", [0, 1, 2]), ("o_proj", [3]), ("gate_up_proj", [4, 5]),
                  ("down_proj", [6])]
    else:
        groups = [(lin.name, [i]) for i, lin in enumerate(wl.linears)]
    g_planes, g_scales, g_shapes, g_in = [], [], [], []
    for name, idx in groups:
        p = torch.cat([enc_planes[i] for i in idx], dim=1).contiguous()
        s = torch.cat([enc_scales[i] for i in idx], dim=1).contiguous()
        g_planes.append(p)
        g_scales.append(s)
        g_shapes.append(rbq.shape(p.shape[1], p.shape[2] * 32, K, group))
        g_in.append(p.shape[2] * 32)
    del enc_planes, enc_scales

    # ---- rotation set: one copy of planes and scales per layer
    layers = []
    for layer in range(args.layers):
        layers.append([(p.clone(), s.clone()) for p, s in zip(g_planes, g_scales)])
    torch.cuda.synchronize()
    xs = {}
    for n_in in g_in:
        if n_in not in xs:
            xa = workloads.workload_activations(wl, n_in, 1)
            xs[n_in] = torch.from_numpy(xa.view(np.float16)[0].copy()).to(dev)
    ys = [torch.empty(sh.out_features, dtype=torch.float16, device=dev) for sh in g_shapes]

    shapes = g_shapes
    per_call = [gemv_bytes(sh.out_features, sh.in_features, K, 1) for sh in g_shapes]
    bytes_per_step = sum(per_call) * args.layers
    calls = []
    for layer in layers:
        for i, (p, s) in enumerate(layer):
            calls.append((p.data_ptr(), s.data_ptr(), shapes[i], xs[g_in[i]].data_ptr(),
                          ys[i].data_ptr(), i))

    def step(st_handle):
        for pp, sp, sh, xp, yp, _ in calls:
            rc = L.rbq_gemv(pp, sp, sh, xp, yp, st_handle)
            if rc != 0:
                raise rbq.RbqError(rc, "rbq_gemv")

    names = path_names(rbq)
    shape_paths = {f"{sh.out_features}x{sh.in_features}":
                   names[rbq.select_path(sh, 1) if path == rbq.PATH_AUTO else path]
                   for sh in shapes}
    path_name = "+".join(sorted(set(shape_paths.values())))

    # ---- whole-job timing: graph replays (or eager steps)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(side.cuda_stream)          # warm the kernels before capture
    side.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step(torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step(stream.cuda_stream)

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
    # (the chain's gate/up epilogue runs in the flat and VALU kernels only)
    layer_chain = decode_layer_chain(args, torch, rbq, L, dev, layers, g_shapes, xs, K, group) \
        if args.layout == "fused" and graph is not None and \
        path in (rbq.PATH_AUTO, rbq.PATH_FLAT, rbq.PATH_VALU) else None

    # ---- per-launch device time of each launch group: its launches over all
    # layers in one graph, replayed between two HIP events on the launch stream
    nlin = len(groups)
    mean_us = [0.0] * nlin
    for i in range(nlin):
        fns = []
        for layer in layers:
            p, s = layer[i]
            fns.append(lambda pp=p.data_ptr(), sp=s.data_ptr(), sh=shapes[i],
                       xp=xs[g_in[i]].data_ptr(), yp=ys[i].data_ptr():
                       L.rbq_gemv(pp, sp, sh, xp, yp, torch.cuda.current_stream(dev).cuda_stream))
        mean_us[i] = graph_launch_us(torch, dev, fns, max(args.kernel_reps, 1) * 4)
    # the dominant kernel: the launch group with the largest share of a step
    dom_i = max(range(nlin), key=lambda i: mean_us[i])
    dom = f"{groups[dom_i][0]} {shapes[dom_i].out_features}x{shapes[dom_i].in_features}"
    achieved = per_call[dom_i] / (mean_us[dom_i] * 1e-6) / 1e9
    dom_key = f"{shapes[dom_i].out_features}x{shapes[dom_i].in_features}"
    tot_us = sum(mean_us)
    per_shape = {}
    for i, (name, _) in enumerate(groups):
        per_shape[name] = {"shape": f"{shapes[i].out_features}x{shapes[i].in_features}",
                           "bytes": per_call[i], "mean_us": round(mean_us[i], 3),
                           "GBps": round(per_call[i] / (mean_us[i] * 1e-6) / 1e9, 1)}

    # ---- dual-scale layer y = sum_k g_k (B_k (h_k x)) on the same planes (the
    # row scales serve as g; h is one input-scale vector per plane and width)
    dual_shape = {}
    hvec = {}
    for i, (name, _) in enumerate(groups):
        n_in = g_in[i]
        if n_in not in hvec:
            hvec[n_in] = torch.ones((K, n_in), dtype=torch.float16, device=dev)
        fns = []
        for layer in layers:
            p, s = layer[i]
            fns.append(lambda pp=p.data_ptr(), sp=s.data_ptr(), hp=hvec[n_in].data_ptr(), sh=shapes[i],
                       xp=xs[n_in].data_ptr(), yp=ys[i].data_ptr():
                       rbq.check(L.rbq_gemv_dual(pp, sp, hp, sh, xp, yp,
                                                 torch.cuda.current_stream(dev).cuda_stream), "rbq_gemv_dual"))
        us = graph_launch_us(torch, dev, fns, max(args.kernel_reps, 1) * 4)
        nb = per_call[i] + 2 * K * n_in
        dual_shape[name] = {"shape": f"{shapes[i].out_features}x{n_in}", "bytes": nb,
                            "mean_us": round(us, 3), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}

    # ---- CPU oracle baseline on a bounded sample (layer 0, one token)
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        planes_np = [p.cpu().numpy().view(np.uint32) for p in g_planes]
        scales_np = [s.cpu().numpy().view(np.uint16) for s in g_scales]
        xs_np = {k: v.cpu().numpy().view(np.uint16)[None, :] for k, v in xs.items()}
        t_start = time.perf_counter()
        done_bytes, reps = 0, 0
        while True:
            for i in range(nlin):
                oracle.gemm(planes_np[i], scales_np[i], xs_np[g_in[i]], group)
                done_bytes += per_call[i]
            reps += 1
            if time.perf_counter() - t_start >= args.cpu_seconds or reps >= 50:
                break
        el = time.perf_counter() - t_start
        cpu = {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{reps} pass(es) over the layer-0 linears at M=1 "
                         f"(fp64 dequantize-and-multiply), {el:.1f} s"}

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
        "dtype": "f32" if path_name == "valu" else "i8",
        "data": "synthetic",
        "config": {"workload": "llama2_7b_decode_gemv", "layers": args.layers,
                   "linears": [f"{l.name} {l.out_features}x{l.in_features}" for l in wl.linears],
                   "layout": args.layout,
                   "launches_per_layer": {name: f"{sh.out_features}x{sh.in_features}"
                                          for (name, _), sh in zip(groups, shapes)},
                   "num_planes": K, "group_size": group, "tokens": 1,
                   "bytes_per_step": bytes_per_step, "graph": graph is not None,
                   "path": path_name, "path_per_shape": shape_paths,
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom_key, shape_paths[dom_key]),
                     "kernel": f"rbq gemv ({shape_paths[dom_key]}) {dom}",
                     "bytes_per_launch": per_call[dom_i], "mean_launch_us": round(mean_us[dom_i], 3),
                     "layer_GBps_from_launch_times": round(sum(per_call) / (tot_us * 1e-6) / 1e9, 1),
                     "per_shape": per_shape},
        "cpu_baseline": cpu,
        "encode": {"linears": len(wl.linears), "ms": round(enc_ms, 4),
                   "GBps": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 1)},
        "refit": {"linears": len(wl.linears), "ms": round(ref_ms, 4),
                  "GBps": round(ref_bytes / (ref_ms * 1e-3) / 1e9, 1)},
        "encode_refit_per_shape": prep,
        "gemv_dual_per_shape": dual_shape,
        "decode_layer_chain": layer_chain,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
