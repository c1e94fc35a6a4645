"""Benchmark: K=2 batch-1 GEMV on the Llama-2-7B decoder linears.

One step is one decode token through the seven linears (q, k, v, o 4096x4096;
gate, up 11008x4096; down 4096x11008) of each of 32 layers: 224 rbq_gemv
calls, captured once in a HIP graph and replayed.  Each layer has its own
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
    ap.add_argument("--path", choices=["auto", "valu", "decode", "stream"], default="auto")
    ap.add_argument("--split", type=int, default=0,
                    help="waves per 16-row tile in the streaming kernel (0 = automatic)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU path is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemm_rbq_encode_amd as rbq
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS["llama2_7b"]
    K, group = wl.num_planes, wl.group_size
    L = rbq.lib()
    path = {"auto": rbq.PATH_AUTO, "valu": rbq.PATH_VALU, "decode": rbq.PATH_DECODE,
            "stream": rbq.PATH_STREAM}[args.path]
    rbq.set_path(path)
    rbq.set_stream_split(args.split)

    # ---- weights: layer 0 from the seeded generator, encoded on the GPU
    stream = torch.cuda.current_stream(dev)
    enc_ev = []
    enc_planes, enc_scales, enc_bytes = [], [], 0
    for i, lin in enumerate(wl.linears):
        W = torch.from_numpy(workloads.workload_weight(wl, i)).to(dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        p, s = rbq.encode(W, K, group)
        e1.record(stream)
        enc_ev.append((e0, e1))
        enc_planes.append(p)
        enc_scales.append(s)
        enc_bytes += 4 * W.numel() + p.numel() * 4 + s.numel() * 2
        del W
    torch.cuda.synchronize()
    enc_ms = sum(a.elapsed_time(b) for a, b in enc_ev)

    # ---- rotation set: one copy of planes and scales per layer
    layers = []
    for layer in range(args.layers):
        layers.append([(p.clone(), s.clone()) for p, s in zip(enc_planes, enc_scales)])
    torch.cuda.synchronize()
    xs = {}
    for lin in wl.linears:
        if lin.in_features not in xs:
            xa = workloads.workload_activations(wl, lin.in_features, 1)
            xs[lin.in_features] = torch.from_numpy(xa.view(np.float16)[0].copy()).to(dev)
    ys = [torch.empty(lin.out_features, dtype=torch.float16, device=dev) for lin in wl.linears]

    shapes = [rbq.shape(lin.out_features, lin.in_features, K, group) for lin in wl.linears]
    per_call = [gemv_bytes(lin.out_features, lin.in_features, K, 1) for lin in wl.linears]
    bytes_per_step = sum(per_call) * args.layers
    calls = []
    for layer in layers:
        for i, (p, s) in enumerate(layer):
            calls.append((p.data_ptr(), s.data_ptr(), shapes[i],
                           xs[wl.linears[i].in_features].data_ptr(), ys[i].data_ptr(), i))

    def step(st_handle):
        for pp, sp, sh, xp, yp, _ in calls:
            rc = L.rbq_gemv(pp, sp, sh, xp, yp, st_handle)
            if rc != 0:
                raise rbq.RbqError(rc, "rbq_gemv")

    chosen = rbq.select_path(shapes[0], 1) if path == rbq.PATH_AUTO else path
    path_name = {rbq.PATH_VALU: "valu", rbq.PATH_DECODE: "decode", rbq.PATH_PREFILL: "prefill",
                 rbq.PATH_STREAM: "stream"}[chosen]

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

    # ---- per-launch kernel timing with HIP events on the launch stream
    nlin = len(wl.linears)
    evs = []
    for rep in range(args.kernel_reps):
        for pp, sp, sh, xp, yp, i in calls:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = L.rbq_gemv(pp, sp, sh, xp, yp, stream.cuda_stream)
            b.record(stream)
            if rc != 0:
                raise rbq.RbqError(rc, "rbq_gemv")
            evs.append((i, a, b))
    torch.cuda.synchronize()
    dur = [[] for _ in range(nlin)]
    for i, a, b in evs:
        dur[i].append(a.elapsed_time(b) * 1e3)          # microseconds
    mean_us = [float(np.mean(d)) for d in dur]
    # the GEMV kernel over all its launches (one kernel family serves every shape)
    tot_bytes = sum(per_call)
    tot_us = sum(mean_us)
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9
    per_shape = {}
    for i, lin in enumerate(wl.linears):
        key = f"{lin.out_features}x{lin.in_features}"
        if key not in per_shape:
            per_shape[key] = {"bytes": per_call[i], "mean_us": round(mean_us[i], 3),
                              "GBps": round(per_call[i] / (mean_us[i] * 1e-6) / 1e9, 1)}

    # ---- CPU oracle baseline on a bounded sample (layer 0, one token)
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        planes_np = [p.cpu().numpy().view(np.uint32) for p in enc_planes]
        scales_np = [s.cpu().numpy().view(np.uint16) for s in enc_scales]
        xs_np = {k: v.cpu().numpy().view(np.uint16)[None, :] for k, v in xs.items()}
        t_start = time.perf_counter()
        done_bytes, reps = 0, 0
        while True:
            for i, lin in enumerate(wl.linears):
                oracle.gemm(planes_np[i], scales_np[i], xs_np[lin.in_features], group)
                done_bytes += per_call[i]
            reps += 1
            if time.perf_counter() - t_start >= args.cpu_seconds or reps >= 50:
                break
        el = time.perf_counter() - t_start
        cpu = {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{reps} pass(es) over the 7 layer-0 linears at M=1 "
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
                   "num_planes": K, "group_size": group, "tokens": 1,
                   "bytes_per_step": bytes_per_step, "graph": graph is not None,
                   "path": path_name, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": f"rbq gemv ({path_name})",
                     "mean_launch_us": round(tot_us / nlin, 3), "per_shape": per_shape},
        "cpu_baseline": cpu,
        "encode": {"linears": nlin, "ms": round(enc_ms, 4),
                   "GBps": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 1)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
