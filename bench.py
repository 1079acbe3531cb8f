#!/usr/bin/env python3
"""Throughput of the Grok-1 top-2-of-8 MoE layer forward pass on one MI355X.

One step = one moe_forward call (router, dispatch, gate/up + GeGLU, down, combine) over
one batch of seeded synthetic inputs already resident in HBM. Default workload: the
Grok-1-shape decode batch (T=8, d=6144, f=32768, E=8, k=2, int8 expert weights with
per-output-channel bf16 scales). Prints ONE JSON line on stdout; progress goes to stderr.

Besides the step time it reports, for the dominant kernel (gate/up + GeGLU), achieved
algorithmic bandwidth (decode) or MFMA throughput (prefill) from HIP events recorded on
the launch stream around that kernel, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
# the launch policy (decode split counts) that the kernels run under
POLICY_SOURCE = "mixture_experts_layer_gemv_amd/csrc/launch_policy.h"
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; % HBM peak (decode T<=64), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(spec, counts):
    """Per-launch algorithmic bytes / FLOPs of the two expert kernels and of the layer.

    Decode units: each touched expert streams its int8 gate+up (2 d f B) and scales (4 f B)
    in the first kernel, its int8 down (d f B) and scales (2 d B) in the second; x is read
    (2 B per element of the real rows). Prefill units: 4 d f FLOPs per assignment for gate/up,
    2 d f for down."""
    touched = int(sum(1 for c in counts if c > 0))
    n_assign = int(sum(counts))
    d, f = spec.d, spec.f
    real = spec.T - spec.n_pad
    gu_bytes = touched * (2 * d * f + 4 * f) + 2 * real * d
    dn_bytes = touched * (d * f + 2 * d)
    layer_bytes = touched * (3 * d * f + 2 * (2 * f + d)) + 2 * spec.T * d + 4 * d * spec.E + 4 * spec.T * d + spec.T
    # prefill gate/up also writes H once (2 B per element); the decode figure leaves out
    # that write, which is below 0.1% of its bytes
    gu_bytes_prefill = touched * (2 * d * f + 4 * f) + 2 * real * d + 2 * n_assign * f
    gu_flops = 4.0 * d * f * n_assign
    dn_flops = 2.0 * d * f * n_assign
    layer_flops = gu_flops + dn_flops + 2.0 * spec.T * d * spec.E
    return dict(touched=touched, n_assign=n_assign, gu_bytes=gu_bytes, dn_bytes=dn_bytes, layer_bytes=layer_bytes,
                gu_bytes_prefill=gu_bytes_prefill, gu_flops=gu_flops, dn_flops=dn_flops, layer_flops=layer_flops)


def recorded_traffic(workload: str, source: str):
    """HBM traffic of the gate/up kernel as measured by rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by the copy calibration) and recorded in profiles/, or None when no record
    matches this workload, the current kernel source and the current launch policy (the
    counters are void once either changes)."""
    import glob
    import hashlib
    import re

    files = [source, POLICY_SOURCE]
    try:
        h = hashlib.sha256()
        for rel in files:
            h.update(open(os.path.join(ROOT, rel), "rb").read())
        digest = h.hexdigest()[:16]
    except OSError:
        return None
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for m in re.finditer(r"<!-- traffic-record (\{.*?\}) -->", open(path).read()):
            rec = json.loads(m.group(1))
            if rec.get("workload") == workload and rec.get("sources") == files and rec.get("sources_sha256_16") == digest:
                rec["profile"] = os.path.relpath(path, ROOT)
                return rec
    return None


def copy_calibration(nbytes: int, steps: int, warmup: int) -> int:
    """A plain copy of known size (torch's device-to-device copy kernel): reads and writes
    nbytes each. Its FETCH_SIZE / WRITE_SIZE counters calibrate the layer's traffic figures,
    and its rate is the practical streaming bandwidth of the part."""
    import torch

    torch.cuda.set_device(0)
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "ms_per_copy": round(ms, 5), "read_plus_write_GBs": round(gbs, 1),
                      "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "batched_decode", "prefill", "skewed", "decode_tp8", "prefill_tp8"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--variant", default="gather", choices=["gather", "dense", "graph", "block"],
                    help="gather: moe_forward (the headline); dense: the one-hot-gated formulation; "
                         "graph: moe_forward replayed from a captured HIP graph; block: the MoE block with "
                         "the pre-norm and post-norm + residual fused")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the layer, time a plain device-to-device copy of BYTES bytes "
                         "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}). The layer would shard over f with one all-reduce of the output; "
              "that path is not built.", file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import mixture_experts_layer_gemv_amd as moe
    import synth

    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps, args.warmup)

    spec = synth.CONFIGS[args.workload]
    T, d, f, E, k = spec.T, spec.d, spec.f, spec.E, spec.k
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    t0 = time.time()
    inp = synth.make_inputs(spec)
    log(f"generated {args.workload} inputs in {time.time() - t0:.1f}s")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    bf = lambda a: to(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
    x, wr, sc = bf(inp["x"]), to(inp["router_w"]), bf(inp["scales"])
    wg, wu, wd = to(inp["w_gate"]), to(inp["w_up"]), to(inp["w_down"])
    pad = None if inp["pad_mask"] is None else to(inp["pad_mask"])
    bias = None if inp["router_bias"] is None else to(inp["router_bias"])
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM after {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    counts_t = torch.empty(E, dtype=torch.int32, device=dev)

    def step(dbg=None):
        moe.moe_forward_ex(x, wr, wg, wu, wd, sc, pad, out, T, d, f, E, k, stream, router_bias=bias, dbg=dbg)

    step(dbg={"counts": counts_t})  # allocates the library workspace (synchronising), outside timing
    torch.cuda.synchronize()
    counts = counts_t.cpu().tolist()
    graph = None
    if args.variant == "dense":
        def step(dbg=None):  # noqa: F811
            moe.moe_forward_dense(x, wr, wg, wu, wd, sc, pad, out, T, d, f, E, k, stream, router_bias=bias)
    elif args.variant == "graph":
        graph = moe.Graph(x, wr, wg, wu, wd, sc, pad, out, T, d, f, E, k, router_bias=bias)

        def step(dbg=None):  # noqa: F811
            graph.launch(stream)
    elif args.variant == "block":
        ones = torch.ones(d, dtype=torch.float32, device=dev)

        def step(dbg=None):  # noqa: F811
            moe.moe_block_forward(x, ones, ones, 1e-5, wr, wg, wu, wd, sc, pad, out, T, d, f, E, k, stream,
                                  router_bias=bias)
    step()
    torch.cuda.synchronize()
    gu_ms = dn_ms = None
    if args.variant == "gather":
        # ---- per-kernel durations (first, so that the GPU is at its steady clocks for the timed
        #      steps after it): the same kernels through the stage entry points, with HIP events
        #      recorded on the launch stream around the two expert kernels
        tk = T * k
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, k), dtype=torch.float32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(max(tk, 1), dtype=torch.int32, device=dev)
        pos = torch.empty((T, k), dtype=torch.int32, device=dev)
        h = torch.empty((tk, f), dtype=torch.float16, device=dev)
        splits = moe.down_splits(T, d, f, E, k)
        y = torch.empty((splits, tk, d), dtype=torch.float32, device=dev)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

        def staged(e=None):
            moe.moe_route(x, wr, bias, pad, ids, wts, T, d, E, k, stream)
            moe.moe_dispatch(ids, pad, counts_t, offsets, perm, pos, T, E, k, stream)
            if e:
                e[0].record(stream)
            moe.moe_gate_up(x, perm, offsets, wg, wu, sc, h, T, d, f, E, k, stream)
            if e:
                e[1].record(stream)
                e[2].record(stream)
            moe.moe_down(h, offsets, wd, sc, y, splits, T, d, f, E, k, stream)
            if e:
                e[3].record(stream)
            moe.moe_combine(y, splits, pos, wts, pad, out, T, d, k, stream)

        # from idle the GPU takes ~15 ms of work to reach its steady clocks: warm the staged
        # passes up for at least 20 of them
        for _ in range(max(20, args.warmup)):
            staged()
        torch.cuda.synchronize()
        for i in range(args.steps):
            staged(evs[i])
        torch.cuda.synchronize()
        gu_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        dn_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
        log(f"gate_up {gu_ms:.4f} ms, down {dn_ms:.4f} ms (splits={splits})")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log(f"{args.steps} steps: {ms_per_step:.4f} ms/step ({args.variant})")
    if args.variant != "gather":
        print(json.dumps({"metric": METRIC, "value": round(T / (ms_per_step * 1e-3), 2), "unit": "tokens/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "variant": args.variant,
                          "config": {"workload": f"{args.workload}: {spec.description}", "T": T, "d": d, "f": f,
                                     "E": E, "k": k, "n_pad": spec.n_pad}}), flush=True)
        return 0

    work = algorithmic_work(spec, counts)
    bm = moe.expert_kernels(T, d, f, E, k)  # 0: streaming kernels, else tiled with bm-row tiles
    streaming = bm == 0
    if streaming:
        gu_ach = work["gu_bytes"] / (gu_ms * 1e-3) / 1e9
        dn_ach = work["dn_bytes"] / (dn_ms * 1e-3) / 1e9
        rec = recorded_traffic(args.workload, "mixture_experts_layer_gemv_amd/csrc/expert_decode.hip")
        roof = {"bound": "hbm", "achieved": round(gu_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_ach / HBM_PEAK_GBS, 4),
                "traffic": rec["gate_up_traffic_bytes"] if rec else None,
                "traffic_source": rec["profile"] if rec else None, "kernel": "gate_up_decode_kernel",
                "algorithmic_bytes_per_launch": work["gu_bytes"], "avg_launch_ms": round(gu_ms, 5)}
        kern = {"down_decode_kernel": {"avg_launch_ms": round(dn_ms, 5), "achieved_GBs": round(dn_ach, 1),
                                       "frac": round(dn_ach / HBM_PEAK_GBS, 4),
                                       "algorithmic_bytes_per_launch": work["dn_bytes"]},
                "layer": {"hbm_GBs": round(work["layer_bytes"] / (ms_per_step * 1e-3) / 1e9, 1),
                          "hbm_frac": round(work["layer_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes": work["layer_bytes"]}}
    else:
        gu_ach = work["gu_flops"] / (gu_ms * 1e-3) / 1e12
        dn_ach = work["dn_flops"] / (dn_ms * 1e-3) / 1e12
        rec = recorded_traffic(args.workload, "mixture_experts_layer_gemv_amd/csrc/expert_prefill.hip")
        roof = {"bound": "mfma", "achieved": round(gu_ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": rec["gate_up_traffic_bytes"] if rec else None,
                "traffic_source": rec["profile"] if rec else None,
                "kernel": f"expert_prefill_kernel<true, {bm}>", "algorithmic_flops_per_launch": work["gu_flops"],
                "algorithmic_bytes_per_launch": work["gu_bytes_prefill"], "avg_launch_ms": round(gu_ms, 5)}
        layer_tf = work["layer_flops"] / (ms_per_step * 1e-3) / 1e12
        kern = {f"expert_prefill_kernel<false, {bm}>": {"avg_launch_ms": round(dn_ms, 5), "achieved_TFLOPs": round(dn_ach, 1),
                                                 "frac": round(dn_ach / MFMA_BF16_PEAK_TFLOPS, 4)},
                "layer": {"TFLOPs": round(layer_tf, 1), "mfma_frac": round(layer_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "algorithmic_flops": work["layer_flops"]}}

    # ---- CPU baseline: the oracle as it stands, on a bounded sample of the same workload
    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        cores = max(1, min(cores, 16))
        rows = np.arange(T) if T <= 16 else np.random.default_rng(0).choice(T, 16, replace=False)
        reps, tok, t_start = 0, 0, time.time()
        while True:
            oracle.forward_inputs(inp, k=k, nthreads=cores, rows=rows)
            reps += 1
            tok += len(rows)
            if time.time() - t_start >= args.cpu_seconds or reps >= 1000:
                break
        el = time.time() - t_start
        cpu = {"value": round(tok / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"{reps} oracle forward(s) of {len(rows)} token rows of the {args.workload} workload "
                         f"({el:.1f} s wall, fp32, {cores} threads)"}
        log(f"cpu oracle: {cpu['value']} tokens/s")

    line = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec.description}", "T": T, "d": d, "f": f, "E": E, "k": k,
                   "n_pad": spec.n_pad, "weights": "int8 + bf16 per-output-channel scales",
                   "touched_experts": work["touched"], "assignments": work["n_assign"], "down_splits": splits,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": kern,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
