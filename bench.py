#!/usr/bin/env python3
"""Throughput of the Grok-1 top-2-of-8 MoE layer forward pass on one MI355X.

One step = one moe_forward call (router, dispatch, gate/up + GeGLU, down, combine) over
one batch of seeded synthetic inputs already resident in HBM. The headline workload is
the Grok-1-shape decode batch (T=8, d=6144, f=32768, E=8, k=2, int8 expert weights with
per-output-channel bf16 scales); the same JSON line carries the other four workloads the
metric is defined on (the tiny layer, batched decode, prefill, skewed routing) under
"configs", each with its own timing, roofline and CPU-oracle baseline, and one GPU's share of
an 8-way tensor-parallel split over f (decode and prefill) under "tp_share". Prints ONE JSON
line on stdout; progress goes to stderr.

For the dominant kernel (gate/up + GeGLU) of each workload it reports achieved algorithmic
bandwidth (streaming kernels, decode) or MFMA throughput (tiled kernels, prefill) from HIP
events recorded on the launch stream around that kernel, and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.abspath(__file__))
# the launch policy (decode split counts) that the kernels run under
POLICY_SOURCE = "mixture_experts_layer_gemv_amd/csrc/launch_policy.h"
# the sources of the expert kernels whose counters the traffic records hold
DECODE_SOURCES = ["mixture_experts_layer_gemv_amd/csrc/expert_decode.hip", "mixture_experts_layer_gemv_amd/csrc/stream_common.h",
                  "mixture_experts_layer_gemv_amd/csrc/device_common.h"]
PREFILL_SOURCES = ["mixture_experts_layer_gemv_amd/csrc/expert_prefill.hip", "mixture_experts_layer_gemv_amd/csrc/device_common.h"]
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; % HBM peak (decode T<=64), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
WORKLOADS = ["tiny", "decode", "batched_decode", "prefill", "skewed", "decode_tp8", "prefill_tp8"]
# the five workloads the metric is defined on; the first after the headline are reported under "configs"
METRIC_WORKLOADS = ["tiny", "decode", "batched_decode", "prefill", "skewed"]
# reported under "tp_share": one GPU's share of the layer split 8 ways over f
TP_SHARE_WORKLOADS = ["decode_tp8", "prefill_tp8"]
# a process driving one GPU is given a share of 16 host cores, whatever the host has in all
HOST_CORE_SHARE = 16


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_info() -> dict:
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "hardware_concurrency": os.cpu_count(), "affinity_cpus": affinity,
            "oracle_threads": max(1, min(affinity, HOST_CORE_SHARE))}


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


def prefill_kernel_name(gate_up: bool, bm: int) -> str:
    """The tiled kernel the library launches for bm-row tiles (256: the 4-wavefront kernel)."""
    return f"expert_wide_kernel<{str(gate_up).lower()}>" if bm == 256 else f"expert_prefill_kernel<{str(gate_up).lower()}, {bm}>"


def recorded_traffic(workload: str, sources: list):
    """HBM traffic of the gate/up kernel as measured by rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by the copy calibration) and recorded in profiles/, or None when no record
    matches this workload, the current kernel source and the current launch policy (the
    counters are void once either changes)."""
    import glob
    import hashlib
    import re

    files = list(sources) + [POLICY_SOURCE]
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


class Inputs:
    """Host inputs of a workload and their device copies (the Grok-shape workloads share one
    weight set, uploaded once)."""

    _weights: dict = {}

    def __init__(self, name: str):
        import numpy as np
        import torch

        import synth

        self.spec = s = synth.WORKLOAD_SPECS[name]
        dev = torch.device("cuda:0")
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        bf = lambda a: to(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
        t0 = time.time()
        wkey = (s.d, s.f, s.E, s.w_set, s.f_full)
        if wkey not in Inputs._weights:
            Inputs._weights.clear()  # keep one weight set resident at a time
            host = {n: synth.expert_weights(s, n.split("_")[1]) for n in ("w_gate", "w_up", "w_down")}
            host["router_w"] = synth.router_w(s)
            host["scales"] = synth.scales(s)
            devw = {n: to(host[n]) for n in ("w_gate", "w_up", "w_down", "router_w")}
            devw["scales"] = bf(host["scales"])
            Inputs._weights[wkey] = (host, devw)
        host, devw = Inputs._weights[wkey]
        self.inp = synth.make_inputs(s, with_weights=False)
        self.inp.update({n: host[n] for n in ("w_gate", "w_up", "w_down", "router_w", "scales")})
        self.x, self.wr, self.sc = bf(self.inp["x"]), devw["router_w"], devw["scales"]
        self.wg, self.wu, self.wd = devw["w_gate"], devw["w_up"], devw["w_down"]
        self.pad = None if self.inp["pad_mask"] is None else to(self.inp["pad_mask"])
        self.bias = None if self.inp["router_bias"] is None else to(self.inp["router_bias"])
        self.out = torch.empty((s.T, s.d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        log(f"{name}: inputs resident in HBM after {time.time() - t0:.1f}s")


def timed_steps(step, steps: int, stream) -> dict:
    """Exactly `steps` calls of step() between two synchronisations, with a HIP event on the
    launch stream before each call and after the last: mean (the headline), median and min."""
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return {"ms_per_step": evs[0].elapsed_time(evs[steps]) / steps, "ms_median": statistics.median(per),
            "ms_min": min(per)}


def cpu_baseline(wl: Inputs, seconds: float, threads: int, name: str):
    """The oracle as it stands on a bounded sample of the workload's token rows (all rows up
    to 16 tokens, else 16 seeded rows, repeated until `seconds` of wall time)."""
    import numpy as np

    import oracle

    T, k = wl.spec.T, wl.spec.k
    rows = np.arange(T) if T <= 16 else np.sort(np.random.default_rng(0).choice(T, 16, replace=False))
    reps, tok, t_start = 0, 0, time.time()
    while True:
        oracle.forward_inputs(wl.inp, k=k, nthreads=threads, rows=rows)
        reps += 1
        tok += len(rows)
        if time.time() - t_start >= seconds or reps >= 1000:
            break
    el = time.time() - t_start
    return {"value": round(tok / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} oracle forward(s) of {len(rows)} token rows of the {name} workload "
                      f"({el:.1f} s wall, fp32, {threads} threads)"}


def measure(name: str, args, host: dict, cpu_seconds: float, graph: bool) -> dict:
    """Staged per-kernel timing, then warm-up and K timed forward steps of one workload."""
    import torch

    import mixture_experts_layer_gemv_amd as moe

    wl = Inputs(name)
    s = wl.spec
    T, d, f, E, k = s.T, s.d, s.f, s.E, s.k
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    counts_t = torch.empty(E, dtype=torch.int32, device=dev)

    def step(dbg=None):
        moe.moe_forward_ex(wl.x, wl.wr, wl.wg, wl.wu, wl.wd, wl.sc, wl.pad, wl.out, T, d, f, E, k, stream,
                           router_bias=wl.bias, dbg=dbg)

    step(dbg={"counts": counts_t})  # grows the library workspace (synchronising), outside timing
    torch.cuda.synchronize()
    counts = counts_t.cpu().tolist()

    # ---- per-kernel durations first (from idle the GPU needs ~15 ms of work to reach its
    #      steady clocks): the same kernels through the stage entry points, HIP events on the
    #      launch stream around the two expert kernels
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
        moe.moe_route(wl.x, wl.wr, wl.bias, wl.pad, ids, wts, T, d, E, k, stream)
        moe.moe_dispatch(ids, wl.pad, counts_t, offsets, perm, pos, T, E, k, stream)
        if e:
            e[0].record(stream)
        moe.moe_gate_up(wl.x, perm, offsets, wl.wg, wl.wu, wl.sc, h, T, d, f, E, k, stream)
        if e:
            e[1].record(stream)
            e[2].record(stream)
        moe.moe_down(h, offsets, wl.wd, wl.sc, y, splits, T, d, f, E, k, stream)
        if e:
            e[3].record(stream)
        moe.moe_combine(y, splits, pos, wts, wl.pad, wl.out, T, d, k, stream)

    for _ in range(max(20, args.warmup)):
        staged()
    torch.cuda.synchronize()
    for i in range(args.steps):
        staged(evs[i])
    torch.cuda.synchronize()
    gu_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dn_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    log(f"{name}: gate_up {gu_ms:.4f} ms, down {dn_ms:.4f} ms (splits={splits})")
    del h, y

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---- timed region: exactly K steps
    t = timed_steps(step, args.steps, stream)
    log(f"{name}: {args.steps} steps: {t['ms_per_step']:.4f} ms/step (median {t['ms_median']:.4f}, "
        f"min {t['ms_min']:.4f})")

    work = algorithmic_work(s, counts)
    bm = moe.expert_kernels(T, d, f, E, k)  # 0: streaming kernels, else tiled with bm-row tiles
    if bm == 0:
        gu_ach = work["gu_bytes"] / (gu_ms * 1e-3) / 1e9
        dn_ach = work["dn_bytes"] / (dn_ms * 1e-3) / 1e9
        rec = recorded_traffic(name, DECODE_SOURCES)
        roof = {"bound": "hbm", "achieved": round(gu_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_ach / HBM_PEAK_GBS, 4),
                "traffic": rec["gate_up_traffic_bytes"] if rec else None,
                "traffic_source": rec["profile"] if rec else None,
                "kernel": "gate_up_decode_kernel" if moe.gate_up_parts(T, d, f, E, k) == 1
                else "gate_up_decode_kernel + geglu_finish_kernel (split contraction; the events bracket both)",
                "algorithmic_bytes_per_launch": work["gu_bytes"], "avg_launch_ms": round(gu_ms, 5)}
        layer_gbs = work["layer_bytes"] / (t["ms_per_step"] * 1e-3) / 1e9
        kern = {"down_decode_kernel": {"avg_launch_ms": round(dn_ms, 5), "achieved_GBs": round(dn_ach, 1),
                                       "frac": round(dn_ach / HBM_PEAK_GBS, 4),
                                       "algorithmic_bytes_per_launch": work["dn_bytes"]},
                "layer": {"bound": "hbm", "hbm_GBs": round(layer_gbs, 1), "hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes": work["layer_bytes"]}}
    else:
        gu_ach = work["gu_flops"] / (gu_ms * 1e-3) / 1e12
        dn_ach = work["dn_flops"] / (dn_ms * 1e-3) / 1e12
        rec = recorded_traffic(name, PREFILL_SOURCES)
        roof = {"bound": "mfma", "achieved": round(gu_ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": rec["gate_up_traffic_bytes"] if rec else None,
                "traffic_source": rec["profile"] if rec else None,
                "kernel": prefill_kernel_name(True, bm), "algorithmic_flops_per_launch": work["gu_flops"],
                "algorithmic_bytes_per_launch": work["gu_bytes_prefill"], "avg_launch_ms": round(gu_ms, 5)}
        layer_tf = work["layer_flops"] / (t["ms_per_step"] * 1e-3) / 1e12
        kern = {prefill_kernel_name(False, bm): {"avg_launch_ms": round(dn_ms, 5),
                                                        "achieved_TFLOPs": round(dn_ach, 1),
                                                        "frac": round(dn_ach / MFMA_BF16_PEAK_TFLOPS, 4)},
                "layer": {"bound": "mfma", "TFLOPs": round(layer_tf, 1),
                          "mfma_frac": round(layer_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "algorithmic_flops": work["layer_flops"]}}
        if s.d * s.f <= (1 << 23):
            kern["layer"]["note"] = "expert matrices of 2^23 weights or fewer: launch- and latency-bound, not a roofline case"

    res = {"T": T, "d": d, "f": f, "E": E, "k": k, "n_pad": s.n_pad, "description": s.description,
           "value": round(T / (t["ms_per_step"] * 1e-3), 2), "unit": "tokens/s",
           "non_pad_tokens_per_s": round((T - s.n_pad) / (t["ms_per_step"] * 1e-3), 2),
           "ms_per_step": round(t["ms_per_step"], 5), "ms_median": round(t["ms_median"], 5),
           "ms_min": round(t["ms_min"], 5), "touched_experts": work["touched"], "assignments": work["n_assign"],
           "down_splits": splits, "expert_kernels": "streaming" if bm == 0 else f"tiled, {bm}-row tiles",
           "roofline": roof, "kernels": kern}

    if graph:
        # the same forward captured once into a HIP graph and replayed (one launch per step)
        ws = torch.empty(moe.workspace_bytes(T, d, f, E, k) + 256, dtype=torch.uint8, device=dev)
        g = moe.Graph(wl.x, wl.wr, wl.wg, wl.wu, wl.wd, wl.sc, wl.pad, wl.out, T, d, f, E, k, router_bias=wl.bias,
                      workspace=ws, workspace_bytes_=ws.numel())
        try:
            for _ in range(args.warmup):
                g.launch(stream)
            tg = timed_steps(lambda: g.launch(stream), args.steps, stream)
        finally:
            g.close()
        res["graph"] = {k2: round(v, 5) for k2, v in tg.items()}
        log(f"{name}: graph replay {tg['ms_per_step']:.4f} ms/step")

    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(wl, cpu_seconds, host["oracle_threads"], name)
        log(f"{name}: cpu oracle {res['cpu_baseline']['value']} tokens/s")
    else:
        res["cpu_baseline"] = None
    return res


def routed(args):
    """The workload's inputs routed and dispatched on the device, with the expert stages' buffers and a
    timer of a callable (mean ms over args.steps calls after a warm-up, HIP events on the launch stream)."""
    import torch

    import mixture_experts_layer_gemv_amd as moe

    wl = Inputs(args.workload)
    s = wl.spec
    T, d, f, E, k = s.T, s.d, s.f, s.E, s.k
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    tk = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(tk, 1), dtype=torch.int32, device=dev)
    pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    h = torch.empty((tk, f), dtype=torch.float16, device=dev)
    splits = moe.down_splits(T, d, f, E, k)
    y = torch.empty((splits, tk, d), dtype=torch.float32, device=dev)
    moe.moe_route(wl.x, wl.wr, wl.bias, wl.pad, ids, wts, T, d, E, k, stream)
    moe.moe_dispatch(ids, wl.pad, counts, offsets, perm, pos, T, E, k, stream)

    def timed(fn) -> float:
        for _ in range(max(20, args.warmup)):
            fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(args.steps):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / args.steps

    def gate_up(x):
        moe.moe_gate_up(x, perm, offsets, wl.wg, wl.wu, wl.sc, h, T, d, f, E, k, stream)

    def down():
        moe.moe_down(h, offsets, wl.wd, wl.sc, y, splits, T, d, f, E, k, stream)

    return SimpleNamespace(wl=wl, s=s, stream=stream, offsets=offsets, h=h, timed=timed, gate_up=gate_up, down=down)


def zero_operands(args) -> int:
    """The expert kernels' durations with the workload's activations and with zeros in their place.
    The routing (hence every tile and launch) is the real inputs'; the MFMA sequence is unchanged,
    so a difference is the clock the operand values allow."""
    import torch

    r = routed(args)
    x0 = torch.zeros_like(r.wl.x)
    res = {}
    res["gate_up_ms_real"] = r.timed(lambda: r.gate_up(r.wl.x))
    res["down_ms_real"] = r.timed(r.down)
    r.h.zero_()
    res["down_ms_zero_h"] = r.timed(r.down)
    res["gate_up_ms_zero_x"] = r.timed(lambda: r.gate_up(x0))
    print(json.dumps({"diagnostic": "expert kernels on the workload's activations and on zeros",
                      "workload": f"{args.workload}: {r.s.description}", "steps": args.steps,
                      **{n: round(v, 4) for n, v in res.items()}}), flush=True)
    return 0


def vendor_gemm(args) -> int:
    """The library's expert kernels beside the vendor GEMM (torch.matmul, which dispatches to
    hipBLASLt) on the same per-expert products: for each expert, its routed row count of the
    workload's activation rows times its gate|up weights as one [d][2f] bf16 matrix, and its rows
    of the layer's real H (fp16) times its down weights as fp16. The vendor GEMMs get the weights
    already converted to 16 bits (twice the weight bytes, no int8 conversion), and do no gather,
    scaling, GeGLU or fp32 output: a plain-GEMM yardstick on the same shapes and operand values."""
    import torch

    r = routed(args)
    s, wl = r.s, r.wl
    r.gate_up(wl.x)
    torch.cuda.synchronize()
    off = r.offsets.cpu().tolist()
    rows = [off[e + 1] - off[e] for e in range(s.E)]
    res = {"rows_per_expert": rows}
    res["gate_up_ms_library"] = r.timed(lambda: r.gate_up(wl.x))
    res["down_ms_library"] = r.timed(r.down)
    a_gu, b_gu, c_gu, a_dn, b_dn, c_dn = [], [], [], [], [], []
    for e in range(s.E):
        if rows[e] == 0:
            continue
        a_gu.append(wl.x[: rows[e]])
        b_gu.append(torch.cat([wl.wg[e], wl.wu[e]], dim=1).to(torch.bfloat16).contiguous())
        c_gu.append(torch.empty((rows[e], 2 * s.f), dtype=torch.bfloat16, device=wl.x.device))
        a_dn.append(r.h[off[e]: off[e + 1]])
        b_dn.append(wl.wd[e].to(torch.float16).contiguous())
        c_dn.append(torch.empty((rows[e], s.d), dtype=torch.float16, device=wl.x.device))

    def vendor(a, b, c):
        for i in range(len(a)):
            torch.matmul(a[i], b[i], out=c[i])

    res["gate_up_ms_vendor_bf16"] = r.timed(lambda: vendor(a_gu, b_gu, c_gu))
    res["down_ms_vendor_fp16"] = r.timed(lambda: vendor(a_dn, b_dn, c_dn))
    n_assign = sum(rows)
    gu_flops, dn_flops = 4.0 * n_assign * s.d * s.f, 2.0 * n_assign * s.d * s.f
    for n in list(res):
        if n.endswith(("_library", "_bf16", "_fp16")):
            pf = (gu_flops if n.startswith("gate_up") else dn_flops) / (res[n] * 1e-3) / 1e15
            res[n] = round(res[n], 4)
            res[n.replace("_ms_", "_pflops_")] = round(pf, 4)
            res[n.replace("_ms_", "_frac_of_2.5P_")] = round(pf / 2.5, 4)
    res["blas_library"] = str(torch.backends.cuda.preferred_blas_library())
    print(json.dumps({"diagnostic": "expert kernels beside the vendor GEMM on the same per-expert products",
                      "workload": f"{args.workload}: {s.description}", "steps": args.steps, **res}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=WORKLOADS)
    ap.add_argument("--configs", default="metric", choices=["metric", "none"],
                    help="metric: also time the other workloads the metric is defined on (reported under "
                         "'configs'); none: only --workload (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the headline workload's oracle baseline (0 = skip)")
    ap.add_argument("--cpu-seconds-other", type=float, default=5.0,
                    help="target CPU time of each other workload's oracle baseline (0 = skip)")
    ap.add_argument("--variant", default="gather", choices=["gather", "dense", "graph", "block"],
                    help="gather: moe_forward (the headline); dense: the one-hot-gated formulation; "
                         "graph: moe_forward replayed from a captured HIP graph; block: the MoE block with "
                         "the pre-norm and post-norm + residual fused")
    ap.add_argument("--zero-operands", action="store_true",
                    help="diagnostic, not a throughput: route and dispatch the workload's own inputs, then time "
                         "the gate/up kernel on them and on zeroed activations, and the down kernel on its real "
                         "H and on a zeroed H (same kernels, same tiles; only the operand values differ)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="diagnostic, not a throughput: the gate/up and down kernels beside torch.matmul "
                         "(hipBLASLt) on the same per-expert products, with 16-bit weights")
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

    import torch

    import mixture_experts_layer_gemv_amd as moe

    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps, args.warmup)

    torch.cuda.set_device(0)
    host = host_info()
    if args.zero_operands:
        return zero_operands(args)
    if args.vendor_gemm:
        return vendor_gemm(args)
    if args.variant != "gather":
        wl = Inputs(args.workload)
        s = wl.spec
        stream = torch.cuda.current_stream()
        if args.variant == "dense":
            def step():
                moe.moe_forward_dense(wl.x, wl.wr, wl.wg, wl.wu, wl.wd, wl.sc, wl.pad, wl.out, s.T, s.d, s.f, s.E, s.k,
                                      stream, router_bias=wl.bias)
        elif args.variant == "graph":
            graph = moe.Graph(wl.x, wl.wr, wl.wg, wl.wu, wl.wd, wl.sc, wl.pad, wl.out, s.T, s.d, s.f, s.E, s.k,
                              router_bias=wl.bias)

            def step():
                graph.launch(stream)
        else:
            ones = torch.ones(s.d, dtype=torch.float32, device="cuda:0")

            def step():
                moe.moe_block_forward(wl.x, ones, ones, 1e-5, wl.wr, wl.wg, wl.wu, wl.wd, wl.sc, wl.pad, wl.out,
                                      s.T, s.d, s.f, s.E, s.k, stream, router_bias=wl.bias)
        step()
        for _ in range(args.warmup):
            step()
        t = timed_steps(step, args.steps, stream)
        log(f"{args.steps} steps: {t['ms_per_step']:.4f} ms/step ({args.variant})")
        print(json.dumps({"metric": METRIC, "value": round(s.T / (t["ms_per_step"] * 1e-3), 2), "unit": "tokens/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": round(t["ms_per_step"], 5), "ms_median": round(t["ms_median"], 5),
                          "ms_min": round(t["ms_min"], 5), "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "variant": args.variant,
                          "config": {"workload": f"{args.workload}: {s.description}", "T": s.T, "d": s.d, "f": s.f,
                                     "E": s.E, "k": s.k, "n_pad": s.n_pad}}), flush=True)
        return 0

    head = measure(args.workload, args, host, args.cpu_seconds, graph=args.workload in ("tiny", "decode"))
    others = {}
    if args.configs == "metric":
        # the Grok-shape workloads share one weight set: run them together, the tiny layer last
        for name in sorted(METRIC_WORKLOADS, key=lambda n: n == "tiny"):
            if name != args.workload:
                others[name] = measure(name, args, host, args.cpu_seconds_other, graph=name in ("tiny", "decode"))
    shares = {}
    if args.configs == "metric":
        # one GPU's share of an 8-way tensor-parallel split of the layer over f, at decode and prefill
        for name in TP_SHARE_WORKLOADS:
            if name != args.workload:
                shares[name] = measure(name, args, host, args.cpu_seconds_other, graph=False)

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_median": head["ms_median"],
        "ms_min": head["ms_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {head['description']}", "T": head["T"], "d": head["d"],
                   "f": head["f"], "E": head["E"], "k": head["k"], "n_pad": head["n_pad"],
                   "weights": "int8 + bf16 per-output-channel scales", "touched_experts": head["touched_experts"],
                   "assignments": head["assignments"], "down_splits": head["down_splits"],
                   "expert_kernels": head["expert_kernels"], "parallelism": "single GPU"},
        "non_pad_tokens_per_s": head["non_pad_tokens_per_s"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "cpu_baseline": head["cpu_baseline"],
        "host": host,
    }
    if "graph" in head:
        line["graph"] = head["graph"]
    if others:
        line["configs"] = {n: {k2: v for k2, v in r.items() if k2 not in ("description",)} | {"workload": r["description"]}
                           for n, r in others.items()}
    if shares:
        line["tp_share"] = {n: {k2: v for k2, v in r.items() if k2 not in ("description",)} | {"workload": r["description"]}
                            for n, r in shares.items()}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
