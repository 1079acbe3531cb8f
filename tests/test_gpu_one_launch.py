"""GPU tests of the one-launch layer (small batches: routing, dispatch, gate/up, down and
combine as work items of one kernel; taken when MOE_ONE_LAUNCH=1). At each of its kernel configurations it must give the
bits of the launch-per-stage sequence (the routing and dispatch arrays and the output) and
agree with the oracle; its control block must stay usable across calls of different sizes,
caller workspaces with stale contents, graph replays and the allocation-free entry point."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import OUT_TOL, exclusions, max_excluded, rms, sample_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mixture_experts_layer_gemv_amd as moe  # noqa: E402

_weights: dict = {}


def inputs(base: str, T: int, n_pad: int = 0, bias=None, x_set: int = 7000):
    """The base workload's expert weights (kept on the device, one set at a time) with T fresh
    activation rows of their own stream."""
    spec = synth.replace(synth.WORKLOAD_SPECS[base], T=T, n_pad=n_pad, bias=bias, x_set=x_set + T)
    if base not in _weights:
        _weights.clear()
        full = synth.make_inputs(synth.WORKLOAD_SPECS[base])
        _weights[base] = ({n: full[n] for n in ("w_gate", "w_up", "w_down")},
                          {n: torch.from_numpy(full[n]).cuda() for n in ("w_gate", "w_up", "w_down")})
    host_w, dev_w = _weights[base]
    inp = synth.make_inputs(spec, with_weights=False)
    inp.update(host_w)
    d = to_dev(inp, with_weights=False)
    d.update(dev_w)
    return spec, inp, d


def run(s, d, monkeypatch, one_launch: bool, how: str = "library"):
    """The forward through one entry point; returns (out, routing and dispatch arrays)."""
    if one_launch:
        monkeypatch.setenv("MOE_ONE_LAUNCH", "1")
    else:
        monkeypatch.delenv("MOE_ONE_LAUNCH", raising=False)
    assert moe.one_launch(s.T, s.d, s.f, s.E, s.k) == int(one_launch)
    out = torch.full((s.T, s.d), float("nan"), device="cuda")
    args = (d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], out, s.T, s.d,
            s.f, s.E, s.k)
    tk = s.T * s.k
    dbg = {"topk_ids": torch.empty(tk, dtype=torch.int32, device="cuda"),
           "topk_w": torch.empty(tk, dtype=torch.float32, device="cuda"),
           "counts": torch.empty(s.E, dtype=torch.int32, device="cuda"),
           "offsets": torch.empty(s.E + 1, dtype=torch.int32, device="cuda"),
           "perm": torch.empty(tk, dtype=torch.int32, device="cuda"),
           "pos": torch.empty(tk, dtype=torch.int32, device="cuda")}
    if how == "library":
        moe.moe_forward_ex(*args, router_bias=d["router_bias"], dbg=dbg)
    elif how == "workspace":
        # a caller workspace holding stale bytes: the call zeroes the control block itself
        ws = torch.full((moe.workspace_bytes(s.T, s.d, s.f, s.E, s.k),), 0xA5, dtype=torch.uint8, device="cuda")
        moe.moe_forward_ex(*args, router_bias=d["router_bias"], workspace=ws, workspace_bytes_=ws.numel(), dbg=dbg)
    elif how == "noalloc":
        moe.moe_forward_noalloc(*args, router_bias=d["router_bias"])
        dbg = None
    else:
        raise ValueError(how)
    torch.cuda.synchronize()
    arrays = None if dbg is None else {n: v.cpu().numpy() for n, v in dbg.items()}
    return out.cpu().numpy(), arrays


def check_oracle(s, inp, got, nrows: int):
    r = oracle.route(inp["x"], inp["router_w"], inp["router_bias"], inp["pad_mask"], s.k)
    excl, _ = exclusions(r)
    assert int(excl.sum()) <= max_excluded(s.T)
    rows = sample_rows(s.T, nrows, seed=s.T)
    ref, _, _ = oracle.forward_inputs(inp, k=s.k, rows=rows)
    keep = ~excl[rows]
    ratio = float(np.max(np.abs(got[rows][keep] - ref[keep])) / rms(ref))
    print(f"{s.name} T={s.T}: {len(rows)} rows vs oracle, max|err|/rms = {ratio:.3e}", flush=True)
    assert ratio <= OUT_TOL
    if inp["pad_mask"] is not None:
        assert np.all(got[inp["pad_mask"] == 0] == 0)


# Every kernel configuration of the one-launch layer: gate/up split over d (tensor-parallel share
# at T <= 16 and T > 16; the Grok-1 shape at T = 1) or whole (the Grok-1 shape at 5-8, 9-16 and
# 17-64 tokens), with padding and a router bias in some.
CASES = [
    ("decode_tp8", 8, 0, None),
    ("decode_tp8", 1, 0, None),
    ("decode_tp8", 3, 0, synth.SKEW_BIAS),
    ("decode_tp8", 17, 2, None),
    ("decode_tp8", 64, 5, None),
    ("decode", 8, 0, None),
    ("decode", 1, 0, None),
    ("decode", 5, 1, None),
    ("decode", 16, 0, synth.SKEW_BIAS),
    ("decode", 33, 3, None),
    ("decode", 64, 6, None),
]


@pytest.mark.parametrize("base,T,n_pad,bias", CASES, ids=[f"{c[0]}-T{c[1]}" for c in CASES])
def test_one_launch_is_bit_identical_to_per_stage(base, T, n_pad, bias, monkeypatch):
    s, inp, d = inputs(base, T, n_pad, bias)
    print(f"case {base} T={T} n_pad={n_pad} bias={bias is not None}", flush=True)
    got, arrays = run(s, d, monkeypatch, one_launch=True)
    ref, ref_arrays = run(s, d, monkeypatch, one_launch=False)
    for n in ref_arrays:
        assert np.array_equal(arrays[n], ref_arrays[n]), n
    assert np.array_equal(got, ref)
    check_oracle(s, inp, got, nrows=16 if s.f <= 4096 else 3)


def test_control_block_stays_clean_across_entry_points(monkeypatch):
    """Calls of different sizes on the library workspace, caller workspaces with stale bytes,
    the allocation-free entry point and graph replays (own and caller workspace), interleaved:
    each one gives the per-stage sequence's bits."""
    cases = {T: inputs("decode_tp8", T, n_pad=1 if T > 8 else 0) for T in (8, 40)}
    ref = {T: run(s, d, monkeypatch, one_launch=False)[0] for T, (s, _, d) in cases.items()}
    order = [(8, "library"), (40, "library"), (8, "workspace"), (8, "noalloc"), (40, "noalloc"), (40, "workspace"),
             (8, "library")]
    for T, how in order:
        s, _, d = cases[T]
        got, _ = run(s, d, monkeypatch, one_launch=True, how=how)
        print(f"T={T} via {how}: bit-identical {bool(np.array_equal(got, ref[T]))}", flush=True)
        assert np.array_equal(got, ref[T]), (T, how)
    monkeypatch.setenv("MOE_ONE_LAUNCH", "1")
    for own in (True, False):
        s, _, d = cases[40]
        out = torch.full((s.T, s.d), float("nan"), device="cuda")
        ws = None
        if not own:
            ws = torch.full((moe.workspace_bytes(s.T, s.d, s.f, s.E, s.k),), 0x5A, dtype=torch.uint8, device="cuda")
        g = moe.Graph(d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], out,
                      s.T, s.d, s.f, s.E, s.k, router_bias=d["router_bias"], workspace=ws,
                      workspace_bytes_=0 if ws is None else ws.numel())
        try:
            for rep in range(3):
                out.fill_(float("nan"))
                torch.cuda.synchronize()
                g.launch()
                torch.cuda.synchronize()
                assert np.array_equal(out.cpu().numpy(), ref[40]), (own, rep)
                # eager calls between replays share nothing with the graph's workspace
                s8, _, d8 = cases[8]
                assert np.array_equal(run(s8, d8, monkeypatch, one_launch=True)[0], ref[8])
        finally:
            g.close()
        print(f"graph ({'own' if own else 'caller'} workspace): 3 replays bit-identical", flush=True)


@pytest.mark.parametrize("base,T", [("decode_tp8", 8), ("decode_tp8", 64), ("decode", 8)])
def test_one_launch_repeats_on_poisoned_workspaces(base, T, monkeypatch):
    """Items pass rp, P, H and Y to each other through the workspace within one launch: a read of a
    stale or unwritten line would show. 60 calls, each on a workspace first filled with NaN
    bytes, must all give the per-stage sequence's bits."""
    s, _, d = inputs(base, T, n_pad=2 if T > 8 else 0)
    ref, _ = run(s, d, monkeypatch, one_launch=False)
    monkeypatch.setenv("MOE_ONE_LAUNCH", "1")
    nbytes = moe.workspace_bytes(s.T, s.d, s.f, s.E, s.k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((s.T, s.d), device="cuda")
    bad = 0
    for rep in range(60):
        ws.fill_(0xFF)
        out.fill_(float("nan"))
        moe.moe_forward_ex(d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"],
                           out, s.T, s.d, s.f, s.E, s.k, router_bias=d["router_bias"], workspace=ws,
                           workspace_bytes_=nbytes)
        torch.cuda.synchronize()
        bad += int(not np.array_equal(out.cpu().numpy(), ref))
    print(f"{base} T={T}: {60 - bad}/60 calls bit-identical", flush=True)
    assert bad == 0
