"""GPU tests of the variants built beside the gather path, each against the oracle:
the dense one-hot formulation, the graph-captured single-launch forward, and the MoE block
with the pre-norm and post-norm + residual fused."""
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

_grok: dict = {}


def grok_case(name: str):
    if name not in _grok:
        spec = synth.WORKLOAD_SPECS[name]
        inp = synth.make_inputs(spec)
        _grok.clear()
        _grok[name] = (spec, inp, to_dev(inp))
    return _grok[name]


def small(name, **kw):
    spec = synth.custom(name, **kw)
    inp = synth.make_inputs(spec)
    return spec, inp, to_dev(inp)


def sparse_out(d, s):
    out = torch.full((s.T, s.d), float("nan"), device="cuda")
    moe.moe_forward_ex(d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], out,
                       s.T, s.d, s.f, s.E, s.k, router_bias=d["router_bias"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ------------------------------------------------------------------------ dense one-hot formulation

# the last case runs the prefill down launch that keeps 1 or 2 parts on the device
@pytest.mark.parametrize("case", ["tiny", "decode", dict(T=300, d=256, f=512, n_pad=30), dict(T=40, d=256, f=256, E=4, k=3),
                                  dict(T=200, d=256, f=8192, n_pad=9)])
def test_dense_onehot_formulation(case):
    s, inp, d = grok_case(case) if isinstance(case, str) else small("dense", **case)
    out = torch.full((s.T, s.d), float("nan"), device="cuda")
    moe.moe_forward_dense(d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"],
                          out, s.T, s.d, s.f, s.E, s.k, router_bias=d["router_bias"])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sp = sparse_out(d, s)
    # the same experts' outputs, added in expert order instead of slot order
    assert np.max(np.abs(got - sp)) <= 1e-5 * rms(sp)
    r = oracle.route(inp["x"], inp["router_w"], inp["router_bias"], inp["pad_mask"], s.k)
    excl, _ = exclusions(r)
    rows = sample_rows(s.T, 16, seed=2)
    ref, _, _ = oracle.forward_inputs(inp, k=s.k, rows=rows)
    keep = ~excl[rows]
    ratio = np.max(np.abs(got[rows][keep] - ref[keep])) / rms(ref)
    print(f"dense {case}: max|err|/rms = {ratio:.3e}, bit-equal to gather path: {bool(np.array_equal(got, sp))}",
          flush=True)
    assert ratio <= OUT_TOL
    if inp["pad_mask"] is not None:
        assert np.all(got[inp["pad_mask"] == 0] == 0)


# ------------------------------------------------------------------------ graph-captured forward

# the last case runs the prefill down kernel that picks its number of parts on the device
@pytest.mark.parametrize("case", ["tiny", "decode", dict(T=200, d=256, f=512, n_pad=10),
                                  dict(T=1500, d=256, f=8192, n_pad=20)])
def test_graph_replays_match_eager(case):
    s, inp, d = grok_case(case) if isinstance(case, str) else small("graph", **case)
    ws = torch.empty(moe.workspace_bytes(s.T, s.d, s.f, s.E, s.k) + 256, dtype=torch.uint8, device="cuda")
    x = d["x"].clone()
    out = torch.full((s.T, s.d), float("nan"), device="cuda")
    g = moe.Graph(x, d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], out, s.T, s.d,
                  s.f, s.E, s.k, router_bias=d["router_bias"], workspace=ws, workspace_bytes_=ws.numel())
    gen = torch.Generator(device="cpu").manual_seed(0)
    try:
        for rep in range(4):
            # eager work between replays: new activations in the graph's input buffer
            if rep:
                x.copy_((torch.randn(s.T, s.d, generator=gen)).to(torch.bfloat16).cuda())
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            eager = sparse_out(dict(d, x=x), s)
            assert np.array_equal(got, eager), rep
            if rep == 0:
                # the first replay runs on the workload's own inputs: against the oracle too
                r = oracle.route(inp["x"], inp["router_w"], inp["router_bias"], inp["pad_mask"], s.k)
                excl, _ = exclusions(r)
                assert int(excl.sum()) <= max_excluded(s.T)
                pads = None if inp["pad_mask"] is None else np.nonzero(inp["pad_mask"] == 0)[0][:2]
                rows = sample_rows(s.T, 24, seed=9, must=pads)
                ref, _, _ = oracle.forward_inputs(inp, k=s.k, rows=rows)
                keep = ~excl[rows]
                ratio = float(np.max(np.abs(got[rows][keep] - ref[keep])) / rms(ref))
                print(f"graph {case}: replay 0 vs oracle max|err|/rms = {ratio:.3e} on {len(rows)} rows", flush=True)
                assert ratio <= OUT_TOL
                if inp["pad_mask"] is not None:
                    assert np.all(got[inp["pad_mask"] == 0] == 0)
    finally:
        g.close()


def test_graph_without_workspace_owns_its_workspace():
    # a graph created without a caller workspace keeps its own: a later, larger call that
    # grows the library workspace (freeing the old buffer) must not affect its replays
    s, inp, d = small("graph_own", T=48, d=256, f=512, n_pad=3)
    out = torch.full((s.T, s.d), float("nan"), device="cuda")
    g = moe.Graph(d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], out, s.T,
                  s.d, s.f, s.E, s.k, router_bias=d["router_bias"])
    try:
        big, _, dbig = small("graph_big", T=3000, d=512, f=1024)
        sparse_out(dbig, big)  # grows the library workspace
        for _ in range(2):
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), sparse_out(d, s))
    finally:
        g.close()


# ------------------------------------------------------------------------ MoE block with fused norms

def block_case(s, inp, d, rows):
    rng = np.random.default_rng(11)
    wpre = (1 + 0.1 * rng.standard_normal(s.d)).astype(np.float32)
    wpost = (1 + 0.1 * rng.standard_normal(s.d)).astype(np.float32)
    eps = 1e-5
    h_out = torch.full((s.T, s.d), float("nan"), device="cuda")
    xn = torch.empty((s.T, s.d), dtype=torch.int16, device="cuda")
    moe.moe_block_forward(d["x"], torch.from_numpy(wpre).cuda(), torch.from_numpy(wpost).cuda(), eps, d["router_w"],
                          d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], h_out, s.T, s.d, s.f, s.E,
                          s.k, router_bias=d["router_bias"], x_norm_out=xn)
    torch.cuda.synchronize()
    got, xg = h_out.cpu().numpy(), xn.cpu().numpy().view(np.uint16)
    pad = None if inp["pad_mask"] is None else inp["pad_mask"][rows]
    ref, xr = oracle.block_forward(np.ascontiguousarray(inp["x"][rows]), wpre, wpost, eps, inp["router_w"],
                                   inp["router_bias"], inp["w_gate"], inp["w_up"], inp["w_down"], inp["scales"],
                                   None if pad is None else np.ascontiguousarray(pad), k=s.k)
    # the MoE input: the same bf16 values up to one ulp where the two sums of squares round apart
    xgv, xrv = synth.bf16_bits_to_f32(xg[rows]), synth.bf16_bits_to_f32(xr)
    assert np.all(np.abs(xgv - xrv) <= 2.0 ** -7 * np.abs(xrv))
    frac_equal = float(np.mean(xg[rows] == xr))
    # routing on the oracle's own MoE input: near ties excluded as for the layer
    r = oracle.route(xr, inp["router_w"], inp["router_bias"], pad, s.k)
    excl, _ = exclusions(r)
    h = synth.bf16_bits_to_f32(inp["x"][rows]).astype(np.float64)
    dm, dr = got[rows] - h, ref - h
    ratio = np.max(np.abs(dm[~excl] - dr[~excl])) / rms(dr)
    print(f"block T={s.T} d={s.d}: x equal {frac_equal:.5f}, max|err(h_out - h)|/rms = {ratio:.3e}", flush=True)
    assert ratio <= OUT_TOL
    if inp["pad_mask"] is not None:
        padded = inp["pad_mask"] == 0
        assert np.array_equal(got[padded], synth.bf16_bits_to_f32(inp["x"][padded]))


# below 1024 tokens the post-norm combine takes two launches over (token, 1024-column chunk)
# workgroups, from 1024 one workgroup per token (and the router 8 tokens per workgroup);
# d = 1280 leaves a partial last chunk
# f = 8192 at T > 160: the down launch keeps 1 or 2 parts on the device and the post-norm
# combine reads the count there (both combine forms)
@pytest.mark.parametrize("case", ["tiny", "decode", "batched_decode", dict(T=500, d=256, f=512, n_pad=40),
                                  dict(T=40, d=1280, f=256, n_pad=5), dict(T=1100, d=1280, f=256, n_pad=60),
                                  dict(T=300, d=256, f=8192, n_pad=11), dict(T=1100, d=256, f=8192, n_pad=7)])
def test_block_parity(case):
    s, inp, d = grok_case(case) if isinstance(case, str) else small("block", **case)
    rows = np.arange(s.T) if s.T * s.d <= 200_000 else sample_rows(s.T, 12, seed=4)
    block_case(s, inp, d, rows)


def test_block_prenorm_is_batch_invariant_bitwise():
    """A token's normalised MoE input is the same bits whether its batch takes the separate norm
    launch (up to 64 tokens), the one-token or the 8-token router workgroups."""
    s, inp, d = small("block_inv", T=1040, d=1280, f=256)
    wpre = torch.from_numpy((1 + 0.1 * np.random.default_rng(12).standard_normal(s.d)).astype(np.float32)).cuda()
    wpost = torch.ones(s.d, dtype=torch.float32, device="cuda")

    def x_norm(T):
        h_out = torch.empty((T, s.d), device="cuda")
        xn = torch.empty((T, s.d), dtype=torch.int16, device="cuda")
        moe.moe_block_forward(d["x"][:T], wpre, wpost, 1e-5, d["router_w"], d["w_gate"], d["w_up"], d["w_down"],
                              d["scales"], None, h_out, T, s.d, s.f, s.E, s.k, router_bias=d["router_bias"],
                              x_norm_out=xn)
        torch.cuda.synchronize()
        return xn.cpu().numpy()

    full = x_norm(s.T)
    assert np.array_equal(full[:24], x_norm(24))
    assert np.array_equal(full[:100], x_norm(100))
