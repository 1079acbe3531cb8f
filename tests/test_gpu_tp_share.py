"""GPU tests of one GPU's share of tensor parallelism over f (Grok-1 Admin & Architecture
Guide, section 6: the expert matmuls under shard_map with a psum over the model axis).

The layer is split into G shares of f / G columns of gate/up (and rows of down) with all
experts in each; each share is an ordinary call of the library at the share's shape, and
the layer's output is the sum of the shares' outputs (the all-reduce, done here on the
host). Routing is the same on every share; H and the down contraction are summed in other
orders (a share splits its narrower contraction differently), so an fp32 value of H can
differ in its last bits and its fp16 rounding flip by one ulp (2^-11 relative): the sum
matches the one-GPU layer to about 1e-4 of its RMS, where a wrong decomposition is O(1)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import OUT_TOL, rms, sample_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import mixture_experts_layer_gemv_amd as moe  # noqa: E402
from test_gpu_parity import check_layer, workload  # noqa: E402

SUM_TOL = 1e-3  # max|sum of shares - layer| / rms(layer): summation order and fp16 ulp flips of H


def forward(d, T, dd, f, E, k):
    out = torch.full((T, dd), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_forward_ex(d["x"], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"], d["pad_mask"], out,
                       T, dd, f, E, k, router_bias=d["router_bias"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def share_dev(d, g, G, f):
    """Share g of G of the device weights (copies made with torch: memory plumbing only)."""
    fs = f // G
    cols = slice(g * fs, (g + 1) * fs)
    sc = d["scales"]
    return dict(d, w_gate=d["w_gate"][:, :, cols].contiguous(), w_up=d["w_up"][:, :, cols].contiguous(),
                w_down=d["w_down"][:, cols, :].contiguous(),
                scales=torch.cat([sc[:, cols], sc[:, f + g * fs:f + (g + 1) * fs], sc[:, 2 * f:]], dim=1).contiguous())


def check_shares_sum(inp, d, G, label):
    T, dd = inp["x"].shape
    E, _, f = inp["w_gate"].shape
    full = forward(d, T, dd, f, E, 2)
    total = np.zeros(full.shape, np.float64)
    for g in range(G):
        sd = share_dev(d, g, G, f)
        total += forward(sd, T, dd, f // G, E, 2)
        del sd
    ratio = float(np.max(np.abs(total - full)) / rms(full))
    print(f"[{label}] G={G} f/G={f // G}: max|sum of shares - layer|/rms = {ratio:.3e}", flush=True)
    assert ratio <= SUM_TOL


def test_tp8_shares_sum_to_the_layer_at_decode():
    inp, d = workload("decode")
    check_shares_sum(inp, d, 8, "decode T=8 d=6144 f=32768")


def test_tp_shares_sum_to_the_layer_on_the_prefill_path():
    spec = synth.custom("tp_prefill", T=300, d=256, f=2048, n_pad=20, scale_jitter=True)
    inp = synth.make_inputs(spec)
    check_shares_sum(inp, to_dev(inp), 8, "T=300 d=256 f=2048")


@pytest.mark.parametrize("name,nrows", [("decode_tp8", None), ("prefill_tp8", 16)])
def test_tp8_share_workload_parity(name, nrows):
    inp, d = workload(name)
    s = synth.WORKLOAD_SPECS[name]
    rows = None if nrows is None else sample_rows(s.T, nrows, seed=5)
    check_layer(inp, d, rows=rows, label=name)
