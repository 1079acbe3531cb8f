"""The allocation-free entry point moe_forward_noalloc, through the C ABI, against
moe_forward_ex (the same kernels with a caller workspace): bit-equal outputs on two calls
in a row, the second with a smaller batch (its scratch keeps the first call's contents),
and a shape above the fixed scratch rejected before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_helpers import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import mixture_experts_layer_gemv_amd as moe  # noqa: E402


def reference(d, T, dd, f, E, k):
    out = torch.full((T, dd), float("nan"), device="cuda")
    ws = torch.empty(moe.workspace_bytes(T, dd, f, E, k) + 256, dtype=torch.uint8, device="cuda")
    moe.moe_forward_ex(d["x"][:T], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"],
                       None if d["pad_mask"] is None else d["pad_mask"][:T], out, T, dd, f, E, k,
                       router_bias=d["router_bias"], workspace=ws, workspace_bytes_=ws.numel())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def noalloc(d, T, dd, f, E, k):
    out = torch.full((T, dd), float("nan"), device="cuda")
    moe.moe_forward_noalloc(d["x"][:T], d["router_w"], d["w_gate"], d["w_up"], d["w_down"], d["scales"],
                            None if d["pad_mask"] is None else d["pad_mask"][:T], out, T, dd, f, E, k,
                            router_bias=d["router_bias"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


# the streaming kernels with a split gate/up contraction (partial sums in the scratch), the
# tiled kernels at a large batch (the down kernel's part count kept in the scratch), and the
# small-batch routing (group sums in the scratch)
@pytest.mark.parametrize("kw,T2", [(dict(T=40, d=6144, f=2048, n_pad=4, bias=(0.5, 0, 0, 0, 0, 0, 0, -0.5)), 9),
                                   (dict(T=1200, d=256, f=8192, n_pad=30), 300),
                                   (dict(T=64, d=256, f=512, n_pad=3), 9)])
def test_noalloc_matches_forward_ex_twice(kw, T2):
    spec = synth.custom("noalloc", E=8, k=2, **kw)
    inp = synth.make_inputs(spec)
    d = to_dev(inp)
    T, dd, f = spec.T, spec.d, spec.f
    for n in (T, T2):  # second call smaller: the scratch holds the first call's arrays
        a = noalloc(d, n, dd, f, 8, 2)
        b = reference(d, n, dd, f, 8, 2)
        assert np.all(np.isfinite(a)), n
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), n
        print(f"noalloc {kw} T={n}: bit-equal to moe_forward_ex", flush=True)


def test_noalloc_rejects_shapes_above_its_scratch():
    # 205 tokens at the Grok-1 shape need more than the fixed 64 MiB: rejected before any
    # launch (the pointers are never dereferenced), out untouched
    out = torch.full((4, 256), 3.0, device="cuda")
    p = out.data_ptr()
    assert moe.workspace_bytes(205, 6144, 32768, 8, 2) > moe.NOALLOC_SCRATCH_BYTES
    assert moe.workspace_bytes(204, 6144, 32768, 8, 2) <= moe.NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(p, p, p, p, p, p, None, p, 205, 6144, 32768, 8, 2)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
