"""Tensor parallelism over the expert FFN width f, as the pages shard the MoE matmuls
(Grok-1 Admin & Architecture Guide, section 6: the expert matmuls under shard_map with one
psum over the model axis): share g of G holds columns [g f/G, (g+1) f/G) of gate and up,
the same rows of down, and all E experts; the layer is the sum of the G shares' outputs.

`tp_share` cuts one share out of a `synth.make_inputs` dict (numpy, host memory)."""
from __future__ import annotations

import numpy as np


def tp_share(inp: dict, g: int, G: int) -> dict:
    E, d, f = inp["w_gate"].shape
    assert f % G == 0
    fs = f // G
    cols = slice(g * fs, (g + 1) * fs)
    sc = inp["scales"]
    out = dict(inp)
    out["w_gate"] = np.ascontiguousarray(inp["w_gate"][:, :, cols])
    out["w_up"] = np.ascontiguousarray(inp["w_up"][:, :, cols])
    out["w_down"] = np.ascontiguousarray(inp["w_down"][:, cols, :])
    out["scales"] = np.ascontiguousarray(np.concatenate(
        [sc[:, cols], sc[:, f + g * fs:f + (g + 1) * fs], sc[:, 2 * f:]], axis=1))
    return out
