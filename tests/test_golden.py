"""Fixtures the pages print: the MoE layer's shape, and the oracle's stored summary."""
import json
import os

import numpy as np

import oracle
import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def ffn_size(emb_size: int, widening_factor: float) -> int:
    # int(widening * emb) * 2 // 3, rounded up to a multiple of 8
    v = int(widening_factor * emb_size) * 2 // 3
    return v + (-v) % 8


def test_grok1_moe_shape_from_pages():
    g = json.load(open(os.path.join(HERE, "grok1_moe_shape.json")))
    assert ffn_size(g["emb_size"], g["widening_factor"]) == g["d_expert"] == 32768
    for name in ("decode", "batched_decode", "prefill", "skewed"):
        s = synth.WORKLOAD_SPECS[name]
        assert (s.d, s.f, s.E, s.k) == (g["emb_size"], g["d_expert"], g["num_experts"], g["num_selected_experts"])
    # cross-check with the pages' parameter counts: the MoE weights of 64 layers hold
    # 64 * 8 * 3 * d * f = 309B of the 314B parameters, and the 2 active experts 77.3B
    # of the 83.8B active per token (attention and embeddings make up the rest)
    moe_total = g["num_layers"] * g["num_experts"] * 3 * g["emb_size"] * g["d_expert"] / 1e9
    moe_active = g["num_layers"] * g["num_selected_experts"] * 3 * g["emb_size"] * g["d_expert"] / 1e9
    assert moe_total < g["total_parameters_billion"] and moe_total > 0.95 * g["total_parameters_billion"]
    assert moe_active < g["active_parameters_billion_modelled"] and moe_active > 0.9 * g["active_parameters_billion_modelled"]


def test_oracle_matches_its_stored_summary():
    """Regression: the tiny workload's oracle output, written by make_golden.py (oracle only)."""
    g = json.load(open(os.path.join(HERE, "tiny_oracle_summary.json")))
    inp = synth.make_inputs(synth.WORKLOAD_SPECS["tiny"])
    out, ids, w = oracle.forward_inputs(inp)
    assert ids.tolist() == g["ids"]
    assert np.array_equal(w.view(np.uint32), np.array(g["w_bits"], np.uint32).reshape(w.shape))
    rows = g["sample_rows"]
    assert np.array_equal(out[rows].view(np.uint32), np.array(g["sample_out_bits"], np.uint32).reshape(len(rows), -1))
    assert float(np.abs(out.astype(np.float64)).sum()) == g["abs_sum"]
