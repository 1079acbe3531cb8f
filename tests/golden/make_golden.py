"""Writes tiny_oracle_summary.json from the oracle alone (run from the repo root:
python tests/golden/make_golden.py). The stored values are a regression fixture of the
oracle's own output on the tiny workload, not values printed by the pages."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

inp = synth.make_inputs(synth.WORKLOAD_SPECS["tiny"])
out, ids, w = oracle.forward_inputs(inp)
rows = [0, 1, 31, 63]
doc = {
    "_source": "oracle.forward on synth workload 'tiny' (seed 42); written by tests/golden/make_golden.py",
    "ids": ids.tolist(),
    "w_bits": w.view(np.uint32).ravel().tolist(),
    "sample_rows": rows,
    "sample_out_bits": out[rows].view(np.uint32).ravel().tolist(),
    "abs_sum": float(np.abs(out.astype(np.float64)).sum()),
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_summary.json"), "w") as fh:
    json.dump(doc, fh)
print("wrote tiny_oracle_summary.json")
