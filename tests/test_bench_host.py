"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the algorithmic byte and FLOP
accounting its roofline fractions rest on (against hand-computed figures for the Grok-1 shape),
the workload lists, and the traffic records' matching rule."""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_refuses_more_than_one_gpu(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_decode_bytes_match_hand_count(bench):
    # T = 8 at the Grok-1 shape with 7 of 8 experts touched: each touched expert streams its int8
    # gate and up matrices (2 x 6144 x 32768 B) and their bf16 scales (2 x 32768 x 2 B), and the 8
    # token rows of x are read once (8 x 6144 x 2 B); down: int8 (6144 x 32768 B) + scales (6144 x 2 B)
    spec = SimpleNamespace(T=8, d=6144, f=32768, E=8, n_pad=0)
    counts = [3, 2, 0, 4, 1, 2, 3, 1]
    w = bench.algorithmic_work(spec, counts)
    assert w["touched"] == 7 and w["n_assign"] == 16
    assert w["gu_bytes"] == 7 * (402_653_184 + 131_072) + 98_304 == 2_819_588_096
    assert w["dn_bytes"] == 7 * (201_326_592 + 12_288) == 1_409_372_160


def test_prefill_flops_match_hand_count(bench):
    # 8192 tokens x 2 assignments: gate/up 2 matrices x 2 FLOPs x d x f per assignment, down half that
    spec = SimpleNamespace(T=8192, d=6144, f=32768, E=8, n_pad=0)
    counts = [2091, 2037, 1997, 2080, 2090, 2006, 2010, 2073]
    w = bench.algorithmic_work(spec, counts)
    assert w["n_assign"] == 16384
    assert w["gu_flops"] == 16384 * 4 * 6144 * 32768 == 13_194_139_533_312
    assert w["dn_flops"] == w["gu_flops"] / 2
    # the layer adds the router GEMV (2 T d E)
    assert w["layer_flops"] == w["gu_flops"] + w["dn_flops"] + 2 * 8192 * 6144 * 8


def test_padded_rows_are_not_counted_as_activations(bench):
    # 64 tokens, 6 padded: 58 real rows of x are read, 116 assignments over all 8 experts
    spec = SimpleNamespace(T=64, d=6144, f=32768, E=8, n_pad=6)
    w = bench.algorithmic_work(spec, [15, 15, 15, 15, 14, 14, 14, 14])
    assert w["n_assign"] == 116 and w["touched"] == 8
    assert w["gu_bytes"] == 8 * (2 * 6144 * 32768 + 4 * 32768) + 2 * 58 * 6144


def test_workload_lists(bench):
    assert set(bench.WORKLOADS) <= set(synth.WORKLOAD_SPECS)
    assert set(bench.METRIC_WORKLOADS) | set(bench.TP_SHARE_WORKLOADS) == set(bench.WORKLOADS)
    assert not set(bench.METRIC_WORKLOADS) & set(bench.TP_SHARE_WORKLOADS)


def test_traffic_record_needs_matching_sources(bench):
    # a record is only used for the exact workload, source list and source contents it was taken with
    assert bench.recorded_traffic("decode", ["mixture_experts_layer_gemv_amd/csrc/no_such_file.hip"]) is None
    assert bench.recorded_traffic("no_such_workload", bench.DECODE_SOURCES) is None
    rec = bench.recorded_traffic("decode", bench.DECODE_SOURCES)
    if rec is not None:
        assert rec["workload"] == "decode" and rec["gate_up_traffic_bytes"] > 0
        assert rec["profile"].startswith("profiles" + os.sep)
