"""The seeded input generator: determinism, slicing, distributions, the workload recipe."""
import math

import numpy as np
import pytest
import torch

import synth


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs are published test values of the
    # generator (Steele, Lea & Flood 2014; also the seeding generator of xoshiro).
    # draw i of a stream is mix64(key + (i+1) * gamma), so key 0 gives them directly.
    d = synth.draws(0, 3)
    assert [int(v) for v in d] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_are_deterministic_and_sliceable():
    k = synth.key(42, 7, 3)
    a = synth.int8_uniform(k, 10000)
    b = synth.int8_uniform(k, 10000)
    assert np.array_equal(a, b)
    # any slice equals the same elements of the full stream (counter-based)
    c = synth.int8_uniform(k, 300, start=4321)
    assert np.array_equal(c, a[4321:4621])
    xa = synth.normal_bf16(k, 5000)
    assert np.array_equal(synth.normal_bf16(k, 100, start=1234), xa[1234:1334])
    assert synth.key(42, 7, 3) != synth.key(42, 7, 4) != synth.key(43, 7, 3)


def test_int8_range_and_uniformity():
    a = synth.int8_uniform(synth.key(1, 2, 3), 1 << 20).astype(np.int64)
    assert a.min() == -127 and a.max() == 127
    counts = np.bincount(a + 127, minlength=255)
    assert counts.size == 255
    expect = a.size / 255
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 400  # 254 dof; mean 254, sd ~22.5


def test_normal_and_student_moments():
    k = synth.key(5, 5, 5)
    z = synth.bf16_bits_to_f32(synth.normal_bf16(k, 1 << 18)).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.02
    t = synth.bf16_bits_to_f32(synth.student4_bf16(k, 1 << 18)).astype(np.float64)
    assert abs(t.mean()) < 0.02
    # unit variance after scaling (t4 variance converges slowly: heavy tails)
    assert 0.85 < t.var() < 1.15
    # heavier tails than the normal
    assert (np.abs(t) > 4).mean() > 5 * (np.abs(z) > 4).mean()
    w = synth.normal_f32(k, 1 << 18, sigma=0.25).astype(np.float64)
    assert abs(w.std() - 0.25) < 0.005


def test_bf16_rounding_matches_torch():
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    v[:4] = [0.0, -0.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8]  # ties at the bf16 midpoint
    ours = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_pad_mask_exact_count_and_seeded():
    k = synth.key(42, 3, synth.TENSOR_PAD)
    m = synth.pad_mask(k, 64, 6)
    assert m.dtype == np.uint8 and m.size == 64 and int((m == 0).sum()) == 6
    assert np.array_equal(m, synth.pad_mask(k, 64, 6))
    assert int((synth.pad_mask(k, 4096, 1024) == 0).sum()) == 1024
    assert synth.pad_mask(k, 5, 5).sum() == 0 and synth.pad_mask(k, 5, 0).sum() == 5
    with pytest.raises(ValueError):
        synth.pad_mask(k, 4, 5)


def test_scale_values_per_recipe():
    # 1/(127 sqrt(fan_in)) rounded to bf16, fan_in = d for gate/up and f for down
    s = synth.scales(synth.WORKLOAD_SPECS["tiny"])
    f = synth.bf16_bits_to_f32(s)
    assert f.shape == (8, 2 * 512 + 256)
    want_gu = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.float32([1 / (127 * math.sqrt(256))])))[0]
    want_d = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.float32([1 / (127 * math.sqrt(512))])))[0]
    assert np.all(f[:, :1024] == want_gu) and np.all(f[:, 1024:] == want_d)
    assert abs(want_gu - 4.920959e-4) < 1e-9 and abs(want_d - 3.471375e-4) < 1e-9
    jit = synth.bf16_bits_to_f32(synth.scales(synth.replace(synth.WORKLOAD_SPECS["tiny"], scale_jitter=True)))
    r = jit[:, :1024] / (1 / (127 * 16))
    assert 0.49 < r.min() and r.max() < 1.51 and r.std() > 0.2


def test_workload_shapes_and_padding():
    c = synth.WORKLOAD_SPECS
    assert (c["decode"].d, c["decode"].f, c["decode"].E, c["decode"].k) == (6144, 32768, 8, 2)
    assert c["batched_decode"].n_pad == round(0.10 * 64)
    assert c["skewed"].n_pad == 1024 and c["skewed"].bias == synth.SKEW_BIAS
    inp = synth.make_inputs(c["tiny"])
    assert inp["x"].shape == (64, 256) and inp["x"].dtype == np.uint16
    assert inp["router_w"].shape == (256, 8) and inp["router_w"].dtype == np.float32
    assert inp["w_gate"].shape == (8, 256, 512) and inp["w_down"].shape == (8, 512, 256)
    assert inp["pad_mask"] is None and inp["router_bias"] is None
    # expert slices of the weights equal the full tensor's experts
    sub = synth.expert_weights(c["tiny"], "down", experts=[5, 2])
    assert np.array_equal(sub[0], inp["w_down"][5]) and np.array_equal(sub[1], inp["w_down"][2])
    rows = synth.x_rows(c["tiny"], np.array([7, 3]))
    assert np.array_equal(rows, inp["x"][[7, 3]])
