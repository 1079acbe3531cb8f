"""Pins of the CPU oracle against what the sources and mathematics fix.

No page prints a worked example or an output value of the MoE layer, so the oracle is
pinned by: library routines for the special cases that reduce to them (numpy fp64 matmul,
torch's tanh-GeLU, scipy's softmax, numpy's stable argsort), closed forms (identity
experts, x = 0), brute-force enumeration (top-k), an fp64 brute force for rounding, and
invariants of the layer (padding, token permutation, expert relabelling, batch
invariance, linearity in the down/up scales). Each test names the mistake it catches.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth


def bf(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64)


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def small(name, T=16, d=48, f=80, E=4, k=2, **kw):
    return synth.make_inputs(synth.custom(name, T=T, d=d, f=f, E=E, k=k, **kw))


def gelu_ref(v):
    return torch.nn.functional.gelu(torch.as_tensor(v, dtype=torch.float64), approximate="tanh").numpy()


def numpy_layer(inp, ids, w):
    """The layer written with numpy fp64 matmuls and torch's tanh-GeLU, given a routing."""
    x = bf(inp["x"])
    E, d, f = inp["w_gate"].shape
    s = bf(inp["scales"])
    out = np.zeros((x.shape[0], d))
    for t in range(x.shape[0]):
        if inp["pad_mask"] is not None and inp["pad_mask"][t] == 0:
            continue
        for j in range(ids.shape[1]):
            e = ids[t, j]
            Wg = inp["w_gate"][e].astype(np.float64) * s[e, :f][None, :]
            Wu = inp["w_up"][e].astype(np.float64) * s[e, f:2 * f][None, :]
            Wd = inp["w_down"][e].astype(np.float64) * s[e, 2 * f:][None, :]
            h = gelu_ref(x[t] @ Wg) * (x[t] @ Wu)
            out[t] += float(w[t, j]) * (h @ Wd)
    return out


# ---------------------------------------------------------------- GeLU (expert step 3)

def test_gelu_is_the_tanh_form():
    v = np.linspace(-8, 8, 2001).astype(np.float32)
    ours = np.array([oracle.gelu_tanh(float(a)) for a in v], np.float64)
    ref = gelu_ref(v.astype(np.float64))
    # fp32 rounding: relative 1e-5, plus ~|v| ulp where 1 + tanh cancels for v << 0
    assert np.all(np.abs(ours - ref) <= 1e-5 * np.abs(ref) + 2e-7 * np.maximum(1, np.abs(v)))
    # and not the erf form (catches the wrong GeLU variant): they differ by up to ~1e-3
    erf = torch.nn.functional.gelu(torch.as_tensor(v, dtype=torch.float64)).numpy()
    assert np.max(np.abs(ours - erf)) > 1e-4


def test_gelu_identities():
    # gelu(v) - gelu(-v) = v exactly in real arithmetic (the tanh term is odd); gelu(0) = 0
    for v in [0.1, 0.5, 1.0, 2.5, 7.0]:
        assert abs(oracle.gelu_tanh(v) - oracle.gelu_tanh(-v) - v) < 4e-7 * max(1, v)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert abs(oracle.gelu_tanh(10.0) - 10.0) < 1e-6 and abs(oracle.gelu_tanh(-10.0)) < 1e-6


# ---------------------------------------------------------------- router (steps 1-2)

def test_router_logits_and_softmax_vs_library():
    inp = small("route-lib", T=64, d=200, E=8, bias=(0.3, -0.2, 0, 0, 1.0, 0, 0, -0.5))
    r = oracle.route(inp["x"], inp["router_w"], inp["router_bias"], None, k=2)
    ref_logits = bf(inp["x"]) @ inp["router_w"].astype(np.float64) + np.asarray(inp["router_bias"])
    bound = 200 * 2.0 ** -23 * (np.abs(bf(inp["x"])) @ np.abs(inp["router_w"].astype(np.float64))) + 1e-7
    assert np.all(np.abs(r["logits"] - ref_logits) <= bound)  # catches a dropped bias or wrong W index
    p_ref = scipy.special.softmax(r["logits"].astype(np.float64), axis=1)
    assert np.max(np.abs(r["probs"] - p_ref)) < 2e-7
    assert np.all(np.abs(r["probs"].astype(np.float64).sum(1) - 1) <= 8 * 2.0 ** -23)


def test_router_x_zero_pins_tie_rule():
    # x = 0 => every logit is 0 => p = 1/E for all => ids (0, 1), w = (1/E, 1/E)
    inp = small("route-zero", T=4, d=32, E=8)
    x0 = np.zeros_like(inp["x"])
    r = oracle.route(x0, inp["router_w"], None, None, k=2)
    assert np.all(r["probs"] == np.float32(1 / 8))
    assert np.array_equal(r["ids"], np.tile([0, 1], (4, 1)))
    assert np.all(r["w"] == np.float32(1 / 8))
    assert np.all(r["gap_sel"] == 0) and np.all(r["gap_order"] == 0)


def test_top_k_equals_brute_force_enumeration():
    # top-k by "(p desc, index asc)" equals the max-sum k-subset, lexicographically lowest on
    # ties, listed by p desc (catches selection on the wrong end, off-by-one, or no tie rule)
    for k, E in [(2, 8), (3, 8), (1, 4), (4, 4)]:
        inp = small(f"topk-{k}-{E}", T=200, d=16, E=E, k=k)
        # force exact ties: experts 1 and 2 share a router column
        wr = inp["router_w"].copy()
        wr[:, 2] = wr[:, 1]
        r = oracle.route(inp["x"], wr, None, None, k=k)
        for t in range(200):
            p = r["probs"][t].astype(np.float64)
            best = max(itertools.combinations(range(E), k),
                       key=lambda c: (sum(p[list(c)]), [-i for i in c]))
            got = r["ids"][t]
            assert sorted(got) == sorted(best), (t, got, best)
            assert all(p[got[j]] >= p[got[j + 1]] for j in range(k - 1))
            assert np.array_equal(r["w"][t], r["probs"][t][got])  # weights = selected probabilities
            if 1 in got and 2 in got:
                assert list(got).index(1) < list(got).index(2)  # equal p: lower index first


def gaps_from_sorted(probs, k, real):
    """The selection and order gaps of each token from numpy's descending sort of its
    probabilities: sel = p_(k) - p_(k+1), order = min over j < k of p_(j) - p_(j+1)
    (1-based ranks; +inf where undefined or padded), in fp32 as the oracle computes them."""
    T, E = probs.shape
    s = -np.sort(-probs, axis=1)  # descending, fp32
    sel = np.full(T, np.inf, np.float32)
    order = np.full(T, np.inf, np.float32)
    if k < E:
        sel = (s[:, k - 1] - s[:, k]).astype(np.float32)
    if k > 1:
        order = np.min(s[:, : k - 1] - s[:, 1:k], axis=1).astype(np.float32)
    sel[~real] = np.inf
    order[~real] = np.inf
    return sel, order


@pytest.mark.parametrize("k,E", [(1, 4), (2, 4), (3, 4), (4, 4), (1, 8), (2, 8), (3, 8), (4, 8)])
def test_near_tie_gaps_equal_sorted_probability_differences(k, E):
    # gap_sel decides which tokens the GPU parity leaves out, so it must be the distance between
    # the k-th and (k+1)-th largest probabilities, not a neighbouring pair: numpy's sort of the
    # same fp32 probabilities gives the same differences bit for bit (an off-by-one in the rank,
    # e.g. p_(k-1) - p_(k), fails on general inputs, where x = 0 cannot tell them apart)
    inp = small(f"gaps-{k}-{E}", T=400, d=64, E=E, k=k, n_pad=13, x_dist="student4")
    r = oracle.route(inp["x"], inp["router_w"], None, inp["pad_mask"], k=k)
    real = inp["pad_mask"] != 0
    sel, order = gaps_from_sorted(r["probs"], k, real)
    assert np.array_equal(r["gap_sel"], sel)
    assert np.array_equal(r["gap_order"], order)
    assert np.all(r["gap_sel"][real] >= 0) and np.all(r["gap_order"][real] >= 0)
    if k < E:
        # the selection gap is the distance from the last selected weight to the best rejected one
        others = r["probs"].copy()
        np.put_along_axis(others, np.maximum(r["ids"], 0), -1, 1)
        assert np.array_equal(r["gap_sel"][real], (r["w"][:, k - 1] - others.max(1))[real])


def test_near_tie_gaps_closed_form():
    # One-hot x picks one router row: the logits are exactly log(q) for a chosen distribution
    # q = (0.05, 0.4, 0.1, 0.3, 0.15) (in a shuffled expert order), so p = q up to fp32 rounding
    # and every gap is known: sorted 0.4, 0.3, 0.15, 0.1, 0.05 ->
    #   k = 1: sel 0.1, order inf; k = 2: sel 0.15, order 0.1; k = 3: sel 0.05, order 0.1;
    #   k = 4: sel 0.05, order 0.05; k = 5 = E: sel inf
    q = np.array([0.05, 0.4, 0.1, 0.3, 0.15])
    d = 8
    wr = np.zeros((d, 5), np.float32)
    wr[3] = np.log(q).astype(np.float32)
    x = np.zeros((1, d), np.uint16)
    x[0, 3] = synth.f32_to_bf16_bits(np.float32([1.0]))[0]
    expect = {1: (0.1, np.inf), 2: (0.15, 0.1), 3: (0.05, 0.1), 4: (0.05, 0.05), 5: (np.inf, 0.05)}
    for k, (sel, order) in expect.items():
        r = oracle.route(x, wr, None, None, k=k)
        assert np.allclose(r["probs"][0], q, rtol=1e-6)
        assert r["ids"][0].tolist() == [1, 3, 4, 2, 0][:k]
        for got, want in ((r["gap_sel"][0], sel), (r["gap_order"][0], order)):
            assert (np.isinf(got) and np.isinf(want)) or abs(got - want) <= 1e-6, (k, got, want)


def test_routing_weights_are_unrenormalised_top2_probabilities(tiny_inputs):
    r = oracle.route(tiny_inputs["x"], tiny_inputs["router_w"], None, None, k=2)
    w, p, ids = r["w"], r["probs"], r["ids"]
    assert np.array_equal(w, np.take_along_axis(p, ids, 1))
    assert np.all(w.sum(1) < 1) and np.all(w[:, 0] >= w[:, 1])
    others = p.copy()
    np.put_along_axis(others, ids, -1, 1)
    assert np.all(w[:, 1] >= others.max(1))


def test_padded_tokens_get_no_route():
    inp = small("route-pad", T=10, d=16, E=4, n_pad=3)
    r = oracle.route(inp["x"], inp["router_w"], None, inp["pad_mask"], k=2)
    pad = inp["pad_mask"] == 0
    assert np.all(r["ids"][pad] == -1) and np.all(r["w"][pad] == 0)
    assert np.all(r["ids"][~pad] >= 0)


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k,n_pad", [(64, 8, 2, 0), (300, 8, 2, 70), (33, 5, 3, 4), (9, 1, 1, 0),
                                         (0, 8, 2, 0), (5, 8, 2, 5)])
def test_dispatch_equals_stable_argsort(T, E, k, n_pad):
    rng = np.random.default_rng(T * 31 + E)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    pad = None
    if n_pad:
        pad = np.ones(T, np.uint8)
        pad[rng.choice(T, n_pad, replace=False)] = 0
    got = oracle.dispatch(ids, pad, E)
    real = np.ones(T, bool) if pad is None else pad.astype(bool)
    tt, jj = np.nonzero(np.broadcast_to(real[:, None], (T, k)))
    ex = ids[tt, jj]
    order = np.argsort(ex, kind="stable")  # library stable sort of the (t, j) pairs by expert
    assert np.array_equal(got["perm"], tt[order])
    assert np.array_equal(got["counts"], np.bincount(ex, minlength=E))
    assert np.array_equal(got["offsets"], np.concatenate([[0], np.cumsum(np.bincount(ex, minlength=E))]))
    pos = -np.ones((T, k), np.int64)
    pos[tt[order], jj[order]] = np.arange(order.size)
    assert np.array_equal(got["pos"], pos)


def test_dispatch_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 9]], np.int32), None, 8)


# ---------------------------------------------------------------- expert FFN (step 3)

@pytest.mark.parametrize("d,f", [(24, 40), (40, 24)])
def test_single_expert_is_the_dense_gated_mlp(d, f):
    # E = k = 1 => p = 1 => out = (gelu(x Wg) * (x Wu)) Wd, checked against numpy fp64 matmuls.
    # d != f and per-channel scale factors catch a transposed weight or a wrong scale index;
    # swapping gate and up, or a dropped scale, fails by far more than the bound.
    inp = small(f"dense-{d}-{f}", T=12, d=d, f=f, E=1, k=1, scale_jitter=True)
    out, ids, w = oracle.forward_inputs(inp, k=1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    ref = numpy_layer(inp, ids, w)
    assert np.max(np.abs(out - ref)) <= 1e-5 * rms(ref)
    swapped = dict(inp, w_gate=inp["w_up"], w_up=inp["w_gate"])
    assert np.max(np.abs(numpy_layer(swapped, ids, w) - ref)) > 1e-2 * rms(ref)


def test_hidden_and_down_stages_vs_numpy():
    inp = small("stages", T=20, d=64, f=96, E=3, scale_jitter=True)
    s = bf(inp["scales"])
    x = bf(inp["x"])
    for e in range(3):
        h, g, u = oracle.expert_hidden(inp["x"], inp["w_gate"], inp["w_up"], inp["scales"], e, with_gu=True)
        gr = x @ (inp["w_gate"][e] * s[e, :96])
        ur = x @ (inp["w_up"][e] * s[e, 96:192])
        assert np.max(np.abs(g - gr)) <= 1e-5 * rms(gr) and np.max(np.abs(u - ur)) <= 1e-5 * rms(ur)
        assert np.max(np.abs(h - gelu_ref(gr) * ur)) <= 1e-5 * rms(h)
        y = oracle.expert_down(h, inp["w_down"], inp["scales"], e)
        yr = h.astype(np.float64) @ (inp["w_down"][e] * s[e, 192:])
        assert np.max(np.abs(y - yr)) <= 1e-5 * rms(yr)


def test_identity_experts_closed_form():
    # d = f, q = 64 I and s = 2^-6 (both exact in int8 / bf16) => every expert matrix is I, so
    # out[t] = (w0 + w1) * gelu(x) * x elementwise, exactly in real arithmetic.
    T, d, E = 16, 32, 4
    inp = small("identity", T=T, d=d, f=d, E=E)
    eye = (64 * np.eye(d)).astype(np.int8)
    for name in ("w_gate", "w_up", "w_down"):
        inp[name] = np.ascontiguousarray(np.broadcast_to(eye, (E, d, d)))
    inp["scales"] = np.full((E, 3 * d), synth.f32_to_bf16_bits(np.float32([2.0 ** -6]))[0], np.uint16)
    out, ids, w = oracle.forward_inputs(inp)
    x = bf(inp["x"])
    ref = w.astype(np.float64).sum(1, keepdims=True) * gelu_ref(x) * x
    assert np.max(np.abs(out - ref)) <= 4e-7 * np.max(np.abs(ref)) + 1e-30


def test_zero_input_gives_zero_output():
    inp = small("zero", T=6, d=16, f=24)
    inp["x"] = np.zeros_like(inp["x"])
    out, ids, w = oracle.forward_inputs(inp)
    assert np.all(out == 0) and np.array_equal(ids, np.tile([0, 1], (6, 1)))


def test_down_and_up_scales_are_linear():
    # doubling every down (or up) scale doubles out bit-exactly (powers of two are exact)
    inp = small("lin", T=16, d=32, f=48, E=4)
    out, _, _ = oracle.forward_inputs(inp)
    for sl in (slice(96, None), slice(48, 96)):
        s2 = bf(inp["scales"]).astype(np.float32)
        s2[:, sl] *= 2
        out2, _, _ = oracle.forward_inputs(dict(inp, scales=synth.f32_to_bf16_bits(s2)))
        assert np.array_equal(out2, 2 * out)


# ---------------------------------------------------------------- the layer (steps 1-4)

@pytest.mark.parametrize("kw", [dict(), dict(n_pad=5), dict(k=3), dict(bias=(1.0, 0.0, -1.0, 0.5)),
                                dict(x_dist="student4", scale_jitter=True)])
def test_sparse_equals_dense_one_hot_formulation(kw):
    # the pages' own formulation: all experts on all tokens, combined with one-hot masks x gate
    inp = small("dense-vs-sparse", T=24, d=40, f=56, E=4, **kw)
    k = kw.get("k", 2)
    out, _, _ = oracle.forward_inputs(inp, k=k)
    dense = oracle.forward_dense(inp["x"], inp["router_w"], inp["router_bias"], inp["w_gate"], inp["w_up"],
                                 inp["w_down"], inp["scales"], inp["pad_mask"], k=k)
    assert np.max(np.abs(out - dense)) <= 1e-5 * rms(dense)
    if k == 2:
        assert np.array_equal(out, dense)  # two terms: addition order cannot matter


def test_fp32_oracle_within_rounding_of_fp64_brute_force(tiny_inputs):
    for inp in [small("bf-a", T=8, d=16, f=16, E=4), small("bf-b", T=8, d=12, f=8, E=3, n_pad=2),
                tiny_inputs]:
        out, ids, _ = oracle.forward_inputs(inp)
        ref, ids64 = oracle.forward_f64(inp["x"][:16], inp["router_w"], inp["router_bias"], inp["w_gate"],
                                        inp["w_up"], inp["w_down"], inp["scales"],
                                        None if inp["pad_mask"] is None else inp["pad_mask"][:16])
        assert np.array_equal(ids[:16], ids64)
        assert np.max(np.abs(out[:16] - ref)) <= 1e-5 * rms(ref)


@pytest.mark.slow
@pytest.mark.parametrize("d,f", [(6144, 64), (64, 32768)])
def test_fp32_oracle_error_at_grok_contraction_lengths(d, f):
    # the two long sums of the real layer: K = 6144 (gate/up) and K = 32768 (down)
    inp = small(f"long-{d}-{f}", T=4, d=d, f=f, E=2)
    out, ids, _ = oracle.forward_inputs(inp)
    ref, ids64 = oracle.forward_f64(inp["x"], inp["router_w"], None, inp["w_gate"], inp["w_up"],
                                    inp["w_down"], inp["scales"], None)
    assert np.array_equal(ids, ids64)
    assert np.max(np.abs(out - ref)) <= 1e-4 * rms(ref)


def test_padded_rows_are_zero_and_do_not_affect_real_rows():
    inp = small("pad-inv", T=20, d=32, f=48, n_pad=6)
    out, ids, _ = oracle.forward_inputs(inp)
    pad = inp["pad_mask"] == 0
    assert np.all(out[pad] == 0) and not np.any(np.signbit(out[pad]))
    x2 = inp["x"].copy()
    x2[pad] = synth.f32_to_bf16_bits(np.full((pad.sum(), 32), 1000.0, np.float32))
    out2, _, _ = oracle.forward_inputs(dict(inp, x=x2))
    assert np.array_equal(out2, out)


def test_token_permutation_commutes(tiny_inputs):
    out, _, _ = oracle.forward_inputs(tiny_inputs)
    perm = np.random.default_rng(1).permutation(64)
    outp, _, _ = oracle.forward_inputs(dict(tiny_inputs, x=np.ascontiguousarray(tiny_inputs["x"][perm])))
    assert np.array_equal(outp, out[perm])


def test_expert_relabelling():
    inp = small("relabel", T=32, d=32, f=40, E=4, bias=(0.1, 0.2, 0.3, 0.4))
    out, ids, _ = oracle.forward_inputs(inp)
    sigma = np.array([2, 0, 3, 1])  # new expert i is old expert sigma[i]
    inv = np.argsort(sigma)
    relab = dict(inp, router_w=np.ascontiguousarray(inp["router_w"][:, sigma]),
                 router_bias=np.ascontiguousarray(np.asarray(inp["router_bias"], np.float32)[sigma]),
                 scales=np.ascontiguousarray(inp["scales"][sigma]))
    for name in ("w_gate", "w_up", "w_down"):
        relab[name] = np.ascontiguousarray(inp[name][sigma])
    out2, ids2, _ = oracle.forward_inputs(relab)
    assert np.array_equal(ids2, inv[ids])
    # the softmax denominator is summed in expert order, so relabelling moves w by an ulp
    assert np.max(np.abs(out2 - out)) <= 1e-6 * rms(out)


def test_batch_invariance_and_thread_count_independence(tiny_inputs):
    out, _, _ = oracle.forward_inputs(tiny_inputs, nthreads=1)
    out8, _, _ = oracle.forward_inputs(tiny_inputs, nthreads=8)
    assert np.array_equal(out, out8)
    for t in (0, 17, 63):
        one, _, _ = oracle.forward_inputs(tiny_inputs, rows=[t])
        assert np.array_equal(one[0], out[t])


def test_empty_batch():
    inp = small("empty", T=0, d=16, f=16)
    out, ids, w = oracle.forward_inputs(inp)
    assert out.shape == (0, 16) and ids.shape == (0, 2)


# ---------------------------------------------------------------- the MoE block of a decoder layer

def test_rms_norm_vs_numpy_and_closed_form():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(300).astype(np.float32) * 3
    scale = (1 + 0.2 * rng.standard_normal(300)).astype(np.float32)
    got = oracle.rms_norm_row(v, scale, 1e-5)
    v64 = v.astype(np.float64)
    ref = v64 / np.sqrt(np.mean(v64 ** 2) + 1e-5) * scale
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    # constant row c: rms = |c|, so out = sign(c) * scale / sqrt(1 + eps / c^2)
    c = np.full(64, -2.5, np.float32)
    out = oracle.rms_norm_row(c, np.ones(64, np.float32), 0.25)
    assert np.allclose(out, -1 / np.sqrt(1 + 0.25 / 6.25), rtol=1e-6)
    # eps matters (catches a dropped eps) and the scale multiplies per feature (catches a dropped scale)
    assert not np.allclose(oracle.rms_norm_row(c, np.ones(64, np.float32), 0.0), out)


def test_block_is_norm_moe_norm_residual():
    inp = small("block", T=20, d=48, f=64, E=4, n_pad=4)
    rng = np.random.default_rng(3)
    wpre = (1 + 0.2 * rng.standard_normal(48)).astype(np.float32)
    wpost = (1 + 0.2 * rng.standard_normal(48)).astype(np.float32)
    h_out, x = oracle.block_forward(inp["x"], wpre, wpost, 1e-5, inp["router_w"], None, inp["w_gate"], inp["w_up"],
                                    inp["w_down"], inp["scales"], inp["pad_mask"])
    h = bf(inp["x"])
    # the MoE input is bf16(rms_norm(h)): numpy fp64 value, rounded, within one bf16 ulp
    xn = h / np.sqrt(np.mean(h ** 2, axis=1, keepdims=True) + 1e-5) * wpre
    assert np.all(np.abs(bf(x) - xn) <= 2.0 ** -7 * np.abs(xn) + 1e-30)
    # h_out - h = rms_norm(moe(x)) with the post scale
    m, _, _ = oracle.forward(x, inp["router_w"], None, inp["w_gate"], inp["w_up"], inp["w_down"], inp["scales"],
                             inp["pad_mask"])
    m64 = m.astype(np.float64)
    post = m64 / np.sqrt(np.mean(m64 ** 2, axis=1, keepdims=True) + 1e-5) * wpost
    assert np.max(np.abs((h_out - h) - post)) <= 1e-5 * rms(post)
    # padded tokens: the MoE contributes 0, so h_out = h exactly
    pad = inp["pad_mask"] == 0
    assert np.array_equal(h_out[pad], h[pad].astype(np.float32))


@pytest.mark.parametrize("G", [2, 4])
def test_tensor_parallel_shares_sum_to_the_layer(G):
    # Splitting f across G shares (all experts in each) and summing the shares' outputs gives
    # the layer: routing is per token and replicated, and every term of the down contraction
    # belongs to exactly one share (Guide section 6, the psum over the model axis).
    from tp_helpers import tp_share

    inp = small("tp", T=24, d=40, f=96, E=4, k=2, n_pad=3, scale_jitter=True)
    full, ids, _ = oracle.forward_inputs(inp, k=2)
    parts = np.zeros(full.shape, np.float64)
    for g in range(G):
        sh = tp_share(inp, g, G)
        out_g, ids_g, _ = oracle.forward_inputs(sh, k=2)
        assert np.array_equal(ids_g, ids)
        parts += out_g
    assert np.max(np.abs(parts - full)) <= 1e-5 * rms(full)
    # a share on its own is not the layer
    assert np.max(np.abs(oracle.forward_inputs(tp_share(inp, 0, G), k=2)[0] - full)) > 0.1 * rms(full)
