"""Shared helpers of the GPU tests: device copies of synth inputs, tolerances, near-tie logic."""
from __future__ import annotations

import numpy as np

import synth

# A token whose 2nd and 3rd (generally k-th and k+1-th) router probabilities are closer than
# this is a near tie: fp32 rounding order may legitimately flip its expert set, so it is
# counted and left out of the id, dispatch and output comparisons.
NEAR_TIE = 1e-5
# max |out_gpu - out_ref| <= OUT_TOL * rms(out_ref)
OUT_TOL = 1e-2
# |w_gpu - w_ref| for routing weights (fp32 exp/sum order differs between CPU and GPU)
W_TOL = 1e-5


def to_dev(inp: dict, with_weights: bool = True) -> dict:
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    t = {
        "x": bf16(inp["x"]),
        "router_w": torch.from_numpy(inp["router_w"]).cuda(),
        "router_bias": None if inp["router_bias"] is None else torch.from_numpy(inp["router_bias"]).cuda(),
        "scales": bf16(inp["scales"]),
        "pad_mask": None if inp["pad_mask"] is None else torch.from_numpy(inp["pad_mask"]).cuda(),
    }
    if with_weights:
        for n in ("w_gate", "w_up", "w_down"):
            t[n] = torch.from_numpy(inp[n]).cuda()
    return t


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def exclusions(route: dict) -> tuple[np.ndarray, np.ndarray]:
    """(excluded, order_ambiguous) masks from the oracle's routing gaps."""
    return route["gap_sel"] < NEAR_TIE, route["gap_order"] < NEAR_TIE


def max_excluded(T: int) -> int:
    """Upper bound on near-tie exclusions in a batch of T tokens. The gap of two neighbouring
    probabilities falls below 1e-5 for about 1-2e-4 of the tokens at the workloads' router
    statistics, so more than max(2, 1e-3 T) means the gap itself is wrong and the comparisons
    would be emptied by it."""
    return max(2, int(1e-3 * T))


def check_excluded_tokens(inp: dict, route: dict, excl: np.ndarray, ids_gpu: np.ndarray, w_gpu: np.ndarray,
                          out_gpu: np.ndarray | None = None, scale: float = 1.0) -> float:
    """Near-tie tokens are left out of the bit-exact id comparison, not out of the checks:
    their GPU ids must be a valid top-k of the oracle's probabilities up to the near-tie
    margin (distinct experts, none worse than the k-th largest probability by more than
    NEAR_TIE, slots in descending order within NEAR_TIE), their weights the oracle's
    probabilities of those experts, and their output row the oracle's expert FFNs evaluated
    on the GPU's choice (when `out_gpu` is given). Returns the worst row error over `scale`."""
    import oracle

    T = excl.size
    n = int(excl.sum())
    assert n <= max_excluded(T), f"{n} near-tie exclusions of {T} tokens"
    k = ids_gpu.shape[1]
    E = route["probs"].shape[1]
    worst = 0.0
    for t in np.nonzero(excl)[0]:
        p = route["probs"][t].astype(np.float64)
        ids = ids_gpu[t]
        assert len(set(ids.tolist())) == k and np.all((ids >= 0) & (ids < E)), (t, ids)
        pk = np.sort(p)[::-1][k - 1]
        assert np.all(p[ids] >= pk - NEAR_TIE), (t, ids, p)
        assert np.all(np.diff(p[ids]) <= NEAR_TIE), (t, ids, p)
        assert np.all(np.abs(w_gpu[t] - p[ids]) <= W_TOL), (t, w_gpu[t], p[ids])
        if out_gpu is None:
            continue
        xr = np.ascontiguousarray(inp["x"][t:t + 1])
        row = np.zeros(inp["x"].shape[1], np.float32)
        for j in range(k):
            e = int(ids[j])
            hrow = oracle.expert_hidden(xr, inp["w_gate"], inp["w_up"], inp["scales"], e)
            y = oracle.expert_down(hrow, inp["w_down"], inp["scales"], e)[0]
            row = row + np.float32(route["probs"][t, e]) * y
        err = float(np.abs(out_gpu[t] - row).max()) / scale
        assert err <= OUT_TOL, (t, err)
        worst = max(worst, err)
    return worst


def compare_ids(ids_gpu: np.ndarray, ids_ref: np.ndarray, excluded: np.ndarray, ambiguous: np.ndarray) -> int:
    """Bit-exact ids on non-excluded tokens (as a set where slot order is a near tie).
    Returns the number of compared tokens."""
    keep = ~excluded
    exact = keep & ~ambiguous
    assert np.array_equal(ids_gpu[exact], ids_ref[exact]), np.nonzero((ids_gpu != ids_ref).any(1) & exact)
    amb = keep & ambiguous
    if amb.any():
        assert np.array_equal(np.sort(ids_gpu[amb], 1), np.sort(ids_ref[amb], 1))
    return int(keep.sum())


def check_dispatch_valid(ids: np.ndarray, pad: np.ndarray | None, E: int, disp: dict) -> None:
    """The dispatch arrays are the stable counting sort of the given ids (properties only)."""
    T, k = ids.shape
    real = np.ones(T, bool) if pad is None else pad.astype(bool)
    counts = np.array([((ids == e) & real[:, None]).sum() for e in range(E)])
    assert np.array_equal(disp["counts"], counts)
    assert np.array_equal(disp["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    n = int(counts.sum())
    perm = disp["perm"][:n]
    pos = disp["pos"]
    for e in range(E):
        seg = perm[disp["offsets"][e]:disp["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all((ids[seg] == e).any(1))
    tt, jj = np.nonzero(real[:, None] & np.ones((1, k), bool))
    assert np.array_equal(perm[pos[tt, jj]], tt)
    assert np.all(pos[~real] == -1)


def sample_rows(T: int, n: int, seed: int, must: np.ndarray | None = None) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, n, replace=False).tolist())
    if must is not None:
        rows |= set(must.tolist())
    return np.array(sorted(rows))


def fp16_from_normal(key_seed: int, shape, sigma: float = 0.5) -> np.ndarray:
    """Seeded synthetic fp16 matrix (normal values rounded to fp16) as an input."""
    n = int(np.prod(shape))
    v = synth.normal_f32(synth.key(key_seed, 4242, 1), n, sigma=sigma)
    return v.astype(np.float16).reshape(shape)
