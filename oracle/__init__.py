"""CPU oracle of the Grok-1 top-2-of-8 MoE layer forward pass (ctypes over liboracle.so).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package. It shares no code with the GPU library.

Each function states the passage of the sources it follows; the C file holds the
arithmetic (fp32, every operation rounded on its own, sums in index order) and the
readings taken where the sources are silent. Arrays are numpy; bf16 tensors are
passed as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB: load another build of the oracle (the sanitizer test's)
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile liboracle.so with g++ (-ffp-contract=off: no fused multiply-add); `sanitize` adds
    AddressSanitizer and UndefinedBehaviorSanitizer, written to `out`."""
    src = os.path.join(_HERE, "moe_oracle.cpp")
    out = out or os.path.join(_HERE, "liboracle.so")
    san = ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"] \
        if sanitize else []
    cmd = ["g++", "-O3", *san, "-mavx2", "-ffp-contract=off", "-fno-fast-math", "-std=c++17", "-fPIC",
           "-shared", "-pthread", src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.oracle_gelu_tanh.argtypes = [ctypes.c_float]
    lib.oracle_gelu_tanh.restype = ctypes.c_float
    lib.oracle_route.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.oracle_dispatch.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_expert_hidden.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, i32]
    lib.oracle_expert_down.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32]
    lib.oracle_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, i32]
    lib.oracle_forward_dense.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32]
    lib.oracle_forward_f64.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.oracle_rms_norm_row.argtypes = [vp, vp, ctypes.c_float, i32, vp]
    lib.oracle_rms_norm_row.restype = None
    lib.oracle_block_forward.argtypes = [vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                         i32, i32, vp, vp, i32]
    lib.oracle_block_forward.restype = ctypes.c_int
    for name in ("oracle_route", "oracle_dispatch", "oracle_expert_hidden", "oracle_expert_down",
                 "oracle_forward", "oracle_forward_dense", "oracle_forward_f64"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray], dtype=None):
    if a is None:
        return None
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    assert a.flags.c_contiguous
    return a.ctypes.data


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def gelu_tanh(v: float) -> float:
    """GeLU, tanh form, fp32 (Grok-1 Admin & Architecture Guide, section 3, MoE step 3)."""
    return float(_load().oracle_gelu_tanh(v))


def route(x, router_w, router_bias, pad_mask, k: int):
    """Router and top-k (Guide section 3, MoE steps 1-2; fp32 routing per section 9).

    Returns dict: logits, probs [T][E]; ids int32 [T][k]; w [T][k]; gap_sel, gap_order [T]."""
    T, d = x.shape
    E = router_w.shape[1]
    out = {
        "logits": np.empty((T, E), np.float32),
        "probs": np.empty((T, E), np.float32),
        "ids": np.empty((T, k), np.int32),
        "w": np.empty((T, k), np.float32),
        "gap_sel": np.empty(T, np.float32),
        "gap_order": np.empty(T, np.float32),
    }
    rc = _load().oracle_route(_p(x, np.uint16), _p(router_w, np.float32), _p(router_bias, np.float32),
                              _p(pad_mask, np.uint8), T, d, E, k,
                              _p(out["logits"]), _p(out["probs"]), _p(out["ids"]), _p(out["w"]),
                              _p(out["gap_sel"]), _p(out["gap_order"]))
    _check(rc, "route")
    return out


def dispatch(ids, pad_mask, E: int):
    """Stable counting sort of the assignments by expert.

    Returns dict: counts [E], offsets [E+1], perm [N_assign], pos [T][k] (int32)."""
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(T * k, 1), np.int32)
    pos = np.empty((T, k), np.int32)
    rc = _load().oracle_dispatch(_p(np.ascontiguousarray(ids, np.int32)), _p(pad_mask, np.uint8), T, E, k,
                                 _p(counts), _p(offsets), _p(perm), _p(pos))
    _check(rc, "dispatch")
    return {"counts": counts, "offsets": offsets, "perm": perm[: int(offsets[E])], "pos": pos}


def expert_hidden(x_rows, w_gate, w_up, scales, e: int, with_gu: bool = False, nthreads: int = 0):
    """h = gelu_tanh(x Wg_e) * (x Wu_e) for rows of x (Guide section 3, MoE step 3 and
    "Quantized weights"). Returns h fp32 [n][f] (and g, u when with_gu)."""
    n, d = x_rows.shape
    E, _, f = w_gate.shape
    h = np.empty((n, f), np.float32)
    g = np.empty((n, f), np.float32) if with_gu else None
    u = np.empty((n, f), np.float32) if with_gu else None
    rc = _load().oracle_expert_hidden(_p(np.ascontiguousarray(x_rows), np.uint16), n, _p(w_gate, np.int8),
                                      _p(w_up, np.int8), _p(scales, np.uint16), d, f, E, e,
                                      _p(h), _p(g), _p(u), nthreads)
    _check(rc, "expert_hidden")
    return (h, g, u) if with_gu else h


def expert_down(h, w_down, scales, e: int, nthreads: int = 0):
    """y = h Wd_e (Guide section 3, MoE step 3 "-> linear_1"). h fp32 [n][f] -> y fp32 [n][d]."""
    n, f = h.shape
    E, _, d = w_down.shape
    y = np.empty((n, d), np.float32)
    rc = _load().oracle_expert_down(_p(np.ascontiguousarray(h, np.float32)), n, _p(w_down, np.int8),
                                    _p(scales, np.uint16), d, f, E, e, _p(y), nthreads)
    _check(rc, "expert_down")
    return y


def forward(x, router_w, router_bias, w_gate, w_up, w_down, scales, pad_mask, k: int = 2, nthreads: int = 0):
    """The layer (Guide section 3, MoE steps 1-4). Returns (out fp32 [T][d], ids, w)."""
    T, d = x.shape
    E, _, f = w_gate.shape
    out = np.empty((T, d), np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = _load().oracle_forward(_p(x, np.uint16), _p(router_w, np.float32), _p(router_bias, np.float32),
                                _p(w_gate, np.int8), _p(w_up, np.int8), _p(w_down, np.int8),
                                _p(scales, np.uint16), _p(pad_mask, np.uint8), T, d, f, E, k,
                                _p(out), _p(ids), _p(w), nthreads)
    _check(rc, "forward")
    return out, ids, w


def forward_dense(x, router_w, router_bias, w_gate, w_up, w_down, scales, pad_mask, k: int = 2, nthreads: int = 0):
    """The pages' dense one-hot-gated formulation (Guide section 3, MoE step 4 and warning)."""
    T, d = x.shape
    E, _, f = w_gate.shape
    out = np.empty((T, d), np.float32)
    rc = _load().oracle_forward_dense(_p(x, np.uint16), _p(router_w, np.float32), _p(router_bias, np.float32),
                                      _p(w_gate, np.int8), _p(w_up, np.int8), _p(w_down, np.int8),
                                      _p(scales, np.uint16), _p(pad_mask, np.uint8), T, d, f, E, k,
                                      _p(out), nthreads)
    _check(rc, "forward_dense")
    return out


def forward_f64(x, router_w, router_bias, w_gate, w_up, w_down, scales, pad_mask, k: int = 2):
    """fp64 brute force of the same definition (tiny shapes only). Returns (out fp64, ids)."""
    T, d = x.shape
    E, _, f = w_gate.shape
    out = np.empty((T, d), np.float64)
    ids = np.empty((T, k), np.int32)
    rc = _load().oracle_forward_f64(_p(x, np.uint16), _p(router_w, np.float32), _p(router_bias, np.float32),
                                    _p(w_gate, np.int8), _p(w_up, np.int8), _p(w_down, np.int8),
                                    _p(scales, np.uint16), _p(pad_mask, np.uint8), T, d, f, E, k,
                                    _p(out), _p(ids))
    _check(rc, "forward_f64")
    return out, ids


def rms_norm_row(v, scale, eps: float):
    """RMSNorm of one fp32 row (Guide section 3 "Transformer stack"; reading: learned scale, given eps)."""
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty_like(v)
    _load().oracle_rms_norm_row(_p(v), _p(np.ascontiguousarray(scale, np.float32)), eps, v.size, _p(out))
    return out


def block_forward(h, norm_pre, norm_post, eps, router_w, router_bias, w_gate, w_up, w_down, scales, pad_mask,
                  k: int = 2, nthreads: int = 0):
    """The decoder layer's MoE block: h + rms_norm(moe(bf16(rms_norm(h)))) (Guide section 3
    "Transformer stack"; grok-field-guide fourth stop). Returns (h_out fp32 [T][d], x bf16 bits)."""
    T, d = h.shape
    E, _, f = w_gate.shape
    out = np.empty((T, d), np.float32)
    x = np.empty((T, d), np.uint16)
    rc = _load().oracle_block_forward(_p(h, np.uint16), _p(np.ascontiguousarray(norm_pre, np.float32)),
                                      _p(np.ascontiguousarray(norm_post, np.float32)), eps,
                                      _p(router_w, np.float32), _p(router_bias, np.float32), _p(w_gate, np.int8),
                                      _p(w_up, np.int8), _p(w_down, np.int8), _p(scales, np.uint16),
                                      _p(pad_mask, np.uint8), T, d, f, E, k, _p(out), _p(x), nthreads)
    _check(rc, "block_forward")
    return out, x


def forward_inputs(inp: dict, k: int = 2, nthreads: int = 0, rows=None):
    """oracle forward on a `synth.make_inputs` dict; `rows` restricts to those token rows
    (rows are independent, so each output row equals its row of the full batch)."""
    x, pad = inp["x"], inp["pad_mask"]
    if rows is not None:
        x = np.ascontiguousarray(x[rows])
        pad = None if pad is None else np.ascontiguousarray(pad[rows])
    return forward(x, inp["router_w"], inp["router_bias"], inp["w_gate"], inp["w_up"], inp["w_down"],
                   inp["scales"], pad, k=k, nthreads=nthreads)
