"""Seeded synthetic inputs for the top-2-of-8 MoE feed-forward layer.

This package only draws numbers; it holds none of the layer's arithmetic. Both the
CPU checker and the GPU path take their inputs from here, as data.

The five named workloads follow the layer shape of the Grok-1 release
(emb 6144, expert FFN 32768, 8 experts, 2 active per token: Grok-1 Admin &
Architecture Guide, section 3 "Configuration objects" and "Mixture of Experts";
llm-architectures-explained "Every architecture field" table), with int8 expert
weights and per-output-channel bf16 scales (Guide section 3 "Quantized weights").

Recipe (all seeded, seed 42 by default):
  * x      bf16, N(0, 1); the skewed workload uses Student-t (4 dof) scaled to unit variance
  * W_r    fp32 [d][E], N(0, 1/d)
  * q      int8 uniform in [-127, 127]: gate/up [E][d][f], down [E][f][d]
  * scales bf16 [E][2f + d] = gate[f] | up[f] | down[d], value 1/(127 sqrt(fan_in))
           (fan_in = d for gate/up, f for down), optionally times U[0.5, 1.5) per channel
  * pad    exact count of padded tokens (mask 0) at seeded random positions
  * bias   optional fp32 [E] added to the router logits (skewed workload only)

Tensor ids within a stream set: x=1, W_r=2, q_gate=3, q_up=4, q_down=5, pad=6,
scale factors=7. Activations and pad masks are keyed by the workload's own set;
router and expert weights by a weight set shared by all Grok-shape workloads
(100 + weight-set id), so the four Grok-shape workloads see one set of weights.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SYNTH_LIB: load another build of the generator (the sanitizer test's)
_LIB_PATH = os.environ.get("MOE_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
_lib = None

TENSOR_X, TENSOR_WR, TENSOR_QG, TENSOR_QU, TENSOR_QD, TENSOR_PAD, TENSOR_SCALE = 1, 2, 3, 4, 5, 6, 7
DEFAULT_SEED = 42


def build(verbose: bool = False, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP for bulk fills); `sanitize` adds AddressSanitizer and
    UndefinedBehaviorSanitizer (host code only), written to `out`."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    out = out or os.path.join(_HERE, "libsynth.so")
    san = ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"] \
        if sanitize else []
    cmd = ["gcc", "-O2", *san, "-fPIC", "-shared", "-fopenmp", "-std=c11", src, "-o", out, "-lm"]
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
    u64, u32, dbl = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.synth_key.argtypes = [u64, u32, u32]
    lib.synth_key.restype = u64
    lib.synth_draw.argtypes = [u64, u64]
    lib.synth_draw.restype = u64
    lib.synth_uniform.argtypes = [u64, u64]
    lib.synth_uniform.restype = dbl
    lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.synth_f32_to_bf16.restype = ctypes.c_uint16
    for name in ("synth_normal_bf16", "synth_normal_f32"):
        getattr(lib, name).argtypes = [vp, u64, u64, u64, dbl]
        getattr(lib, name).restype = None
    lib.synth_student4_bf16.argtypes = [vp, u64, u64, u64]
    lib.synth_student4_bf16.restype = None
    lib.synth_int8.argtypes = [vp, u64, u64, u64]
    lib.synth_int8.restype = None
    lib.synth_uniform_f64.argtypes = [vp, u64, u64, u64]
    lib.synth_uniform_f64.restype = None
    lib.synth_pad_mask.argtypes = [vp, ctypes.c_int, ctypes.c_int, u64]
    lib.synth_pad_mask.restype = ctypes.c_int
    _lib = lib
    return lib


def key(seed: int, stream_set: int, tensor: int) -> int:
    return int(_load().synth_key(seed, stream_set, tensor))


def draws(k: int, n: int, start: int = 0) -> np.ndarray:
    lib = _load()
    return np.array([lib.synth_draw(k, start + i) for i in range(n)], dtype=np.uint64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even), returned as uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(k: int, n: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(out.ctypes.data, start, n, k, sigma)
    return out


def student4_bf16(k: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().synth_student4_bf16(out.ctypes.data, start, n, k)
    return out


def normal_f32(k: int, n: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(out.ctypes.data, start, n, k, sigma)
    return out


def int8_uniform(k: int, n: int, start: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, dtype=np.int8)
    assert out.dtype == np.int8 and out.flags.c_contiguous and out.size == n
    _load().synth_int8(out.ctypes.data, start, n, k)
    return out


def uniform_f64(k: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(out.ctypes.data, start, n, k)
    return out


def pad_mask(k: int, T: int, n_pad: int) -> np.ndarray:
    out = np.empty(max(T, 1), dtype=np.uint8)
    rc = _load().synth_pad_mask(out.ctypes.data, T, n_pad, k)
    if rc != 0:
        raise ValueError("bad pad-mask sizes")
    return out[:T]


@dataclass(frozen=True)
class Spec:
    """One synthetic workload of the MoE layer."""

    name: str
    T: int
    d: int
    f: int
    E: int = 8
    k: int = 2
    n_pad: int = 0
    x_dist: str = "normal"  # "normal" | "student4"
    bias: Optional[Sequence[float]] = None
    x_set: int = 1
    w_set: int = 1
    scale_jitter: bool = False
    seed: int = DEFAULT_SEED
    f_full: Optional[int] = None  # FFN width of the whole layer when f is one GPU's share of it
    description: str = field(default="", compare=False)

    @property
    def n_real(self) -> int:
        return self.T - self.n_pad


SKEW_BIAS = (2.0, 1.0, 0.5, 0.0, 0.0, 0.0, 0.0, -1.0)

WORKLOAD_SPECS = {
    "tiny": Spec("tiny", T=64, d=256, f=512, x_set=1, w_set=1,
                 description="T=64, d=256, f=512, E=8, top-2, no padding"),
    "decode": Spec("decode", T=8, d=6144, f=32768, x_set=2, w_set=2,
                   description="Grok-1 shape, decode: T=8, no padding"),
    "batched_decode": Spec("batched_decode", T=64, d=6144, f=32768, n_pad=6, x_set=3, w_set=2,
                           description="Grok-1 shape, batched decode: T=64, 6 padded tokens"),
    "prefill": Spec("prefill", T=8192, d=6144, f=32768, x_set=4, w_set=2,
                    description="Grok-1 shape, prefill at max context: T=8192, no padding"),
    "skewed": Spec("skewed", T=4096, d=6144, f=32768, n_pad=1024, x_dist="student4", bias=SKEW_BIAS,
                   x_set=5, w_set=2,
                   description="Grok-1 shape, skewed routing: T=4096, 1024 padded, Student-t x, biased router"),
    # One GPU's share of an 8-way tensor-parallel split over f (all 8 experts, f / 8 columns
    # of gate/up and rows of down): what each GPU computes before the all-reduce of out.
    "decode_tp8": Spec("decode_tp8", T=8, d=6144, f=4096, f_full=32768, x_set=2, w_set=6,
                       description="one GPU's share of 8-way tensor parallelism over f: T=8, d=6144, f=4096"),
    "prefill_tp8": Spec("prefill_tp8", T=8192, d=6144, f=4096, f_full=32768, x_set=4, w_set=6,
                        description="one GPU's share of 8-way tensor parallelism over f: T=8192, d=6144, f=4096"),
}


def x_rows(spec: Spec, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Activation rows (bf16 bits, [len(rows)][d]); all T rows when rows is None."""
    kx = key(spec.seed, spec.x_set, TENSOR_X)
    gen = student4_bf16 if spec.x_dist == "student4" else normal_bf16
    if rows is None:
        return gen(kx, spec.T * spec.d).reshape(spec.T, spec.d)
    out = np.empty((len(rows), spec.d), dtype=np.uint16)
    for i, t in enumerate(rows):
        out[i] = gen(kx, spec.d, start=int(t) * spec.d)
    return out


def router_w(spec: Spec) -> np.ndarray:
    kw = key(spec.seed, 100 + spec.w_set, TENSOR_WR)
    return normal_f32(kw, spec.d * spec.E, sigma=1.0 / math.sqrt(spec.d)).reshape(spec.d, spec.E)


def expert_weights(spec: Spec, which: str, experts: Optional[Sequence[int]] = None,
                   out: Optional[np.ndarray] = None) -> np.ndarray:
    """int8 weights of 'gate' | 'up' ([E][d][f]) or 'down' ([E][f][d]).

    With `experts`, only those experts' slices are drawn (same values as in the full tensor)."""
    tid = {"gate": TENSOR_QG, "up": TENSOR_QU, "down": TENSOR_QD}[which]
    kq = key(spec.seed, 100 + spec.w_set, tid)
    per = spec.d * spec.f
    shape_tail = (spec.d, spec.f) if which != "down" else (spec.f, spec.d)
    ex = list(range(spec.E)) if experts is None else list(experts)
    if out is None:
        out = np.empty((len(ex),) + shape_tail, dtype=np.int8)
    for i, e in enumerate(ex):
        int8_uniform(kq, per, start=e * per, out=out[i].reshape(-1))
    return out


def scales(spec: Spec) -> np.ndarray:
    """bf16 bits [E][2f + d]: gate[f] | up[f] | down[d] per expert.

    Value 1/(127 sqrt(fan_in)) in fp64, times a per-channel factor U[0.5, 1.5) when
    scale_jitter is set, rounded fp64 -> fp32 -> bf16 (nearest even both times)."""
    n_ch = 2 * spec.f + spec.d
    fan_in_down = spec.f_full or spec.f
    base = np.concatenate([np.full(2 * spec.f, 1.0 / (127.0 * math.sqrt(spec.d))),
                           np.full(spec.d, 1.0 / (127.0 * math.sqrt(fan_in_down)))])
    vals = np.broadcast_to(base, (spec.E, n_ch)).copy()
    if spec.scale_jitter:
        ks = key(spec.seed, 100 + spec.w_set, TENSOR_SCALE)
        vals *= 0.5 + uniform_f64(ks, spec.E * n_ch).reshape(spec.E, n_ch)
    return f32_to_bf16_bits(vals.astype(np.float32))


def pad(spec: Spec) -> Optional[np.ndarray]:
    if spec.n_pad == 0:
        return None
    return pad_mask(key(spec.seed, spec.x_set, TENSOR_PAD), spec.T, spec.n_pad)


def bias(spec: Spec) -> Optional[np.ndarray]:
    return None if spec.bias is None else np.asarray(spec.bias, dtype=np.float32)


def make_inputs(spec: Spec, with_weights: bool = True) -> dict:
    """All inputs of one workload as numpy arrays (bf16 tensors as uint16 bits)."""
    inp = {
        "spec": spec,
        "x": x_rows(spec),
        "router_w": router_w(spec),
        "router_bias": bias(spec),
        "scales": scales(spec),
        "pad_mask": pad(spec),
    }
    if with_weights:
        inp["w_gate"] = expert_weights(spec, "gate")
        inp["w_up"] = expert_weights(spec, "up")
        inp["w_down"] = expert_weights(spec, "down")
    return inp


def custom(name: str, T: int, d: int, f: int, E: int = 8, k: int = 2, **kw) -> Spec:
    """A small workload for tests: its own stream sets (x_set/w_set default 1000+)."""
    kw.setdefault("x_set", 1000)
    kw.setdefault("w_set", 1000)
    return Spec(name, T=T, d=d, f=f, E=E, k=k, **kw)


__all__ = ["Spec", "WORKLOAD_SPECS", "make_inputs", "custom", "replace", "build", "f32_to_bf16_bits", "bf16_bits_to_f32"]
