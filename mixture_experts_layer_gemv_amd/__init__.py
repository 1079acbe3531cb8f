"""MI355X (gfx950) forward pass of Grok-1's top-2-of-8 Mixture-of-Experts layer.

A thin ctypes binding over libmoe.so, whose C ABI is declared in include/moe.h. The
functions here only marshal arguments: every step of the layer runs in the library's
HIP kernels. PyTorch supplies device memory and streams. If libmoe.so is not built,
every call raises; there is no other implementation to fall back to.

Tensor arguments may be torch tensors (their data_ptr() is passed) or raw device
addresses (int); None passes NULL. `stream` defaults to torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_NOMEM = range(5)
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_HIP", 4: "MOE_ERR_NOMEM"}

# Every symbol include/moe.h declares, with its ctypes signature.
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "moe_forward": ([_vp] * 8 + [_i32] * 5 + [_vp], _i32),
    "moe_forward_ex": ([_vp] * 8 + [_i32] * 5 + [_vp, _vp, _vp, _sz, _vp], _i32),
    "moe_route": ([_vp] * 6 + [_i32] * 4 + [_vp], _i32),
    "moe_dispatch": ([_vp] * 6 + [_i32] * 3 + [_vp], _i32),
    "moe_gate_up": ([_vp] * 7 + [_i32] * 5 + [_vp], _i32),
    "moe_down": ([_vp] * 5 + [_i32] * 6 + [_vp], _i32),
    "moe_down_splits": ([_i32] * 5, _i32),
    "moe_expert_kernels": ([_i32] * 5, _i32),
    "moe_gate_up_parts": ([_i32] * 5, _i32),
    "moe_one_launch": ([_i32] * 5, _i32),
    "moe_combine": ([_vp] + [_i32] + [_vp] * 4 + [_i32] * 3 + [_vp], _i32),
    "moe_workspace_bytes": ([_i32] * 5, _sz),
    "moe_forward_noalloc": ([_vp] * 8 + [_i32] * 5 + [_vp, _vp], _i32),
    "moe_forward_dense": ([_vp] * 8 + [_i32] * 5 + [_vp, _vp, _vp, _sz], _i32),
    "moe_workspace_bytes_dense": ([_i32] * 5, _sz),
    "moe_block_forward": ([_vp, _vp, _vp, ctypes.c_float] + [_vp] * 7 + [_i32] * 5 + [_vp, _vp, _vp, _sz, _vp], _i32),
    "moe_workspace_bytes_block": ([_i32] * 5, _sz),
    "moe_graph_create": ([ctypes.POINTER(_vp)] + [_vp] * 8 + [_i32] * 5 + [_vp, _vp, _sz], _i32),
    "moe_graph_launch": ([_vp, _vp], _i32),
    "moe_graph_destroy": ([_vp], None),
    "moe_release_workspace": ([], None),
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_abi_version": ([], _i32),
}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class DebugOut(ctypes.Structure):
    _fields_ = [("topk_ids", _vp), ("topk_w", _vp), ("counts", _vp), ("offsets", _vp), ("perm", _vp), ("pos", _vp)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the MoE layer has no implementation other than its HIP kernels)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, last_error())


def last_error() -> str:
    return lib().moe_last_error().decode()


def abi_version() -> int:
    return lib().moe_abi_version()


def workspace_bytes(T: int, d: int, f: int, E: int, k: int) -> int:
    return lib().moe_workspace_bytes(T, d, f, E, k)


def down_splits(T: int, d: int, f: int, E: int, k: int) -> int:
    return lib().moe_down_splits(T, d, f, E, k)


def expert_kernels(T: int, d: int, f: int, E: int, k: int) -> int:
    """0: the streaming expert kernels run; 128 / 256: the tiled ones, with tiles of that many rows."""
    return lib().moe_expert_kernels(T, d, f, E, k)


def gate_up_parts(T: int, d: int, f: int, E: int, k: int) -> int:
    """Parts of gate/up's contraction over d (more than 1: a finish launch adds them)."""
    return lib().moe_gate_up_parts(T, d, f, E, k)


def one_launch(T: int, d: int, f: int, E: int, k: int) -> int:
    """1 if the forward runs this shape as one kernel launch, 0 if one launch per stage."""
    return lib().moe_one_launch(T, d, f, E, k)


def release_workspace() -> None:
    lib().moe_release_workspace()


def moe_forward(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, stream=None) -> None:
    _check(lib().moe_forward(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(scales),
                             _ptr(pad_mask), _ptr(out), T, d, f, E, k, _stream(stream)))


def moe_forward_ex(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, stream=None,
                   router_bias=None, workspace=None, workspace_bytes_: int = 0, dbg: Optional[dict] = None) -> None:
    dbg_struct = None
    if dbg is not None:
        dbg_struct = DebugOut(*(_ptr(dbg.get(n)) for n in ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos")))
    _check(lib().moe_forward_ex(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(scales),
                                _ptr(pad_mask), _ptr(out), T, d, f, E, k, _stream(stream), _ptr(router_bias),
                                _ptr(workspace), workspace_bytes_,
                                ctypes.byref(dbg_struct) if dbg_struct is not None else None))


def moe_forward_noalloc(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, stream=None,
                        router_bias=None) -> None:
    """moe_forward_ex whose scratch is the library's fixed per-device array (allocates nothing)."""
    _check(lib().moe_forward_noalloc(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(scales),
                                     _ptr(pad_mask), _ptr(out), T, d, f, E, k, _stream(stream), _ptr(router_bias)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_dense(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, stream=None,
                      router_bias=None, workspace=None, workspace_bytes_: int = 0) -> None:
    """The dense one-hot-gated formulation (every expert on every token): a baseline."""
    _check(lib().moe_forward_dense(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(scales),
                                   _ptr(pad_mask), _ptr(out), T, d, f, E, k, _stream(stream), _ptr(router_bias),
                                   _ptr(workspace), workspace_bytes_))


def workspace_bytes_dense(T: int, d: int, f: int, E: int, k: int) -> int:
    return lib().moe_workspace_bytes_dense(T, d, f, E, k)


def moe_block_forward(h, norm_pre, norm_post, eps, router_w, w_gate, w_up, w_down, scales, pad_mask, h_out,
                      T, d, f, E, k, stream=None, router_bias=None, workspace=None, workspace_bytes_: int = 0,
                      x_norm_out=None) -> None:
    """The decoder layer's MoE block with the pre-norm and post-norm + residual fused."""
    _check(lib().moe_block_forward(_ptr(h), _ptr(norm_pre), _ptr(norm_post), float(eps), _ptr(router_w),
                                   _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(scales), _ptr(pad_mask), _ptr(h_out),
                                   T, d, f, E, k, _stream(stream), _ptr(router_bias), _ptr(workspace),
                                   workspace_bytes_, _ptr(x_norm_out)))


def workspace_bytes_block(T: int, d: int, f: int, E: int, k: int) -> int:
    return lib().moe_workspace_bytes_block(T, d, f, E, k)


class Graph:
    """A captured single-launch forward (moe_graph_*): fixed buffers, one hipGraphLaunch per call."""

    def __init__(self, x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k,
                 router_bias=None, workspace=None, workspace_bytes_: int = 0):
        handle = _vp()
        _check(lib().moe_graph_create(ctypes.byref(handle), _ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up),
                                      _ptr(w_down), _ptr(scales), _ptr(pad_mask), _ptr(out), T, d, f, E, k,
                                      _ptr(router_bias), _ptr(workspace), workspace_bytes_))
        self._handle = handle
        self._keep = (x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, router_bias, workspace)

    def launch(self, stream=None) -> None:
        _check(lib().moe_graph_launch(self._handle, _stream(stream)))

    def close(self) -> None:
        if self._handle:
            lib().moe_graph_destroy(self._handle)
            self._handle = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_route(x, router_w, router_bias, pad_mask, topk_ids, topk_w, T, d, E, k, stream=None) -> None:
    _check(lib().moe_route(_ptr(x), _ptr(router_w), _ptr(router_bias), _ptr(pad_mask), _ptr(topk_ids),
                           _ptr(topk_w), T, d, E, k, _stream(stream)))


def moe_dispatch(topk_ids, pad_mask, counts, offsets, perm, pos, T, E, k, stream=None) -> None:
    _check(lib().moe_dispatch(_ptr(topk_ids), _ptr(pad_mask), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(pos),
                              T, E, k, _stream(stream)))


def moe_gate_up(x, perm, offsets, w_gate, w_up, scales, h, T, d, f, E, k, stream=None) -> None:
    _check(lib().moe_gate_up(_ptr(x), _ptr(perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(scales), _ptr(h),
                             T, d, f, E, k, _stream(stream)))


def moe_down(h, offsets, w_down, scales, y, splits, T, d, f, E, k, stream=None) -> None:
    _check(lib().moe_down(_ptr(h), _ptr(offsets), _ptr(w_down), _ptr(scales), _ptr(y), splits, T, d, f, E, k,
                          _stream(stream)))


def moe_combine(y, splits, pos, topk_w, pad_mask, out, T, d, k, stream=None) -> None:
    _check(lib().moe_combine(_ptr(y), splits, _ptr(pos), _ptr(topk_w), _ptr(pad_mask), _ptr(out), T, d, k,
                             _stream(stream)))


def forward(x, router_w, w_gate, w_up, w_down, scales, pad_mask=None, router_bias=None, k: int = 2,
            out=None, stream=None, dbg: Optional[dict] = None):
    """Convenience wrapper: shapes from the tensors, `out` allocated with torch if None.

    x bf16 [T][d]; router_w fp32 [d][E]; w_gate/w_up int8 [E][d][f]; w_down int8 [E][f][d];
    scales bf16 [E][2f+d]; pad_mask uint8 [T] or None; router_bias fp32 [E] or None."""
    import torch

    T, d = x.shape
    E, _, f = w_gate.shape
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    moe_forward_ex(x, router_w, w_gate, w_up, w_down, scales, pad_mask, out, T, d, f, E, k, stream,
                   router_bias=router_bias, dbg=dbg)
    return out
