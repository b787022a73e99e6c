"""MI355X-native Qwen3 decoder-stack forward: HIP kernels for gfx950 behind a C ABI.

This module is the thin Python binding of ``libqwen3.so``: functions carry the C
names (``qwen3_init``, ``qwen3_reset``, ``qwen3_forward``, ``qwen3_forward_hidden``,
``qwen3_moe_block``, ...) and only marshal torch tensors (device memory) and the
current HIP stream into the C calls.  Every step of the layer runs in the library's
kernels; there is no Python or CPU fallback, and a missing library raises.
"""
from __future__ import annotations

import atexit
import ctypes
import sys
import weakref

import torch

from . import _lib
from ._lib import BF16, FP32, Qwen3Error
from .config import PRESETS, Qwen3Config

__all__ = ["Qwen3Config", "PRESETS", "Qwen3Error", "Seat", "qwen3_init", "qwen3_reset", "qwen3_forward",
           "qwen3_forward_hidden", "qwen3_moe_block", "qwen3_forward_batch", "qwen3_head", "qwen3_set_length", "qwen3_get_length",
           "qwen3_destroy", "qwen3_workspace_bytes", "qwen3_rope_table", "ops"]

DTYPES = {"bf16": BF16, "fp32": FP32}
TORCH_DTYPES = {BF16: torch.bfloat16, FP32: torch.float32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def c_config(cfg: Qwen3Config, max_tokens: int) -> _lib.Config:
    return _lib.Config(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate,
                       cfg.vocab, cfg.capacity, cfg.rms_eps, cfg.rope_theta, DTYPES[cfg.dtype], cfg.n_experts,
                       cfg.top_k, cfg.moe_intermediate, cfg.norm_topk_prob, cfg.quant_bits, cfg.quant_group,
                       max_tokens, cfg.sliding_window)


def qwen3_workspace_bytes(cfg: Qwen3Config, max_tokens: int) -> int:
    c = c_config(cfg, max_tokens)
    return _lib.load().qwen3_workspace_bytes(ctypes.byref(c))


_live = weakref.WeakSet()  # handles not yet destroyed


def _destroy_all() -> None:
    """Destroy every live handle while the HIP runtime is still up (registered with atexit,
    so it runs before interpreter teardown and before the runtime's own exit handlers):
    the handle's timer events are released by hipEventDestroy, which must not run after
    the runtime has begun to shut down."""
    hs = list(_live)
    if not hs:
        return
    if torch.cuda.is_initialized():
        torch.cuda.synchronize()
    for h in hs:
        h.close()


atexit.register(_destroy_all)


class _Handle:
    """Owns the C handle plus references to every borrowed buffer, so none is freed early."""

    def __init__(self, ptr, cfg, keep):
        self.ptr = ptr
        self.cfg = cfg
        self.keep = keep
        _live.add(self)

    def close(self) -> None:
        if getattr(self, "ptr", None) and _lib._lib is not None:
            _lib._lib.qwen3_destroy(self.ptr)
        self.ptr = None
        _live.discard(self)

    def __del__(self, _finalizing=sys.is_finalizing):
        # during interpreter teardown the atexit hook has already destroyed every handle;
        # make no library call then (module globals may already be gone: the check is bound here)
        if not _finalizing():
            self.close()


def qwen3_init(cfg: Qwen3Config, weights: dict, k_cache: torch.Tensor, v_cache: torch.Tensor,
               max_tokens: int, workspace: torch.Tensor | None = None, stream=None,
               rope: tuple | None = None) -> _Handle:
    """Create a seat.  ``weights``: {"layers": [dict per layer], "final_norm", optional "embed"}
    with the layer keys of ``qwen3.h`` (in_norm, post_norm, q_norm, k_norm, qkv, o, gate_up, down,
    qkv_s, ..., router, exp_gate_up, exp_down).  The workspace is allocated with torch when not given."""
    L = _lib.load()
    c = c_config(cfg, max_tokens)
    need = L.qwen3_workspace_bytes(ctypes.byref(c))
    if need == 0:
        raise Qwen3Error(_lib.ERR_ARG, "invalid configuration")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k_cache.device)
        if stream is not None:
            workspace.record_stream(stream)  # the library's kernels use it on that stream
    if stream is not None and stream != torch.cuda.current_stream():
        # weights, caches and the workspace block may still have writes queued on the current
        # stream (torch reuses freed blocks in stream order); the library's stream waits for them
        stream.wait_stream(torch.cuda.current_stream())
    arr = (_lib.LayerWeights * cfg.n_layers)()
    for i, lw in enumerate(weights["layers"]):
        for name in _lib.LAYER_FIELDS:
            t = lw.get(name)
            if t is None and name in ("qkv", "o", "gate_up", "down", "router", "exp_gate_up", "exp_down"):
                t = lw.get(name + "_q")
            setattr(arr[i], name, None if t is None else t.data_ptr())
    w = _lib.Weights(_ptr(weights.get("embed")), _ptr(weights["final_norm"]),
                     _ptr(rope[0]) if rope else None, _ptr(rope[1]) if rope else None, arr)
    h = ctypes.c_void_p()
    rc = L.qwen3_init(ctypes.byref(c), ctypes.byref(w), _ptr(k_cache), _ptr(v_cache), _ptr(workspace),
                      workspace.numel(), _stream(stream), ctypes.byref(h))
    _lib.check(rc)
    return _Handle(h, cfg, (weights, k_cache, v_cache, workspace, rope, arr))


def qwen3_reset(h: _Handle) -> None:
    _lib.check(_lib.load().qwen3_reset(h.ptr), h.ptr)


def qwen3_forward(h: _Handle, tokens: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    _lib.check(_lib.load().qwen3_forward(h.ptr, _ptr(tokens), tokens.numel(), _ptr(out)), h.ptr)
    return out


def qwen3_forward_hidden(h: _Handle, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    _lib.check(_lib.load().qwen3_forward_hidden(h.ptr, _ptr(x), x.shape[0], _ptr(out)), h.ptr)
    return out


def qwen3_moe_block(h: _Handle, layer: int, x: torch.Tensor, out: torch.Tensor, topk_idx=None, topk_w=None):
    _lib.check(_lib.load().qwen3_moe_block(h.ptr, layer, _ptr(x), x.shape[0], _ptr(out), _ptr(topk_idx),
                                           _ptr(topk_w)), h.ptr)
    return out


def qwen3_forward_batch(handles, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """One decode step for len(handles) seats of the same model: row b of x is seat b's token."""
    arr = (ctypes.c_void_p * len(handles))(*[hd.ptr.value if isinstance(hd.ptr, ctypes.c_void_p) else hd.ptr
                                               for hd in handles])
    _lib.check(_lib.load().qwen3_forward_batch(ctypes.cast(arr, ctypes.c_void_p), len(handles), _ptr(x), _ptr(out)),
               handles[0].ptr)
    return out


def qwen3_head(h: _Handle, hs: torch.Tensor, head: torch.Tensor | None = None, logits: torch.Tensor | None = None,
               argmax: torch.Tensor | None = None):
    """Output head + greedy token on final-norm hidden states hs [T][hidden]: logits (fp32 [T][V])
    and/or argmax (int32 [T]); head [V][hidden] or None for the tied embedding table."""
    V = head.shape[0] if head is not None else h.cfg.vocab
    _lib.check(_lib.load().qwen3_head(h.ptr, _ptr(hs), hs.shape[0], _ptr(head), V, _ptr(logits), _ptr(argmax)),
               h.ptr)
    return logits, argmax


def qwen3_set_length(h: _Handle, length: int) -> None:
    _lib.check(_lib.load().qwen3_set_length(h.ptr, length), h.ptr)


def qwen3_get_length(h: _Handle) -> int:
    return _lib.load().qwen3_get_length(h.ptr)


def qwen3_set_stream(h: _Handle, stream=None) -> None:
    _lib.check(_lib.load().qwen3_set_stream(h.ptr, _stream(stream)), h.ptr)


def qwen3_check_device_errors(h: _Handle) -> None:
    _lib.check(_lib.load().qwen3_check_device_errors(h.ptr), h.ptr)


def qwen3_set_decode_path(h: _Handle, path: int) -> None:
    """0: automatic, 1: one kernel per step of the layer, 2: the persistent decode kernel."""
    _lib.check(_lib.load().qwen3_set_decode_path(h.ptr, path), h.ptr)


def qwen3_get_decode_path(h: _Handle) -> int:
    return _lib.load().qwen3_get_decode_path(h.ptr)


def qwen3_destroy(h: _Handle) -> None:
    _lib.load()
    h.close()


def qwen3_rope_table(capacity: int, head_dim: int, theta: float, dtype: str, device="cuda", stream=None):
    dt = DTYPES[dtype]
    c = torch.empty((capacity, head_dim), dtype=TORCH_DTYPES[dt], device=device)
    s = torch.empty_like(c)
    _lib.check(_lib.load().qwen3_rope_table(capacity, head_dim, theta, dt, _ptr(c), _ptr(s), _stream(stream)))
    return c, s


class Seat:
    """Convenience wrapper: one seat with its KV cache, output buffers and handle."""

    def __init__(self, cfg: Qwen3Config, weights: dict, max_tokens: int, k_cache=None, v_cache=None,
                 device="cuda", stream=None):
        dt = TORCH_DTYPES[DTYPES[cfg.dtype]]
        shape = (cfg.n_layers, cfg.n_kv_heads, cfg.capacity, cfg.head_dim)
        self.cfg = cfg
        self.k = k_cache if k_cache is not None else torch.zeros(shape, dtype=dt, device=device)
        self.v = v_cache if v_cache is not None else torch.zeros(shape, dtype=dt, device=device)
        self.handle = qwen3_init(cfg, weights, self.k, self.v, max_tokens, stream=stream)
        self.dtype = dt

    def forward_hidden(self, x, out=None):
        out = out if out is not None else torch.empty((x.shape[0], self.cfg.hidden), dtype=self.dtype,
                                                      device=x.device)
        return qwen3_forward_hidden(self.handle, x, out)

    def forward(self, tokens, out=None):
        out = out if out is not None else torch.empty((tokens.numel(), self.cfg.hidden), dtype=self.dtype,
                                                      device=tokens.device)
        return qwen3_forward(self.handle, tokens, out)

    def moe_block(self, layer, x, out=None, topk_idx=None, topk_w=None):
        out = out if out is not None else torch.empty_like(x)
        return qwen3_moe_block(self.handle, layer, x, out, topk_idx, topk_w)

    def reset(self):
        qwen3_reset(self.handle)

    @property
    def length(self) -> int:
        return qwen3_get_length(self.handle)

    @length.setter
    def length(self, n: int) -> None:
        qwen3_set_length(self.handle, n)


from . import ops  # noqa: E402  (single-kernel entry points)
