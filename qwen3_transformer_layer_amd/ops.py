"""Single-kernel entry points (include/qwen3_ops.h) for per-kernel parity tests.

Argument marshalling only: torch device tensors in, the library's kernel out.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import BF16, FP32

EPI_STORE, EPI_RESID, EPI_SWIGLU = 0, 1, 2


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def add_rmsnorm(h_in, w, eps, res=None, h_out=None):
    _contig(h_in, w, res, h_out)
    T, n = h_in.shape
    y = torch.empty_like(h_in)
    _lib.check(_lib.load().qwen3_op_add_rmsnorm(_dt(h_in), _p(h_in), _p(res), _p(w), _p(h_out), _p(y), T, n, eps,
                                                 _s()))
    return y


def stream_read(buf):
    """Streaming-read probe over a contiguous device tensor (its byte size a multiple of 16):
    returns the 65536 per-thread XOR words (uint32 values in an int32 tensor)."""
    _contig(buf)
    out = torch.empty(256 * 256, dtype=torch.int32, device=buf.device)
    _lib.check(_lib.load().qwen3_op_stream_read(_p(buf), buf.numel() * buf.element_size(), _p(out), _s()))
    return out


def linear(x, W, epilogue=EPI_STORE, res=None):
    _contig(x, W, res)
    M, K = x.shape
    N = W.shape[0] // 2 if epilogue == EPI_SWIGLU else W.shape[0]
    out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _lib.check(_lib.load().qwen3_op_linear(_dt(x), _p(x), M, K, _p(W), N, epilogue, _p(res), _p(out), _s()))
    return out


def linear_q8(x, codes, scale, bias, epilogue=EPI_STORE, res=None):
    _contig(x, codes, scale, bias, res)
    M, K = x.shape
    N = codes.shape[0] // 2 if epilogue == EPI_SWIGLU else codes.shape[0]
    out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _lib.check(_lib.load().qwen3_op_linear_q8(_p(x), M, K, _p(codes), _p(scale), _p(bias), N, epilogue, _p(res),
                                               _p(out), _s()))
    return out


def qknorm_rope_kv(qkv, H, KV, D, q_norm, k_norm, eps, cos_t, sin_t, p0, k_cache, v_cache):
    """qkv [T][(H+2KV)D]; caches [KV][cap][D] updated in place; returns q [T][H][D]."""
    _contig(qkv, q_norm, k_norm, cos_t, sin_t, k_cache, v_cache)
    T = qkv.shape[0]
    cap = k_cache.shape[1]
    q = torch.empty((T, H, D), dtype=qkv.dtype, device=qkv.device)
    _lib.check(_lib.load().qwen3_op_qknorm_rope_kv(_dt(qkv), _p(qkv), T, H, KV, D, _p(q_norm), _p(k_norm), eps,
                                                    _p(cos_t), _p(sin_t), p0, cap, _p(q), _p(k_cache), _p(v_cache),
                                                    _s()))
    return q


def attention(q, k_cache, v_cache, p0):
    """q [T][H][D]; caches [KV][cap][D]; returns [T][H*D]."""
    _contig(q, k_cache, v_cache)
    T, H, D = q.shape
    KV, cap, _ = k_cache.shape
    L = _lib.load()
    nbytes = L.qwen3_op_attention_workspace(T, H, KV, D, cap)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty((T, H * D), dtype=q.dtype, device=q.device)
    _lib.check(L.qwen3_op_attention(_dt(q), _p(q), _p(k_cache), _p(v_cache), T, H, KV, D, cap, p0, _p(out), _p(ws),
                                    ws.numel(), _s()))
    return out


def moe(x, router, exp_gate_up, exp_down, k, norm=True):
    """Returns (out [T][hid], idx int32 [T][k], w [T][k])."""
    _contig(x, router, exp_gate_up, exp_down)
    T, hid = x.shape
    E = router.shape[0]
    Ie = exp_gate_up.shape[1] // 2
    L = _lib.load()
    dt = _dt(x)
    nbytes = L.qwen3_op_moe_workspace(dt, T, hid, E, k, Ie)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=x.dtype, device=x.device)
    out = torch.empty_like(x)
    _lib.check(L.qwen3_op_moe(dt, _p(x), T, hid, _p(router), E, k, int(bool(norm)), Ie, _p(exp_gate_up),
                              _p(exp_down), _p(idx), _p(w), _p(out), _p(ws), ws.numel(), _s()))
    return out, idx, w
