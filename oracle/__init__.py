"""CPU oracle for the Qwen3 decoder-layer path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this module.  The GPU library never imports, links or calls it.

This is a thin ctypes/numpy wrapper around ``liboracle.so`` (plain C++ built
from ``oracle.cpp``); every function documents the page passage it restates in
``oracle.h``.  All arrays are float32 numpy arrays; in bf16 mode they hold
bf16-representable values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

BF16 = 0
FP32 = 1
MODES = {"bf16": BF16, "fp32": FP32}

ERR_ARG, ERR_CAPACITY, ERR_MODE = -1, -2, -3

_lib = None


def build() -> str:
    """Compile liboracle.so with g++ (strict IEEE: no contraction, no fast-math)."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", os.path.join(HERE, "oracle.cpp"), "-o", LIB_PATH + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim",
                                            "intermediate", "capacity")] + \
               [("rms_eps", ctypes.c_float), ("mode", ctypes.c_int)] + \
               [(n, ctypes.c_int) for n in ("n_experts", "top_k", "moe_intermediate", "norm_topk_prob", "qk_norm",
                                            "attention_bias", "window")]


_P = ctypes.c_void_p


class OrcLayer(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("in_norm", "post_norm", "q_norm", "k_norm", "qkv", "o", "gate_up",
                                  "down", "router", "exp_gate_up", "exp_down", "qkv_bias")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        f, i, p = ctypes.c_float, ctypes.c_int, ctypes.c_void_p
        L.orc_round.restype = f
        L.orc_round.argtypes = [f, i]
        L.orc_round_array.argtypes = [p, ctypes.c_size_t, i]
        L.orc_rmsnorm.argtypes = [p, p, i, f, i, p]
        L.orc_linear.argtypes = [p, i, i, p, i, i, p]
        L.orc_head.argtypes = [p, i, i, p, i, i, p, p]
        L.orc_rope_table.argtypes = [i, i, ctypes.c_double, i, p, p]
        L.orc_rope.argtypes = [p, i, p, p, i, p]
        L.orc_attention.argtypes = [p, p, p, i, i, i, i, i, i, i, i, p, p]
        L.orc_swiglu.argtypes = [p, i, i, i, p]
        L.orc_router.argtypes = [p, i, i, p, i, i, i, i, p, p, p]
        L.orc_moe_block.argtypes = [p, i, i, p, i, i, i, i, p, p, i, i, p, p, p]
        L.orc_q8_dequant.argtypes = [p, p, p, i, i, i, p]
        L.orc_q8_quantize.argtypes = [p, i, i, i, p, p, p]
        L.orc_forward.restype = i
        L.orc_forward.argtypes = [ctypes.POINTER(OrcConfig), ctypes.POINTER(OrcLayer), p, p, p, p, p,
                                  ctypes.POINTER(ctypes.c_int), p, i, p]
        L.orc_set_threads.argtypes = [i]
        L.orc_get_threads.restype = i
        _lib = L
    return _lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return lib().orc_get_threads()


def round_(x, mode="bf16") -> np.ndarray:
    """rho: round to the model dtype (bf16 RNE, or identity in fp32 mode)."""
    y = _f32(x).copy()
    lib().orc_round_array(_ptr(y), y.size, _mode(mode))
    return y


def rmsnorm(v, w, eps, mode="bf16") -> np.ndarray:
    """Row-wise RMSNorm with two roundings over the last axis."""
    v = _f32(v)
    w = _f32(w)
    n = v.shape[-1]
    rows = v.reshape(-1, n)
    out = np.empty_like(rows)
    for r in range(rows.shape[0]):
        lib().orc_rmsnorm(_ptr(rows[r]), _ptr(w), n, float(eps), _mode(mode), _ptr(out[r]))
    return out.reshape(v.shape)


def linear(x, W, mode="bf16") -> np.ndarray:
    """rho(x @ W^T), W [N][K]."""
    x = _f32(x)
    W = _f32(W)
    T, K = x.reshape(-1, x.shape[-1]).shape
    N = W.shape[0]
    assert W.shape[1] == K
    out = np.empty((T, N), np.float32)
    lib().orc_linear(_ptr(x), T, K, _ptr(W), N, _mode(mode), _ptr(out))
    return out.reshape(x.shape[:-1] + (N,))


def head(hs, W, mode="bf16"):
    """(logits fp32 [T][V] = rho(hs @ W^T), argmax int32 [T]: lowest index of the largest)."""
    hs = _f32(hs)
    W = _f32(W)
    T, K = hs.reshape(-1, hs.shape[-1]).shape
    V = W.shape[0]
    assert W.shape[1] == K
    logits = np.empty((T, V), np.float32)
    am = np.empty(T, np.int32)
    lib().orc_head(_ptr(hs), T, K, _ptr(W), V, _mode(mode), _ptr(logits), am.ctypes.data_as(ctypes.c_void_p))
    return logits, am


def rope_table(capacity, head_dim, theta, mode="bf16"):
    """(cos, sin), each [capacity][head_dim], halves duplicated."""
    c = np.empty((capacity, head_dim), np.float32)
    s = np.empty((capacity, head_dim), np.float32)
    lib().orc_rope_table(capacity, head_dim, float(theta), _mode(mode), _ptr(c), _ptr(s))
    return c, s


def rope(x, cos_row, sin_row, mode="bf16") -> np.ndarray:
    """Rotate-half RoPE of one or more head vectors at one position."""
    x = _f32(x)
    D = x.shape[-1]
    rows = x.reshape(-1, D)
    out = np.empty_like(rows)
    c, s = _f32(cos_row), _f32(sin_row)
    for r in range(rows.shape[0]):
        lib().orc_rope(_ptr(rows[r]), D, _ptr(c), _ptr(s), _mode(mode), _ptr(out[r]))
    return out.reshape(x.shape)


def attention(q, K, V, p0, mode="bf16", want_probs=False, window=0):
    """q [T][H][D]; K, V [KV][cap][D]; returns a [T][H*D] (and probs [T][H][p0+T]).
    window > 0: each query sees only the `window` most recent positions up to its own."""
    q, K, V = _f32(q), _f32(K), _f32(V)
    T, H, D = q.shape
    KV, cap, D2 = K.shape
    assert D2 == D and V.shape == K.shape and p0 + T <= cap
    out = np.empty((T, H * D), np.float32)
    probs = np.empty((T, H, p0 + T), np.float32) if want_probs else None
    lib().orc_attention(_ptr(q), _ptr(K), _ptr(V), T, H, KV, D, cap, int(p0), int(window), _mode(mode), _ptr(out),
                        _ptr(probs))
    return (out, probs) if want_probs else out


def swiglu(gu, mode="bf16") -> np.ndarray:
    gu = _f32(gu)
    T, I2 = gu.reshape(-1, gu.shape[-1]).shape
    out = np.empty((T, I2 // 2), np.float32)
    lib().orc_swiglu(_ptr(gu), T, I2 // 2, _mode(mode), _ptr(out))
    return out


def router(y2, Wr, k, norm=True, mode="bf16"):
    """(idx int32 [T][k], w [T][k], probs [T][E])."""
    y2, Wr = _f32(y2), _f32(Wr)
    T, hid = y2.shape
    E = Wr.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    probs = np.empty((T, E), np.float32)
    lib().orc_router(_ptr(y2), T, hid, _ptr(Wr), E, k, int(bool(norm)), _mode(mode), _ptr(idx), _ptr(w),
                     _ptr(probs))
    return idx, w, probs


def moe_block(y2, Wr, Wgu_e, Wd_e, k, norm=True, sorted_order=False, mode="bf16"):
    """(out [T][hid], idx [T][k], w [T][k])."""
    y2, Wr, Wgu_e, Wd_e = _f32(y2), _f32(Wr), _f32(Wgu_e), _f32(Wd_e)
    T, hid = y2.shape
    E, I2, hid2 = Wgu_e.shape
    assert hid2 == hid and Wd_e.shape == (E, hid, I2 // 2) and Wr.shape == (E, hid)
    out = np.empty((T, hid), np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().orc_moe_block(_ptr(y2), T, hid, _ptr(Wr), E, k, I2 // 2, int(bool(norm)), _ptr(Wgu_e), _ptr(Wd_e),
                        int(bool(sorted_order)), _mode(mode), _ptr(out), _ptr(idx), _ptr(w))
    return out, idx, w


def q8_dequant(q, s, b, group=64) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s, b = _f32(s), _f32(b)
    N, K = q.shape
    out = np.empty((N, K), np.float32)
    lib().orc_q8_dequant(_ptr(q), _ptr(s), _ptr(b), N, K, group, _ptr(out))
    return out


def q8_quantize(w, group=64):
    w = _f32(w)
    N, K = w.shape
    q = np.empty((N, K), np.uint8)
    s = np.empty((N, K // group), np.float32)
    b = np.empty((N, K // group), np.float32)
    lib().orc_q8_quantize(_ptr(w), N, K, group, _ptr(q), _ptr(s), _ptr(b))
    return q, s, b


class Stack:
    """The oracle's view of one seat: config, host fp32 weights, K/V cache and length.

    ``layers`` is a list of dicts with keys in_norm, post_norm, q_norm, k_norm, qkv, o,
    gate_up, down (dense) or router, exp_gate_up, exp_down (MoE), as float32 arrays.
    """

    def __init__(self, cfg, layers, final_norm, mode, cos=None, sin=None, kcache=None, vcache=None):
        self.cfg = cfg
        self.mode = _mode(mode)
        self.layers = [{k: (None if v is None else _f32(v)) for k, v in L.items()} for L in layers]
        self.final_norm = _f32(final_norm)
        L, KV, cap, D = cfg.n_layers, cfg.n_kv_heads, cfg.capacity, cfg.head_dim
        if cos is None:
            cos, sin = rope_table(cap, D, cfg.rope_theta, self.mode)
        self.cos, self.sin = _f32(cos), _f32(sin)
        self.k = _f32(kcache) if kcache is not None else np.zeros((L, KV, cap, D), np.float32)
        self.v = _f32(vcache) if vcache is not None else np.zeros((L, KV, cap, D), np.float32)
        self.length = 0
        self._c = OrcConfig(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                            cfg.intermediate, cfg.capacity, cfg.rms_eps, self.mode, cfg.n_experts, cfg.top_k,
                            cfg.moe_intermediate, cfg.norm_topk_prob, int(bool(cfg.qk_norm)),
                            int(bool(cfg.attention_bias)), cfg.sliding_window)
        arr = (OrcLayer * cfg.n_layers)()
        for i, Ld in enumerate(self.layers):
            for name, _ in OrcLayer._fields_:
                setattr(arr[i], name, _ptr(Ld.get(name)))
        self._layers = arr

    def reset(self):
        self.k[...] = 0
        self.v[...] = 0
        self.length = 0

    def forward(self, x) -> np.ndarray:
        x = _f32(x)
        T = x.shape[0]
        out = np.empty((T, self.cfg.hidden), np.float32)
        n = ctypes.c_int(self.length)
        rc = lib().orc_forward(ctypes.byref(self._c), self._layers, _ptr(self.final_norm), _ptr(self.cos),
                               _ptr(self.sin), _ptr(self.k), _ptr(self.v), ctypes.byref(n), _ptr(x), T, _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle forward failed with code {rc}")
        self.length = n.value
        return out
