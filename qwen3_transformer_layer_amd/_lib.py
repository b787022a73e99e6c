"""ctypes declarations of libqwen3.so (include/qwen3.h and include/qwen3_ops.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqwen3.so")

BF16, FP32 = 0, 1
OK = 0
ERR = {-1: "QWEN3_ERR_ARG", -2: "QWEN3_ERR_DTYPE", -3: "QWEN3_ERR_CAPACITY", -4: "QWEN3_ERR_NULL_WEIGHT",
       -5: "QWEN3_ERR_UNSUPPORTED", -6: "QWEN3_ERR_HIP", -7: "QWEN3_ERR_WORKSPACE"}
ERR_ARG, ERR_DTYPE, ERR_CAPACITY, ERR_NULL_WEIGHT, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = -1, -2, -3, -4, -5, -6, -7

_P = ctypes.c_void_p
_I = ctypes.c_int


class Config(ctypes.Structure):
    _fields_ = [(n, _I) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate",
                                  "vocab", "capacity")] + \
               [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double), ("dtype", _I)] + \
               [(n, _I) for n in ("n_experts", "top_k", "moe_intermediate", "norm_topk_prob", "quant_bits",
                                  "quant_group", "max_tokens", "sliding_window")]


LAYER_FIELDS = ("in_norm", "post_norm", "q_norm", "k_norm", "qkv", "o", "gate_up", "down", "qkv_s", "qkv_b", "o_s",
                "o_b", "gate_up_s", "gate_up_b", "down_s", "down_b", "router", "exp_gate_up", "exp_down",
                "router_s", "router_b", "exp_gate_up_s", "exp_gate_up_b", "exp_down_s", "exp_down_b", "qkv_bias")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("rope_cos", _P), ("rope_sin", _P),
                ("layers", ctypes.POINTER(LayerWeights))]


class Qwen3Error(RuntimeError):
    def __init__(self, code: int, msg: str = ""):
        self.code = code
        super().__init__(f"{ERR.get(code, code)}: {msg}" if msg else ERR.get(code, str(code)))


_lib = None


def load():
    """Load libqwen3.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with qwen3_transformer_layer_amd.build.build() "
                          "(the HIP kernels are the only implementation)")
    L = ctypes.CDLL(LIB_PATH)
    sz, H = ctypes.c_size_t, _P
    sig = {
        "qwen3_workspace_bytes": (sz, [ctypes.POINTER(Config)]),
        "qwen3_init": (_I, [ctypes.POINTER(Config), ctypes.POINTER(Weights), _P, _P, _P, sz, _P, ctypes.POINTER(H)]),
        "qwen3_reset": (_I, [H]),
        "qwen3_forward": (_I, [H, _P, _I, _P]),
        "qwen3_forward_hidden": (_I, [H, _P, _I, _P]),
        "qwen3_moe_block": (_I, [H, _I, _P, _I, _P, _P, _P]),
        "qwen3_head": (_I, [H, _P, _I, _P, _I, _P, _P]),
        "qwen3_forward_batch": (_I, [_P, _I, _P, _P]),
        "qwen3_head_static": (_I, [_I, _P, _I, _I, _P, _I, _P, _P, _P]),
        "qwen3_set_length": (_I, [H, _I]),
        "qwen3_get_length": (_I, [H]),
        "qwen3_set_stream": (_I, [H, _P]),
        "qwen3_check_device_errors": (_I, [H]),
        "qwen3_set_decode_path": (_I, [H, _I]),
        "qwen3_get_decode_path": (_I, [H]),
        "qwen3_last_error": (ctypes.c_char_p, [H]),
        "qwen3_status_string": (ctypes.c_char_p, [_I]),
        "qwen3_destroy": (None, [H]),
        "qwen3_rope_table": (_I, [_I, _I, ctypes.c_double, _I, _P, _P, _P]),
        "qwen3_op_add_rmsnorm": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, ctypes.c_float, _P]),
        "qwen3_op_stream_read": (_I, [_P, ctypes.c_size_t, _P, _P]),
        "qwen3_op_linear": (_I, [_I, _P, _I, _I, _P, _I, _I, _P, _P, _P]),
        "qwen3_op_linear_q8": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P]),
        "qwen3_op_qknorm_rope_kv": (_I, [_I, _P, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _P, _I, _I, _P, _P, _P,
                                         _P]),
        "qwen3_op_attention_workspace": (sz, [_I, _I, _I, _I, _I]),
        "qwen3_op_attention": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, sz, _P]),
        "qwen3_op_moe_workspace": (sz, [_I, _I, _I, _I, _I, _I]),
        "qwen3_kernel_timer": (_I, [H, _I, _I]),
        "qwen3_kernel_timer_read": (_I, [H, _I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I)]),
        "qwen3_op_moe": (_I, [_I, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, sz, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(code: int, handle=None) -> None:
    if code != OK:
        msg = ""
        if handle is not None and _lib is not None:
            msg = (_lib.qwen3_last_error(handle) or b"").decode()
        raise Qwen3Error(code, msg)
