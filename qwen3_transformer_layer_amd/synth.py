"""Seeded synthetic inputs: random-init weights, pre-filled K/V caches, hidden states, token ids.

This module only draws numbers; it performs none of the layer's arithmetic.  It is
the one piece of code shared by the GPU path's tests and the CPU oracle's tests,
so both sides see byte-identical inputs.

Every tensor gets its own generator, seeded with FNV-1a-64 of
"{config seed}/{tensor name}" (low 63 bits), and is drawn as float32 normals:
linear weights 0.02*z, norm weights 1 + 0.1*z, q/k/v biases 0.5*z, K/V pre-fill and
hidden states z,
then cast (round-to-nearest-even) to the model dtype.  8-bit quantised
projections are drawn directly in their stored form: codes around 127.5 with
spread 42.5, per-group scales near 3.8e-4 and biases near -127.5*scale, which is
what an affine 8-bit quantiser gives for N(0, 0.02) weights in groups of 64.
"""
from __future__ import annotations

import torch

from .config import Qwen3Config


def fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for b in text.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def tensor_seed(cfg: Qwen3Config, name: str) -> int:
    return fnv1a64(f"{cfg.seed}/{name}") & ((1 << 63) - 1)


def _gen(cfg, name, device):
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(cfg, name))
    return g


def randn(cfg: Qwen3Config, name: str, shape, device="cpu") -> torch.Tensor:
    return torch.randn(tuple(shape), generator=_gen(cfg, name, device), device=device, dtype=torch.float32)


def model_dtype(cfg: Qwen3Config) -> torch.dtype:
    if cfg.dtype == "bf16":
        return torch.bfloat16
    if cfg.dtype == "fp32":
        return torch.float32
    raise ValueError(f"unsupported model dtype {cfg.dtype!r}")


def linear_weight(cfg, name, shape, device="cpu"):
    return (0.02 * randn(cfg, name, shape, device)).to(model_dtype(cfg))


def norm_weight(cfg, name, n, device="cpu"):
    return (1.0 + 0.1 * randn(cfg, name, (n,), device)).to(model_dtype(cfg))


def q8_weight(cfg, name, rows, cols, device="cpu"):
    """(codes u8 [rows][cols], scale bf16 [rows][cols/g], bias bf16 [rows][cols/g])."""
    g = cfg.quant_group
    z = randn(cfg, name + ".codes", (rows, cols), device)
    codes = torch.clamp(torch.round(127.5 + 42.5 * z), 0, 255).to(torch.uint8)
    zs = randn(cfg, name + ".scale", (rows, cols // g), device)
    scale = (3.8e-4 * (1.0 + 0.1 * zs)).to(torch.bfloat16)
    zb = randn(cfg, name + ".bias", (rows, cols // g), device)
    bias = (-127.5 * scale.float() * (1.0 + 0.05 * zb)).to(torch.bfloat16)
    return codes, scale, bias


PROJ_SHAPES = ("qkv", "o", "gate_up", "down")


def proj_shape(cfg: Qwen3Config, name: str):
    hid, HD, I = cfg.hidden, cfg.n_heads * cfg.head_dim, cfg.intermediate
    return {"qkv": (cfg.qkv_rows, hid), "o": (hid, HD), "gate_up": (2 * I, hid), "down": (hid, I)}[name]


def layer_weights(cfg: Qwen3Config, layer: int, device="cpu") -> dict:
    """One layer's weights in the library's layout (row-major [out][in]; q|k|v and
    gate|up rows fused, gate rows first)."""
    p = f"layers.{layer}."
    hid, D = cfg.hidden, cfg.head_dim
    w = {
        "in_norm": norm_weight(cfg, p + "in_norm", hid, device),
        "post_norm": norm_weight(cfg, p + "post_norm", hid, device),
    }
    if cfg.qk_norm:
        w["q_norm"] = norm_weight(cfg, p + "q_norm", D, device)
        w["k_norm"] = norm_weight(cfg, p + "k_norm", D, device)
    if cfg.attention_bias:  # N(0, 0.5): the size of a projection output at hidden ~ 1000
        w["qkv_bias"] = (0.5 * randn(cfg, p + "qkv_bias", (cfg.qkv_rows,), device)).to(model_dtype(cfg))
    moe_layer = cfg.is_moe_layer(layer)
    names = ("qkv", "o") if moe_layer else PROJ_SHAPES
    for n in names:
        rows, cols = proj_shape(cfg, n)
        if cfg.quant_bits == 8:
            w[n + "_q"], w[n + "_s"], w[n + "_b"] = q8_weight(cfg, p + n, rows, cols, device)
        else:
            w[n] = linear_weight(cfg, p + n, (rows, cols), device)
    if moe_layer:
        E, Ie = cfg.n_experts, cfg.moe_intermediate
        shapes = {"router": (E, hid), "exp_gate_up": (E, 2 * Ie, hid), "exp_down": (E, hid, Ie)}
        for n, shape in shapes.items():
            if cfg.quant_bits == 8:  # stacked experts: groups of 64 along each row's input axis
                rows = shape[0] * (shape[1] if len(shape) == 3 else 1)
                q, sc, bi = q8_weight(cfg, p + n, rows, shape[-1], device)
                w[n + "_q"] = q.reshape(shape)
                w[n + "_s"] = sc.reshape(shape[:-1] + (shape[-1] // cfg.quant_group,))
                w[n + "_b"] = bi.reshape(shape[:-1] + (shape[-1] // cfg.quant_group,))
            else:
                w[n] = linear_weight(cfg, p + n, shape, device)
    return w


def model_weights(cfg: Qwen3Config, device="cpu", n_layers: int | None = None) -> dict:
    n = cfg.n_layers if n_layers is None else n_layers
    out = {"layers": [layer_weights(cfg, l, device) for l in range(n)],
           "final_norm": norm_weight(cfg, "final_norm", cfg.hidden, device)}
    if cfg.vocab:
        out["embed"] = linear_weight(cfg, "embed", (cfg.vocab, cfg.hidden), device)
    return out


def kv_cache(cfg: Qwen3Config, filled: int, device="cpu", n_layers: int | None = None):
    """K, V [L][KV][capacity][D]: N(0,1) at positions < filled, zeros after."""
    n = cfg.n_layers if n_layers is None else n_layers
    shape = (n, cfg.n_kv_heads, cfg.capacity, cfg.head_dim)
    dt = model_dtype(cfg)
    K = torch.zeros(shape, dtype=dt, device=device)
    V = torch.zeros(shape, dtype=dt, device=device)
    if filled:
        for l in range(n):
            sub = (cfg.n_kv_heads, filled, cfg.head_dim)
            K[l, :, :filled] = randn(cfg, f"kcache.{l}", sub, device).to(dt)
            V[l, :, :filled] = randn(cfg, f"vcache.{l}", sub, device).to(dt)
    return K, V


def hidden_states(cfg: Qwen3Config, T: int, device="cpu", name: str = "x"):
    return randn(cfg, name, (T, cfg.hidden), device).to(model_dtype(cfg))


def token_ids(cfg: Qwen3Config, n: int, device="cpu", name: str = "tokens"):
    return torch.randint(0, cfg.vocab, (n,), generator=_gen(cfg, name, device), device=device,
                         dtype=torch.int32)
