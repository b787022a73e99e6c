"""Pins for the oracle's bf16 rounding points.

The fp32 mode of each oracle function is pinned elsewhere against float64 library
routines.  Here the placement of the model-dtype roundings is pinned:

- functions whose bf16 result is their fp32 result rounded once ("maya2_mlx/backbone.py",
  Backbone._rope: fp32 maths on the bf16 table, one rounding; module docstring: fp32
  softmax attention, one rounding) must equal rho(fp32 mode) bit for bit on bf16 inputs;
- SwiGLU rounds twice (SiLU in fp32 rounded once, then the model-dtype product with the up
  half), pinned against an independent torch statement;
- the whole dense stack (Backbone.forward) and the MoE block ("@mlx-bun/inference"
  qwen3-moe.ts, Qwen3MoeSparseMoeBlock.forward) in bf16 against the independent torch
  statement in tests/page_ref.py.

Each comparison also checks that the inputs can tell one rounding more or fewer apart, so
a dropped or added rounding in the oracle fails here.
"""
import numpy as np
import pytest
import torch

import page_ref


def bf(a):
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def ordered(a):
    """bf16 values as integers in order (adjacent bf16 numbers differ by 1)."""
    u = (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.int64)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def ulps(a, b):
    return np.abs(ordered(a) - ordered(b))


def is_bf16(a):
    return np.all((np.asarray(a, np.float32).view(np.uint32) & 0xFFFF) == 0)


# ------------------------------------------------------------------ RoPE: one rounding

@pytest.mark.parametrize("D,theta", [(64, 1e6), (128, 1e6), (128, 1e7)])
def test_rope_bf16_is_fp32_rotation_rounded_once(orc, D, theta):
    rng = np.random.default_rng(100 + D)
    c, s = orc.rope_table(4096, D, theta, "bf16")
    x = bf(rng.standard_normal((64, D)) * 2)
    for p in (1, 7, 100, 2047, 4095):
        got = orc.rope(x, c[p], s[p], "bf16")
        once = bf(orc.rope(x, c[p], s[p], "fp32"))
        assert np.array_equal(got, once), p
        # power: rounding each product before the difference changes some results
        half = D // 2
        x1, x2 = x[:, :half], x[:, half:]
        per_product = bf(np.concatenate([bf(x1 * c[p, :half]) - bf(x2 * s[p, :half]),
                                         bf(x2 * c[p, half:]) + bf(x1 * s[p, half:])], -1))
        assert np.mean(per_product != once) > 0.05


def test_rope_table_matches_independent_statement(orc):
    for D, theta, mode in ((128, 1e6, "bf16"), (64, 1e7, "bf16"), (128, 1e6, "fp32")):
        c, s = orc.rope_table(8192, D, theta, mode)
        rc, rs = page_ref.rope_table(8192, D, theta, mode)
        assert np.array_equal(c, rc.numpy()) and np.array_equal(s, rs.numpy()), (D, theta, mode)


# ------------------------------------------------------------------ attention: one rounding

@pytest.mark.parametrize("T,H,KV,D,p0,window", [(1, 4, 2, 64, 40, 0), (5, 8, 2, 32, 11, 0), (7, 4, 4, 16, 0, 0),
                                                (3, 16, 8, 128, 200, 0), (6, 4, 1, 32, 30, 9)])
def test_attention_bf16_is_fp32_attention_rounded_once(orc, T, H, KV, D, p0, window):
    rng = np.random.default_rng(7 * T + H + D)
    cap = p0 + T + 3
    q = bf(rng.standard_normal((T, H, D)))
    K = np.zeros((KV, cap, D), np.float32)
    V = np.zeros((KV, cap, D), np.float32)
    K[:, : p0 + T] = bf(rng.standard_normal((KV, p0 + T, D)))
    V[:, : p0 + T] = bf(rng.standard_normal((KV, p0 + T, D)))
    got = orc.attention(q, K, V, p0, "bf16", window=window)
    full = orc.attention(q, K, V, p0, "fp32", window=window)
    assert is_bf16(got)
    assert np.array_equal(got, bf(full))
    # power: the fp32 outputs of queries that see two or more keys are mostly not bf16
    # values, so a missing final rounding shows
    many = (p0 + np.arange(T) >= 1)
    assert np.mean(full[many] != bf(full[many])) > 0.9


def test_attention_bf16_against_independent_statement(orc):
    """fp32 softmax over bf16 scores inputs, never rounding the probabilities."""
    rng = np.random.default_rng(5)
    T, H, KV, D, p0 = 4, 4, 2, 64, 60
    cap = p0 + T
    q = bf(rng.standard_normal((T, H, D)) * 3)
    K = bf(rng.standard_normal((KV, cap, D)))
    V = bf(rng.standard_normal((KV, cap, D)))
    got = orc.attention(q, K, V, p0, "bf16").reshape(T, H, D)
    md = page_ref.ModelDtype("bf16")
    want = np.stack([np.stack([md.attention_row(torch.from_numpy(q[t, h]), torch.from_numpy(K[h // 2, : p0 + t + 1]),
                                                torch.from_numpy(V[h // 2, : p0 + t + 1]), D ** -0.5).numpy()
                               for h in range(H)]) for t in range(T)])
    assert ulps(got, want).max() <= 1 and np.mean(got == want) > 0.99
    # power: rounding the probabilities to bf16 before the product with V moves many outputs
    pr = np.stack([np.stack([bf(torch.softmax((torch.from_numpy(K[h // 2, : p0 + t + 1]).double()
                                               @ torch.from_numpy(q[t, h]).double()).float() * np.float32(D ** -0.5),
                                              0).numpy()) @ V[h // 2, : p0 + t + 1].astype(np.float64)
                             for h in range(H)]) for t in range(T)])
    assert np.mean(bf(pr) != want) > 0.2


# ------------------------------------------------------------------ SwiGLU: two roundings

def test_swiglu_bf16_rounds_silu_then_product(orc):
    rng = np.random.default_rng(31)
    I = 4096
    g = bf(rng.standard_normal((4, I)) * 3)
    u = bf(rng.standard_normal((4, I)) * 3)
    got = orc.swiglu(np.concatenate([g, u], -1), "bf16")
    want = page_ref.ModelDtype("bf16").silu_times_up(torch.from_numpy(g), torch.from_numpy(u)).numpy()
    assert is_bf16(got)
    assert ulps(got, want).max() <= 1 and np.mean(got == want) > 0.999
    # power: one rounding fewer (SiLU kept in fp32) or more (the gate rounded after SiLU's
    # division only) changes a clear share of the outputs
    silu32 = torch.from_numpy(g) / (1.0 + torch.exp(-torch.from_numpy(g)))
    once = bf((silu32 * torch.from_numpy(u)).numpy())
    assert np.mean(once != want) > 0.05


# ------------------------------------------------------------------ whole dense stack

def _stack_pair(orc, cfg, w):
    cos, sin = page_ref.rope_table(cfg.capacity, cfg.head_dim, cfg.rope_theta, cfg.dtype)
    ref = page_ref.PageStack(cfg, w, cos, sin, cfg.dtype)
    layers = [{k: v.float().numpy() for k, v in L.items()} for L in w["layers"]]
    st = orc.Stack(cfg, layers, w["final_norm"].float().numpy(), cfg.dtype)
    return st, ref


def test_stack_bf16_matches_independent_statement(orc):
    """Backbone.forward in bf16, two layers: a 16-token prefill then 8 decode steps; every
    output and every cache entry agrees with the torch statement of the page's roundings."""
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(dtype="bf16")
    w = synth.model_weights(cfg)
    x = synth.hidden_states(cfg, 24).float()
    st, ref = _stack_pair(orc, cfg, w)
    got = np.concatenate([st.forward(x[:16].numpy())] + [st.forward(x[i:i + 1].numpy()) for i in range(16, 24)])
    want = torch.cat([ref.forward(x[:16])] + [ref.forward(x[i:i + 1]) for i in range(16, 24)]).numpy()
    d = ulps(got, want)
    assert is_bf16(got)
    assert d.max() <= 1 and np.mean(d == 0) > 0.99, (d.max(), np.mean(d == 0))
    dk = ulps(st.k[:, :, :24], ref.K[:, :, :24].numpy())
    dv = ulps(st.v[:, :, :24], ref.V[:, :, :24].numpy())
    assert dk.max() <= 1 and dv.max() <= 1 and np.mean(dk == 0) > 0.99 and np.mean(dv == 0) > 0.99


# ------------------------------------------------------------------ MoE block

def test_moe_block_bf16_matches_independent_statement(orc):
    rng = np.random.default_rng(41)
    T, hid, E, Ie, k = 12, 128, 16, 64, 4
    y2 = bf(rng.standard_normal((T, hid)))
    Wr = bf(rng.standard_normal((E, hid)) * 0.3)
    Wgu = bf(rng.standard_normal((E, 2 * Ie, hid)) * 0.1)
    Wd = bf(rng.standard_normal((E, hid, Ie)) * 0.1)
    out, idx, w = orc.moe_block(y2, Wr, Wgu, Wd, k, True, False, "bf16")
    rout, ridx, rw = page_ref.moe_block(*(torch.from_numpy(a) for a in (y2, Wr, Wgu, Wd)), k, "bf16")
    assert np.array_equal(idx, ridx.numpy())
    assert np.array_equal(w, rw.numpy())
    d = ulps(out, rout.numpy())
    assert d.max() <= 1 and np.mean(d == 0) > 0.99


# ------------------------------------------------------------------ 8-bit weights: no rounding of w

def test_q8_dequant_is_fp32_not_model_dtype(orc):
    """The dequantised weight s*q + b stays an fp32 value (the affine form is evaluated in
    fp32 from the bf16 scale and bias and never rounded to bf16): each value is within two
    fp32 roundings of the exact s*q + b, and most are not bf16 values."""
    rng = np.random.default_rng(51)
    N, K, g = 16, 256, 64
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)
    s = bf(3.8e-4 * (1 + 0.1 * rng.standard_normal((N, K // g))))
    b = bf(-127.5 * s * (1 + 0.05 * rng.standard_normal((N, K // g))))
    wh = orc.q8_dequant(q, s, b, g)
    exact = np.repeat(s, g, 1).astype(np.float64) * q + np.repeat(b, g, 1).astype(np.float64)
    assert np.all(np.abs(wh - exact) <= 2 * np.spacing(np.abs(exact).astype(np.float32)) + 1e-30)
    assert np.mean(wh != bf(wh)) > 0.5
