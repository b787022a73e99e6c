"""A second, independent statement of the layer's model-dtype arithmetic, in torch.

Test infrastructure: it pins the oracle's bf16 rounding points.  It is written from the
rounding rules the pages state, not from the oracle's code:

- "maya2_mlx/backbone.py", module docstring and Backbone.forward: every array of the
  model dtype is a bf16 tensor here, so each elementwise op and each matmul on such arrays
  ends in one round-to-nearest-even; the residual adds are "one rounding"; RMSNorm has
  Qwen3's two roundings (the normalised value, then the product with the weight); SiLU is
  evaluated in fp32 on the rounded gate and rounded once; the product with the up half is a
  model-dtype product (one more rounding); attention is an fp32 softmax with one rounding
  of the output.
- same page, Backbone._rope: the rotation is fp32 arithmetic on the bf16 table values,
  rounded once.
- "@mlx-bun/inference" qwen3-moe.ts, Qwen3MoeSparseMoeBlock.forward: router logits,
  softmax output, the renormalising sum and quotient, each expert's matmul outputs, each
  weighted expert output and the slot sum are model-dtype arrays.

Matmuls accumulate exactly (float64 products and sums) and round to fp32, then to the
model dtype: the reading that an fp32-accumulated product is its exact value rounded
once.  Values travel as float32 tensors holding bf16 values; `rb` is torch's own
round-to-nearest-even cast.  In fp32 mode every `rb` is the identity.
"""
from __future__ import annotations

import torch


class ModelDtype:
    """Rounding to the model dtype: bf16 RNE, or nothing in fp32 mode."""

    def __init__(self, mode: str):
        assert mode in ("bf16", "fp32")
        self.mode = mode

    def rb(self, x: torch.Tensor) -> torch.Tensor:
        x = x.to(torch.float32)
        return x.to(torch.bfloat16).to(torch.float32) if self.mode == "bf16" else x

    def matmul(self, x: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
        """rho(x @ W^T), exact accumulation rounded to fp32 first."""
        return self.rb((x.double() @ W.double().T).to(torch.float32))

    def rms_norm(self, v: torch.Tensor, w: torch.Tensor, eps: float) -> torch.Tensor:
        """Rows of v: r = 1/sqrt(mean(v^2) + eps) in fp32; rho(w * rho(v * r))."""
        ms = ((v.double() ** 2).sum(-1, keepdim=True) / v.shape[-1]).to(torch.float32)
        r = torch.ones_like(ms) / torch.sqrt(ms + torch.tensor(eps, dtype=torch.float32))
        return self.rb(w * self.rb(v * r))

    def rope(self, x: torch.Tensor, c: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
        """Rotate-half RoPE of head vectors x [..., D] with table rows c, s [D] (fp32 maths)."""
        half = x.shape[-1] // 2
        a, b = x[..., :half], x[..., half:]
        first = a * c[:half] - b * s[:half]
        second = b * c[half:] + a * s[half:]
        return self.rb(torch.cat([first, second], -1))

    def attention_row(self, q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, scale: float) -> torch.Tensor:
        """One query q [D] against keys K [n][D], values V [n][D]: fp32 softmax, one rounding."""
        sc = (K.double() @ q.double()).to(torch.float32) * torch.tensor(scale, dtype=torch.float32)
        p = torch.softmax(sc, 0)
        return self.rb((p.double() @ V.double()).to(torch.float32))

    def silu_times_up(self, g: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
        """rho(rho(silu(g)) * u), SiLU as g / (1 + exp(-g)) in fp32."""
        act = self.rb(g / (1.0 + torch.exp(-g)))
        return self.rb(act * u)

    def add(self, a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
        return self.rb(a + b)


class PageStack:
    """One seat of the dense decoder stack: weights (float32 tensors of model-dtype values,
    layouts [out][in], q|k|v and gate|up rows fused), a K/V cache per layer and a length."""

    def __init__(self, cfg, weights: dict, cos: torch.Tensor, sin: torch.Tensor, mode: str):
        self.cfg = cfg
        self.md = ModelDtype(mode)
        self.w = [{k: v.to(torch.float32) for k, v in L.items()} for L in weights["layers"]]
        self.final_norm = weights["final_norm"].to(torch.float32)
        self.cos, self.sin = cos.to(torch.float32), sin.to(torch.float32)
        L, KV, cap, D = cfg.n_layers, cfg.n_kv_heads, cfg.capacity, cfg.head_dim
        self.K = torch.zeros(L, KV, cap, D)
        self.V = torch.zeros(L, KV, cap, D)
        self.length = 0

    def _attention(self, layer: int, q: torch.Tensor, p: int) -> torch.Tensor:
        """q [H][D] at absolute position p: every head over keys 0..p of its kv head."""
        cfg = self.cfg
        group = cfg.n_heads // cfg.n_kv_heads
        heads = []
        for hh in range(cfg.n_heads):
            g = hh // group
            heads.append(self.md.attention_row(q[hh], self.K[layer, g, : p + 1], self.V[layer, g, : p + 1],
                                               cfg.head_dim ** -0.5))
        return torch.cat(heads)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """x [T][hidden] at positions length..length+T-1 -> final-norm hidden states."""
        cfg, md = self.cfg, self.md
        H, KV, D, hid, I = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden, cfg.intermediate
        T, p0 = x.shape[0], self.length
        assert p0 + T <= cfg.capacity
        h = x.to(torch.float32).clone()
        pend = None
        for l, L in enumerate(self.w):
            if pend is not None:
                h = md.add(h, pend)
            y = md.rms_norm(h, L["in_norm"], cfg.rms_eps)
            qkv = md.matmul(y, L["qkv"])
            qh = qkv[:, : H * D].reshape(T, H, D)
            kh = qkv[:, H * D:(H + KV) * D].reshape(T, KV, D)
            vh = qkv[:, (H + KV) * D:].reshape(T, KV, D)
            qn = md.rms_norm(qh, L["q_norm"], cfg.rms_eps)
            kn = md.rms_norm(kh, L["k_norm"], cfg.rms_eps)
            q_all = torch.empty(T, H, D)
            for t in range(T):  # every new position is written before any query reads it
                p = p0 + t
                q_all[t] = md.rope(qn[t], self.cos[p], self.sin[p])
                self.K[l, :, p] = md.rope(kn[t], self.cos[p], self.sin[p])
                self.V[l, :, p] = vh[t]
            a = torch.stack([self._attention(l, q_all[t], p0 + t) for t in range(T)])
            h = md.add(h, md.matmul(a, L["o"]))
            y2 = md.rms_norm(h, L["post_norm"], cfg.rms_eps)
            gu = md.matmul(y2, L["gate_up"])
            m = md.silu_times_up(gu[:, :I], gu[:, I:])
            pend = md.matmul(m, L["down"])
        h = md.add(h, pend)
        self.length = p0 + T
        return md.rms_norm(h, self.final_norm, cfg.rms_eps)


def moe_block(y2: torch.Tensor, Wr: torch.Tensor, Wgu: torch.Tensor, Wd: torch.Tensor, k: int, mode: str):
    """The sparse MoE block on normalised rows y2 [T][hid]: softmax over all experts, the k
    largest (ties to the lower index, slots in descending probability), renormalised weights,
    each chosen expert's SwiGLU MLP, and the weighted sum over the slots.
    Returns (out [T][hid], idx [T][k], weights [T][k])."""
    md = ModelDtype(mode)
    T = y2.shape[0]
    Ie = Wgu.shape[1] // 2
    logits = md.matmul(y2, Wr)                                   # [T][E], model dtype
    probs = md.rb(torch.softmax(logits, -1))                     # fp32 softmax, stored in the model dtype
    outs, idxs, wts = [], [], []
    for t in range(T):
        order = sorted(range(probs.shape[1]), key=lambda e: (-float(probs[t, e]), e))[:k]
        sel = probs[t, order]
        den = md.rb(sel.double().sum().to(torch.float32))       # the renormalising sum, model dtype
        w = md.rb(sel / den)
        acc = torch.zeros(y2.shape[1], dtype=torch.float64)
        for s, e in enumerate(order):
            gu = md.matmul(y2[t:t + 1], Wgu[e])
            m = md.silu_times_up(gu[:, :Ie], gu[:, Ie:])
            ye = md.matmul(m, Wd[e])[0]
            acc += md.rb(ye * w[s]).double()                    # each weighted expert output rounded
        outs.append(md.rb(acc.to(torch.float32)))               # the slot sum rounded once
        idxs.append(order)
        wts.append(w)
    return torch.stack(outs), torch.tensor(idxs, dtype=torch.int32), torch.stack(wts)


def rope_table(capacity: int, D: int, theta: float, mode: str):
    """cos, sin [capacity][D] with duplicated halves: inverse frequencies theta^(-2j/D) in
    double rounded to fp32 (and, in bf16, to the bf16 buffer the model holds), angles as one
    fp32 product p * inv_j, cos and sin of that angle rounded to fp32 and then stored in the
    model dtype."""
    md = ModelDtype(mode)
    j = torch.arange(D // 2, dtype=torch.float64)
    inv = md.rb((1.0 / theta ** (2.0 * j / D)).to(torch.float32))
    p = torch.arange(capacity, dtype=torch.float32)
    ang = p[:, None] * inv[None, :]                              # fp32 products
    c = md.rb(torch.cos(ang.double()).to(torch.float32))
    s = md.rb(torch.sin(ang.double()).to(torch.float32))
    return torch.cat([c, c], -1), torch.cat([s, s], -1)
