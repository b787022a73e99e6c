"""Model configurations of the Qwen3 decoder stack (shapes and constants only).

The fields mirror the config keys the pages read: "maya2_mlx/backbone.py"
(Backbone.__init__: num_hidden_layers, num_attention_heads, num_key_value_heads,
head_dim, hidden_size, rms_norm_eps, capacity), "@mlx-bun/inference" qwen3-moe.ts
(numExperts, topKExperts, normTopkProb, moe_intermediate, rope_theta) and the
8-bit affine group format of the quantised projections.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Qwen3Config:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    capacity: int
    dtype: str = "bf16"            # "bf16" (production) or "fp32" (strict)
    vocab: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    n_experts: int = 0             # 0: dense SwiGLU MLP in every layer
    top_k: int = 0
    moe_intermediate: int = 0
    norm_topk_prob: int = 1
    quant_bits: int = 0            # 0: bf16/fp32 weights; 8: u8 codes + bf16 scale/bias per group
    quant_group: int = 64
    seed: int = 0
    qk_norm: bool = True           # page 2 Qwen3DecoderSpec switches: per-head q/k RMSNorm (Qwen3;
    attention_bias: bool = False   # Qwen2 skips it), q/k/v projection bias (Qwen2) and the
    sliding_window: int = 0        # attention mask: 0 causal, w > 0 SlidingWindow(w)
    decoder_sparse_step: int = 1   # MoE layer selection ("@mlx-bun/inference" qwen3-moe.ts,
    mlp_only_layers: tuple = ()    # Qwen3MoeDecoderLayer): see is_moe_layer

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    def is_moe_layer(self, layer: int) -> bool:
        """A layer runs the sparse MoE block unless its index is in mlp_only_layers or
        (index + 1) is not a multiple of decoder_sparse_step; otherwise the dense MLP."""
        return self.n_experts > 0 and layer not in self.mlp_only_layers and (layer + 1) % self.decoder_sparse_step == 0

    def replace(self, **kw) -> "Qwen3Config":
        return dataclasses.replace(self, **kw)


# Tiny fp32 stack: 2 layers, 16-token prefill then 16 single-token decode steps.
TINY_FP32 = Qwen3Config("tiny-fp32", n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                        intermediate=768, capacity=64, dtype="fp32", vocab=1024, seed=0)

# Qwen3-1.7B shape, bf16, decode at context 4096 (K/V pre-filled at 0..4094).
QWEN3_1P7B_DECODE = Qwen3Config("qwen3-1.7b-decode", n_layers=28, hidden=2048, n_heads=16, n_kv_heads=8,
                                head_dim=128, intermediate=6144, capacity=4096, seed=0)

# Same shape, one 2048-token causal prefill from an empty cache of capacity 8192.
QWEN3_1P7B_PREFILL = QWEN3_1P7B_DECODE.replace(name="qwen3-1.7b-prefill", capacity=8192, seed=1)

# Qwen3-MoE shape: 48 layers, 128 experts, top-8 renormalised, expert intermediate 768.
QWEN3_MOE = Qwen3Config("qwen3-moe", n_layers=48, hidden=2048, n_heads=32, n_kv_heads=4, head_dim=128,
                        intermediate=0, capacity=2048, rope_theta=1e7, n_experts=128, top_k=8,
                        moe_intermediate=768, norm_topk_prob=1, seed=0)

# Qwen3-1.7B shape with 8-bit affine group-quantised projections (groups of 64 along K).
QWEN3_1P7B_Q8 = QWEN3_1P7B_DECODE.replace(name="qwen3-1.7b-q8", quant_bits=8, quant_group=64)

PRESETS = {c.name: c for c in (TINY_FP32, QWEN3_1P7B_DECODE, QWEN3_1P7B_PREFILL, QWEN3_MOE, QWEN3_1P7B_Q8)}
