"""MoE stacks with dense layers and 8-bit MoE weights through the C ABI, against the CPU oracle.

Layer kinds follow the Qwen3-MoE decoder layer's rule ("@mlx-bun/inference" qwen3-moe.ts,
Qwen3MoeDecoderLayer): a layer is sparse unless it is listed in mlp_only_layers or (index + 1)
is not a multiple of decoder_sparse_step; the synthetic builder gives a dense layer gate_up /
down of width `intermediate` and no router, and the library dispatches on the router.

8-bit MoE weights (the quantised gate Linear and QuantizedSwitchLinear experts): router and
stacked experts as u8 codes with bf16 scale and bias per group of 64 inputs; the oracle gets
the weights dequantised by its own routine.  Top-k: the GPU folds each group as s * (x . q) +
b * sum(x) in fp32 while the oracle sums dequantised products, so a router logit can round to
the neighbouring bf16 value; a pick that differs from the oracle's must then be an expert
whose oracle probability is within one bf16 step of the k-th largest (a tie up to that
rounding).  Gates: bf16 per-row relative L2 <= 2e-2 per layer."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, gate, host_layers, max_row_rel_l2, np32, oracle_threads, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def _cfg(**kw):
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    return QWEN3_MOE.replace(**kw)


def _oracle(orc, cfg, w):
    return orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), cfg.dtype)


def _check_topk(gidx, ridx, probs):
    """Exact picks, or picks that differ only among experts tied with the k-th largest oracle
    probability up to one bf16 step."""
    diff = 0
    for t in range(gidx.shape[0]):
        g, r = set(gidx[t].tolist()), set(ridx[t].tolist())
        if g == r:
            continue
        kth = np.sort(probs[t])[-len(r)]
        step = 2.0 ** (np.floor(np.log2(kth)) - 7)
        for e in g ^ r:
            assert abs(probs[t, e] - kth) <= step, f"token {t}: expert {e} p={probs[t, e]:.4e}, k-th {kth:.4e}"
        diff += 1
    return diff


def test_mixed_stack_prefill_then_decode(orc):
    """Three layers, mlp_only_layers (1,): MoE, dense (I = 6144), MoE, at hidden 2048 with 128
    experts; a 64-token prefill (sorted experts) then a decode step (one-token routing)."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = _cfg(n_layers=3, intermediate=6144, mlp_only_layers=(1,))
    w = synth.model_weights(cfg, DEV)
    assert ["router" in L for L in w["layers"]] == [True, False, True]
    seat = q3.Seat(cfg, w, max_tokens=64)
    x = synth.hidden_states(cfg, 65, DEV)
    say("mixed MoE stack (MoE, dense, MoE): T=64 prefill then T=1 decode")
    got = torch.cat([seat.forward_hidden(x[:64]), seat.forward_hidden(x[64:65])])
    torch.cuda.synchronize()
    st = _oracle(orc, cfg, w)
    xn = np32(x)
    ref = np.concatenate([st.forward(xn[:64]), st.forward(xn[64:65])])
    e = max_row_rel_l2(np32(got), ref)
    ek = max_row_rel_l2(np32(seat.k)[1, :, :65], st.k[1, :, :65])  # the dense layer's keys
    say(f"mixed MoE stack 3 layers, 64 + 1 tokens: out rel L2 {e:.2e}, layer-1 K {ek:.2e}")
    assert e <= 3 * BF16_TOL and ek <= 2 * BF16_TOL
    with pytest.raises(q3.Qwen3Error):  # the block entry point refuses a dense layer
        seat.moe_block(1, x[:2])


def test_mixed_stack_dense_layer_equals_dense_stack():
    """A one-layer MoE configuration whose only layer is listed in mlp_only_layers runs exactly
    the dense stack's kernels: the outputs are bitwise equal."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    dense = QWEN3_1P7B_DECODE.replace(n_layers=1, capacity=256)
    mixed = dense.replace(n_experts=16, top_k=4, moe_intermediate=128, mlp_only_layers=(0,))
    w = synth.model_weights(dense, DEV)
    assert not mixed.is_moe_layer(0)
    a = q3.Seat(dense, w, max_tokens=16)
    b = q3.Seat(mixed, w, max_tokens=16)
    x = synth.hidden_states(dense, 17, DEV)
    q3.qwen3_set_decode_path(a.handle, 1)  # the MoE configuration has no persistent decode kernel
    ga = torch.cat([a.forward_hidden(x[:16]), a.forward_hidden(x[16:])])
    gb = torch.cat([b.forward_hidden(x[:16]), b.forward_hidden(x[16:])])
    torch.cuda.synchronize()
    assert torch.equal(ga, gb)


@pytest.mark.parametrize("T", [1, 5, 64])
def test_q8_moe_block_real_shape(orc, T):
    """8-bit router and experts at the Qwen3-MoE shape on identical inputs."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = _cfg(n_layers=1, quant_bits=8, quant_group=64)
    w = synth.model_weights(cfg, DEV)
    L = w["layers"][0]
    assert L["router_q"].dtype == torch.uint8 and L["exp_gate_up_q"].shape == (128, 1536, 2048)
    assert L["exp_down_s"].shape == (128, 2048, 12)
    seat = q3.Seat(cfg, w, max_tokens=64)
    x = synth.hidden_states(cfg, T, DEV, name="moe_x")
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=DEV)
    wt = torch.empty((T, cfg.top_k), dtype=torch.bfloat16, device=DEV)
    out = seat.moe_block(0, x, topk_idx=idx, topk_w=wt)
    torch.cuda.synchronize()
    H = host_layers(orc, cfg, w)[0]
    ref, ridx, rw = orc.moe_block(np32(x), H["router"], H["exp_gate_up"], H["exp_down"], cfg.top_k, True, False,
                                  "bf16")
    _, _, probs = orc.router(np32(x), H["router"], cfg.top_k, True, "bf16")
    gidx = idx.cpu().numpy()
    diff = _check_topk(gidx, ridx, probs)
    e = gate(np32(out), ref, "bf16") if diff == 0 else max_row_rel_l2(np32(out), ref)
    say(f"q8 MoE block T={T}: tokens with a tie-swapped pick {diff}, out rel L2 {e:.2e}")
    if diff:  # rows whose routing agrees meet the gate
        same = [t for t in range(T) if set(gidx[t]) == set(ridx[t])]
        gate(np32(out)[same], ref[same], "bf16")


def test_q8_moe_stack_with_dense_layer(orc):
    """8-bit everywhere, decoder_sparse_step 2: layer 0 dense (8-bit gate_up / down), layer 1
    MoE (8-bit router and experts); 24-token prefill then two decode steps."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = _cfg(n_layers=2, intermediate=6144, decoder_sparse_step=2, quant_bits=8, quant_group=64)
    w = synth.model_weights(cfg, DEV)
    assert "gate_up_q" in w["layers"][0] and "router_q" in w["layers"][1]
    seat = q3.Seat(cfg, w, max_tokens=24)
    x = synth.hidden_states(cfg, 26, DEV)
    say("q8 MoE stack (dense, MoE): T=24 prefill then 2 x T=1")
    got = torch.cat([seat.forward_hidden(x[:24]), seat.forward_hidden(x[24:25]), seat.forward_hidden(x[25:26])])
    torch.cuda.synchronize()
    st = _oracle(orc, cfg, w)
    xn = np32(x)
    ref = np.concatenate([st.forward(xn[:24]), st.forward(xn[24:25]), st.forward(xn[25:26])])
    e = max_row_rel_l2(np32(got), ref)
    say(f"q8 MoE stack 2 layers, 24 + 1 + 1 tokens: out rel L2 {e:.2e}")
    assert e <= 2 * BF16_TOL


def test_q8_moe_batched_decode(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = _cfg(n_layers=1, quant_bits=8, quant_group=64)
    w = synth.model_weights(cfg, DEV)
    fills = [300, 0, 17, 2047]
    seats = []
    for i, f in enumerate(fills):
        K, V = synth.kv_cache(cfg, f, DEV)
        if f:
            K[:, :, :f] = K[:, :, :f].roll(i + 1, dims=2)
        st = q3.Seat(cfg, w, max_tokens=len(fills), k_cache=K, v_cache=V)
        st.length = f
        seats.append(st)
    hk = [np32(s.k) for s in seats]
    hv = [np32(s.v) for s in seats]
    x = synth.hidden_states(cfg, len(fills), DEV, name="xq")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch([s.handle for s in seats], x, out)
    torch.cuda.synchronize()
    worst = 0.0
    for b, f in enumerate(fills):
        st = orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), "bf16", kcache=hk[b], vcache=hv[b])
        st.length = f
        worst = max(worst, gate(np32(out)[b:b + 1], st.forward(np32(x)[b:b + 1]), "bf16"))
    say(f"q8 MoE batched decode B={len(fills)}: worst row {worst:.2e}")


def test_init_checks_per_layer_kind():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = _cfg(n_layers=2, intermediate=256, decoder_sparse_step=2, quant_bits=8, quant_group=64, hidden=256,
               n_heads=4, n_kv_heads=2, n_experts=8, top_k=2, moe_intermediate=64, capacity=64)
    w = synth.model_weights(cfg, DEV)
    q3.Seat(cfg, w, max_tokens=4)  # valid
    bad = {**w, "layers": [w["layers"][0], {k: v for k, v in w["layers"][1].items() if k != "router_s"}]}
    with pytest.raises(q3.Qwen3Error):  # an 8-bit MoE layer without its router scales
        q3.Seat(cfg, bad, max_tokens=4)
    with pytest.raises(q3.Qwen3Error):  # a dense layer in a configuration with no dense width
        q3.Seat(cfg.replace(intermediate=0), w, max_tokens=4)
