"""Whole-stack parity through the C ABI (qwen3_init / qwen3_forward / qwen3_forward_hidden /
qwen3_moe_block) against the CPU oracle on identical seeded inputs, for the five
configurations: tiny fp32 stack, Qwen3-1.7B-shaped bf16 decode and prefill, Qwen3-MoE
shape, and 8-bit group-quantised projections.

Gates: fp32 max|d|/RMS <= 1e-4; bf16 per-row relative L2 <= 2e-2 after one layer (deeper
stacks are reported); router top-k indices exact on identical block inputs."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, gate, host_layers, max_rel_rms, max_row_rel_l2, np32, oracle_threads, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def build(cfg, n_layers=None, filled=0):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = cfg.replace(n_layers=n_layers) if n_layers else cfg
    w = synth.model_weights(cfg, DEV)
    K, V = synth.kv_cache(cfg, filled, DEV)
    return cfg, w, K, V


def oracle_stack(orc, cfg, w, K=None, V=None):
    st = orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), cfg.dtype,
                   kcache=None if K is None else np32(K), vcache=None if V is None else np32(V))
    return st


def test_tiny_fp32_prefill_then_decode_tokens(orc):
    """16 token ids prefilled in one call, then 16 single-token decode steps; outputs at
    every position and the final caches against the oracle (strict fp32 gate)."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32 as cfg
    cfg_, w, K, V = build(cfg)
    seat = q3.Seat(cfg, w, max_tokens=16, k_cache=K, v_cache=V)
    ids = synth.token_ids(cfg, 32, DEV)
    outs = [seat.forward(ids[:16])] + [seat.forward(ids[16 + i:17 + i]) for i in range(16)]
    torch.cuda.synchronize()
    got = np.concatenate([np32(o) for o in outs])
    assert seat.length == 32
    st = oracle_stack(orc, cfg, w)
    E = np32(w["embed"])
    idn = ids.cpu().numpy()
    ref = np.concatenate([st.forward(E[idn[:16]])] + [st.forward(E[idn[16 + i:17 + i]]) for i in range(16)])
    e = gate(got, ref, "fp32")
    ek = max_rel_rms(np32(seat.k)[:, :, :32], st.k[:, :, :32])
    ev = max_rel_rms(np32(seat.v)[:, :, :32], st.v[:, :, :32])
    say(f"tiny fp32 16+16x1: out {e:.2e}, K {ek:.2e}, V {ev:.2e}")
    assert ek <= 1e-4 and ev <= 1e-4
    q3.qwen3_check_device_errors(seat.handle)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tiny_prefill_then_decode_matches_one_prefill_on_gpu(dtype):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(dtype=dtype)
    cfg, w, K, V = build(cfg)
    x = synth.hidden_states(cfg, 32, DEV)
    a = q3.Seat(cfg, w, max_tokens=32)
    outs = [a.forward_hidden(x[:16])] + [a.forward_hidden(x[i:i + 1]) for i in range(16, 32)]
    b = q3.Seat(cfg, w, max_tokens=32)
    full = b.forward_hidden(x)
    torch.cuda.synchronize()
    got = torch.cat(outs)
    e = max_row_rel_l2(np32(got), np32(full))
    say(f"tiny {dtype}: 16 + 16x1 vs one 32-token prefill on the GPU: {e:.2e}")
    assert e <= (1e-5 if dtype == "fp32" else BF16_TOL)


def test_tiny_bf16_vs_oracle(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(dtype="bf16", n_layers=1)
    cfg, w, K, V = build(cfg)
    x = synth.hidden_states(cfg, 24, DEV)
    seat = q3.Seat(cfg, w, max_tokens=16)
    got = torch.cat([seat.forward_hidden(x[:16])] + [seat.forward_hidden(x[i:i + 1]) for i in range(16, 24)])
    torch.cuda.synchronize()
    st = oracle_stack(orc, cfg, w)
    xn = np32(x)
    ref = np.concatenate([st.forward(xn[:16])] + [st.forward(xn[i:i + 1]) for i in range(16, 24)])
    e = gate(np32(got), ref, "bf16")
    say(f"tiny bf16 one layer 16+8x1: {e:.2e}")


def _decode_case(orc, cfg, n_layers, filled):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg, w, K, V = build(cfg, n_layers=n_layers, filled=filled)
    st = oracle_stack(orc, cfg, w, K, V)  # host copies taken before the GPU touches the cache
    st.length = filled
    seat = q3.Seat(cfg, w, max_tokens=1, k_cache=K, v_cache=V)
    seat.length = filled
    x = synth.hidden_states(cfg, 1, DEV)
    say(f"{cfg.name}: {cfg.n_layers} layer(s), decode at position {filled}")
    out = seat.forward_hidden(x)
    torch.cuda.synchronize()
    ref = st.forward(np32(x))
    kv_e = max(max_row_rel_l2(np32(seat.k)[:, :, filled], st.k[:, :, filled]),
               max_row_rel_l2(np32(seat.v)[:, :, filled], st.v[:, :, filled]))
    return np32(out), ref, kv_e, seat


def test_qwen3_1p7b_decode_one_layer(orc):
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    got, ref, kv_e, _ = _decode_case(orc, QWEN3_1P7B_DECODE, 1, 4095)
    e = gate(got, ref, "bf16")
    say(f"1.7B decode, 1 layer, ctx 4096: out {e:.2e}, new K/V entries {kv_e:.2e}")
    assert kv_e <= BF16_TOL


def test_qwen3_1p7b_decode_full_stack(orc):
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    got, ref, kv_e, _ = _decode_case(orc, QWEN3_1P7B_DECODE, None, 4095)
    e = max_row_rel_l2(got, ref)
    say(f"1.7B decode, 28 layers, ctx 4096: out rel L2 {e:.2e} (reported), new K/V entries {kv_e:.2e}")
    # regression bound: the 28-layer bf16 drift measures ~2.8% on both decode paths
    assert e < 0.05


def test_qwen3_1p7b_prefill_one_layer(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_PREFILL
    cfg, w, K, V = build(QWEN3_1P7B_PREFILL, n_layers=1)
    seat = q3.Seat(cfg, w, max_tokens=2048, k_cache=K, v_cache=V)
    x = synth.hidden_states(cfg, 2048, DEV)
    say("1.7B prefill, 1 layer, T=2048")
    got = seat.forward_hidden(x)
    torch.cuda.synchronize()
    st = oracle_stack(orc, cfg, w)
    ref = st.forward(np32(x))
    e = gate(np32(got), ref, "bf16")
    ek = max_row_rel_l2(np32(seat.k)[0, :, :2048], st.k[0, :, :2048])
    say(f"1.7B prefill, 1 layer, T=2048: out {e:.2e}, K {ek:.2e}")
    assert ek <= BF16_TOL and seat.length == 2048


@pytest.mark.parametrize("T", [1, 64])
def test_moe_block_real_shape(orc, T):
    """Isolated MoE block at the Qwen3-MoE shape on identical inputs: exact top-k indices."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    cfg, w, K, V = build(QWEN3_MOE, n_layers=1)
    seat = q3.Seat(cfg, w, max_tokens=64, k_cache=K, v_cache=V)
    x = synth.hidden_states(cfg, T, DEV, name="moe_x")
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=DEV)
    wt = torch.empty((T, cfg.top_k), dtype=torch.bfloat16, device=DEV)
    out = seat.moe_block(0, x, topk_idx=idx, topk_w=wt)
    torch.cuda.synchronize()
    L = w["layers"][0]
    ref, ridx, rw = orc.moe_block(np32(x), np32(L["router"]), np32(L["exp_gate_up"]), np32(L["exp_down"]),
                                  cfg.top_k, True, False, "bf16")
    gidx = idx.cpu().numpy()
    mism = int(np.sum(gidx != ridx))
    e = gate(np32(out), ref, "bf16")
    say(f"MoE block T={T}: top-k mismatches {mism}, out {e:.2e}, distinct experts {len(np.unique(gidx))}")
    assert mism == 0


def test_moe_stack_prefill_then_decode(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    cfg, w, K, V = build(QWEN3_MOE, n_layers=2)
    seat = q3.Seat(cfg, w, max_tokens=64, k_cache=K, v_cache=V)
    x = synth.hidden_states(cfg, 65, DEV)
    say("MoE 2-layer stack: T=64 prefill then T=1 decode")
    got = torch.cat([seat.forward_hidden(x[:64]), seat.forward_hidden(x[64:65])])
    torch.cuda.synchronize()
    st = oracle_stack(orc, cfg, w)
    xn = np32(x)
    ref = np.concatenate([st.forward(xn[:64]), st.forward(xn[64:65])])
    e = max_row_rel_l2(np32(got), ref)
    say(f"MoE 2 layers, 64 + 1 tokens: rel L2 {e:.2e}")
    assert e <= 2 * BF16_TOL


def test_moe_decode_one_layer_ctx2048(orc):
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    got, ref, kv_e, _ = _decode_case(orc, QWEN3_MOE, 1, 2047)
    e = gate(got, ref, "bf16")
    say(f"MoE decode, 1 layer, ctx 2048: out {e:.2e}, new K/V {kv_e:.2e}")


def test_q8_decode_and_prefill_one_layer(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_Q8
    got, ref, kv_e, _ = _decode_case(orc, QWEN3_1P7B_Q8, 1, 4095)
    e = gate(got, ref, "bf16")
    say(f"q8 decode, 1 layer, ctx 4096: out {e:.2e}")
    cfg, w, K, V = build(QWEN3_1P7B_Q8, n_layers=1)
    seat = q3.Seat(cfg, w, max_tokens=512, k_cache=K, v_cache=V)
    x = synth.hidden_states(cfg, 512, DEV)
    out = seat.forward_hidden(x)
    torch.cuda.synchronize()
    st = oracle_stack(orc, cfg, w)
    ref = st.forward(np32(x))
    e = gate(np32(out), ref, "bf16")
    say(f"q8 prefill, 1 layer, T=512: out {e:.2e}")


def test_errors_leave_the_seat_unchanged():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import _lib, synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg, w, K, V = build(TINY_FP32)
    seat = q3.Seat(cfg, w, max_tokens=16)
    seat.forward_hidden(synth.hidden_states(cfg, 16, DEV))
    seat.length = 60
    torch.cuda.synchronize()
    k0, v0 = seat.k.clone(), seat.v.clone()
    out = torch.full((5, cfg.hidden), 7.0, device=DEV)
    with pytest.raises(q3.Qwen3Error) as ei:
        q3.qwen3_forward_hidden(seat.handle, synth.hidden_states(cfg, 5, DEV), out)
    assert ei.value.code == _lib.ERR_CAPACITY
    with pytest.raises(q3.Qwen3Error) as ei:
        q3.qwen3_forward_hidden(seat.handle, synth.hidden_states(cfg, 17, DEV), out)
    assert ei.value.code == _lib.ERR_ARG
    with pytest.raises(q3.Qwen3Error) as ei:
        seat.length = 65
    torch.cuda.synchronize()
    assert seat.length == 60 and torch.equal(seat.k, k0) and torch.equal(seat.v, v0) and bool((out == 7.0).all())
    seat.reset()
    torch.cuda.synchronize()
    assert seat.length == 0 and not seat.k.any() and not seat.v.any()


def test_bad_token_id_is_flagged():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import _lib
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg, w, K, V = build(TINY_FP32)
    seat = q3.Seat(cfg, w, max_tokens=4)
    seat.forward(torch.tensor([1, 2, 5000, 3], dtype=torch.int32, device=DEV))
    with pytest.raises(q3.Qwen3Error) as ei:
        q3.qwen3_check_device_errors(seat.handle)
    assert ei.value.code == _lib.ERR_ARG
    q3.qwen3_check_device_errors(seat.handle)  # cleared
