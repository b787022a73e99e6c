"""The persistent decode step of Qwen3-MoE stacks (one kernel for all layers of a T = 1 call)
against the CPU oracle and against the one-kernel-per-step decode path, through the C ABI.

Shape: hidden 2048, 32 q / 4 kv heads of 128, 128 experts, top 8 renormalised, expert
intermediate 768 ("@mlx-bun/inference" qwen3-moe.ts, Qwen3MoeSparseMoeBlock; attention as
"maya2_mlx/backbone.py" Backbone.forward).  Covers one layer at positions with 32 keys per
attention split, fewer keys than splits and a single key; the full 48-layer stack; several
consecutive steps; page 2's switches (no q/k norm, q|k|v bias, a sliding window); HIP-graph
replays against the eager step; the fallback for stacks with a dense-MLP layer; and every
weight 8-bit (router and experts included).

Top-k: both GPU paths and the oracle round each router logit to bf16 after an fp32 (GPU) or
float64 (oracle) dot, so a logit can land on the neighbouring bf16 value and the k-th pick
can differ where two probabilities tie up to one bf16 step; the fixed seeds here give no such
tie (a differing pick would show as a large output error).  Gates: bf16 per-row relative L2
<= 2e-2 against the oracle per layer (and per step over 2-4 layers); the 48-layer stack is
reported, with a bound that separates the drift both decode paths show there from a broken step."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, gate, host_layers, max_row_rel_l2, np32, oracle_threads, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def _seats(cfg, n_layers, filled):
    """Two seats over identical weights and identical (separate) caches: path 2 and path 1."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = cfg.replace(n_layers=n_layers) if n_layers else cfg
    w = synth.model_weights(cfg, DEV)
    K, V = synth.kv_cache(cfg, filled, DEV)
    K2, V2 = K.clone(), V.clone()
    mk = q3.Seat(cfg, w, max_tokens=1, k_cache=K, v_cache=V)
    q3.qwen3_set_decode_path(mk.handle, 2)
    assert q3.qwen3_get_decode_path(mk.handle) == 2
    ref = q3.Seat(cfg, w, max_tokens=1, k_cache=K2, v_cache=V2)
    q3.qwen3_set_decode_path(ref.handle, 1)
    assert q3.qwen3_get_decode_path(ref.handle) == 1
    mk.length = filled
    ref.length = filled
    return cfg, w, mk, ref


def _oracle(orc, cfg, w, seat, filled):
    st = orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), cfg.dtype,
                   kcache=np32(seat.k), vcache=np32(seat.v))
    st.length = filled
    return st


@pytest.mark.parametrize("filled", [2047, 0, 5, 31, 64, 1000])
def test_moe_persistent_one_layer_vs_oracle_and_kernels(orc, filled):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    say(f"persistent MoE decode, 1 layer, position {filled}")
    cfg, w, mk, ref = _seats(QWEN3_MOE, 1, filled)
    st = _oracle(orc, cfg, w, mk, filled)  # host copies taken before the GPU touches the cache
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e, e_ref = max_row_rel_l2(np32(a), o), max_row_rel_l2(np32(b), o)
    e_paths = max_row_rel_l2(np32(a), np32(b))
    ek = max_row_rel_l2(np32(mk.k)[:, :, filled], st.k[:, :, filled])
    ev = max_row_rel_l2(np32(mk.v)[:, :, filled], st.v[:, :, filled])
    say(f"  vs oracle {e:.2e} (one-kernel-per-step path {e_ref:.2e}), vs that path {e_paths:.2e}, "
        f"new K {ek:.2e}, new V {ev:.2e}")
    gate(np32(a), o, "bf16")
    assert max(ek, ev) <= BF16_TOL and e_paths <= BF16_TOL
    assert np.array_equal(np32(mk.v)[:, :, filled], np32(ref.v)[:, :, filled])  # raw v rows
    assert mk.length == filled + 1


def test_moe_persistent_capacity_8192_last_position(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    cfg0 = QWEN3_MOE.replace(capacity=8192)
    filled = 8191
    say(f"persistent MoE decode, 1 layer, capacity 8192, position {filled}")
    cfg, w, mk, ref = _seats(cfg0, 1, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    e = gate(np32(a), st.forward(np32(x)), "bf16")
    e_paths = max_row_rel_l2(np32(a), np32(b))
    say(f"  vs oracle {e:.2e}, vs one-kernel-per-step path {e_paths:.2e}")
    assert e_paths <= BF16_TOL


def test_moe_persistent_full_stack(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    filled = 2047
    say("persistent MoE decode, 48 layers, ctx 2048")
    cfg, w, mk, ref = _seats(QWEN3_MOE, None, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e, e_ref, e_paths = max_row_rel_l2(np32(a), o), max_row_rel_l2(np32(b), o), max_row_rel_l2(np32(a), np32(b))
    ekv = max(max_row_rel_l2(np32(mk.k)[l, :, filled], st.k[l, :, filled]) for l in range(cfg.n_layers))
    say(f"  vs oracle {e:.2e} (one-kernel-per-step path {e_ref:.2e}), vs that path {e_paths:.2e}, "
        f"new K of every layer vs oracle {ekv:.2e}")
    # 48 MoE layers: reported, with a bound that separates drift from a broken step (an unrelated
    # output is ~1.4 away).  Each single layer agrees with the oracle within the gate, but a top-8
    # pick is discontinuous: an fp32 summation-order change anywhere (measured: only the order of
    # the split merge) moves the 48-layer distance between 0.08 and 0.16 for both paths.
    assert e < 0.35 and e_paths < 0.35


def test_moe_persistent_consecutive_steps(orc):
    """Six steps in a row from position 100 over two layers (fresh exchange tags per call, the
    previous calls' cache entries read back)."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    filled, n = 100, 6
    say(f"persistent MoE decode, 2 layers, {n} steps from position {filled}")
    cfg, w, mk, ref = _seats(QWEN3_MOE, 2, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, n, DEV)
    outs = [mk.forward_hidden(x[i:i + 1]) for i in range(n)]
    outs_ref = [ref.forward_hidden(x[i:i + 1]) for i in range(n)]
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    xs = np32(x)
    worst = worst_paths = 0.0
    for i in range(n):
        worst = max(worst, max_row_rel_l2(np32(outs[i]), st.forward(xs[i:i + 1])))
        worst_paths = max(worst_paths, max_row_rel_l2(np32(outs[i]), np32(outs_ref[i])))
    say(f"  worst step vs oracle {worst:.2e}, vs one-kernel-per-step path {worst_paths:.2e}")
    assert worst <= 2 * BF16_TOL and worst_paths <= BF16_TOL
    assert mk.length == filled + n


def test_moe_persistent_qwen2_switches(orc):
    """No per-head q/k norm, a q|k|v bias and a sliding window of 40 keys: four steps from
    position 60 over two layers."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    cfg0 = QWEN3_MOE.replace(qk_norm=False, attention_bias=True, sliding_window=40)
    filled, n = 60, 4
    say(f"persistent MoE decode with Qwen2 switches, 2 layers, {n} steps from position {filled}")
    cfg, w, mk, ref = _seats(cfg0, 2, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, n, DEV)
    outs = [mk.forward_hidden(x[i:i + 1]) for i in range(n)]
    outs_ref = [ref.forward_hidden(x[i:i + 1]) for i in range(n)]
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    xs = np32(x)
    worst = 0.0
    for i in range(n):
        worst = max(worst, max_row_rel_l2(np32(outs[i]), st.forward(xs[i:i + 1])))
        assert max_row_rel_l2(np32(outs[i]), np32(outs_ref[i])) <= BF16_TOL
    say(f"  worst step vs oracle {worst:.2e}")
    assert worst <= 2 * BF16_TOL


def test_moe_persistent_graph_replays_match_eager():
    """One captured step replayed five times (the position is baked into the graph; each
    replay rewrites the same cache row), with eager calls between replays: every replay's
    output equals the eager step's bit for bit, and no exchange times out."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    filled = 1500
    cfg, w, mk, _ = _seats(QWEN3_MOE, 4, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    out = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.Stream()
    q3.qwen3_set_stream(mk.handle, stream)
    with torch.cuda.stream(stream):
        mk.length = filled
        q3.qwen3_forward_hidden(mk.handle, x, out)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        mk.length = filled
        q3.qwen3_forward_hidden(mk.handle, x, out)
    for r in range(5):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        with torch.cuda.stream(stream):
            mk.length = filled
            q3.qwen3_forward_hidden(mk.handle, x, out)  # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    q3.qwen3_set_stream(mk.handle, None)
    q3.qwen3_check_device_errors(mk.handle)
    say("persistent MoE decode: 5 graph replays equal the eager step")


def test_moe_stack_with_a_dense_layer_takes_the_kernel_path():
    """mlp_only_layers makes layer 1 dense: the persistent MoE kernel has no dense MLP, so the
    seat decodes one kernel per step and refuses path 2."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import _lib, synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    cfg = QWEN3_MOE.replace(n_layers=2, intermediate=6144, mlp_only_layers=(1,))
    w = synth.model_weights(cfg, DEV)
    seat = q3.Seat(cfg, w, max_tokens=1)
    assert q3.qwen3_get_decode_path(seat.handle) == 1
    with pytest.raises(q3.Qwen3Error) as ei:
        q3.qwen3_set_decode_path(seat.handle, 2)
    assert ei.value.code == _lib.ERR_UNSUPPORTED


# ------------------------------------------------------------------ 8-bit weights

def _q8(cfg):
    return cfg.replace(quant_bits=8, quant_group=64)


@pytest.mark.parametrize("filled", [2047, 0, 31, 1000])
def test_moe_persistent_q8_one_layer_vs_oracle_and_kernels(orc, filled):
    """Every weight 8-bit (router and experts included): one layer against the oracle (weights
    dequantised exactly) and against the one-kernel-per-step path."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    say(f"persistent MoE decode, 8-bit weights, 1 layer, position {filled}")
    cfg, w, mk, ref = _seats(_q8(QWEN3_MOE), 1, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e, e_ref = max_row_rel_l2(np32(a), o), max_row_rel_l2(np32(b), o)
    e_paths = max_row_rel_l2(np32(a), np32(b))
    ek = max_row_rel_l2(np32(mk.k)[:, :, filled], st.k[:, :, filled])
    ev = max_row_rel_l2(np32(mk.v)[:, :, filled], st.v[:, :, filled])
    say(f"  vs oracle {e:.2e} (one-kernel-per-step path {e_ref:.2e}), vs that path {e_paths:.2e}, "
        f"new K {ek:.2e}, new V {ev:.2e}")
    gate(np32(a), o, "bf16")
    assert max(ek, ev) <= BF16_TOL and e_paths <= BF16_TOL


def test_moe_persistent_q8_stack_steps(orc):
    """8-bit weights, 4 layers, three steps in a row from position 1200, against the oracle and
    the one-kernel-per-step path."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    filled, n = 1200, 3
    say(f"persistent MoE decode, 8-bit weights, 4 layers, {n} steps from position {filled}")
    cfg, w, mk, ref = _seats(_q8(QWEN3_MOE), 4, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, n, DEV)
    outs = [mk.forward_hidden(x[i:i + 1]) for i in range(n)]
    outs_ref = [ref.forward_hidden(x[i:i + 1]) for i in range(n)]
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    xs = np32(x)
    worst = worst_paths = 0.0
    for i in range(n):
        worst = max(worst, max_row_rel_l2(np32(outs[i]), st.forward(xs[i:i + 1])))
        worst_paths = max(worst_paths, max_row_rel_l2(np32(outs[i]), np32(outs_ref[i])))
    say(f"  worst step vs oracle {worst:.2e}, vs one-kernel-per-step path {worst_paths:.2e}")
    assert worst <= 2 * BF16_TOL and worst_paths <= 2 * BF16_TOL


def test_moe_persistent_q8_full_stack(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    filled = 2047
    say("persistent MoE decode, 8-bit weights, 48 layers, ctx 2048")
    cfg, w, mk, ref = _seats(_q8(QWEN3_MOE), None, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e, e_ref, e_paths = max_row_rel_l2(np32(a), o), max_row_rel_l2(np32(b), o), max_row_rel_l2(np32(a), np32(b))
    say(f"  vs oracle {e:.2e} (one-kernel-per-step path {e_ref:.2e}), vs that path {e_paths:.2e}")
    assert e < 0.35 and e_paths < 0.35  # reported; see the bf16 48-layer test
