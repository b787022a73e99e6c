"""The persistent decode step (one kernel for all layers of a T = 1 call) against the CPU
oracle and against the one-kernel-per-step decode path, through the C ABI.

Covers: the Qwen3-1.7B shape at ctx 4096 (32 keys per attention split's chunk of 128) for
one layer and the full 28-layer stack; positions with fewer keys than attention splits
(empty splits) and a single key; capacity 8192 with 256-key chunks; several consecutive
steps (fresh exchange tags per call, cache entries written by earlier calls); and HIP-graph
replays of one captured step, each checked against the eager step."""
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


@pytest.mark.parametrize("filled", [4095, 0, 5, 31, 32, 1000])
def test_persistent_one_layer_vs_oracle_and_kernels(orc, filled):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    say(f"persistent decode, 1 layer, position {filled}")
    cfg, w, mk, ref = _seats(QWEN3_1P7B_DECODE, 1, filled)
    st = _oracle(orc, cfg, w, mk, filled)  # host copies taken before the GPU touches the cache
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e = gate(np32(a), o, "bf16")
    e_paths = max_row_rel_l2(np32(a), np32(b))
    kv = max(max_row_rel_l2(np32(mk.k)[:, :, filled], st.k[:, :, filled]),
             max_row_rel_l2(np32(mk.v)[:, :, filled], st.v[:, :, filled]))
    say(f"  vs oracle {e:.2e}, vs one-kernel-per-step path {e_paths:.2e}, new K/V {kv:.2e}")
    assert kv <= BF16_TOL and e_paths <= BF16_TOL
    assert np.array_equal(np32(mk.v)[:, :, filled], np32(ref.v)[:, :, filled])  # raw v rows
    assert mk.length == filled + 1


def test_persistent_capacity_8192_last_position(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_PREFILL
    filled = QWEN3_1P7B_PREFILL.capacity - 1
    say(f"persistent decode, 1 layer, capacity 8192, position {filled}")
    cfg, w, mk, ref = _seats(QWEN3_1P7B_PREFILL, 1, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    e = gate(np32(a), st.forward(np32(x)), "bf16")
    say(f"  vs oracle {e:.2e}, vs one-kernel-per-step path {max_row_rel_l2(np32(a), np32(b)):.2e}")
    with pytest.raises(q3.Qwen3Error):
        mk.forward_hidden(x)  # the cache is full


def test_persistent_full_stack(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    filled = 4095
    say("persistent decode, 28 layers, ctx 4096")
    cfg, w, mk, ref = _seats(QWEN3_1P7B_DECODE, None, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e = max_row_rel_l2(np32(a), o)
    e_ref = max_row_rel_l2(np32(b), o)
    e_paths = max_row_rel_l2(np32(a), np32(b))
    # layer 0's new K/V rows depend on x alone and are gated; deeper layers' rows inherit the
    # bf16 drift of the residual stream and are reported, like the output
    kv0 = max(max_row_rel_l2(np32(mk.k)[0, :, filled], st.k[0, :, filled]),
              max_row_rel_l2(np32(mk.v)[0, :, filled], st.v[0, :, filled]))
    kv = max(max_row_rel_l2(np32(mk.k)[:, :, filled], st.k[:, :, filled]),
             max_row_rel_l2(np32(mk.v)[:, :, filled], st.v[:, :, filled]))
    say(f"  vs oracle {e:.2e} (one-kernel-per-step path {e_ref:.2e}), vs that path {e_paths:.2e}, "
        f"new K/V layer 0 {kv0:.2e}, all layers {kv:.2e}")
    # Through 28 layers both paths drift from the oracle (and from each other: the two differ
    # in fp32 summation order) by bf16 rounding chains, so the deep-stack figures are reported
    # with a regression bound (the drift measures ~2.8%); the gated parity is the one-layer test above.
    assert e < 0.05 and e_paths < 0.05 and kv0 <= BF16_TOL


def test_persistent_consecutive_steps(orc):
    """Eight steps in a row from position 60: every output and the cache rows written by the
    steps, against the oracle stack stepped alike (two layers, so layer l > 0 is exercised)."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    filled, n = 60, 8
    say(f"persistent decode, 2 layers, {n} steps from position {filled}")
    cfg, w, mk, ref = _seats(QWEN3_1P7B_DECODE, 2, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, n, DEV)
    outs = [mk.forward_hidden(x[i:i + 1]) for i in range(n)]
    outs_ref = [ref.forward_hidden(x[i:i + 1]) for i in range(n)]
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    xs = np32(x)
    worst = 0.0
    for i in range(n):
        o = st.forward(xs[i:i + 1])
        worst = max(worst, max_row_rel_l2(np32(outs[i]), o))
        assert max_row_rel_l2(np32(outs[i]), np32(outs_ref[i])) <= BF16_TOL
    kv = max(max_row_rel_l2(np32(mk.k)[:, :, filled:filled + n], st.k[:, :, filled:filled + n]),
             max_row_rel_l2(np32(mk.v)[:, :, filled:filled + n], st.v[:, :, filled:filled + n]))
    say(f"  worst step vs oracle {worst:.2e}, cache rows {kv:.2e}")
    assert worst <= 2 * BF16_TOL and kv <= 2 * BF16_TOL
    assert mk.length == filled + n


def test_persistent_graph_replays_match_eager():
    """One captured step replayed five times (the position is baked into the graph; each
    replay rewrites the same cache row), with eager work between replays: every replay's
    output equals the eager step's bit for bit, since both run the same kernel on the same
    inputs, and no exchange times out (fresh tags per replay)."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    filled = 777
    cfg, w, mk, _ = _seats(QWEN3_1P7B_DECODE, 3, filled)
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
    say("persistent decode: 5 graph replays equal the eager step")


def test_decode_path_selection():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32
    w = synth.model_weights(cfg, DEV)
    seat = q3.Seat(cfg, w, max_tokens=4)
    assert q3.qwen3_get_decode_path(seat.handle) == 1  # fp32: no persistent kernel
    with pytest.raises(q3.Qwen3Error):
        q3.qwen3_set_decode_path(seat.handle, 2)
    with pytest.raises(q3.Qwen3Error):
        q3.qwen3_set_decode_path(seat.handle, 3)
    q3.qwen3_set_decode_path(seat.handle, 0)


# ------------------------------------------------------------------ 8-bit weights

@pytest.mark.parametrize("filled", [4095, 0, 31, 1000])
def test_persistent_q8_one_layer_vs_oracle_and_kernels(orc, filled):
    """The persistent step with 8-bit group-quantised projections (the 1.7B shape's q8
    configuration): one layer against the oracle (weights dequantised exactly, never rounded)
    and against the one-kernel-per-step path."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_Q8
    say(f"persistent decode, 8-bit weights, 1 layer, position {filled}")
    cfg, w, mk, ref = _seats(QWEN3_1P7B_Q8, 1, filled)
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


def test_persistent_q8_full_stack(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_Q8
    filled = 4095
    say("persistent decode, 8-bit weights, 28 layers, ctx 4096")
    cfg, w, mk, ref = _seats(QWEN3_1P7B_Q8, None, filled)
    st = _oracle(orc, cfg, w, mk, filled)
    x = synth.hidden_states(cfg, 1, DEV)
    a = mk.forward_hidden(x)
    b = ref.forward_hidden(x)
    torch.cuda.synchronize()
    q3.qwen3_check_device_errors(mk.handle)
    o = st.forward(np32(x))
    e, e_ref, e_paths = max_row_rel_l2(np32(a), o), max_row_rel_l2(np32(b), o), max_row_rel_l2(np32(a), np32(b))
    say(f"  vs oracle {e:.2e} (one-kernel-per-step path {e_ref:.2e}), vs that path {e_paths:.2e}")
    assert e < 0.05 and e_paths < 0.05


def test_persistent_q8_consecutive_steps_with_qwen2_switches(orc):
    """8-bit weights with page 2's switches (no q/k norm, q|k|v bias, a sliding window of 40):
    six steps in a row from position 50 over two layers, against the oracle and the kernel path."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_Q8
    cfg0 = QWEN3_1P7B_Q8.replace(qk_norm=False, attention_bias=True, sliding_window=40)
    filled, n = 50, 6
    say(f"persistent decode, 8-bit weights + Qwen2 switches, 2 layers, {n} steps from position {filled}")
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
