"""Multi-seat batched decode (qwen3_forward_batch through the C ABI): B seats of one model, one
token each, every seat with its own cache and position.  Each output row is checked against the
oracle stack of that seat alone (rows are independent in the method), plus the new cache rows,
the seat lengths, agreement with one-seat-at-a-time steps, the fp32 / MoE / 8-bit configurations
and the error paths (which must leave every seat unchanged)."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, gate, host_layers, max_row_rel_l2, np32, oracle_threads, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def _seats(cfg, fills, max_tokens=None):
    """One weight set; one seat per entry of fills, cache pre-filled up to that position."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    w = synth.model_weights(cfg, DEV)
    seats = []
    for i, f in enumerate(fills):
        K, V = synth.kv_cache(cfg, f, DEV)
        if f:  # distinct contents per seat
            K[:, :, :f] = K[:, :, :f].roll(i + 1, dims=2)
            V[:, :, :f] = V[:, :, :f].roll(2 * i + 1, dims=2)
        st = q3.Seat(cfg, w, max_tokens=max_tokens or len(fills), k_cache=K, v_cache=V)
        st.length = f
        seats.append(st)
    return w, seats


def _oracle_row(orc, cfg, w, seat_k, seat_v, fill, x_row):
    st = orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), cfg.dtype, kcache=seat_k, vcache=seat_v)
    st.length = fill
    return st.forward(x_row), st


@pytest.mark.parametrize("n_layers", [1, 2])
def test_batch_1p7b_vs_oracle(orc, n_layers):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg = QWEN3_1P7B_DECODE.replace(n_layers=n_layers)
    fills = [4095, 100, 0, 2047, 31]
    w, seats = _seats(cfg, fills)
    hk = [np32(s.k) for s in seats]  # host copies before the step writes the caches
    hv = [np32(s.v) for s in seats]
    x = synth.hidden_states(cfg, len(fills), DEV, name="xb")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch([s.handle for s in seats], x, out)
    torch.cuda.synchronize()
    worst, worst_kv = 0.0, 0.0
    for b, f in enumerate(fills):
        ref, st = _oracle_row(orc, cfg, w, hk[b], hv[b], f, np32(x)[b:b + 1])
        e = max_row_rel_l2(np32(out)[b:b + 1], ref)
        kv = max(max_row_rel_l2(np32(seats[b].k)[:, :, f], st.k[:, :, f]),
                 max_row_rel_l2(np32(seats[b].v)[:, :, f], st.v[:, :, f]))
        worst, worst_kv = max(worst, e), max(worst_kv, kv)
        assert seats[b].length == f + 1
    say(f"batched decode 1.7B, {n_layers} layer(s), B={len(fills)}: worst row {worst:.2e}, new K/V {worst_kv:.2e}")
    tol = BF16_TOL * n_layers
    assert worst <= tol and worst_kv <= tol


def test_batch_matches_one_seat_steps():
    """The batched step and B single-seat steps (one kernel per step, the same projection
    kernels at M = 1) from identical states agree within the bf16 gate."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg = QWEN3_1P7B_DECODE.replace(n_layers=2)
    fills = [500, 7, 4000]
    w, seats = _seats(cfg, fills)
    _, single = _seats(cfg, fills, max_tokens=1)
    x = synth.hidden_states(cfg, len(fills), DEV, name="xs")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch([s.handle for s in seats], x, out)
    outs = []
    for b, s in enumerate(single):
        q3.qwen3_set_decode_path(s.handle, 1)
        outs.append(s.forward_hidden(x[b:b + 1]))
    torch.cuda.synchronize()
    e = max_row_rel_l2(np32(out), np32(torch.cat(outs)))
    say(f"batched vs one-seat steps: {e:.2e}")
    assert e <= BF16_TOL
    for b in range(len(fills)):  # new cache rows (the norms' sums run in different orders)
        assert max_row_rel_l2(np32(seats[b].v[:, :, fills[b]]), np32(single[b].v[:, :, fills[b]])) <= BF16_TOL
        assert max_row_rel_l2(np32(seats[b].k[:, :, fills[b]]), np32(single[b].k[:, :, fills[b]])) <= BF16_TOL


def test_batch_tiny_fp32(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32
    fills = [10, 0, 63 - 1]
    w, seats = _seats(cfg, fills)
    hk = [np32(s.k) for s in seats]
    hv = [np32(s.v) for s in seats]
    x = synth.hidden_states(cfg, 3, DEV, name="xt")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch([s.handle for s in seats], x, out)
    torch.cuda.synchronize()
    for b, f in enumerate(fills):
        ref, _ = _oracle_row(orc, cfg, w, hk[b], hv[b], f, np32(x)[b:b + 1])
        gate(np32(out)[b:b + 1], ref, "fp32")


@pytest.mark.parametrize("which", ["moe", "q8"])
def test_batch_moe_and_q8(orc, which):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_Q8, QWEN3_MOE
    cfg = (QWEN3_MOE if which == "moe" else QWEN3_1P7B_Q8).replace(n_layers=1)
    fills = [cfg.capacity - 1, 64, 3]
    w, seats = _seats(cfg, fills)
    hk = [np32(s.k) for s in seats]
    hv = [np32(s.v) for s in seats]
    x = synth.hidden_states(cfg, 3, DEV, name="xm")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch([s.handle for s in seats], x, out)
    torch.cuda.synchronize()
    worst = 0.0
    for b, f in enumerate(fills):
        ref, _ = _oracle_row(orc, cfg, w, hk[b], hv[b], f, np32(x)[b:b + 1])
        worst = max(worst, gate(np32(out)[b:b + 1], ref, "bf16"))
    say(f"batched decode {which}, B=3: worst row {worst:.2e}")


def test_batch_sixteen_seats_and_errors():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(dtype="bf16")
    fills = [3 * i for i in range(16)]
    w, seats = _seats(cfg, fills, max_tokens=17)
    handles = [s.handle for s in seats]
    x = synth.hidden_states(cfg, 17, DEV, name="x16")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch(handles, x[:16], out[:16])
    torch.cuda.synchronize()
    assert [s.length for s in seats] == [f + 1 for f in fills]
    _, extra = _seats(cfg, [0], max_tokens=17)
    with pytest.raises(q3.Qwen3Error):  # 17 seats
        q3.qwen3_forward_batch(handles + [extra[0].handle], x, out)
    with pytest.raises(q3.Qwen3Error):  # a seat twice
        q3.qwen3_forward_batch([handles[0], handles[1], handles[0]], x[:3], out[:3])
    w2 = synth.model_weights(cfg.replace(seed=5), DEV)
    other = q3.Seat(cfg, w2, max_tokens=4)
    with pytest.raises(q3.Qwen3Error):  # another weight set
        q3.qwen3_forward_batch([handles[0], other.handle], x[:2], out[:2])
    seats[3].length = cfg.capacity  # full
    with pytest.raises(q3.Qwen3Error):
        q3.qwen3_forward_batch(handles[:5], x[:5], out[:5])
    assert [s.length for s in seats[:3]] == [f + 1 for f in fills[:3]]  # unchanged by the failed calls
