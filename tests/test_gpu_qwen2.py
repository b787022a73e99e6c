"""Page 2's decoder switches through the C ABI against the CPU oracle ("rlx_flow/blocks/
qwen3_decoder.rs", Qwen3DecoderSpec): qk_norm off (Qwen2: RoPE on the projections), q/k/v bias
(each element rho(x + b) after the projection) and the SlidingWindow(w) mask (the query at p
sees keys max(0, p-w+1)..p), alone and together, on every attention kernel: split-K decode
(one seat and batched), the head_dim-128 flash prefill, the head_dim-64 MFMA prefill and the
fp32 row-wise kernel.  Windows cut keys inside tiles, at tile edges, below the first tile of a
block, and in both the prefill and the decode phase; w = 1 and w >= capacity are covered.

Gates: fp32 max|d|/RMS <= 1e-4; bf16 per-row relative L2 <= 2e-2 per layer."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, gate, host_layers, max_row_rel_l2, np32, oracle_threads, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def _run(orc, cfg, chunks, filled=0, max_tokens=None, path=None):
    """GPU seat and oracle stack from the same weights and pre-fill; forward each chunk length."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    w = synth.model_weights(cfg, DEV)
    K, V = synth.kv_cache(cfg, filled, DEV)
    st = orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), cfg.dtype, kcache=np32(K), vcache=np32(V))
    st.length = filled
    seat = q3.Seat(cfg, w, max_tokens=max_tokens or max(chunks), k_cache=K, v_cache=V)
    seat.length = filled
    if path is not None:
        q3.qwen3_set_decode_path(seat.handle, path)
    x = synth.hidden_states(cfg, sum(chunks), DEV)
    outs, refs, t = [], [], 0
    for n in chunks:
        outs.append(seat.forward_hidden(x[t:t + n]))
        t += n
    torch.cuda.synchronize()
    xn, t = np32(x), 0
    for n in chunks:
        refs.append(st.forward(xn[t:t + n]))
        t += n
    return seat, st, np32(torch.cat(outs)), np.concatenate(refs)


@pytest.mark.parametrize("qk_norm,bias,window", [(False, True, 0), (False, True, 5), (True, False, 7),
                                                 (True, True, 1), (False, False, 64)])
def test_tiny_fp32_switches(orc, qk_norm, bias, window):
    """fp32 row-wise prefill and split-K decode: a 20-token prefill then 5 decode steps."""
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(qk_norm=qk_norm, attention_bias=bias, sliding_window=window)
    seat, st, got, ref = _run(orc, cfg, [20, 1, 1, 1, 1, 1])
    e = gate(got, ref, "fp32")
    say(f"tiny fp32 qk_norm={qk_norm} bias={bias} window={window}: max|d|/RMS {e:.2e}")
    assert np.array_equal(np32(seat.k)[:, :, :25] != 0, st.k[:, :, :25] != 0)


@pytest.mark.parametrize("window,chunks", [(3, [100, 1, 1]), (64, [130, 1]), (70, [57, 64, 1]), (1, [33, 1])])
def test_head_dim64_bf16_window(orc, window, chunks):
    """head_dim 64, bf16: the 16x16x32 MFMA prefill (64-key tiles) with windows inside a tile, of
    one tile, across tiles, and of one key; a second prefill call starts at p0 > 0."""
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(dtype="bf16", n_layers=1, sliding_window=window, capacity=256)
    _, _, got, ref = _run(orc, cfg, chunks)
    e = gate(got, ref, "bf16")
    say(f"head_dim 64 bf16 window={window} chunks={chunks}: {e:.2e}")


@pytest.mark.parametrize("window,T", [(1, 1024), (33, 1024), (512, 1024), (5000, 1024), (700, 2048)])
def test_1p7b_prefill_window(orc, window, T):
    """The 1.7B shape (head_dim 128, flash prefill), one layer from an empty cache: a window
    smaller than a 32-query tile, one spanning tile boundaries, a long one and one wider than
    the context (causal); at T = 2048 the flash kernel pairs query tiles (63 and 0, 62 and 1, ...)."""
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_PREFILL
    cfg = QWEN3_1P7B_PREFILL.replace(n_layers=1, sliding_window=window, capacity=2048)
    seat, st, got, ref = _run(orc, cfg, [T])
    e = gate(got, ref, "bf16")
    ek = max_row_rel_l2(np32(seat.k)[0, :, :T], st.k[0, :, :T])
    say(f"1.7B prefill T={T} window={window}: out {e:.2e}, K {ek:.2e}")
    assert ek <= BF16_TOL


@pytest.mark.parametrize("qk_norm,bias", [(True, False), (False, True), (True, True)])
def test_1p7b_prefill_fused_qkv_epilogue(orc, qk_norm, bias):
    """Two 1600-token prefill calls on the 1.7B attention shape, the second at p0 = 1600: both
    take the q|k|v GEMM whose epilogue does the q/k norm, RoPE and K/V cache write (256 x 128
    tiles, the last row tile ragged), with and without the q/k norm and bias; the MLP is
    narrowed to keep the oracle quick."""
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_PREFILL
    cfg = QWEN3_1P7B_PREFILL.replace(n_layers=1, qk_norm=qk_norm, attention_bias=bias, intermediate=512,
                                     capacity=3200)
    seat, st, got, ref = _run(orc, cfg, [1600, 1600])
    e = gate(got, ref, "bf16")
    ek = max_row_rel_l2(np32(seat.k)[0, :, :3200], st.k[0, :, :3200])
    ev = max_row_rel_l2(np32(seat.v)[0, :, :3200], st.v[0, :, :3200])
    say(f"1.7B fused q|k|v prefill qk_norm={qk_norm} bias={bias}: out {e:.2e}, K {ek:.2e}, V {ev:.2e}")
    assert ek <= BF16_TOL and ev <= BF16_TOL and seat.length == 3200


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("qk_norm,bias,window", [(True, False, 1000), (False, True, 0), (False, True, 300)])
def test_1p7b_decode_switches(orc, qk_norm, bias, window, path):
    """Decode at position 4095 (ctx 4096) on the kernel-per-step path (1) and on the persistent
    kernel (2: bias as its own rounded add, no q/k norm, attention splits over the window's
    keys), then a 64-token chunk at p0 = 4096."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg = QWEN3_1P7B_DECODE.replace(n_layers=1, qk_norm=qk_norm, attention_bias=bias, sliding_window=window,
                                    capacity=4160)
    seat, st, got, ref = _run(orc, cfg, [1, 64], filled=4095, path=path)
    assert q3.qwen3_get_decode_path(seat.handle) == path
    q3.qwen3_check_device_errors(seat.handle)
    e1 = gate(got[:1], ref[:1], "bf16")
    e2 = gate(got[1:], ref[1:], "bf16")
    say(f"1.7B decode qk_norm={qk_norm} bias={bias} window={window}: decode {e1:.2e}, chunk {e2:.2e}")


@pytest.mark.parametrize("window,filled", [(1, 0), (1, 4095), (7, 3), (7, 40), (300, 299), (300, 300), (5000, 4095)])
def test_persistent_decode_window_edges(orc, window, filled):
    """The persistent kernel's window bounds at one decode step: a window of one key, windows
    just wider and just narrower than p + 1, one wider than the context, and position 0."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg = QWEN3_1P7B_DECODE.replace(n_layers=1, sliding_window=window, capacity=4096)
    seat, st, got, ref = _run(orc, cfg, [1], filled=filled, path=2)
    assert q3.qwen3_get_decode_path(seat.handle) == 2
    q3.qwen3_check_device_errors(seat.handle)
    e = gate(got, ref, "bf16")
    say(f"persistent decode window={window} at position {filled}: {e:.2e}")


@pytest.mark.parametrize("path", [1, 2])
def test_window_wider_than_capacity_is_causal_bitwise(path):
    """sliding_window >= capacity changes nothing: identical outputs and caches, on either decode
    path."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    base = QWEN3_1P7B_DECODE.replace(n_layers=2, capacity=512)
    wide = base.replace(sliding_window=512)
    w = synth.model_weights(base, DEV)
    a = q3.Seat(base, w, max_tokens=100)
    b = q3.Seat(wide, w, max_tokens=100)
    q3.qwen3_set_decode_path(a.handle, path)
    q3.qwen3_set_decode_path(b.handle, path)
    x = synth.hidden_states(base, 103, DEV)
    ga = torch.cat([a.forward_hidden(x[:100])] + [a.forward_hidden(x[100 + i:101 + i]) for i in range(3)])
    gb = torch.cat([b.forward_hidden(x[:100])] + [b.forward_hidden(x[100 + i:101 + i]) for i in range(3)])
    torch.cuda.synchronize()
    assert torch.equal(ga, gb) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)


def test_batched_decode_switches(orc):
    """Batched decode with bias, no q/k norm and a window of 200: seats before, at and far past
    the window length."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg = QWEN3_1P7B_DECODE.replace(n_layers=1, qk_norm=False, attention_bias=True, sliding_window=200,
                                    capacity=2048)
    w = synth.model_weights(cfg, DEV)
    fills = [50, 199, 200, 2047, 0]
    seats, hk, hv = [], [], []
    for i, f in enumerate(fills):
        K, V = synth.kv_cache(cfg, f, DEV)
        if f:
            K[:, :, :f] = K[:, :, :f].roll(i + 1, dims=2)
        s = q3.Seat(cfg, w, max_tokens=len(fills), k_cache=K, v_cache=V)
        s.length = f
        seats.append(s)
        hk.append(np32(K))
        hv.append(np32(V))
    x = synth.hidden_states(cfg, len(fills), DEV, name="xb")
    out = torch.empty_like(x)
    q3.qwen3_forward_batch([s.handle for s in seats], x, out)
    torch.cuda.synchronize()
    worst = 0.0
    for b, f in enumerate(fills):
        st = orc.Stack(cfg, host_layers(orc, cfg, w), np32(w["final_norm"]), "bf16", kcache=hk[b], vcache=hv[b])
        st.length = f
        worst = max(worst, gate(np32(out)[b:b + 1], st.forward(np32(x)[b:b + 1]), "bf16"))
        assert max_row_rel_l2(np32(seats[b].v)[:, :, f], st.v[:, :, f]) <= BF16_TOL  # v + bias in the cache
    say(f"batched decode, Qwen2 switches, window 200: worst row {worst:.2e}")


def test_moe_decode_window(orc):
    """The MoE stack's attention with a window (decode at 2047, window 256)."""
    from qwen3_transformer_layer_amd.config import QWEN3_MOE
    cfg = QWEN3_MOE.replace(n_layers=1, sliding_window=256)
    _, _, got, ref = _run(orc, cfg, [1], filled=2047)
    e = gate(got, ref, "bf16")
    say(f"MoE decode window 256: {e:.2e}")


def test_switch_weight_errors():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(n_layers=1)
    w = synth.model_weights(cfg, DEV)
    bad = {**w, "layers": [{k: v for k, v in w["layers"][0].items() if k != "k_norm"}]}
    with pytest.raises(q3.Qwen3Error):  # q_norm without k_norm
        q3.Seat(cfg, bad, max_tokens=4)
    with pytest.raises(q3.Qwen3Error):
        q3.Seat(cfg.replace(sliding_window=-1), w, max_tokens=4)
