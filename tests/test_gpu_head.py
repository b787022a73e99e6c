"""Output head + greedy token (qwen3_head through the C ABI) against the CPU oracle.

Logits: per-row relative L2 against the oracle's fp32(rho(hs . W^T)) (bf16: one rounding of an
fp32-accumulated dot on both sides, so they differ only where the two summation orders round
to neighbouring bf16 values).  Greedy token: exact against the first maximum of the kernel's
own logits (both decisions in the same precision); against the oracle exact wherever the
oracle's top-2 margin exceeds two bf16 steps of the top logit, else the pick's oracle logit must
be within that margin of the maximum.  Covers the page's 2049-row head and a 151,936-row
vocabulary at hidden 2048, T = 1 / 5 / 20 (20 takes two 16-row passes), the tied embedding in
fp32, duplicate-row ties, NaN rows and the error paths."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, max_row_rel_l2, np32, oracle_threads, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


def _seat(cfg, max_tokens):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    cfg = cfg.replace(n_layers=1)
    w = synth.model_weights(cfg, DEV)
    return cfg, w, q3.Seat(cfg, w, max_tokens=max_tokens)


def _check_pick(gl, ga, ol, oa):
    """gl/ol: GPU / oracle logits [T][V]; ga/oa: picks [T]."""
    for t in range(gl.shape[0]):
        row = gl[t]
        assert ga[t] == int(np.argmax(row)), f"row {t}: pick {ga[t]} is not the first maximum of its own logits"
        top2 = np.sort(ol[t])[-2:]
        margin = 2.0 * 2.0 ** (np.floor(np.log2(abs(top2[1]) + 1e-30)) - 7)
        if top2[1] - top2[0] > margin:
            assert ga[t] == oa[t], f"row {t}: pick {ga[t]} vs oracle {oa[t]} (margin {top2[1] - top2[0]:.3e})"
        else:
            assert ol[t, ga[t]] >= top2[1] - margin


@pytest.mark.parametrize("V,T", [(2049, 1), (2049, 20), (151936, 1), (151936, 5)])
def test_head_bf16_vs_oracle(orc, V, T):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg, _, seat = _seat(QWEN3_1P7B_DECODE, 32)
    W = synth.linear_weight(cfg, "head", (V, cfg.hidden), DEV)
    hs = synth.hidden_states(cfg, T, DEV, name="hs")
    logits = torch.empty((T, V), dtype=torch.float32, device=DEV)
    am = torch.empty(T, dtype=torch.int32, device=DEV)
    q3.qwen3_head(seat.handle, hs, W, logits, am)
    am_only = torch.empty(T, dtype=torch.int32, device=DEV)
    q3.qwen3_head(seat.handle, hs, W, None, am_only)  # argmax without the logits pass-through
    torch.cuda.synchronize()
    ol, oa = orc.head(np32(hs), np32(W), "bf16")
    gl, ga = np32(logits), am.cpu().numpy()
    e = max_row_rel_l2(gl, ol)
    say(f"head bf16 V={V} T={T}: logits row rel L2 {e:.2e}, equal {np.mean(gl == ol):.4f}, picks {ga.tolist()[:5]}")
    assert e < 6e-3
    _check_pick(gl, ga, ol, oa)
    assert np.array_equal(am_only.cpu().numpy(), ga)


def test_head_tied_embedding_fp32(orc):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg, w, seat = _seat(TINY_FP32, 8)
    hs = synth.hidden_states(cfg, 7, DEV, name="hs")
    logits = torch.empty((7, cfg.vocab), dtype=torch.float32, device=DEV)
    am = torch.empty(7, dtype=torch.int32, device=DEV)
    q3.qwen3_head(seat.handle, hs, None, logits, am)
    torch.cuda.synchronize()
    ol, oa = orc.head(np32(hs), np32(w["embed"]), "fp32")
    e = float(np.max(np.abs(np32(logits) - ol)) / np.sqrt(np.mean(ol.astype(np.float64) ** 2)))
    say(f"head fp32 tied V={cfg.vocab}: max|d|/RMS {e:.2e}")
    assert e <= 1e-4
    _check_pick(np32(logits), am.cpu().numpy(), ol, oa)


def test_head_ties_and_nan_rows():
    """Rows 7, 31 and 40 are copies of the best row: the pick is 7.  Row 3 is NaN: never picked."""
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg, _, seat = _seat(QWEN3_1P7B_DECODE, 4)
    hs = synth.hidden_states(cfg, 1, DEV, name="hs")
    W = synth.linear_weight(cfg, "head_ties", (64, cfg.hidden), DEV)
    W = -(W.float().abs() * torch.sign(hs.float())).to(torch.bfloat16)  # every row scores <= 0
    best = synth.linear_weight(cfg, "head_best", (1, cfg.hidden), DEV)
    best = (best.float().abs() * torch.sign(hs.float())).to(torch.bfloat16)  # scores > 0
    for r in (7, 31, 40):
        W[r] = best[0]
    W[3] = float("nan")
    W = W.contiguous()
    logits = torch.empty((1, 64), dtype=torch.float32, device=DEV)
    am = torch.empty(1, dtype=torch.int32, device=DEV)
    q3.qwen3_head(seat.handle, hs, W, logits, am)
    torch.cuda.synchronize()
    gl = np32(logits)[0]
    assert gl[7] == gl[31] == gl[40] and gl[7] > 0 and np.isnan(gl[3])
    assert int(am.item()) == 7


def test_head_errors():
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    cfg, _, seat = _seat(QWEN3_1P7B_DECODE, 4)  # no vocab: no embedding table
    hs = synth.hidden_states(cfg, 2, DEV, name="hs")
    am = torch.empty(2, dtype=torch.int32, device=DEV)
    with pytest.raises(q3.Qwen3Error):
        q3.qwen3_head(seat.handle, hs, None, None, am)  # tied, but no table
    W = synth.linear_weight(cfg, "head", (100, cfg.hidden), DEV)
    with pytest.raises(q3.Qwen3Error):
        q3.qwen3_head(seat.handle, hs, W, None, None)  # nothing requested
    big = synth.hidden_states(cfg, 5, DEV, name="hs5")
    with pytest.raises(q3.Qwen3Error):
        q3.qwen3_head(seat.handle, big, W, None, torch.empty(5, dtype=torch.int32, device=DEV))  # T > max_tokens
