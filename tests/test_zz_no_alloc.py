"""qwen3_head_static (no handle, no workspace, no allocation: its greedy-token keys sit in the
library's per-device static array) against qwen3_head on the same inputs, through the C ABI:
two calls in a row, the second with fewer rows and a shorter head, in bf16 and fp32; logits
must be identical and the greedy tokens equal (integer results: exact)."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import np32, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_head_static_matches_head(dtype):
    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import _lib, synth
    from qwen3_transformer_layer_amd.config import TINY_FP32
    cfg = TINY_FP32.replace(dtype=dtype, n_layers=1)
    w = synth.model_weights(cfg, DEV)
    seat = q3.Seat(cfg, w, max_tokens=64)
    L = _lib.load()
    code = q3.DTYPES[dtype]
    stream = torch.cuda.current_stream()
    for T, V in ((40, 5003), (7, 3001)):  # the second call is smaller: stale keys must not leak
        say(f"head_static {dtype}: T={T} V={V}")
        hs = synth.hidden_states(cfg, T, DEV, name=f"hs{T}")
        W = synth.linear_weight(cfg, f"head{V}", (V, cfg.hidden), DEV)
        lg_a = torch.full((T, V), float("nan"), device=DEV)
        am_a = torch.full((T,), -1, dtype=torch.int32, device=DEV)
        q3.qwen3_head(seat.handle, hs, W, lg_a, am_a)
        lg_b = torch.full((T, V), float("nan"), device=DEV)
        am_b = torch.full((T,), -1, dtype=torch.int32, device=DEV)
        rc = L.qwen3_head_static(code, _p(hs), T, cfg.hidden, _p(W), V, _p(lg_b), _p(am_b),
                                 ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, rc
        am_only = torch.full((T,), -1, dtype=torch.int32, device=DEV)
        rc = L.qwen3_head_static(code, _p(hs), T, cfg.hidden, _p(W), V, None, _p(am_only),
                                 ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, rc
        torch.cuda.synchronize()
        a, b = np32(lg_a), np32(lg_b)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(am_a.cpu().numpy(), am_b.cpu().numpy())
        assert np.array_equal(am_a.cpu().numpy(), am_only.cpu().numpy())
        assert np.array_equal(am_b.cpu().numpy(), np.argmax(b, axis=1))
    q3.qwen3_check_device_errors(seat.handle)


def test_head_static_rejects_bad_arguments_before_launch():
    from qwen3_transformer_layer_amd import _lib
    L = _lib.load()
    x = torch.zeros((300, 256), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((10, 256), dtype=torch.bfloat16, device=DEV)
    am = torch.zeros(300, dtype=torch.int32, device=DEV)
    assert L.qwen3_head_static(0, _p(x), 257, 256, _p(W), 10, None, _p(am), None) == _lib.ERR_ARG  # T > 256
    assert L.qwen3_head_static(0, _p(x), 0, 256, _p(W), 10, None, _p(am), None) == _lib.ERR_ARG
    assert L.qwen3_head_static(0, _p(x), 4, 256, _p(W), 10, None, None, None) == _lib.ERR_ARG    # no output
    assert L.qwen3_head_static(3, _p(x), 4, 256, _p(W), 10, None, _p(am), None) == _lib.ERR_DTYPE
    assert L.qwen3_head_static(0, ctypes.c_void_p(x.data_ptr() + 2), 4, 256, _p(W), 10, None, _p(am), None) == \
        _lib.ERR_ARG                                                                                    # misaligned
