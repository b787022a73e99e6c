"""Host-only checks of the C ABI: the library loads, exports every function the
headers declare, and rejects bad configurations before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in ("qwen3.h", "qwen3_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(qwen3_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from qwen3_transformer_layer_amd import _lib
    return _lib.load()


def test_headers_declare_the_boundary():
    names = declared_functions()
    for required in ("qwen3_init", "qwen3_reset", "qwen3_forward", "qwen3_forward_hidden", "qwen3_moe_block",
                     "qwen3_workspace_bytes", "qwen3_set_length", "qwen3_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_library_has_no_oracle_dependency():
    import subprocess
    from qwen3_transformer_layer_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "orc_" not in out
    deps = subprocess.run(["ldd", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def _cfg(**kw):
    from qwen3_transformer_layer_amd import c_config
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
    return c_config(QWEN3_1P7B_DECODE.replace(**kw), 1)


def test_workspace_bytes_valid_and_invalid(lib):
    good = _cfg()
    assert lib.qwen3_workspace_bytes(ctypes.byref(good)) > 0
    for bad in (dict(head_dim=96), dict(n_kv_heads=3), dict(dtype="fp32", quant_bits=8),
                dict(intermediate=100), dict(n_layers=0)):
        from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE
        try:
            c = _cfg(**bad)
        except KeyError:
            continue
        assert lib.qwen3_workspace_bytes(ctypes.byref(c)) == 0, bad


def test_init_rejects_bad_configs_before_any_gpu_work(lib):
    from qwen3_transformer_layer_amd import _lib
    h = ctypes.c_void_p()
    layers = (_lib.LayerWeights * 28)()
    w = _lib.Weights(None, None, None, None, layers)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every check runs before device work
    c = _cfg()
    c.dtype = 7
    assert lib.qwen3_init(ctypes.byref(c), ctypes.byref(w), fake, fake, fake, 1 << 40, None, ctypes.byref(h)) == \
        _lib.ERR_DTYPE
    c = _cfg(head_dim=96)
    assert lib.qwen3_init(ctypes.byref(c), ctypes.byref(w), fake, fake, fake, 1 << 40, None, ctypes.byref(h)) == \
        _lib.ERR_UNSUPPORTED
    c = _cfg()
    assert lib.qwen3_init(ctypes.byref(c), ctypes.byref(w), fake, fake, fake, 16, None, ctypes.byref(h)) == \
        _lib.ERR_WORKSPACE
    assert lib.qwen3_init(ctypes.byref(c), ctypes.byref(w), fake, fake, fake, 1 << 40, None, ctypes.byref(h)) == \
        _lib.ERR_NULL_WEIGHT
    assert not h.value


def test_ops_reject_bad_arguments_before_launch(lib):
    from qwen3_transformer_layer_amd import _lib
    fake = ctypes.c_void_p(1 << 20)
    assert lib.qwen3_op_linear(5, fake, 1, 64, fake, 8, 0, None, fake, None) == _lib.ERR_DTYPE
    assert lib.qwen3_op_linear(0, fake, 1, 100, fake, 8, 0, None, fake, None) == _lib.ERR_ARG      # K % 64
    assert lib.qwen3_op_linear(0, fake, 1, 64, fake, 8, 1, None, fake, None) == _lib.ERR_ARG       # RESID, no res
    assert lib.qwen3_op_attention(0, fake, fake, fake, 1, 6, 2, 128, 64, 0, fake, fake, 1 << 30, None) == \
        _lib.ERR_UNSUPPORTED                                                                        # group of 3
    assert lib.qwen3_op_attention(0, fake, fake, fake, 4, 4, 2, 128, 64, 61, fake, fake, 1 << 30, None) == \
        _lib.ERR_ARG                                                                                # p0 + T > cap
    assert lib.qwen3_rope_table(64, 96, 1e6, 0, fake, fake, None) == _lib.ERR_ARG
    assert lib.qwen3_op_stream_read(fake, 24, fake, None) == _lib.ERR_ARG                        # not 16-byte words
    assert lib.qwen3_op_stream_read(ctypes.c_void_p((1 << 20) + 8), 64, fake, None) == _lib.ERR_ARG  # misaligned
    assert lib.qwen3_op_stream_read(None, 64, fake, None) == _lib.ERR_ARG
    assert lib.qwen3_status_string(-3) == b"context exceeds capacity"


def test_init_rejects_misaligned_pointers_before_any_gpu_work(lib):
    """Every weight, cache and table pointer must be 16-byte aligned (the kernels read rows
    with 16-byte vector loads); a misaligned one is rejected on the host, before any HIP
    call, so this runs without a GPU and the fake addresses are never dereferenced."""
    from qwen3_transformer_layer_amd import _lib
    c = _cfg(n_layers=2)
    need = lib.qwen3_workspace_bytes(ctypes.byref(c))
    base = 1 << 32
    fields = [n for n, _ in _lib.LayerWeights._fields_]
    plain = {"in_norm", "post_norm", "q_norm", "k_norm", "qkv", "o", "gate_up", "down"}
    for bad in ("in_norm", "q_norm", "qkv", "down", "kc", "vc", "embed", "final_norm", "rope"):
        layers = (_lib.LayerWeights * 2)()
        for l in range(2):
            for i, name in enumerate(fields):
                if name in plain:
                    setattr(layers[l], name, base + (1 + l * 64 + i) * 4096 + (2 if bad == name and l == 1 else 0))
        emb = base + 900 * 4096 + (8 if bad == "embed" else 0)
        fn = base + 901 * 4096 + (2 if bad == "final_norm" else 0)
        rc_ = (base + 902 * 4096 + (4 if bad == "rope" else 0), base + 903 * 4096)
        w = _lib.Weights(emb, fn, rc_[0], rc_[1], layers)
        kc = ctypes.c_void_p(base + 904 * 4096 + (2 if bad == "kc" else 0))
        vc = ctypes.c_void_p(base + 905 * 4096 + (6 if bad == "vc" else 0))
        ws = ctypes.c_void_p(base + 4096 * 4096)
        h = ctypes.c_void_p()
        assert lib.qwen3_init(ctypes.byref(c), ctypes.byref(w), kc, vc, ws, need, None, ctypes.byref(h)) == \
            _lib.ERR_ARG, bad
        assert not h.value
