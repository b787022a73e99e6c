"""Per-kernel parity: each HIP kernel (through the C ABI in qwen3_ops.h) against the CPU
oracle on identical seeded inputs, at sizes spanning several tiles and ragged tails."""
import numpy as np
import pytest
import torch

from helpers import BF16_TOL, max_rel_rms, max_row_rel_l2, np32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    from qwen3_transformer_layer_amd import ops as o
    o._lib.load()
    return o


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def randn(shape, seed, scale=1.0, dtype=torch.bfloat16):
    return (scale * torch.randn(shape, generator=_gen(seed), device=DEV)).to(dtype)


TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_table_bitwise(orc, dtype, D):
    from qwen3_transformer_layer_amd import qwen3_rope_table
    for theta in (1e6, 1e7):
        c, s = qwen3_rope_table(8192, D, theta, dtype)
        torch.cuda.synchronize()
        oc, os_ = orc.rope_table(8192, D, theta, dtype)
        nc = int(np.sum(np32(c) != oc))
        ns = int(np.sum(np32(s) != os_))
        say(f"rope table {dtype} D={D} theta={theta}: cos mismatches {nc}, sin mismatches {ns}")
        assert nc == 0 and ns == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n", [256, 2048, 4096])
def test_add_rmsnorm(orc, dtype, n, ops):
    dt = TDT[dtype]
    h = randn((7, n), 1, 1.0, dt)
    r = randn((7, n), 2, 1.0, dt)
    w = (1 + randn((n,), 3, 0.1, torch.float32)).to(dt)
    hout = torch.empty_like(h)
    y = ops.add_rmsnorm(h, w, 1e-6, res=r, h_out=hout)
    y0 = ops.add_rmsnorm(h, w, 1e-6)
    torch.cuda.synchronize()
    hs = orc.round_(np32(h) + np32(r), dtype)
    assert np.array_equal(np32(hout), hs)  # one rounding of an exact fp32 sum
    ref = orc.rmsnorm(hs, np32(w), 1e-6, dtype)
    ref0 = orc.rmsnorm(np32(h), np32(w), 1e-6, dtype)
    for got, rf in ((np32(y), ref), (np32(y0), ref0)):
        if dtype == "fp32":
            assert max_rel_rms(got, rf) < 1e-6
        else:
            assert np.mean(got == rf) > 0.99 and max_row_rel_l2(got, rf) < 4e-3


# 2 <= M <= 16 in bf16 with K % 256 == 0: the skinny MFMA GEMV, on 8 outputs per block for K 2048 /
# 4096 / 6144 when 16-output blocks would be too few ((3, 2048, 384), (5, 4096, 1000), (7, 6144, 130),
# ragged N) and on 16 otherwise ((16, 256, 512)); M = 1 the plain GEMV.  MFMA tilings (the largest
# with >= 192 tiles): (520, 128, 8200) 256 x 128 (SWIGLU 128 x 256); (2000, 128, 1900) and
# (1600, 256, 1800) 128 x 128 in two K groups (SWIGLU 128 x 256); (300, 192, 4100) SWIGLU
# 128 x 128 with 8 waves, the others 128 x 64 in two K groups; the remaining M > 16 cases
# 128 x 64 in two K groups (SWIGLU 64 x 128).  Ragged M and N.
LIN_CASES = [(1, 2048, 4096), (3, 2048, 384), (16, 256, 512), (40, 512, 384), (300, 2048, 640), (130, 6144, 256),
             (520, 128, 8200), (2000, 128, 1900), (300, 192, 4100), (17, 64, 200), (7, 6144, 130),
             (5, 4096, 1000), (1600, 256, 1800)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("epi", [0, 1, 2])
@pytest.mark.parametrize("M,K,N", LIN_CASES)
def test_linear(orc, ops, dtype, epi, M, K, N):
    dt = TDT[dtype]
    x = randn((M, K), 10 + M, 1.0, dt)
    rows = 2 * N if epi == 2 else N
    W = randn((rows, K), 20 + K, 0.02, dt)
    res = randn((M, N), 30, 1.0, dt) if epi == 1 else None
    out = ops.linear(x, W, epi, res)
    torch.cuda.synchronize()
    acc = orc.linear(np32(x), np32(W), dtype)
    if epi == 0:
        ref = acc
    elif epi == 1:
        ref = orc.round_(np32(res) + acc, dtype)
    else:
        ref = orc.swiglu(acc, dtype)
    got = np32(out)
    e = max_row_rel_l2(got, ref)
    say(f"linear {dtype} epi={epi} M={M} K={K} N={N}: row rel L2 {e:.2e}, equal {np.mean(got == ref):.4f}")
    assert e < (2e-5 if dtype == "fp32" else 6e-3)


@pytest.mark.parametrize("epi", [0, 1, 2])
# K = 320 (an odd number of groups) takes the register-staged 8-bit GEMM; the other M > 16
# cases the LDS-DMA one, whose tiling follows the tile count: (1030, 256, 5400) 128 x 256 with
# 8 waves for every epilogue; (1030, 256, 2800) that tiling for SwiGLU, 64 x 128 with 8 waves
# (copies padded with dummies) otherwise; (1030, 256, 1400) 128 x 128 for SwiGLU; the smaller
# ones 64 x 64 (store, residual: 2 K groups of 4 waves) and 64 x 128 (SwiGLU) with 4 waves
@pytest.mark.parametrize("M,K,N", [(1, 2048, 4096), (5, 6144, 256), (40, 2048, 384), (512, 2048, 640),
                                   (200, 6144, 136), (40, 320, 96), (1030, 256, 2800), (1030, 256, 5400),
                                   (1030, 256, 1400), (17, 128, 72)])
def test_linear_q8(orc, ops, epi, M, K, N):
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_Q8
    rows = 2 * N if epi == 2 else N
    q, s, b = synth.q8_weight(QWEN3_1P7B_Q8, f"t{M}.{K}.{N}", rows, K, DEV)
    x = randn((M, K), 40 + M)
    res = randn((M, N), 41) if epi == 1 else None
    out = ops.linear_q8(x, q, s, b, epi, res)
    torch.cuda.synchronize()
    W = orc.q8_dequant(q.cpu().numpy(), np32(s), np32(b), 64)
    acc = orc.linear(np32(x), W, "bf16")
    ref = acc if epi == 0 else (orc.round_(np32(res) + acc, "bf16") if epi == 1 else orc.swiglu(acc, "bf16"))
    e = max_row_rel_l2(np32(out), ref)
    say(f"linear_q8 epi={epi} M={M} K={K} N={N}: row rel L2 {e:.2e}")
    assert e < 6e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("H,KV,D", [(16, 8, 128), (32, 4, 128), (4, 2, 64)])
def test_qknorm_rope_kv(orc, ops, dtype, H, KV, D):
    dt = TDT[dtype]
    T, cap, p0 = 5, 64, 17
    qkv = randn((T, (H + 2 * KV) * D), 50, 1.0, dt)
    qn = (1 + randn((D,), 51, 0.1, torch.float32)).to(dt)
    kn = (1 + randn((D,), 52, 0.1, torch.float32)).to(dt)
    c, s = orc.rope_table(cap, D, 1e6, dtype)
    ct, st = torch.from_numpy(c).to(DEV, dt), torch.from_numpy(s).to(DEV, dt)
    kc = torch.zeros((KV, cap, D), dtype=dt, device=DEV)
    vc = torch.zeros_like(kc)
    q = ops.qknorm_rope_kv(qkv, H, KV, D, qn, kn, 1e-6, ct, st, p0, kc, vc)
    torch.cuda.synchronize()
    x = np32(qkv).reshape(T, H + 2 * KV, D)
    wq, wk = np32(qn), np32(kn)
    ref_q = np.stack([orc.rope(orc.rmsnorm(x[t, :H], wq, 1e-6, dtype), c[p0 + t], s[p0 + t], dtype) for t in range(T)])
    ref_k = np.stack([orc.rope(orc.rmsnorm(x[t, H:H + KV], wk, 1e-6, dtype), c[p0 + t], s[p0 + t], dtype)
                      for t in range(T)])
    gk = np32(kc)
    gv = np32(vc)
    e_q = max_row_rel_l2(np32(q), ref_q)
    e_k = max_row_rel_l2(gk[:, p0:p0 + T].transpose(1, 0, 2), ref_k)
    say(f"qknorm_rope_kv {dtype} H={H} KV={KV} D={D}: q {e_q:.2e} k {e_k:.2e}")
    tol = 1e-6 if dtype == "fp32" else 8e-3
    assert e_q < tol and e_k < tol
    assert np.array_equal(gv[:, p0:p0 + T].transpose(1, 0, 2), x[:, H + KV:])
    assert not gk[:, :p0].any() and not gk[:, p0 + T:].any() and not gv[:, p0 + T:].any()


ATT_DECODE = [(16, 8, 128, 4096, 4095), (16, 8, 128, 4096, 0), (16, 8, 128, 4096, 63), (32, 4, 128, 2048, 2047),
              (32, 4, 128, 2048, 64), (4, 2, 64, 64, 31), (8, 8, 64, 300, 257), (8, 1, 128, 128, 100)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("H,KV,D,cap,p0", ATT_DECODE)
def test_attention_decode(orc, ops, dtype, H, KV, D, cap, p0):
    dt = TDT[dtype]
    q = randn((1, H, D), 60, 1.0, dt)
    kc = randn((KV, cap, D), 61, 1.0, dt)
    vc = randn((KV, cap, D), 62, 1.0, dt)
    out = ops.attention(q, kc, vc, p0)
    torch.cuda.synchronize()
    ref = orc.attention(np32(q), np32(kc), np32(vc), p0, dtype)
    e = max_row_rel_l2(np32(out).reshape(H, D), ref.reshape(H, D))
    say(f"attention decode {dtype} H={H} KV={KV} D={D} p0={p0}: {e:.2e}")
    assert e < (2e-6 if dtype == "fp32" else 8e-3)


# head_dim 128 takes attn_prefill_fa_kernel (G = 2, 4, 8 and 1 below), head_dim 64 the
# 16x16x32 kernel.  (513, 7, 32, 32, ...) has 17 query tiles x 32 kv heads, enough blocks for the
# flash kernel's paired query tiles (16 and 0, 15 and 1, ..., 8 alone).
ATT_PREFILL = [(2, 0, 16, 8, 128, 64), (40, 7, 16, 4, 128, 64), (33, 0, 16, 16, 64, 64), (70, 0, 16, 8, 128, 128),
               (64, 5, 4, 2, 64, 128), (200, 100, 32, 4, 128, 512), (130, 0, 8, 8, 64, 256), (16, 48, 4, 2, 64, 64),
               (97, 30, 8, 8, 128, 160), (513, 7, 32, 32, 128, 576)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T,p0,H,KV,D,cap", ATT_PREFILL)
def test_attention_prefill(orc, ops, dtype, T, p0, H, KV, D, cap):
    dt = TDT[dtype]
    q = randn((T, H, D), 70, 1.0, dt)
    kc = randn((KV, cap, D), 71, 1.0, dt)
    vc = randn((KV, cap, D), 72, 1.0, dt)
    out = ops.attention(q, kc, vc, p0)
    torch.cuda.synchronize()
    ref = orc.attention(np32(q), np32(kc), np32(vc), p0, dtype)
    e = max_row_rel_l2(np32(out).reshape(T * H, D), ref.reshape(T * H, D))
    say(f"attention prefill {dtype} T={T} p0={p0} H={H} KV={KV} D={D}: {e:.2e}")
    assert e < (2e-6 if dtype == "fp32" else 8e-3)


MOE_CASES = [(1, 2048, 128, 8, 768), (5, 2048, 128, 8, 768), (64, 2048, 128, 8, 768), (20, 128, 16, 4, 64),
             (3, 256, 8, 8, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T,hid,E,k,Ie", MOE_CASES)
def test_moe_block_op(orc, ops, dtype, T, hid, E, k, Ie):
    dt = TDT[dtype]
    x = randn((T, hid), 80 + T, 1.0, dt)
    Wr = randn((E, hid), 81, 0.02, dt)
    Wgu = randn((E, 2 * Ie, hid), 82, 0.02, dt)
    Wd = randn((E, hid, Ie), 83, 0.02, dt)
    out, idx, w = ops.moe(x, Wr, Wgu, Wd, k)
    torch.cuda.synchronize()
    ref, ridx, rw = orc.moe_block(np32(x), np32(Wr), np32(Wgu), np32(Wd), k, True, False, dtype)
    gidx = idx.cpu().numpy()
    mism = int(np.sum(np.sort(gidx, -1) != np.sort(ridx, -1)))
    e = max_row_rel_l2(np32(out), ref)
    say(f"moe {dtype} T={T} hid={hid} E={E} k={k} Ie={Ie}: idx mismatches {mism}, out {e:.2e}")
    assert mism == 0
    assert np.array_equal(gidx, ridx)   # same slot order: descending probability, ties to the lower index
    np.testing.assert_allclose(np32(w), rw, rtol=1e-5 if dtype == "fp32" else 2 ** -7, atol=0)
    assert e < (2e-5 if dtype == "fp32" else BF16_TOL)


def test_moe_nan_router_row_gets_valid_experts(orc, ops):
    """A token whose router logits are all NaN still receives k distinct experts in [0, E):
    NaN ranks as -inf, so ties go to the lowest indices 0..k-1.  The other tokens' routing and
    outputs equal the oracle's on the same rows (no routed row is lost or misplaced)."""
    T, hid, E, k, Ie = 6, 128, 16, 4, 64
    dt = TDT["bf16"]
    x = randn((T, hid), 90, 1.0, dt)
    x[2, 5] = float("nan")
    Wr = randn((E, hid), 91, 0.02, dt)
    Wgu = randn((E, 2 * Ie, hid), 92, 0.02, dt)
    Wd = randn((E, hid, Ie), 93, 0.02, dt)
    out, idx, w = ops.moe(x, Wr, Wgu, Wd, k)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    assert ((gidx >= 0) & (gidx < E)).all()
    assert list(gidx[2]) == list(range(k))
    good = [0, 1, 3, 4, 5]
    ref, ridx, _ = orc.moe_block(np32(x)[good], np32(Wr), np32(Wgu), np32(Wd), k, True, False, "bf16")
    assert np.array_equal(gidx[good], ridx)
    assert max_row_rel_l2(np32(out)[good], ref) < BF16_TOL


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) * 16 * 9 + 1040])
def test_stream_read_probe_xor(ops, nbytes):
    """The streaming-read probe behind the measured HBM peak: thread t XORs the 32-bit words of
    16-byte words t, t + 65536, ...; checked word for word against numpy on the same bytes
    (short, ragged and multi-round buffers)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    got = ops.stream_read(host.to("cuda")).cpu().numpy().view(np.uint32)
    words = host.numpy().view(np.uint32).reshape(-1, 4)
    n16, grid = words.shape[0], 256 * 256
    per16 = np.bitwise_xor.reduce(words, axis=1)
    pad = np.zeros(((n16 + grid - 1) // grid) * grid, np.uint32)
    pad[:n16] = per16
    ref = np.bitwise_xor.reduce(pad.reshape(-1, grid), axis=0)
    assert np.array_equal(got, ref)
