"""Shared helpers of the GPU parity tests: host copies for the oracle and error metrics.

Tolerances (the layer's stated gates): strict fp32 mode max|d| / RMS(ref) <= 1e-4;
bf16 mode per-row ||d||_2 / ||ref||_2 <= 2e-2 after one layer.
"""
import os
import sys

import numpy as np
import torch

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def max_rel_rms(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


def max_row_rel_l2(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    return float(np.max(np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)))


def gate(got, ref, dtype: str) -> float:
    """Return the gated metric and assert it (fp32: max|d|/RMS; bf16: per-row relative L2)."""
    if dtype == "fp32":
        e = max_rel_rms(got, ref)
        assert e <= FP32_TOL, f"fp32 max|d|/RMS = {e:.3e} > {FP32_TOL}"
    else:
        e = max_row_rel_l2(got, ref)
        assert e <= BF16_TOL, f"bf16 per-row rel L2 = {e:.3e} > {BF16_TOL}"
    return e


def oracle_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_layers(orc, cfg, weights):
    """Oracle-side fp32 host copies of the layer weights (8-bit weights dequantised by the oracle)."""
    out = []
    for lw in weights["layers"]:
        d = {}
        for k, v in lw.items():
            if k.endswith(("_q", "_s", "_b")):
                continue
            d[k] = np32(v)
        for name in ("qkv", "o", "gate_up", "down", "router", "exp_gate_up", "exp_down"):
            if name + "_q" in lw:  # stacked experts [E][rows][cols] dequantised as E*rows rows
                q = lw[name + "_q"].cpu().numpy()
                d[name] = orc.q8_dequant(q.reshape(-1, q.shape[-1]), np32(lw[name + "_s"]).reshape(-1, q.shape[-1] // cfg.quant_group),
                                         np32(lw[name + "_b"]).reshape(-1, q.shape[-1] // cfg.quant_group),
                                         cfg.quant_group).reshape(q.shape)
        out.append(d)
    return out
