"""Benchmark of the Qwen3 decoder-stack forward on one MI355X.

Headline (one JSON line on stdout): decode tokens/s of the Qwen3-1.7B-shaped bf16 stack
(28 layers, hidden 2048, 16 q / 8 kv heads, head_dim 128, intermediate 6144), T = 1 at
position 4095 over a K/V cache pre-filled with N(0,1) values (ctx 4096), random-init
weights.  A "step" is one full forward call through all 28 layers (embedding-free
hidden-state input, final norm output); the seat length is rewound to 4095 before each
step on the host.  Also reported: HBM GB/s of the step (algorithmic bytes / time), the
2048-token causal prefill in TFLOP/s (algorithmic FLOPs / time), the dominant kernel's
roofline fraction from HIP events on the library's stream, and the CPU oracle on a
bounded sample of the same decode step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# Algorithmic bytes of one 1.7B decode step at ctx 4096 (weights of 28 layers, the K/V
# read of 4096 positions, norm vectors, the new K/V entries).
DECODE_STEP_BYTES = 3_288_692_736
# gate|up projection launch at T = 1: weight [12288][2048] bf16 + the normalised input
# row (2048 bf16) + the SwiGLU output row (6144 bf16).
GU_LAUNCH_BYTES = 12288 * 2048 * 2 + 2048 * 2 + 6144 * 2
# Algorithmic FLOPs of the 28-layer 2048-token causal prefill: projections
# 2*T*(4096*2048 + 2048*2048 + 12288*2048 + 2048*6144) per layer plus causal attention
# 4*D*H*T(T+1)/2 per layer.
PREFILL_T = 2048
PREFILL_FLOPS = 28 * (2 * PREFILL_T * (4096 * 2048 + 2048 * 2048 + 12288 * 2048 + 2048 * 6144)
                      + 4 * 128 * 16 * PREFILL_T * (PREFILL_T + 1) // 2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device-to-device copy of known size (torch's copy kernel), run before the
    decode leg when hardware counters are collected: its FETCH_SIZE / WRITE_SIZE per dispatch
    against nbytes gives the counters' scale."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")
    del src, dst
    torch.cuda.empty_cache()


def decode_bench(steps: int, warmup: int, compare: bool = True):
    """Time `steps` replays of one captured decode step (HIP graph on a side stream), then
    `steps` eager steps with HIP events around the dominant kernel's launches on the
    library's stream.  Done for the default T = 1 path (the persistent decode kernel) and,
    for comparison, for the one-kernel-per-step path."""
    import ctypes

    import torch

    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import _lib, synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE as cfg

    dev = "cuda"
    log(f"decode: building {cfg.n_layers}-layer weights and a {cfg.capacity}-position cache")
    w = synth.model_weights(cfg, dev)
    K, V = synth.kv_cache(cfg, 4095, dev)
    stream = torch.cuda.Stream()
    seat = q3.Seat(cfg, w, max_tokens=1, k_cache=K, v_cache=V, stream=stream)
    x = synth.hidden_states(cfg, 1, dev)
    out = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device=dev)
    L = _lib.load()
    torch.cuda.synchronize()

    def step():
        seat.length = 4095
        q3.qwen3_forward_hidden(seat.handle, x, out)

    def run(path):
        q3.qwen3_set_decode_path(seat.handle, path)
        used = q3.qwen3_get_decode_path(seat.handle)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        del graph
        # eager pass with the timer on the dominant kernel: the whole-step kernel on the
        # persistent path, the gate|up projection otherwise
        kind = 5 if used == 2 else 2
        L.qwen3_kernel_timer(seat.handle.ptr, kind, 1)
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for _ in range(steps):
                step()
        torch.cuda.synchronize()
        dt_eager = (time.perf_counter() - t0) / steps
        tot, cnt = ctypes.c_double(), ctypes.c_int()
        _lib.check(L.qwen3_kernel_timer_read(seat.handle.ptr, kind, ctypes.byref(tot), ctypes.byref(cnt)))
        L.qwen3_kernel_timer(seat.handle.ptr, kind, 0)
        q3.qwen3_check_device_errors(seat.handle)
        k_us = tot.value * 1e3 / max(cnt.value, 1)
        log(f"decode path {used}: graph {dt * 1e6:.1f} us/step, eager {dt_eager * 1e6:.1f} us/step, "
            f"timed kernel {k_us:.2f} us/launch over {cnt.value} launches")
        return {"path": used, "ms_per_step": dt * 1e3, "eager_ms_per_step": dt_eager * 1e3,
                "tokens_per_s": 1.0 / dt, "hbm_gbps": DECODE_STEP_BYTES / dt / 1e9, "kernel_us": k_us,
                "launches": cnt.value}

    res = run(0)
    res["kernels_path"] = run(1) if res["path"] == 2 and compare else None
    q3.qwen3_set_decode_path(seat.handle, 0)
    del seat, w, K, V
    torch.cuda.empty_cache()
    return res


def prefill_bench(iters: int):
    import torch

    import qwen3_transformer_layer_amd as q3
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_PREFILL as cfg

    dev = "cuda"
    log("prefill: building weights (seed 1), capacity 8192, T=2048")
    w = synth.model_weights(cfg, dev)
    seat = q3.Seat(cfg, w, max_tokens=PREFILL_T)
    x = synth.hidden_states(cfg, PREFILL_T, dev)
    out = torch.empty((PREFILL_T, cfg.hidden), dtype=torch.bfloat16, device=dev)

    def call():
        seat.length = 0
        q3.qwen3_forward_hidden(seat.handle, x, out)

    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / iters
    log(f"prefill: {dt * 1e3:.2f} ms per 2048-token call")
    del seat, w
    torch.cuda.empty_cache()
    return {"ms": dt * 1e3, "tflops": PREFILL_FLOPS / dt / 1e12}


def cpu_baseline(sample_layers: int = 4):
    """The oracle on the host: a decode step of the same shape over `sample_layers` layers
    (same per-layer work as the 28-layer step), scaled to a 28-layer step."""
    import numpy as np
    import torch

    import oracle
    from qwen3_transformer_layer_amd import synth
    from qwen3_transformer_layer_amd.config import QWEN3_1P7B_DECODE

    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    cfg = QWEN3_1P7B_DECODE.replace(n_layers=sample_layers)
    w = synth.model_weights(cfg, "cuda")
    K, V = synth.kv_cache(cfg, 4095, "cuda")
    layers = [{k: v.float().cpu().numpy() for k, v in L.items()} for L in w["layers"]]
    st = oracle.Stack(cfg, layers, w["final_norm"].float().cpu().numpy(), "bf16", kcache=K.float().cpu().numpy(),
                      vcache=V.float().cpu().numpy())
    x = synth.hidden_states(cfg, 1, "cuda").float().cpu().numpy()
    times = []
    for _ in range(3):
        st.length = 4095
        t0 = time.perf_counter()
        st.forward(x)
        times.append(time.perf_counter() - t0)
    t_layer = float(np.median(times)) / sample_layers
    t_step = t_layer * 28
    return {"value": 1.0 / t_step, "unit": "tokens/s", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": f"{sample_layers} of 28 layers of the ctx-4096 T=1 decode step, median of 3, "
                      f"scaled x{28 / sample_layers:g} to a full step ({t_step * 1e3:.1f} ms/step)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-iters", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill leg (for profiling)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the one-kernel-per-step decode path (for profiling)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run a 1 GiB device copy first (hardware-counter scale for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.prefill_only:
        pre = prefill_bench(args.prefill_iters)
        print(json.dumps({"prefill_ms": pre["ms"], "prefill_tflops": pre["tflops"]}), flush=True)
        return
    if args.copy_calib:
        copy_calibration()
    dec = decode_bench(args.steps, args.warmup, compare=not args.no_compare)
    pre = None if args.no_prefill else prefill_bench(args.prefill_iters)
    cpu = None if args.no_cpu else cpu_baseline()

    if dec["path"] == 2:
        rl_kernel = "persistent decode kernel (all 28 layers of a T=1 step, final norm)"
        rl_bytes = DECODE_STEP_BYTES
    else:
        rl_kernel = "gate|up projection GEMV with SwiGLU epilogue (T=1)"
        rl_bytes = GU_LAUNCH_BYTES
    achieved = rl_bytes / (dec["kernel_us"] * 1e-6) / 1e9
    kp = dec["kernels_path"]
    line = {
        "metric": "decode tokens/s + HBM GB/s (T=1, ctx 4096); prefill TFLOP/s at T=2048",
        "value": round(dec["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "eager_ms_per_step": round(dec["eager_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: random-init weights N(0,0.02), norms 1+N(0,0.1), K/V pre-fill and input N(0,1)",
        "config": {"workload": "Qwen3-1.7B-shaped bf16 decode, T=1 at position 4095 (ctx 4096), 28 layers, "
                               "hidden 2048, 16 q / 8 kv heads, head_dim 128, intermediate 6144",
                   "global_batch": 1, "seq_len": 4096, "parallelism": "single GPU"},
        "decode_path": "persistent kernel" if dec["path"] == 2 else "one kernel per step",
        "hbm_gbps": round(dec["hbm_gbps"], 1),
        "hbm_frac": round(dec["hbm_gbps"] / HBM_PEAK_GBPS, 4),
        "kernels_path_ms_per_step": None if kp is None else round(kp["ms_per_step"], 4),
        "prefill_tflops": None if pre is None else round(pre["tflops"], 1),
        "prefill_mfma_frac": None if pre is None else round(pre["tflops"] / BF16_PEAK_TFLOPS, 4),
        "prefill_ms": None if pre is None else round(pre["ms"], 3),
        "roofline": {"kernel": rl_kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": rl_bytes, "avg_launch_us": round(dec["kernel_us"], 3),
                     "launches": dec["launches"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
