"""Build libqwen3.so (HIP for gfx950) in-tree with hipcc.

Each source under csrc/ is compiled to an object in parallel, then linked into
qwen3_transformer_layer_amd/libqwen3.so.  Packed-fp32 instructions are disabled
for all device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqwen3.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["kernels_elem.hip", "kernels_linear.hip", "kernels_gemm.hip", "kernels_attn.hip", "kernels_moe.hip",
           "kernels_q8.hip", "kernels_decode_mk.hip", "kernels_decode_moe.hip", "kernels_head.hip", "qwen3_api.cpp", "qwen3_ops.cpp"]
ARCH = os.environ.get("QWEN3_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqwen3)")


def flags() -> list[str]:
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; the persistent decode kernel's
    # LDS-DMA asm names M0, which the compiler reports as a reserved register
    noise = ("is not a recognized feature for this target", "contains reserved registers: m0",
             "Reserved registers on the clobber list", "warning generated", "warnings generated")
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
