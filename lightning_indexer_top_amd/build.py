"""Build liblit.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Every HIP source is compiled on its own (in parallel), then linked into
``lightning_indexer_top_amd/liblit.so``.  Packed-FP32 instructions are disabled for
the device code; the host pass warns that it does not know that feature, which is
harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build", "lit")
LIB = os.path.join(HERE, "liblit.so")
SOURCES = ["lit_api.hip", "indexer.hip", "topk.hip", "attention.hip", "produce.hip", "fused_decode.hip",
           "fused_e4m3.hip", "fused_e2m1.hip", "fused_e4m3_cand.hip", "fused_e2m1_cand.hip",
           "fused_e4m3_qkv.hip", "fused_e2m1_qkv.hip", "fused_e4m3_layers.hip", "fused_e2m1_layers.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# MFMA results are written to VGPRs rather than AGPRs: no accumulator reads before the
# epilogues, and the kernels here have the VGPRs to spare.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=true"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
