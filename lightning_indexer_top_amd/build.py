"""Build liblit.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Every HIP source is compiled on its own (in parallel; fused_forms.hip once per fused
kernel form), then linked into
``lightning_indexer_top_amd/liblit.so``.  Packed-FP32 instructions are disabled for
the device code; the host pass warns that it does not know that feature, which is
harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build", "lit")
LIB = os.path.join(HERE, "liblit.so")
SOURCES = ["lit_api.hip", "indexer.hip", "topk.hip", "attention.hip", "produce.hip", "fused_decode.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# MFMA results are written to VGPRs rather than AGPRs: no accumulator reads before the
# epilogues, and the kernels here have the VGPRs to spare.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=true"]


def fused_forms() -> list:
    """Names of the fused kernel's forms, from the LIT_FUSED_FORMS list in lit_internal.h."""
    with open(os.path.join(CSRC, "lit_internal.h")) as fh:
        text = fh.read()
    block = text[text.index("#define LIT_FUSED_FORMS(X)"):]
    block = block[:block.index("\n#define", 1)] if "\n#define" in block[1:] else block
    return re.findall(r"^\s*X\((\w+),", block, flags=re.M)


def _compile(unit) -> str:
    src, form = unit
    name = os.path.splitext(src)[0] + (f"_{form}" if form else "")
    obj = os.path.join(BUILD, name + ".o")
    defs = [f"-DLIT_FORM={form}"] if form else []
    cmd = [HIPCC, *CFLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    forms = fused_forms()
    if not forms:
        raise RuntimeError("no fused forms found in lit_internal.h")
    # the fused forms first: they take longest
    units = [("fused_forms.hip", f) for f in forms] + [(s, None) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(units), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(_compile, units))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
