"""Build libsage.so (the HIP kernels + the C ABI) for gfx950, in-tree.

    python -m quantized_attention_02_amd.build [--resource-usage]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsage.so")
SOURCES = ["api.cpp", "quant.hip", "attn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results stay in ordinary VGPRs (no accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libsage.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [HIPCC] + FLAGS + extra + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        return obj, out

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for _, out in results:
        if out.strip() and (verbose or resource_usage):
            print(out)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for o, _ in results] + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, verbose=True))
