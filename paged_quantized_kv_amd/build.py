"""Build libpkv.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 and linked into
paged_quantized_kv_amd/libpkv.so next to this file.  Object files go to
_build/ at the repository root.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "gather_indexer_k_fp8.hip",
    "store_indexer_k_fp8.hip",
    "store_kv_fp4.hip",
    "gather_dequant.hip",
    "mqa_logits.hip",
    "paged_attention.hip",
    "diag_codecs.hip",
]

CXXFLAGS = [
    f"--offload-arch={ARCH}",
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",  # only the PKV_API entry points are exported
    # IEEE binary32 step by step: no a*b+c contraction except the explicit
    # fma calls; divisions stay correctly rounded; subnormals are kept.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments preloaded into SGPRs by the command processor (gfx950
    # supports it; each code object keeps a fallback that loads them as usual
    # where the firmware does not): short bandwidth-bound kernels start their
    # address arithmetic without the kernel-argument round trip (0.3-0.5 us
    # of an 11-12 us gather).
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libpkv.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
