"""Compile libmoe.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled with packed-fp32 instructions disabled; the
router is compiled without floating-point contraction so that its fixed
summation order is exactly the one written in the source.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")

ARCH = "gfx950"
SOURCES = {
    "route.hip": ["-ffp-contract=off"],
    "group.hip": [],
    "prep.hip": [],
    "ffn.hip": [],
    "ffn_large.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "combine.hip": [],
    "api.cpp": [],
}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    p = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _compile(src: str, extra) -> str:
    out = os.path.join(OBJ, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
