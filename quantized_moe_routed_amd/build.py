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
    "host.cpp": [],
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


# Sources with hand-written DPP instructions in inline assembly: the compiler does not check
# those for the two wait states a DPP operand needs after a vector write, so the build does.
DPP_CHECKED = ["route.hip"]


def _dpp_hazards(asm_text: str):
    """(write, dpp) pairs where a DPP instruction reads, as its first source, a VGPR written by a
    vector instruction fewer than two wait states before (s_nop N counts N + 1)."""
    import re

    def regs(tok):
        m = re.match(r"v\[(\d+):(\d+)\]", tok)
        if m:
            return set(range(int(m.group(1)), int(m.group(2)) + 1))
        m = re.match(r"v(\d+)$", tok)
        return {int(m.group(1))} if m else set()

    ins = [l.strip() for l in asm_text.splitlines()]
    ins = [l for l in ins if l and not l.startswith((";", ".")) and not l.endswith(":")]
    found = []
    for i, line in enumerate(ins):
        parts = line.split(None, 1)
        if "_dpp" not in parts[0] or len(parts) < 2:
            continue
        src0 = regs(parts[1].split(",")[1].strip())
        ws, j = 0, i - 1
        while j >= 0 and ws < 2:
            p = ins[j].split(None, 1)
            if p[0] == "s_nop":
                ws += int(p[1], 0) + 1
            else:
                if p[0].startswith("v_") and len(p) > 1 and regs(p[1].split(",")[0].strip()) & src0:
                    found.append((ins[j], line))
                    break
                ws += 1
            j -= 1
    return found


def _check_dpp(src: str, extra) -> None:
    out = os.path.join(OBJ, src + ".s")
    cmd = [hipcc(), *COMMON, *extra, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    bad = _dpp_hazards(open(out).read())
    if bad:
        raise RuntimeError(f"{src}: DPP operand written fewer than 2 wait states before use: {bad[:3]}")


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
        list(ex.map(lambda src: _check_dpp(src, SOURCES[src]), DPP_CHECKED))
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
