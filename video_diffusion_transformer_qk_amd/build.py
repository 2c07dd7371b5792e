"""Builds libh3attn.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libh3attn.so")
SOURCES = ["qk_norm_rope.hip", "attention.hip", "attention_fp8.hip", "fp8_quant.hip", "subblock_select.hip",
           "block_ops.hip", "cache_gate.hip", "index_check.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags(debug: bool = False):
    flags = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
             # packed fp32 VALU ops are kept off for every HIP translation unit
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
    flags += ["-O0", "-g"] if debug else ["-O3"]
    return flags


# Per-source flags. The attention kernels never see NaN operands (masked keys are -inf), so
# max() needs no NaN quieting of MFMA results before the v_max3 tree.
EXTRA_FLAGS = {"attention.hip": ["-fno-honor-nans"], "attention_fp8.hip": ["-fno-honor-nans"]}


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + common_flags(debug) + EXTRA_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, debug: bool = False) -> str:
    """Compile every source and link libh3attn.so next to this file. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv)
