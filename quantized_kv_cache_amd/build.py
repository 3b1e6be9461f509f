"""Build the gfx950 HIP library libflk.so in-tree (and the CPU oracle beside it).

    python -m quantized_kv_cache_amd.build

Every HIP source is compiled with -ffp-contract=off (the codec is specified one IEEE step at
a time) and with packed FP32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libflk.so")
SOURCES = ["flk_api.cpp", "flk_encode.hip", "flk_reconstruct.hip", "flk_attn.hip", "flk_attn_split.hip", "flk_sparse.hip",
           "flk_select.hip", "flk_fp4.hip"]
ARCH = os.environ.get("FLK_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip() and "1 warning generated" not in ln
            and "warnings generated" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + (r.stdout + r.stderr))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_check(src: str, verbose: bool = True) -> str:
    """Compile a standalone gfx950 check program (test infrastructure, not part of the
    library) next to its source, with the library's flags."""
    exe = os.path.splitext(src)[0]
    tmp = exe + ".tmp"
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-fPIC", "-ffp-contract=off")], src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + (r.stdout + r.stderr))
    os.replace(tmp, exe)
    if verbose:
        print(f"built {exe}")
    return exe


if __name__ == "__main__":
    build()
