"""Build libnf4moe.so (HIP, gfx950) in-tree.

    python -m grouped_nf4_gemm_quantize_amd.build [--jobs N] [--save-temps]

Every source under ``csrc/`` is compiled with hipcc for gfx950 into
``_build/`` and linked into ``grouped_nf4_gemm_quantize_amd/libnf4moe.so``.
Packed-fp32 VALU instructions are disabled (``-packed-fp32-ops``); float
division and square root stay correctly rounded and denormals are kept (no
fast-math), which the bit-exact quantiser relies on.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnf4moe.so")
ARCH = "gfx950"

SOURCES = ["quantize.hip", "route.hip", "gemm.hip", "gemm16.hip", "dgrad.hip", "lora.hip", "gemv.hip",
           "noalloc.hip", "abi.cpp"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # the GEMM's direct-to-LDS copies name M0 in their clobber list on purpose
    "-Wno-inline-asm",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnf4moe.so)")


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if save_temps:
        cmd.append("--save-temps")
    res = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn:
        sys.stderr.write(f"[{src}]\n{warn}\n")
    return obj


def build(jobs: int = 0, save_temps: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--save-temps", action="store_true")
    args = ap.parse_args()
    build(args.jobs, args.save_temps)


if __name__ == "__main__":
    main()
