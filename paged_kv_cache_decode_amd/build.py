"""Build libpa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m paged_kv_cache_decode_amd.build           # build
    python -m paged_kv_cache_decode_amd.build --isa     # also dump AMDGCN assembly

Every source is compiled with hipcc for gfx950 with packed-fp32 instruction
selection disabled, then linked into ``paged_kv_cache_decode_amd/libpa.so``.
Objects go to ``paged_kv_cache_decode_amd/_build/``.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "api.cpp", "block_manager.cpp", "decode.hip", "prefill.hip",
           "shared_prefix.hip", "write_kv.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libpa.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning
    # is expected and dropped.
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(isa: bool = False, jobs: int = 4, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if isa and src.endswith(".hip"):
            asm = os.path.join(BUILD, src + ".s")
            _run([hipcc, *COMMON_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
                  os.path.join(CSRC, src), "-o", asm])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", action="store_true", help="also write AMDGCN assembly")
    ap.add_argument("-j", type=int, default=4)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args(argv)
    print(build(isa=a.isa, jobs=a.j, verbose=a.v))


if __name__ == "__main__":
    sys.exit(main())
