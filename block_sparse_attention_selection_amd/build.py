"""Build libmsa_kvouter.so (HIP, gfx950) in-tree with hipcc, and the rate
measurement program lib/msa_rates (run by `python bench.py --micro`).

    python -m block_sparse_attention_selection_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmsa_kvouter.so")
OBJDIR = os.path.join(ROOT, "_build", "msa")
SOURCES = ["msa_api.hip", "msa_index.hip", "msa_forward.hip", "msa_tiles.hip", "msa_store.hip", "msa_select.hip"]
RATES_SRC = "msa_rates.hip"  # a standalone program, not part of the library
RATES = os.path.join(LIBDIR, "msa_rates")
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled for all device code: they are only
# ever produced by the compiler here, never written by hand.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def _build_rates() -> None:
    tmp = RATES + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], os.path.join(CSRC, RATES_SRC), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {RATES_SRC}:\n{r.stderr}")
    os.replace(tmp, RATES)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        rates = ex.submit(_build_rates)
        objs = list(ex.map(_compile, SOURCES))
        rates.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, "and", RATES)
    return LIB


if __name__ == "__main__":
    build()
