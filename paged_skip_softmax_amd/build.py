"""Builds libattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m paged_skip_softmax_amd.build`` (always recompiles).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["decode.hip", "smallseq.hip", "prefill.hip", "prefill_d128.hip", "prefill_bwd.hip", "check.hip", "api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code (the compiler would otherwise form them
# from plain float code).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-source extras.  No NaN reaches a used value in the D=128 prefill kernels: every K / V row they use
# arrives by their own loads (rows past a sequence read as zero), and LDS left over from earlier work is
# only read for the scores of the tile past the last, which are discarded; so max() of MFMA results
# needs no NaN canonicalisation.
EXTRA = {"prefill_d128.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    out = os.path.join(OBJ, src + ".o")
    flags = [*FLAGS, *EXTRA.get(src, [])]
    cmd = ["hipcc", *flags, "-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd = ["hipcc", *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return out


# Measurement only, outside the library's ABI: the matrix-core loop the bench reports as the achievable
# bf16 MFMA rate.
PROBE_SRC = "probe.hip"
PROBE_LIB = os.path.join(HERE, "libattn_probe.so")


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        fut_probe = ex.submit(_compile, PROBE_SRC)
        objs = list(ex.map(_compile, SOURCES))
        probe_obj = fut_probe.result()
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, probe_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
