"""Builds the HIP library ``libint4kv.so`` in-tree for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into one shared library exporting the C ABI of ``include/int4kv.h``.
The cache-write kernel is compiled without FMA contraction so its fp32
sequence is the one the encoding defines; the LDS-staged decode kernel is
compiled without NaN semantics (its scores are finite or -inf by construction)
so its 16-lane maxima are single DPP instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libint4kv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", "-Wno-unused-variable",
          # packed fp32 ops are never emitted (see the project's design notes)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(HERE, "..", "include")]
# The LDS-staged decode kernel and the prefill kernel never produce NaN
# logits (masked keys are selected as -inf, not computed), so their maxima
# need no NaN quieting.
PER_FILE = {"write.hip": ["-ffp-contract=off"], "write_int8.hip": ["-ffp-contract=off"],
            "write_int2.hip": ["-ffp-contract=off"], "decode_lds.hip": ["-fno-honor-nans"],
            "prefill.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
