"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

fp32 steps must be single correctly rounded operations: no FMA contraction,
no fast-math, no flush-to-zero.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "int4kv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (CPU
# only, single-threaded), loaded by the oracle tests when ORACLE_SANITIZED=1
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fno-finite-math-only", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fPIC", "-shared", "-Wall",
             "-Wextra"]
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False, sanitized: bool = False) -> str:
    out = LIB_SAN if sanitized else LIB
    cmd = ["gcc", *(SAN_FLAGS if sanitized else CFLAGS), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitized="--sanitized" in sys.argv))
