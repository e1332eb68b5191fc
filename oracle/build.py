"""Compile the CPU oracle (oracle/moe_oracle.c) into oracle/libmoe_oracle.so with gcc.

Test infrastructure only: the oracle is the checker, never part of the product path.
Floating-point contraction is switched off so that every `a * b + c` in the source rounds twice
and every intended fused multiply-add is an explicit fmaf() call.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")
SAN_LIB = os.path.join(HERE, "libmoe_oracle_san.so")

FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
         "-Wall", "-Wno-unknown-pragmas"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *FLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer (any finding aborts), for the
    CPU test that runs the oracle's pins against it with the ASan runtime preloaded."""
    flags = [f for f in FLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                                "-fno-sanitize-recover=undefined"]
    cmd = ["gcc", *flags, SRC, "-o", SAN_LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
