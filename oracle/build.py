"""Build the CPU oracle library (plain C, gcc, no fast-math).

Test infrastructure only: the product library never links or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "halo_oracle.c")
LIB = os.path.join(HERE, "libhalo_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out: str, verbose: bool = False) -> str:
    """The same oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc), for
    the CPU test that runs the oracle's pins under them; any finding aborts."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-o", out, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
