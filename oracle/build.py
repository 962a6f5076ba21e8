"""Build the CPU oracle (test infrastructure) as a shared library with gcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "velox_oracle.c")
LIB = os.path.join(HERE, "libvelox_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    # -ffp-contract=off keeps every float operation separately rounded (no FMA);
    # no fast-math.
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose="-v" in sys.argv))
