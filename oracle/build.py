"""Build the CPU oracle (test infrastructure only): liboracle.so next to this file."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           os.path.join(HERE, "oracle.c"), "-o", SO + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
