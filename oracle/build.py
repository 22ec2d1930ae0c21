"""Build the fp64 CPU oracle (oracle.c -> liboracle.so) with gcc.

Test infrastructure: the oracle is loaded only by the tests, the smoke check and
the benchmark's CPU-baseline leg.  No floating-point contraction or fast-math, so
every product and sum is an ordinary IEEE double operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
