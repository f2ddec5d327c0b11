"""Build the C oracle into oracle/libar_oracle.so (test infrastructure only).

Plain gcc, -O2 -fno-fast-math, OpenMP for the optional multi-threaded timing
loop.  No flag that would change binary32 semantics (no -ffast-math, no
-ffp-contract=fast, no flush-to-zero start-up code) is used.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ar_oracle.c")
LIB = os.path.join(HERE, "libar_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
           "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra", "-Werror",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
