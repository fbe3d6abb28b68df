"""Builds the C oracle (``liboracle_swa.so``) with gcc.

Test infrastructure: the oracle is the fp64 CPU reference that the HIP
library is checked against.  It is compiled separately from the HIP library
and shares no source with it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "swa_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle_swa.so")


def build(verbose: bool = False) -> str:
    """Compiles the oracle (always, even when a built copy exists)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SOURCE, "-o", LIBRARY + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
