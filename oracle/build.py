"""Build step for the CPU oracle: compiles oracle.c into liboracle.so with gcc.

Test infrastructure only (see oracle/__init__.py). Strict IEEE double
arithmetic: -O2 -ffp-contract=off, no fast-math, so every operation the C
source writes is the one executed.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile `src` (oracle.c by default) into the shared library `lib`."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", lib, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
