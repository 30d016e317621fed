"""Compile the CPU oracle (plain C, fp64, OpenMP) into oracle/libbsa_oracle.so.

Test infrastructure only: see oracle/__init__.py.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsa_oracle.c")
LIB = os.path.join(HERE, "libbsa_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile src (the oracle, or a copy of it) into the shared library lib."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-Wextra", "-shared", "-fPIC",
           src, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
