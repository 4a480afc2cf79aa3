"""Compile the oracle's C++ source into a host shared library.

The oracle is test infrastructure: it is built next to its source so that the
test suite, the smoke check and the benchmark's CPU-baseline leg can load it.
Plain g++ with IEEE semantics: no fast-math and no FMA contraction, so every
operation in the source rounds exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfr_oracle.cpp")
LIB = os.path.join(HERE, "libmfr_oracle.so")

CXXFLAGS = ["-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
            "-Wall", "-Wextra"]


def compile_source(src, out, verbose=False):
    """Compile one oracle source file into a shared library at `out`."""
    cmd = ["g++", *CXXFLAGS, "-o", out + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose=False):
    return compile_source(SRC, LIB, verbose=verbose)


if __name__ == "__main__":
    print(build(verbose=True))
