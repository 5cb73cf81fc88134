"""Build the C oracle (test infrastructure) into oracle/liboracle.so with gcc.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
the library that this script builds.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ref_decode.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", SOURCE, "-o", LIBRARY + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
