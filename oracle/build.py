"""Compile the C oracle (kda_oracle.c) into liboracle.so next to it.

Test infrastructure only.  Plain gcc, fp64, IEEE semantics (no fast-math).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def compile_oracle(src: str, out: str, verbose: bool = False, werror: bool = True) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]
    cmd += ["-Werror"] if werror else ["-w"]
    cmd += ["-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    return compile_oracle(SRC, OUT, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
