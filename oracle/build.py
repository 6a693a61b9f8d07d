"""Compile the C oracle (kda_oracle.c) into liboracle.so next to it.

Test infrastructure only.  Plain gcc, IEEE semantics (no fast-math).  The
library holds the fp64 oracle and its fp32 twin: the same source instantiated
with float for double (expf for exp), built from a copy generated here, so
the two cannot drift apart.  The fp32 twin is a diagnostic only: it shows how
close plain fp32 arithmetic of the same recurrence gets to the fp64 result.
"""
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def fp32_twin(src_text: str) -> str:
    """The oracle source with every double made float: exp -> expf, the
    exported names' _f64 suffix -> _f32 (and the thread-count query renamed)."""
    t = re.sub(r"\bdouble\b", "float", src_text)
    t = re.sub(r"\bexp\(", "expf(", t)
    t = t.replace("_f64(", "_f32(").replace("kda_oracle_num_threads", "kda_oracle_num_threads_f32")
    t = t.replace("kda_oracle_set_num_threads", "kda_oracle_set_num_threads_f32")
    return t


def compile_oracle(src: str, out: str, verbose: bool = False, werror: bool = True,
                   twin: bool = False) -> str:
    with tempfile.TemporaryDirectory() as td:
        srcs = [src]
        if twin:
            tw = os.path.join(td, "kda_oracle_f32.c")
            with open(src) as f, open(tw, "w") as g:
                g.write(fp32_twin(f.read()))
            srcs.append(tw)
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]
        cmd += ["-Werror"] if werror else ["-w"]
        cmd += ["-o", out + ".tmp"] + srcs + ["-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    return compile_oracle(SRC, OUT, verbose, twin=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
