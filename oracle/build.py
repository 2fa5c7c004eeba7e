"""Build the CPU oracle shared library (test infrastructure).

gcc, -O2, no fast-math, -ffp-contract=off: every fp32 operation of the
definition is rounded once, in the order written.  x86-64 evaluates float
arithmetic in SSE registers (FLT_EVAL_METHOD 0), so nothing is carried at
extended precision.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zq_oracle.c")
LIB = os.path.join(HERE, "libzq_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-frounding-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


def ensure_built() -> str:
    override = os.environ.get("ZQ_ORACLE_LIB")
    if override:  # a separately built oracle (e.g. a planted-mistake copy)
        return override
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
