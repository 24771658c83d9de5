"""Build step for the CPU oracle (test infrastructure only).

Compiles ``tq1_oracle.c`` with plain gcc into ``oracle/_build/libtq1_oracle.so``.
No intrinsics and no fast-math; floating-point contraction is off so every
fp32 operation rounds exactly once, as the definitions state.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq1_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libtq1_oracle.so")

CFLAGS = [
    "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
]


def build(force: bool = True) -> str:
    """Compile the oracle library; returns its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
