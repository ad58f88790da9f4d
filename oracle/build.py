"""Build step for the reference library ``liboracle.so`` (plain C, gcc, OpenMP).

Test infrastructure only: the library it builds is loaded by the test suite, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, n) for n in ("attn_ref.c", "attn_bwd_ref.c", "attn_window_ref.c", "attn_dropout_ref.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the reference sources into liboracle.so next to them and return the path."""
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(s) for s in SRCS):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp] + SRCS + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
