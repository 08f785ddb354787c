"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles ``oracle.c`` into ``liboracle.so`` beside it with the host C compiler.
No fast-math and no floating-point contraction, so the oracle's roundings are
the ones its source spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def build(cc: str = None, out: str = LIB, extra_cflags=(), source: str = None) -> str:
    """Compile the oracle (or a given source text file) into a shared library."""
    cc = cc or os.environ.get("CC", "gcc")
    src = source or os.path.join(HERE, "oracle.c")
    tmp = out + ".tmp"
    cmd = [cc, *CFLAGS, *extra_cflags, "-I", HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(out=sys.argv[1] if len(sys.argv) > 1 else LIB))
