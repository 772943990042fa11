"""Build the C oracle: oracle/_build/libmoe_ref.so from oracle/moe_ref.c alone.

TEST INFRASTRUCTURE ONLY (the checker, not the product). gcc, C11, -O2 without
-ffast-math, so float64 arithmetic keeps IEEE semantics and the source's order.
`python oracle/build_ref.py` or build() from Python.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_ref.c")
OUT = os.path.join(HERE, "_build", "libmoe_ref.so")
FLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
         "-Werror", "-fPIC", "-shared", "-pthread"]


def build(src: str = SRC, out: str = OUT, extra=()) -> str:
    """Compile src into the shared library out (written through a temporary name, so a
    process that has the old library loaded keeps a whole file)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", *FLAGS, *extra, "-I", HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
