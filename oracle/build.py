"""Build step for the CPU oracle (test infrastructure only).

Compiles ``oracle/oracle.c`` into ``oracle/liboracle.so`` with the host C
compiler.  ``extra_cflags`` and ``source``/``out`` let the mutation tests build
deliberately broken copies of the oracle in a temporary directory.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(source=SOURCE, out=LIBRARY, extra_cflags=(), quiet=False):
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
           *extra_cflags, "-o", out + ".tmp", source, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if res.stderr and not quiet:
        print(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
