"""Build the oracle's shared library with gcc (plain C11, -O2, no fast-math).

Usage: ``python oracle/build.py`` (also called by ``__graft_entry__.build()``).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rownorm_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-fPIC", "-shared", "-o", OUT + ".tmp", SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
