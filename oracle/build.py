"""Build the CPU oracle (plain C) into oracle/liboracle.so.

Test infrastructure only: the oracle is the checker the GPU path is compared
against, never part of that path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = [os.path.join(HERE, "fmoe_oracle.c"), os.path.join(HERE, "fmoe_oracle_next.c")]
LIB = os.path.join(HERE, "liboracle.so")

# -O2 without fast-math; no contraction so every expression rounds as written.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, *SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
