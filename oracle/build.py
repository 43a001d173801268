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


# AddressSanitizer + UBSan variant (CPU runs with the sanitizer runtimes preloaded).
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False) -> str:
    lib = SAN_LIB if sanitize else LIB
    if not force and os.path.exists(lib):
        return lib
    tmp = lib + ".tmp"
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else []), "-o", tmp, *SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(sanitize="--sanitize" in sys.argv))
