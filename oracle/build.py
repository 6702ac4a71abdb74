"""Build the CPU oracle (test infrastructure) into oracle/libcoat_oracle.so.

Plain gcc, no GPU toolchain: the oracle shares nothing with the HIP library.
-ffp-contract=off keeps FP32 expressions in the order they are written (no
fused multiply-add), which is how the oracle states the AdamW arithmetic.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcoat_oracle.so")
SRC = os.path.join(HERE, "coat_oracle.c")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Werror",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
