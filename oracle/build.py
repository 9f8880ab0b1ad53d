"""Build the CPU oracle shared library (test infrastructure only).

Compiles ``k8v4_oracle.c`` with gcc into ``liborc_k8v4.so`` next to this
file.  Strict IEEE fp32: no fused multiply-add contraction, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "k8v4_oracle.c")
LIB = os.path.join(HERE, "liborc_k8v4.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
