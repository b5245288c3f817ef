"""Build the CPU oracle library (test infrastructure only).

gcc with -ffp-contract=off -fno-fast-math: the emulator page ("GPU Arithmetic
Emulator", section "Compiler flags") notes that without it the host compiler
fuses a multiply and an add into one FMA and changes the rounding.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bg_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
         "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = ["gcc", *FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
