"""Build liboracle.so (gcc; no FMA contraction, no fast-math, OpenMP)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                    "-shared", "-std=c11", "-Wall", "-o", os.path.join(HERE, "liboracle.so"),
                    os.path.join(HERE, "oracle.c"), "-lm"], check=True)


if __name__ == "__main__":
    build()
