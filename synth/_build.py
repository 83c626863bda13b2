"""Compile the shared input generator once, with gcc, into synth/synth.o.

Both the CPU oracle and the HIP library link this same object, so both sides
draw bit-identical synthetic weights and prompts.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth.c")
OBJ = os.path.join(HERE, "synth.o")
FLAGS = ["-O2", "-fPIC", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build_synth():
    r = subprocess.run(["gcc", *FLAGS, "-c", SRC, "-o", OBJ], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("synth build failed:\n" + r.stdout + r.stderr)
    return OBJ


if __name__ == "__main__":
    print(build_synth())
