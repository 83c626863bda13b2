"""Build the CPU oracle (test infrastructure).

The oracle is plain C built with gcc -O3 and no fast-math (the pages' default
flags: openai.wiki "llama2.c | Baby LLaMA", section "Performance optimisation"),
linked with the shared input generator object synth/synth.o.
"""
import importlib.util
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
ORACLE_LIB = os.path.join(ROOT, "oracle", "liboracle.so")

CFLAGS = ["-O3", "-fPIC", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def _synth():
    spec = importlib.util.spec_from_file_location("synth_build", os.path.join(ROOT, "synth", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


SYNTH_OBJ = _synth().OBJ


def build_synth():
    return _synth().build_synth()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))


def build_oracle(src=ORACLE_SRC, out=ORACLE_LIB, extra=()):
    """Compile an oracle source (the real one, or a planted-mistake copy made by a test)."""
    if not os.path.exists(SYNTH_OBJ):
        build_synth()
    _run(["gcc", *CFLAGS, *extra, "-I", os.path.join(ROOT, "oracle"), "-I", os.path.join(ROOT, "synth"),
          "-shared", "-Wl,-Bsymbolic", src, SYNTH_OBJ, "-o", out, "-lm", "-lpthread"])
    return out


ORACLE_TIMING_LIB = os.path.join(ROOT, "oracle", "liboracle_accf.so")


def build_oracle_timing():
    """The timing-only build with float accumulators (-DOR_ACC=float): the pages'
    plain fp32 C loop, for the CPU baseline's comparison; never used for parity."""
    return build_oracle(out=ORACLE_TIMING_LIB, extra=("-DOR_ACC=float",))


def build():
    build_synth()
    build_oracle()
    build_oracle_timing()


if __name__ == "__main__":
    build()
    print(ORACLE_LIB)
