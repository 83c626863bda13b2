"""Compile the HIP decode library for gfx950 into transformer_llama_decode_amd/libld.so.

Each kernel file is compiled separately (in parallel) with hipcc for gfx950
only, then linked with the host engine and the shared input generator object.
"""
import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libld.so")
ARCH = "gfx950"

KERNELS = ["k_gemv.hip", "k_attn.hip", "k_attn_prefill.hip", "k_gemm.hip", "k_misc.hip", "static_scratch.hip"]
HOST = ["engine.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "synth")]
# no packed-fp32 instructions in any generated code
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _synth_obj():
    spec = importlib.util.spec_from_file_location("synth_build", os.path.join(ROOT, "synth", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build_synth()


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
               "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    synth_obj = _synth_obj()
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, KERNELS + HOST))
    objs = [o for o, _ in results]
    if verbose:
        for o, err in results:
            if err.strip():
                print(o, err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-Bsymbolic", "-o", tmp,
           *objs, synth_obj, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
