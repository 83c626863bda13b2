"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle/check_sanitize.c drives every oracle entry point on small models (every
attention variant, bfloat16 weights, the window past max_seq; cached forward
against recomputation); built with gcc -fsanitize=address,undefined it must
run clean.  Host code only: nothing here touches the GPU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_is_clean_under_address_and_undefined_behaviour_sanitizers():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "check_sanitize")
        cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "oracle"), "-I", os.path.join(ROOT, "synth"),
               os.path.join(ROOT, "oracle", "check_sanitize.c"), os.path.join(ROOT, "oracle", "oracle.c"),
               os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm", "-lpthread"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0 and "asan" in (r.stderr or "").lower() and "cannot find" in r.stderr:
            pytest.skip("sanitizer runtime not installed")
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
