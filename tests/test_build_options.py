"""The documented build option of the kernels still compiles (CPU only: hipcc
cross-compiles for gfx950 without a GPU).

LD_TICKET_ACQ_REL makes the cross-workgroup tickets (attention chunk merge,
split-K slices) take an explicit device-scope release/acquire pair instead of
the relaxed ticket that follows the partials' completed device-scope stores.
"""
import os
import shutil
import subprocess

import pytest

from transformer_llama_decode_amd import _build

HIPCC = _build.HIPCC


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.parametrize("src", ["k_attn.hip", "k_gemm.hip"])
def test_ticket_acq_rel_option_compiles(src, tmp_path):
    out = tmp_path / (src + ".o")
    cmd = [HIPCC, *_build.COMMON, *_build.DEVICE, "-DLD_TICKET_ACQ_REL", "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    # the release before every ticket and the acquire of the last arrival
    assert "buffer_wbl2" in asm and "buffer_inv" in asm
