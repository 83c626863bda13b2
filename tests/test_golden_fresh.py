"""The stored oracle outputs under tests/golden/ were written by the oracle as it
stands: each file records a hash of the oracle and generator sources it came
from, and a file written by an older oracle must be regenerated
(tests/golden/make_golden.py) before the GPU parity tests may compare against
it.  Checked here on the CPU, so a stale file shows up before any GPU run."""
import glob
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")

from tests.golden.make_golden import PLAN, source_hash  # noqa: E402


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLD, "*.npz"))),
                         ids=lambda p: os.path.basename(p))
def test_stored_outputs_match_current_oracle(path):
    z = np.load(path, allow_pickle=False)
    name = os.path.splitext(os.path.basename(path))[0]
    assert str(z["workload"]) == name
    assert str(z["source_hash"]) == source_hash(), (
        "%s was written by another version of the oracle: run tests/golden/make_golden.py %s" % (name, name))


def test_every_planned_workload_is_stored():
    stored = {os.path.splitext(os.path.basename(p))[0] for p in glob.glob(os.path.join(GOLD, "*.npz"))}
    assert set(PLAN) <= stored, sorted(set(PLAN) - stored)
