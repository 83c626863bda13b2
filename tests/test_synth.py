"""Pins of the seeded input generator (synth/), CPU only.

The generator is checked against (a) the published SplitMix64 reference outputs,
(b) an independent pure-Python implementation of its definition, and (c) the
statistics of the distributions it must draw from.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O

M64 = (1 << 64) - 1
PHI = 0x9E3779B97F4A7C15


def _mix(z):
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & M64
    z ^= z >> 31
    return z


def _u(seed, stream, c):
    k = _mix(_mix(seed) ^ ((stream * PHI) & M64))
    return _mix((k + c * PHI) & M64)


def _normal(seed, stream, e, std=0.02):
    j = e >> 1
    a, b = _u(seed, stream, 2 * j), _u(seed, stream, 2 * j + 1)
    u1 = ((a >> 11) + 1) * 2.0 ** -53
    u2 = (b >> 11) * 2.0 ** -53
    r = math.sqrt(-2.0 * math.log(u1))
    th = 2 * math.pi * u2
    z = r * math.sin(th) if e & 1 else r * math.cos(th)
    return np.float32(std * z)


def test_splitmix64_reference_values(oracle_lib):
    # SplitMix64 (Steele, Lea & Flood 2014) seeded with 0: outputs are mix(i*PHI).
    import ctypes
    oracle_lib.synth_mix64.argtypes = [ctypes.c_uint64]
    oracle_lib.synth_mix64.restype = ctypes.c_uint64
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [oracle_lib.synth_mix64((i * PHI) & M64) for i in (1, 2, 3)]
    assert got == want


@pytest.mark.parametrize("seed,stream", [(0, 0), (4, 1 + 7 * 31 + 4), (123456789, 225)])
def test_normal_matches_independent_python(seed, stream):
    idx = [0, 1, 2, 3, 1001, 1002, 65535, 65536, 10 ** 9 + 7]
    for e in idx:
        c = O.synth_normal(seed, stream, e, 1)[0]
        assert c == _normal(seed, stream, e), (seed, stream, e)


def test_u64_matches_independent_python(oracle_lib):
    for s, t, c in [(0, 0, 0), (1, 2, 3), (M64, M64, M64), (7, 0x50524F4D, 99)]:
        assert oracle_lib.synth_u64(s, t, c) == _u(s, t, c)


def test_normal_chunking_and_threads_do_not_change_values():
    full = O.synth_normal(3, 5, 0, 300001)
    part = O.synth_normal(3, 5, 123457, 1000)           # odd start: splits a pair
    assert np.array_equal(full[123457:124457], part)
    mt = O.synth_normal(3, 5, 0, 300001, nthreads=7)
    assert np.array_equal(full, mt)


def test_normal_statistics():
    n = 2_000_000
    w = O.synth_normal(0, 0, 0, n, nthreads=8).astype(np.float64)
    z = w / 0.02
    assert abs(z.mean()) < 4 / math.sqrt(n)
    assert abs(z.std() - 1.0) < 4 * math.sqrt(0.5 / n)
    tail = np.mean(np.abs(z) > 3.0)
    p = 0.0026998
    assert abs(tail - p) < 4 * math.sqrt(p * (1 - p) / n)
    # even (cos) and odd (sin) halves are uncorrelated
    r = np.corrcoef(z[0::2], z[1::2])[0, 1]
    assert abs(r) < 4 / math.sqrt(n / 2)


def test_prompt_range_and_uniformity():
    n = 400_000
    t = O.synth_prompt(2, 0, n)
    assert t.min() >= 3 and t.max() <= 31999
    bins = 100
    h, _ = np.histogram(t, bins=bins, range=(3, 32000))
    # bins of 319.97 tokens; chi-square with 99 dof, 5-sigma bound
    expect = n / bins
    chi2 = ((h - expect) ** 2 / expect).sum()
    assert chi2 < 99 + 5 * math.sqrt(2 * 99)


def test_prompt_independent_python():
    for seed, seq in [(1, 0), (2, 255), (4, 0)]:
        t = O.synth_prompt(seed, seq, 50)
        for j in range(50):
            u = _u(seed, 0x50524F4D + seq, j) >> 32
            assert t[j] == 3 + ((u * 31997) >> 32)
