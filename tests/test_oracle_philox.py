"""Pins of the oracle's Philox4x32-10 generator and of its uniforms.

The external pin is rocRAND's own Philox4x32-10 engine (an independent
library implementation of Salmon et al., "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11), compiled here for the host from its public header and run
on the same counter/key pairs.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.stats

HERE = os.path.dirname(os.path.abspath(__file__))


def _pairs(n, seed=7):
    rng = np.random.default_rng(seed)
    rows = []
    # edge counters/keys, then random ones (word 1 kept below 2^30 so the
    # engine's 64-bit output offset, 4 per block, does not wrap)
    rows.append([0, 0, 0, 0, 0, 0])
    rows.append([0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF])
    rows.append([1, 0, 0, 0, 0, 0])
    rows.append([0, 0, 0, 0, 1, 0])
    for _ in range(n):
        r = rng.integers(0, 2**32, size=6, dtype=np.uint64)
        r[1] &= 0x3FFFFFFF
        rows.append([int(v) for v in r])
    return rows


@pytest.fixture(scope="module")
def rocrand_driver(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND driver")
    out = tmp_path_factory.mktemp("philox") / "rocrand_pin"
    subprocess.check_call([hipcc, "-O1", os.path.join(HERE, "philox_rocrand_pin.cpp"),
                           "-o", str(out)], stderr=subprocess.DEVNULL)
    return str(out)


def test_philox_matches_rocrand(oracle_mod, rocrand_driver):
    pairs = _pairs(200)
    stdin = "\n".join(" ".join(f"{v:x}" for v in p) for p in pairs) + "\n"
    res = subprocess.run([rocrand_driver], input=stdin, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    for p, line in zip(pairs, res):
        want = [int(t, 16) for t in line.split()]
        got = oracle_mod.philox4x32_10(p[:4], p[4:]).tolist()
        assert got == want, (p, got, want)


def test_philox_is_a_bijection_sample(oracle_mod):
    # distinct counters under one key must give distinct blocks
    seen = set()
    for row in range(64):
        for pos in range(16):
            for off in (0, 1, 2**32, 2**63 + 5):
                blk = tuple(oracle_mod.philox4x32_10(
                    [pos, row, off & 0xFFFFFFFF, off >> 32], [0x1234, 0x5678]).tolist())
                assert blk not in seen
                seen.add(blk)


def test_uniforms_are_24bit_words_0_and_1(oracle_mod):
    seed, offset = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    for row, pos in [(0, 0), (5, 3), (2**31, 7), (12345, 0)]:
        u_acc, u_smp = oracle_mod.uniforms(seed, offset, row, pos)
        blk = oracle_mod.philox4x32_10(
            [pos, row, offset & 0xFFFFFFFF, offset >> 32],
            [seed & 0xFFFFFFFF, seed >> 32])
        assert u_acc == (int(blk[0]) >> 8) / 2**24
        assert u_smp == (int(blk[1]) >> 8) / 2**24
        # exact in fp32
        assert np.float32(u_acc) == u_acc and np.float32(u_smp) == u_smp
        assert 0.0 <= u_acc < 1.0 and 0.0 <= u_smp < 1.0


def test_uniforms_chi_square(oracle_mod):
    us = []
    for row in range(200):
        for pos in range(50):
            us.extend(oracle_mod.uniforms(99, 3, row, pos))
    us = np.asarray(us)
    counts, _ = np.histogram(us, bins=64, range=(0.0, 1.0))
    assert scipy.stats.chisquare(counts).pvalue > 1e-4
    # the acceptance and sampling uniforms of one block are uncorrelated
    a, s = us[0::2], us[1::2]
    assert abs(np.corrcoef(a, s)[0, 1]) < 4.5 / np.sqrt(len(a))
