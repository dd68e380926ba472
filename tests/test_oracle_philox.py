"""Pins of the oracle's Philox4x32-10 (CPU only)."""
import json
from pathlib import Path

import numpy as np
import pytest
from scipy import stats

from oracle import philox

GOLDEN = Path(__file__).parent / "golden"


def _kat():
    return json.loads((GOLDEN / "philox_kat.json").read_text())["cases"]


@pytest.mark.parametrize("case", _kat())
def test_known_answers_pure(case):
    ctr = [int(x, 16) for x in case["counter"]]
    key = [int(x, 16) for x in case["key"]]
    assert philox.philox4x32_10(ctr, key) == tuple(int(x, 16) for x in case["out"])


@pytest.mark.parametrize("case", _kat())
def test_known_answers_numpy(case):
    c = [np.uint32(int(x, 16)) for x in case["counter"]]
    k = [int(x, 16) for x in case["key"]]
    out = philox.philox4x32_10_np(*c, *k)
    assert tuple(int(o) for o in out) == tuple(int(x, 16) for x in case["out"])


def test_numpy_matches_pure_on_random_counters():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 2 ** 32, size=(4, 2000), dtype=np.uint64)
    for key in [(0, 0), (0xDEADBEEF, 0x12345678), (0xFFFFFFFF, 1)]:
        out = philox.philox4x32_10_np(*c, *key)
        for j in range(0, 2000, 97):
            ref = philox.philox4x32_10([int(c[r, j]) for r in range(4)], key)
            assert tuple(int(o[j]) for o in out) == ref


def test_block_uniforms_layout():
    seed, offset = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    u, v = philox.block_uniforms(seed, offset, b=3, i=5)
    x = philox.philox4x32_10((5, 3, offset & 0xFFFFFFFF, offset >> 32),
                             (seed & 0xFFFFFFFF, seed >> 32))
    assert u == x[0] / 2.0 ** 32
    assert v == (x[1] * 2 ** 21 + (x[2] >> 11)) / 2.0 ** 53
    uu, vv = philox.block_uniforms_np(seed, offset, np.array([3]), np.array([5]))
    assert uu[0] == u and vv[0] == v
    assert 0.0 <= u < 1.0 and 0.0 <= v < 1.0


def test_uniformity_chi_square():
    n = 200_000
    u, v = philox.block_uniforms_np(42, 7, np.arange(n) % 8, np.arange(n) // 8)
    for x in (u, v):
        counts = np.bincount((x * 100).astype(int), minlength=100)
        assert stats.chisquare(counts).pvalue > 1e-4
    # u and v of one draw are not correlated
    assert abs(np.corrcoef(u, v)[0, 1]) < 0.01
