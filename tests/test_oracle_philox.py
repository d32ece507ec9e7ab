"""Pins for the oracle's Philox4x32-10: published known-answer vectors, the vectorized
form against the scalar form, and uniformity of the derived float32 uniforms."""
import json
import os

import numpy as np
from scipy import stats

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_known_answer_vectors():
    kat = json.load(open(GOLDEN))
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        out = [int(x, 16) for x in v["out"]]
        assert list(philox.philox4x32_10(ctr, key)) == out


def test_vectorized_matches_scalar():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(4, 257), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = philox.philox4x32_10_np(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(c.shape[1]):
        ref = philox.philox4x32_10([int(c[w, i]) for w in range(4)], (k0, k1))
        assert tuple(int(vec[w][i]) for w in range(4)) == ref


def test_uniform_is_24bit_and_in_range():
    u = philox.uniforms_np(7, np.arange(4096), 3, 0, philox.STREAM_ACCEPT)
    assert u.dtype == np.float32
    assert np.all(u >= 0) and np.all(u < 1)
    scaled = u.astype(np.float64) * 2**24
    assert np.array_equal(scaled, np.floor(scaled))
    # scalar and vector paths agree
    for i in (0, 1, 17, 4095):
        assert philox.uniform(7, i, 3, 0, philox.STREAM_ACCEPT) == u[i]


def test_uniformity_chi2():
    u = philox.uniforms_np(0, np.arange(1 << 16), np.arange(1 << 16) % 7, 1, 2)
    counts, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
    p = stats.chisquare(counts).pvalue
    assert p > 1e-6


def test_streams_and_counters_differ():
    a = philox.uniform(1, 1, 0, 0, 0)
    b = philox.uniform(1, 1, 0, 0, 1)
    c = philox.uniform(1, 2, 0, 0, 0)
    d = philox.uniform(2, 1, 0, 0, 0)
    assert len({float(a), float(b), float(c), float(d)}) == 4
