"""Pins for the oracle's Philox4x32-10 and uniform map (CPU only)."""
import os

import numpy as np

from oracle import philox4x32_10, philox_scalar, uniform01
from oracle.philox import mulhi_token


def _kat(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(v, 16) for v in line.split()])
    return rows


def test_known_answer_vectors_vectorised(golden_dir):
    for r in _kat(golden_dir):
        ctr, key, want = r[:4], r[4:6], r[6:]
        seed = key[0] | (key[1] << 32)
        got = philox4x32_10(*[np.array([c], np.uint32) for c in ctr], seed)
        assert [int(g[0]) for g in got] == want


def test_known_answer_vectors_scalar(golden_dir):
    for r in _kat(golden_dir):
        assert list(philox_scalar(r[:4], r[4:6])) == r[6:]


def test_vectorised_matches_scalar_on_random_counters():
    rng = np.random.default_rng(7)
    ctr = rng.integers(0, 2**32, size=(4, 50), dtype=np.uint64)
    seed = int(rng.integers(0, 2**63)) * 2 + 1
    got = philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], seed)
    for j in range(50):
        want = philox_scalar(ctr[:, j], (seed & 0xFFFFFFFF, seed >> 32))
        assert tuple(int(g[j]) for g in got) == want


def test_uniform_endpoints_and_exactness():
    w = np.array([0, 511, 512, 0xFFFFFFFF, 0x80000000], dtype=np.uint32)
    u = uniform01(w)
    assert u.dtype == np.float32
    assert u[0] == np.float32(2.0 ** -24) and u[1] == u[0]
    assert u[2] == np.float32(3 * 2.0 ** -24)
    assert u[3] == np.float32(1 - 2.0 ** -24)
    assert u[4] == np.float32(0.5 + 2.0 ** -24)
    # every value sits strictly inside (0, 1) and is exact in float32
    ww = np.random.default_rng(0).integers(0, 2**32, size=100000, dtype=np.uint64).astype(np.uint32)
    uu = uniform01(ww)
    assert np.all(uu > 0) and np.all(uu < 1)
    exact = ((ww >> np.uint32(9)).astype(np.float64) * 2 + 1) / 2.0 ** 24
    assert np.array_equal(uu.astype(np.float64), exact)


def test_mulhi_token_is_uniform_partition():
    # floor(w * V / 2^32) maps exactly 2^32 / V words onto each token when V | 2^32
    V = 8
    edges = np.arange(V, dtype=np.uint64) * np.uint64(2**32 // V)
    assert np.array_equal(mulhi_token(edges, V), np.arange(V))
    assert np.array_equal(mulhi_token(edges - np.uint64(1), V)[1:], np.arange(V - 1))
    assert mulhi_token(np.uint64(2**32 - 1), V) == V - 1
