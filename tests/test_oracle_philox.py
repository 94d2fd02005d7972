"""Pins for the oracle's Philox4x64-10 and the uniform / Gumbel mapping.

Pinned against (a) the published known-answer vectors of the generator
(tests/golden/philox4x64_10_kat.txt) and (b) numpy's own Philox4x64-10 bit
generator, a library routine independent of the oracle's implementation."""

import os

import numpy as np

from oracle import philox

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x64_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = line.split("|")
        rows.append(([int(x, 16) for x in a.split()], [int(x, 16) for x in b.split()]))
    return rows


def test_known_answer_vectors():
    rows = _kat()
    assert len(rows) == 3
    for inp, out in rows:
        got = philox.philox4x64_10(*[np.uint64(x) for x in inp])
        assert [int(x) for x in got] == out


def _numpy_block(ctr, key):
    """Block at counter ctr from numpy's Philox.  numpy increments the 256-bit
    counter before producing a block, so start one below."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(ctr))
    g = np.random.Philox(counter=(c - 1) % (1 << 256), key=key[0] | (key[1] << 64))
    return [int(x) for x in g.random_raw(4)]


def test_matches_numpy_philox():
    rng = np.random.default_rng(123)
    ctrs = rng.integers(0, 2**63, size=(64, 4), dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=(64, 4), dtype=np.uint64)
    keys = rng.integers(0, 2**63, size=(64, 2), dtype=np.uint64)
    got = philox.philox4x64_10(ctrs[:, 0], ctrs[:, 1], ctrs[:, 2], ctrs[:, 3],
                               keys[:, 0], keys[:, 1])
    for i in range(64):
        ref = _numpy_block([int(x) for x in ctrs[i]], [int(keys[i, 0]), int(keys[i, 1])])
        assert [int(g[i]) for g in got] == ref


def test_stream_layout_against_numpy():
    # element j of stream (purpose, seq, pos, cycle): block j//8, word (j//2)%4,
    # high half first; counter = (j//8, pos, seq, cycle<<8 | purpose), key = (seed, 0)
    seed, purpose, seq, pos, cycle = 7, 2, 5, 3, 11
    j = np.arange(40, dtype=np.uint64)
    got = philox.raw32(seed, purpose, seq, pos, cycle, j)
    for t in range(5):
        words = _numpy_block([t, pos, seq, (cycle << 8) | purpose], [seed, 0])
        halves = []
        for w in words:
            halves += [w >> 32, w & 0xFFFFFFFF]
        assert [int(x) for x in got[8 * t:8 * t + 8]] == halves


def test_uniform_range_and_exactness():
    u = philox.uniform(3, 1, np.arange(100)[:, None], np.arange(16)[None, :], 9, 0)
    k = u * 2.0 ** 24
    assert np.all(k == np.round(k))
    assert np.all(k % 2 == 1)           # (x >> 8) | 1 is odd
    assert u.min() >= 2.0 ** -24 and u.max() <= 1 - 2.0 ** -24
    assert np.all(u.astype(np.float32) == u)   # exact in float32


def test_uniform_is_uniform():
    u = philox.uniform(0, 0, 0, 0, 0, np.arange(200000, dtype=np.uint64))
    # Kolmogorov-Smirnov against U(0,1)
    from scipy import stats
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    g = philox.gumbel(0, 0, 0, 0, 0, np.arange(200000, dtype=np.uint64))
    assert stats.kstest(g, "gumbel_r").pvalue > 1e-4
    assert abs(np.mean(g) - np.euler_gamma) < 0.01
