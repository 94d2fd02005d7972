"""Philox4x64-10 counter-based generator and the uniforms / Gumbel draws the
path consumes.  Test infrastructure only (see the package docstring).

Philox is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11), section 3 (the Philox
S-box: two 64x64->128-bit multiplies per round, Weyl key schedule), ten rounds.
Counter-based draws let the oracle replay exactly the numbers the GPU drew,
which the verification step needs (DStill "Inference": standard
rejection-sampling verifier; the draws are inputs to it).

Stream layout (a reading; the pages fix none):
  counter = (t, pos, seq, (cycle << 8) | purpose), key = (seed, 0)
  element j of a stream lives in block t = j // 8, 64-bit word (j // 2) % 4,
  32-bit half j % 2 (high half first);
  u = ((x >> 8) | 1) * 2^-24   in [2^-24, 1 - 2^-24], exact in float32;
  Gumbel g = -log(-log u).
Purposes: 0 draft Gumbel, 1 accept uniform, 2 residual / bonus Gumbel,
3 shared Gumbel (seq forced to 0, pos = block slot).
"""

from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_RESIDUAL = 2
PURPOSE_SHARED = 3


def _mulhilo(a, b):
    """Full 128-bit product of 64-bit words, as (high, low) uint64."""
    a0, a1 = a & _LO32, a >> _S32
    b0, b1 = b & _LO32, b >> _S32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    return hi, a * b


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox-4x64 rounds on broadcastable uint64 arrays; returns 4 words."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3))
        k0 = np.asarray(k0, dtype=np.uint64)
        k1 = np.asarray(k1, dtype=np.uint64)
        for _ in range(10):
            hi0, lo0 = _mulhilo(_M0, c0)
            hi1, lo1 = _mulhilo(_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            k0 = k0 + _W0
            k1 = k1 + _W1
    return c0, c1, c2, c3


def raw32(seed, purpose, seq, pos, cycle, j):
    """32-bit draw number j of stream (purpose, seq, pos, cycle); all
    arguments broadcast against each other."""
    j = np.asarray(j, dtype=np.uint64)
    t = j >> np.uint64(3)
    word = (j >> np.uint64(1)) & np.uint64(3)
    half = j & np.uint64(1)
    c3 = (np.asarray(cycle, dtype=np.uint64) << np.uint64(8)) | np.asarray(
        purpose, dtype=np.uint64)
    w = philox4x64_10(t, np.asarray(pos, dtype=np.uint64),
                      np.asarray(seq, dtype=np.uint64), c3,
                      np.uint64(seed), np.uint64(0))
    w0, w1, w2, w3, word, half = np.broadcast_arrays(*w, word, half)
    picked = np.choose(word.astype(np.int64), [w0, w1, w2, w3])
    return np.where(half == 0, picked >> _S32, picked & _LO32)


def uniform(seed, purpose, seq, pos, cycle, j):
    """Uniform in [2^-24, 1 - 2^-24] (float64, exactly float32-representable)."""
    x = raw32(seed, purpose, seq, pos, cycle, j)
    return ((x >> np.uint64(8)) | np.uint64(1)).astype(np.float64) * 2.0 ** -24


def gumbel(seed, purpose, seq, pos, cycle, j):
    """Standard Gumbel draw -log(-log u), float64."""
    u = uniform(seed, purpose, seq, pos, cycle, j)
    return -np.log(-np.log(u))


def gumbel_row(seed, purpose, seq, pos, cycle, n):
    """The first n Gumbel draws of one stream, shape [n]."""
    return gumbel(seed, purpose, seq, pos, cycle, np.arange(n, dtype=np.uint64))
