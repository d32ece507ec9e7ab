"""Philox4x32-10 (oracle side).

Written from the definition in Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11): a 4x32-bit counter and a 2x32-bit key; each of
the 10 rounds multiplies counter words 0 and 2 by two fixed odd constants, takes the
high and low halves of the 64-bit products, and mixes them with words 1 and 3 and the
round key; the key advances by the two Weyl constants between rounds.

The pages do not say which random numbers the accept rule draws; the uniforms here
come from this generator, keyed by the run seed and indexed by a counter
(slot, round, sequence, stream) so that the oracle and the kernels draw the same
numbers without passing them around.  Streams: 0 = draft sampling, 1 = accept test,
2 = residual / bonus sample.  A uniform is word 0 shifted right by 8, times 2^-24,
which is exact in float32 and lies in [0, 1 - 2^-24].
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
MUL0 = 0xD2511F53
MUL1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85

STREAM_DRAFT = 0
STREAM_ACCEPT = 1
STREAM_RESIDUAL = 2


def philox4x32_10(ctr, key):
    """One block: ctr = 4 uint32, key = 2 uint32 -> 4 uint32 (Python ints)."""
    c0, c1, c2, c3 = (int(c) & MASK32 for c in ctr)
    k0, k1 = (int(k) & MASK32 for k in key)
    for r in range(10):
        if r:
            k0 = (k0 + WEYL0) & MASK32
            k1 = (k1 + WEYL1) & MASK32
        p0 = MUL0 * c0
        p1 = MUL1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorized over counters (uint32-valued numpy arrays), same arithmetic in uint64."""
    m = np.uint64(MASK32)
    c0 = np.asarray(c0, dtype=np.uint64) & m
    c1 = np.asarray(c1, dtype=np.uint64) & m
    c2 = np.asarray(c2, dtype=np.uint64) & m
    c3 = np.asarray(c3, dtype=np.uint64) & m
    k0 = int(k0) & MASK32
    k1 = int(k1) & MASK32
    for r in range(10):
        if r:
            k0 = (k0 + WEYL0) & MASK32
            k1 = (k1 + WEYL1) & MASK32
        p0 = np.uint64(MUL0) * c0
        p1 = np.uint64(MUL1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return c0, c1, c2, c3


def seed_key(seed: int):
    return int(seed) & MASK32, (int(seed) >> 32) & MASK32


def uniform(seed: int, slot: int, rnd: int, seq: int, stream: int) -> np.float32:
    """The float32 uniform for counter (slot, round, seq, stream) under key = seed."""
    x0 = philox4x32_10((slot, rnd, seq, stream), seed_key(seed))[0]
    return np.float32((x0 >> 8) * (1.0 / 16777216.0))


def uniforms_np(seed: int, slot, rnd, seq, stream) -> np.ndarray:
    """Vectorized ``uniform`` (broadcasting counter arrays)."""
    slot, rnd, seq, stream = np.broadcast_arrays(np.asarray(slot), np.asarray(rnd),
                                                 np.asarray(seq), np.asarray(stream))
    k0, k1 = seed_key(seed)
    x0 = philox4x32_10_np(slot, rnd, seq, stream, k0, k1)[0]
    return ((x0 >> np.uint64(8)).astype(np.float64) * (1.0 / 16777216.0)).astype(np.float32)
