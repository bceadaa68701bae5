"""Philox4x32-10 counter-based generator and the dropout keep mask, in numpy.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle). Nothing in the product path
may import this module; the GPU kernels carry their own implementation.

The dropout rule comes from "Lecture 7 - Backward Pass and Validation",
section "Dropout": the kernel draws a Bernoulli keep mask from a Philox
generator seeded by (seed, offset), and a checker must draw the same mask.
The page gives no mapping from (seed, offset, element) to Philox words, so
this oracle fixes one: the seed is the key, the offset the low counter
words, the element the high ones.  Each Philox block (128 bits) serves
eight keys of one row, 16 bits each: two runs of four keys eight apart,
j0 .. j0 + 3 and j0 + 8 .. j0 + 11 with j0 = 16 m or 16 m + 4 (so a block of
16 consecutive keys is served by two Philox blocks).  For key j:

    j0      = (j - j mod 16) + (j mod 8 - j mod 4)    (the block's first key)
    pos     = 4 * ((j mod 16) div 8) + j mod 4       (0 .. 7 within the block)
    key     = (low 32 bits of seed, high 32 bits of seed)
    counter = (low 32 bits of offset, high 32 bits of offset,
               (i << 16) | j0, (b << 16) | h)
    w       = word (pos div 2) of Philox4x32-10(counter, key)
    x       = the low 16 bits of w for even pos, the high 16 bits for odd pos
    keep    = x >= T,  T = ceil(p * 2**16)   (exactly x / 2**16 >= p)

so a key is kept with probability 1 - T / 2**16, within 2**-16 of 1 - p.

The block function is Philox4x32 with 10 rounds as published by Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
each round multiplies counter words 0 and 2 by two fixed odd constants,
keeps both halves of the 64-bit products and mixes them with words 1 and 3
and the key; the key is advanced by two Weyl constants between rounds.
"""

import math

import numpy as np

# Round multipliers and key-schedule (Weyl) increments of Philox4x32 (SC'11).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

_MASK32 = np.uint64(0xFFFFFFFF)


def _u64(x):
    return np.asarray(x, dtype=np.uint64)


def philox4x32_10(counter, key, rounds=10):
    """Apply the Philox4x32 bijection to a (broadcastable) batch of counters.

    counter: 4 integer arrays (each element < 2**32); key: 2 integers/arrays.
    Returns the 4 output words as uint32 arrays.  All arithmetic is done in
    uint64 so the 32x32 -> 64-bit products are exact.
    """
    c0, c1, c2, c3 = (_u64(c) for c in counter)
    k0, k1 = (_u64(k) for k in key)
    for r in range(rounds):
        if r > 0:  # key schedule: bump the key before every round but the first
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        prod0 = np.uint64(PHILOX_M0) * c0  # < 2**64, exact
        prod1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & _MASK32
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def keep_threshold(p):
    """Integer threshold T = ceil(p * 2**16); keep iff the 16-bit draw >= T.

    p * 2**16 is exact in binary64 (a power-of-two scaling), so T is exact.
    """
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    t = math.ceil(p * 65536.0)
    if t > 0xFFFF:
        raise ValueError("dropout probability too close to 1")
    return t


def dropout_uniform_bits(seed, offset, b, h, rows, cols):
    """The 16-bit draw x for every (i, j) in rows x cols of head (b, h)."""
    rows = _u64(rows).reshape(-1, 1)
    cols = _u64(cols).reshape(1, -1)
    if (rows.size and rows.max() >= 65536) or (cols.size and cols.max() >= 65536):
        raise ValueError("row/column index must be < 65536 for the dropout counter")
    if b >= 65536 or h >= 65536:
        raise ValueError("batch/head index must be < 65536 for the dropout counter")
    seed = int(seed)
    offset = int(offset)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    group = (cols & ~np.uint64(15)) | (cols & np.uint64(4))   # j0, the block's first key
    pos = ((cols >> np.uint64(1)) & np.uint64(4)) | (cols & np.uint64(3))
    word = (pos >> np.uint64(1)).astype(np.int64)
    half = (pos & np.uint64(1)) * np.uint64(16)   # bit position of the key's half
    w2 = (rows << np.uint64(16)) | group
    w3 = np.uint64((int(b) << 16) | int(h))
    shape = w2.shape
    counter = (
        np.full(shape, offset & 0xFFFFFFFF, dtype=np.uint64),
        np.full(shape, (offset >> 32) & 0xFFFFFFFF, dtype=np.uint64),
        w2,
        np.full(shape, w3, dtype=np.uint64),
    )
    words = np.stack(philox4x32_10(counter, key))       # [4, rows, cols]
    word = np.broadcast_to(word, shape)
    w = np.take_along_axis(words, word[None], axis=0)[0].astype(np.uint64)
    return ((w >> np.broadcast_to(half, shape)) & np.uint64(0xFFFF)).astype(np.uint32)


def dropout_keep(seed, offset, b, h, rows, cols, p):
    """Keep mask Z (uint8, 1 = kept) for rows x cols of head (b, h)."""
    t = keep_threshold(p)
    x = dropout_uniform_bits(seed, offset, b, h, rows, cols)
    return (x.astype(np.uint64) >= np.uint64(t)).astype(np.uint8)
