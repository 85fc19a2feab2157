"""Philox4x32-10 counter-based generator (test infrastructure only).

Written from the definition in Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC 2011): a 128-bit counter (four 32-bit words)
and a 64-bit key (two words) go through ten rounds.  Each round multiplies
words 0 and 2 by the constants M0 and M1, keeps the high and low halves of the
64-bit products, and mixes them with words 1 and 3 and the round key; the key
is advanced by the Weyl constants W0 and W1 between rounds.

Canvas use (uniform-state noise): a draw for canvas position ``i`` uses the
counter ``(i, step_tag, canvas, block)`` and the key ``(seed mod 2**32,
seed >> 32)``; the token id is output word 0 modulo the vocabulary size.
``step_tag`` is 0 for the initial canvas and ``s + 1`` for the re-noise that
follows denoise step ``s``.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(ctr, key):
    """Apply Philox4x32-10.

    ``ctr``: array-like of shape (4, n) (or (4,)) of 32-bit words; ``key``: (k0, k1).
    Returns a uint64 array of the same shape holding the four 32-bit output words.
    """
    c = np.array(ctr, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = (c[0].copy(), c[1].copy(), c[2].copy(), c[3].copy())
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    m0, m1 = np.uint64(M0), np.uint64(M1)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & 0xFFFFFFFF
            k1 = (k1 + W1) & 0xFFFFFFFF
        p0 = m0 * c0                       # < 2**64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> _SH, p0 & _MASK
        hi1, lo1 = p1 >> _SH, p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
    return np.stack([c0, c1, c2, c3])


def seed_key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def canvas_draw(seed: int, positions, step_tag: int, canvas: int, block: int, vocab: int):
    """Token ids for ``positions`` under counter ``(pos, step_tag, canvas, block)``."""
    pos = np.asarray(positions, dtype=np.uint64)
    n = pos.shape[0]
    ctr = np.stack([pos,
                    np.full(n, step_tag & 0xFFFFFFFF, np.uint64),
                    np.full(n, canvas & 0xFFFFFFFF, np.uint64),
                    np.full(n, block & 0xFFFFFFFF, np.uint64)])
    x = philox4x32_10(ctr, seed_key(seed))
    return (x[0] % np.uint64(vocab)).astype(np.int64)
