"""Philox4x32-10 counter-based generator and the fixed H32 sign mask.

The pages fix only that stochastic-rounding state is a seed plus a counter
offset that is checkpointed so a resumed run never reuses draws
("Format-Aware Fusion for Fast FP4 Pretraining", App. A.1).  The generator is
Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw ("Parallel random
numbers: as easy as 1, 2, 3", SC'11): a four-word counter, a two-word key, ten
rounds of two 32x32->64 multiplies with xors, and a Weyl-sequence key bump
between rounds.

Counter layout (a reading; the pages are silent):
  key     = (lo32(seed), hi32(seed))
  counter = (lo32(i >> 2), hi32(i >> 2), lo32(offset), hi32(offset))
  draw(i) = output word (i & 3)
where i is the element's row-major index in the logical tensor.  Draws depend
only on (seed, offset, i), never on tiling, and distinct offsets address
disjoint counter ranges.

Pins: published known-answer vectors are not available offline, so the tests
check this module against an independent implementation of the same generator,
rocRAND's host-callable Philox4x32-10 engine compiled from its open-source
header (every draw and the sign mask, with the SR offset as rocRAND's
subsequence and the element index as its offset), besides structure
(bijectivity of a round, key-schedule and layout invariants) and statistics.
Agreement with the GPU generator is checked separately.

Parity unpinned: the sign vector itself (sign_mask_from_seed).  The pages fix
one 16-entry vector for both Wgrad operands but do not print its entries; the
tests pin the generator that derives it, not its agreement with the pages.
"""

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo(a, b):
    p = np.asarray(a, dtype=np.uint64) * np.uint64(b)
    return (p >> np.uint64(32)), (p & MASK32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four output words for counters (c0..c3) under key (k0, k1).

    All arguments are broadcastable uint32-valued arrays; outputs are uint64
    arrays holding 32-bit values.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & MASK32
        hi0, lo0 = _mulhilo(c0, PHILOX_M0)
        hi1, lo1 = _mulhilo(c2, PHILOX_M1)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def draws(seed, offset, index):
    """32-bit SR draw for each logical element index (uint64 array)."""
    index = np.asarray(index, dtype=np.uint64)
    blk = index >> np.uint64(2)
    seed, offset = int(seed), int(offset)
    out = philox4x32_10(blk & MASK32, blk >> np.uint64(32),
                        offset & 0xFFFFFFFF, (offset >> 32) & 0xFFFFFFFF,
                        seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    word = index & np.uint64(3)
    res = np.where(word == 0, out[0], np.where(word == 1, out[1], np.where(word == 2, out[2], out[3])))
    return res.astype(np.uint64)


def sign_mask_from_seed(seed):
    """Fixed 16-entry sign vector as a bit mask (bit j set => d_j = -1).

    The pages reuse a literal 16-sign constant that is not reproduced here; a
    synthetic fixed vector is drawn instead: the low 16 bits of word 0 of
    Philox4x32-10 at counter (0,0,0,0) under key (lo32(seed), hi32(seed)).
    """
    seed = int(seed)
    out = philox4x32_10(0, 0, 0, 0, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return int(out[0]) & 0xFFFF
