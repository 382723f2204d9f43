"""Philox4x32-10 counter-based generator, written from [SC11].

TEST INFRASTRUCTURE ONLY (see the package docstring).

Philox-4x32 maps a 128-bit counter (four 32-bit words) and a 64-bit key (two
32-bit words) to 128 random bits by applying R=10 rounds of a keyed bijection.
One round multiplies words 0 and 2 by two fixed odd 32-bit multipliers, keeping
the full 64-bit products; the high halves are XORed with the opposite odd words
and with the round key, and the words are permuted.  Between rounds the key is
advanced by two Weyl increments (the golden ratio and sqrt(3)-1 in 32-bit fixed
point).  The constants below are the ones the paper gives for Philox4x32.

The functions work on whole NumPy arrays of counters at once; each word is held
in a uint64 array whose values stay below 2**32, so the 32x32 -> 64 products are
exact.

Parity: pinned by ``tests/test_oracle_philox.py`` against the independent
Philox4x32-10 engine in rocRAND's source headers (built for the host with g++),
plus statistical checks of the dropout decisions derived from it.
"""

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)

# Round multipliers and key increments for Philox4x32 [SC11, sec. 4].
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)
PHILOX_W1 = np.uint64(0xBB67AE85)
PHILOX_ROUNDS = 10


def _u32(a):
    return np.asarray(a, dtype=np.uint64) & MASK32


def philox4x32(counter, key, rounds=PHILOX_ROUNDS):
    """Apply the Philox4x32 bijection.

    counter: tuple of four arrays (or ints) -- words c0..c3, each < 2**32,
             broadcast against one another.
    key:     tuple of two ints (k0, k1), each < 2**32.
    Returns a tuple of four uint64 arrays holding the 32-bit output words.
    """
    c0, c1, c2, c3 = (_u32(c) for c in counter)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for r in range(rounds):
        if r > 0:
            # Key schedule: the key for round r is the original key plus r Weyl steps.
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * c0          # full 64-bit product of the 32-bit words
        prod1 = PHILOX_M1 * c2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & MASK32
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox_words(block_index, seed, stream):
    """128 random bits for each block index, as a (n, 4) uint64 array of words.

    The counter is (lo32(block), hi32(block), lo32(stream), hi32(stream)) and
    the key is (lo32(seed), hi32(seed)).  ``block_index`` is a 1-D integer array
    (values below 2**64); ``seed`` and ``stream`` are Python ints below 2**64.
    """
    b = np.asarray(block_index, dtype=np.uint64)
    seed = int(seed)
    stream = int(stream)
    words = philox4x32(
        (b & MASK32, b >> np.uint64(32), stream & 0xFFFFFFFF, (stream >> 32) & 0xFFFFFFFF),
        (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF),
    )
    return np.stack(words, axis=-1)


def random_fields(index, bits, seed, stream):
    """The ``bits``-wide random field that belongs to element ``index``.

    One Philox call yields 128 bits, cut into 128/bits fields.  Element i uses
    call number i // (128/bits) and field i % (128/bits); fields are taken from
    word 0 upward and, inside a word, from the least significant end upward.
    ``index`` is a 1-D integer array of flat element indices.
    """
    if bits not in (8, 16, 32):
        raise ValueError("bits must be 8, 16 or 32")
    per_call = 128 // bits
    idx = np.asarray(index, dtype=np.uint64).reshape(-1)
    if idx.size == 0:
        return np.zeros(0, dtype=np.uint64)
    block = idx // np.uint64(per_call)
    bmin, bmax = int(block.min()), int(block.max())
    if bmax - bmin + 1 <= idx.size:
        # Dense index set (the usual case, a whole tensor): one call per block.
        blocks = np.arange(bmin, bmax + 1, dtype=np.uint64)
        first = bmin
    else:
        blocks = np.unique(block)
        first = None
    words = philox_words(blocks, seed, stream)                  # (nb, 4)
    mask = np.uint64((1 << bits) - 1)
    # fields[b, f] = field f of call b: word f*bits//32, shifted from the low end.
    fields = np.empty((blocks.size, per_call), dtype=np.uint64)
    for f in range(per_call):
        pos = f * bits
        fields[:, f] = (words[:, pos // 32] >> np.uint64(pos % 32)) & mask
    if first is not None:
        return fields.reshape(-1)[(idx - np.uint64(first * per_call)).astype(np.int64)]
    row = np.searchsorted(blocks, block)
    return fields[row, (idx % np.uint64(per_call)).astype(np.int64)]
