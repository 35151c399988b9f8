"""Counter-based uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11), written from its published definition.

The pages say nothing about how random draws are made; the reading used here (and by the
HIP path, which carries its own implementation) is:

* key     = (seed, 0)
* counter = (index // 4, row, purpose, offset)      (four 64-bit words)
* the draw for `index` is output word ``index % 4`` of the block
* u = ((word >> 41) + 0.5) * 2**-23: the top 23 bits, centred in their cell, so that
  2u * 2**23 is an odd integer below 2**24 -- exactly representable in float32 -- and u
  lies strictly inside (0, 1), in [2**-24, 1 - 2**-24].

Purposes: 0 draft group, 1 draft element, 2 verify accept, 3 residual group,
4 residual element, 5 bonus group, 6 bonus element.
"""
import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
MASK64 = (1 << 64) - 1
ROUNDS = 10

PURPOSE_DRAFT_GROUP = 0
PURPOSE_DRAFT_ELEM = 1
PURPOSE_ACCEPT = 2
PURPOSE_RESID_GROUP = 3
PURPOSE_RESID_ELEM = 4
PURPOSE_BONUS_GROUP = 5
PURPOSE_BONUS_ELEM = 6


def philox4x64_10(counter, key):
    """One Philox4x64-10 block on Python integers: 4 x 64-bit counter, 2 x 64-bit key."""
    c = [int(v) & MASK64 for v in counter]
    k = [int(v) & MASK64 for v in key]
    for rnd in range(ROUNDS):
        if rnd:
            k = [(k[0] + W0) & MASK64, (k[1] + W1) & MASK64]
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return c


def word_to_uniform(word):
    """Top 23 bits of a 64-bit word -> float in (0,1), centred in its 2^-23 cell."""
    return ((int(word) >> 41) + 0.5) * 2.0 ** -23


def uniform(seed, offset, purpose, row, index):
    """Scalar uniform for (seed, offset, purpose, row, index)."""
    block = philox4x64_10((index // 4, row, purpose, offset), (seed, 0))
    return word_to_uniform(block[index % 4])


# ---- vectorised variant (same arithmetic on numpy uint64 lanes, 32-bit limbs for mulhi) ----

_L32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a_const, b):
    """(hi, lo) of a_const * b for a Python-int constant and a uint64 array."""
    a_lo = np.uint64(a_const & 0xFFFFFFFF)
    a_hi = np.uint64(a_const >> 32)
    b_lo = b & _L32
    b_hi = b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _L32) + (hl & _L32)
    lo = (ll & _L32) | ((mid & _L32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10_vec(c0, c1, c2, c3, seed):
    """Philox4x64-10 over arrays of counters (broadcastable uint64), key (seed, 0)."""
    with np.errstate(over="ignore"):
        c = [np.asarray(v, dtype=np.uint64) for v in np.broadcast_arrays(c0, c1, c2, c3)]
        k0 = int(seed) & MASK64
        k1 = 0
        for rnd in range(ROUNDS):
            if rnd:
                k0 = (k0 + W0) & MASK64
                k1 = (k1 + W1) & MASK64
            hi0, lo0 = _mulhilo(M0, c[0])
            hi1, lo1 = _mulhilo(M1, c[2])
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return c


def uniforms(seed, offset, purpose, row, indices):
    """Vectorised uniforms for an array of indices (row may be an array broadcast with it)."""
    idx = np.asarray(indices, dtype=np.uint64)
    row = np.asarray(row, dtype=np.uint64)
    idx, row = np.broadcast_arrays(idx, row)
    words = philox4x64_10_vec(idx >> np.uint64(2), row, np.uint64(purpose), np.uint64(offset), seed)
    sel = (idx & np.uint64(3)).astype(np.int64)
    w = np.choose(sel, words)
    return ((w >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(u):
    """Standard Gumbel transform of a uniform: -log(-log u), float64."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))
