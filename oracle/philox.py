"""Philox4x32-10 and the uniform map (oracle side, numpy).

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 128-bit counter and a
64-bit key go through ten rounds of two 32x32->64-bit multiplies and xors,
with a Weyl increment of the key between rounds.

Counter layout used by every draw of the path (the pages fix none; this is the
layout both sides implement):

    key     = (seed & 0xffffffff, seed >> 32)
    counter = (index >> 2, position, request_id, tag)
    value   = output word (index & 3)

``index`` is the vocabulary index of the element being drawn for (0 for scalar
draws), ``position`` the draft position in the block, ``request_id`` the
caller's 32-bit request id, ``tag`` the purpose of the draw:

    TAG_DRAFT   0  Gumbel noise of the Markov-loop sampler
    TAG_ACCEPT  1  acceptance uniform of the rejection test
    TAG_RESID   2  exponential race of the residual resample
    TAG_BONUS   3  exponential race of the bonus token
    TAG_TARGET  4  Gumbel noise of a target id outside the draft vocabulary
                   (Gumbel-coupled verification)

Uniform map: ``u = ((w >> 8) | 1) * 2**-24`` -- exact in float32, odd
multiples of 2**-24, so never 0 and never 1.

Pins: the published known-answer vectors of Philox4x32-10 (tests/golden);
Kolmogorov-Smirnov uniformity of ``u``.
"""
from __future__ import annotations

import numpy as np

TAG_DRAFT, TAG_ACCEPT, TAG_RESID, TAG_BONUS, TAG_TARGET = 0, 1, 2, 3, 4

_MASK = np.uint64(0xFFFFFFFF)
_MUL0 = np.uint64(0xD2511F53)   # multiplier of counter word 0
_MUL1 = np.uint64(0xCD9E8D57)   # multiplier of counter word 2
_WEYL0 = 0x9E3779B9             # key increments (golden ratio, sqrt(3)-1)
_WEYL1 = 0xBB67AE85


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox rounds on broadcastable uint32-valued arrays.

    Returns the four output words as uint64 arrays holding 32-bit values.
    """
    x0 = np.asarray(c0, dtype=np.uint64)
    x1 = np.asarray(c1, dtype=np.uint64)
    x2 = np.asarray(c2, dtype=np.uint64)
    x3 = np.asarray(c3, dtype=np.uint64)
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    key0 = int(k0) & 0xFFFFFFFF
    key1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            key0 = (key0 + _WEYL0) & 0xFFFFFFFF
            key1 = (key1 + _WEYL1) & 0xFFFFFFFF
        p0 = _MUL0 * x0                      # < 2**64, no wrap
        p1 = _MUL1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(key0), lo1,
                          hi0 ^ x3 ^ np.uint64(key1), lo0)
    return x0, x1, x2, x3


def words(seed: int, index, position, request_id, tag) -> np.ndarray:
    """The 32-bit word drawn for (seed, index, position, request_id, tag).

    All of index/position/request_id/tag may be arrays (broadcast).
    """
    idx = np.asarray(index, dtype=np.uint64)
    out = philox4x32_10(idx >> np.uint64(2), position, request_id, tag,
                        int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    sel = (idx & np.uint64(3)).astype(np.int64)
    stacked = np.stack(np.broadcast_arrays(*out), axis=-1)
    sel = np.broadcast_to(sel, stacked.shape[:-1])
    return np.take_along_axis(stacked, sel[..., None], axis=-1)[..., 0]


def uniform(w) -> np.ndarray:
    """Uniform map of a 32-bit word to float32 in (0, 1), exact."""
    w = np.asarray(w, dtype=np.uint64)
    q = ((w >> np.uint64(8)) | np.uint64(1)).astype(np.float32)   # < 2**24: exact
    return q * np.float32(2.0 ** -24)


def uniforms(seed: int, index, position, request_id, tag) -> np.ndarray:
    return uniform(words(seed, index, position, request_id, tag))
