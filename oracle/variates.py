"""Variates built on the uniform map (oracle side).

Gumbel-max (stage 2).  Sampling x ~ softmax(l / T) by taking the argmax of
l_j / T + G_j with G_j = -ln(-ln u_j) i.i.d. standard Gumbel; the pages name
this sampler for the Markov loop (DSpark 的实现和测评, §2.2 and §5).  Here in
fp64.  Pins: KS test of G against the Gumbel CDF; chi-square of Gumbel-max
samples against softmax.

Exponential race (stage 3).  Sampling y with P(y = v) = r_v / sum(r) as the
argmax of r_v / E_v, E_v i.i.d. exponential.  E_v = -plog2(u_v): the base of
the logarithm only rescales every E_v by the same factor, which does not move
the argmax.  The comparison of two candidates (r_a, E_a), (r_b, E_b) is made
exactly: r_a * E_b against r_b * E_a, each a product of two float32 values and
hence exact in float64; ties go to the smaller index.  Pins: chi-square of race
winners against r / sum(r); order independence.

Portable log2 (``plog2``).  A log2 built only from IEEE float32 add, multiply
and divide (round to nearest even, no fused multiply-add), in one fixed order,
so that the GPU reproduces it bit for bit.  Method: write u = m * 2**e with
m in [sqrt(2)/2, sqrt(2)); then log2(u) = e + 2*atanh(s)/ln 2 with
s = (m - 1)/(m + 1), and 2*atanh(s)/ln 2 = s * (c1 + c3 s^2 + c5 s^4 + c7 s^6
+ c9 s^8 + ...), c_k = 2 / (k ln 2), truncated after c9 (|s| <= 0.1716, so the
dropped tail is below 1e-9) and evaluated by Horner's rule.  Pins: within a few
float32 ulp of math.log2, monotone, exact at powers of two.
"""
from __future__ import annotations

import math

import numpy as np

from . import philox

_F = np.float32
SQRT2_F32 = _F(np.uint32(0x3FB504F3).view(np.float32))   # float32 nearest sqrt(2), below it
_C = {k: _F(2.0 / (k * math.log(2.0))) for k in (1, 3, 5, 7, 9)}


def plog2(u) -> np.ndarray:
    """Portable float32 log2 of positive normal float32 values."""
    u = np.ascontiguousarray(u, dtype=np.float32)
    bits = u.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - 127
    m = ((bits & np.uint32(0x7FFFFF)) | np.uint32(0x3F800000)).view(np.float32)
    big = m > SQRT2_F32
    m = np.where(big, m * _F(0.5), m).astype(np.float32)      # exact halving
    e = np.where(big, e + 1, e)
    s = (m - _F(1.0)) / (m + _F(1.0))
    z = s * s
    p = _C[9]
    p = p * z + _C[7]       # numpy: multiply then add, two roundings
    p = p * z + _C[5]
    p = p * z + _C[3]
    p = p * z + _C[1]
    return (e.astype(np.float32) + s * p).astype(np.float32)


def gumbel(u) -> np.ndarray:
    """Standard Gumbel noise -ln(-ln u) in fp64."""
    u64 = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u64))


def race_exponentials(seed: int, n: int, position: int, request_id: int, tag: int) -> np.ndarray:
    """E_v = -plog2(u_v) for v = 0..n-1 (float32, strictly positive)."""
    u = philox.uniforms(seed, np.arange(n, dtype=np.uint64), position, request_id, tag)
    return (-plog2(u)).astype(np.float32)


def race_argmax(r, E) -> int:
    """Index maximising r_v / E_v under the exact comparison (ties -> smaller v).

    r: float32 >= 0, E: float32 > 0.  A candidate is found with a rounded
    ratio, then replaced by any element that beats it exactly, until none does.
    """
    r32 = np.asarray(r, dtype=np.float32)
    E32 = np.asarray(E, dtype=np.float32)
    r64 = r32.astype(np.float64)
    E64 = E32.astype(np.float64)
    idx = np.arange(r64.size)
    c = int(np.argmax(r64 / E64))
    while True:
        lhs = r64 * E64[c]          # r_v * E_c   (exact)
        rhs = r64[c] * E64          # r_c * E_v   (exact)
        beats = (lhs > rhs) | ((lhs == rhs) & (idx < c))
        if not beats.any():
            return c
        cand = np.nonzero(beats)[0]
        c = int(cand[np.argmax(r64[cand] / E64[cand])])


def race_top2_margin(r, E) -> float:
    """Relative gap between the best and second-best r/E (for near-tie accounting)."""
    q = np.asarray(r, dtype=np.float64) / np.asarray(E, dtype=np.float64)
    if q.size < 2:
        return math.inf
    top = np.partition(q, q.size - 2)[-2:]
    hi, lo = max(top), min(top)
    return math.inf if hi == 0 else float((hi - lo) / hi)
