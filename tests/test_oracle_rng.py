"""Pins of the oracle's random-number layer: Philox, uniform map, variates."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import philox, variates


def _kat(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    return rows


def test_philox_known_answers(golden_dir):
    rows = _kat(golden_dir)
    assert len(rows) == 3
    for r in rows:
        out = philox.philox4x32_10(*r[:4], r[4], r[5])
        assert [int(o) for o in out] == r[6:10]


def test_philox_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(4, 64), dtype=np.uint64)
    k0, k1 = 0x01234567, 0x89ABCDEF
    vec = philox.philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(64):
        one = philox.philox4x32_10(int(c[0, i]), int(c[1, i]), int(c[2, i]), int(c[3, i]), k0, k1)
        assert [int(v[i]) for v in vec] == [int(o) for o in one]


def test_counter_layout_word_selection():
    # index v uses counter word v>>2 and output word v&3
    seed = (7 << 32) | 11
    w = philox.words(seed, np.arange(8), 3, 5, 2)
    for v in range(8):
        out = philox.philox4x32_10(v >> 2, 3, 5, 2, 11, 7)
        assert int(w[v]) == int(out[v & 3])


def test_uniform_map_exact_and_open_interval():
    w = np.array([0, 0xFF, 0x100, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = philox.uniform(w)
    expect = [1 * 2**-24, 1 * 2**-24, 1 * 2**-24, (2**24 - 1) * 2**-24, (2**23 + 1) * 2**-24]
    assert u.dtype == np.float32
    assert [float(x) for x in u] == expect
    assert (u > 0).all() and (u < 1).all()


def test_uniform_is_uniform_ks():
    u = philox.uniforms(0, np.arange(200_000), 0, 0, 0).astype(np.float64)
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # different tags / positions / requests give different streams
    u2 = philox.uniforms(0, np.arange(1000), 0, 0, 1)
    u3 = philox.uniforms(0, np.arange(1000), 1, 0, 0)
    u4 = philox.uniforms(0, np.arange(1000), 0, 1, 0)
    assert not np.array_equal(u[:1000].astype(np.float32), u2)
    assert not np.array_equal(u2, u3) and not np.array_equal(u3, u4)


def test_plog2_close_to_log2_and_monotone():
    rng = np.random.default_rng(1)
    u = np.concatenate([
        rng.random(400_000, dtype=np.float32),
        1.0 - np.arange(1, 2000, dtype=np.float32) * np.float32(2**-24),   # near 1
        np.arange(1, 2000, dtype=np.float32) * np.float32(2**-24),         # near 0
    ]).astype(np.float32)
    u = u[(u > 0) & (u < 1)]
    got = variates.plog2(u).astype(np.float64)
    ref = np.log2(u.astype(np.float64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 4.0
    s = np.sort(np.unique(u))
    g = variates.plog2(s)
    assert np.all(np.diff(g.astype(np.float64)) >= 0)


def test_plog2_exact_at_powers_of_two():
    for k in range(1, 60):
        assert float(variates.plog2(np.array([2.0 ** -k], np.float32))[0]) == -k
    assert float(variates.plog2(np.array([1.0], np.float32))[0]) == 0.0


def test_gumbel_ks():
    u = philox.uniforms(3, np.arange(100_000), 0, 0, 0)
    g = variates.gumbel(u)
    assert stats.kstest(g, "gumbel_r").pvalue > 1e-3


def test_race_exponentials_positive_and_exponential():
    E = variates.race_exponentials(9, 100_000, 2, 4, philox.TAG_RESID).astype(np.float64)
    assert (E > 0).all()
    # E = -log2(u) = Exp(1) / ln 2
    assert stats.kstest(E * math.log(2.0), "expon").pvalue > 1e-3


def test_race_chi_square_matches_weights():
    r = np.array([0.05, 0.0, 0.3, 0.15, 0.5], dtype=np.float32)
    n = 40_000
    counts = np.zeros(r.size)
    for req in range(n):
        E = variates.race_exponentials(1, r.size, 0, req, philox.TAG_BONUS)
        counts[variates.race_argmax(r, E)] += 1
    assert counts[1] == 0                      # zero weight never wins
    p = r.astype(np.float64) / r.astype(np.float64).sum()
    nz = p > 0
    chi2 = stats.chisquare(counts[nz], n * p[nz])
    assert chi2.pvalue > 1e-4


def test_race_exact_ties_and_zero_rows():
    # r and E chosen so that r_a * E_b == r_b * E_a exactly: smaller index wins
    r = np.array([0.25, 0.5, 0.125], dtype=np.float32)
    E = np.array([0.5, 1.0, 0.25], dtype=np.float32)
    assert variates.race_argmax(r, E) == 0
    assert variates.race_argmax(np.zeros(5, np.float32), np.ones(5, np.float32)) == 0
    # near-equal ratios that fp64 division could misorder are decided exactly
    r = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(2.0))], dtype=np.float32)
    E = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(2.0))], dtype=np.float32)
    assert variates.race_argmax(r, E) == 0     # equal ratios exactly -> index 0
