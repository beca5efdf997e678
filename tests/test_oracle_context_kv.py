"""Pins of the context-KV oracle (oracle/context_kv.py) against hand-worked values,
closed forms, brute force and properties the pages' definitions fix."""
import numpy as np
import pytest

from oracle import context_kv as ck


def _bits_of(values):
    """float32-exact values -> bf16 bits by truncation (values chosen exactly representable)."""
    return (np.asarray(values, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_hand_worked():
    e8, e30 = 2.0 ** -8, 2.0 ** -30
    cases = [
        (1.0, 0x3F80),
        (1.0 + e8, 0x3F80),               # exact midpoint of 1 and 1 + 2^-7: ties to even (down)
        (1.0 + 3 * e8, 0x3F82),           # midpoint of 0x3F81 (odd) and 0x3F82 (even): up
        (1.0 + e8 + e30, 0x3F81),         # just above the midpoint, below float32 precision
        (1.0 + e8 - e30, 0x3F80),         # just below it
        (-(1.0 + e8 + e30), 0xBF81),
        (-2.5, 0xC020),
        (0.0, 0x0000),
    ]
    for x, want in cases:
        got = int(ck.bf16_round(np.array([x]))[0])
        assert got == want, f"{x!r}: got {got:#06x}, want {want:#06x}"


def test_bf16_round_matches_brute_force_nearest():
    g = np.random.default_rng(3)
    x = np.concatenate([g.normal(0, 1, 4000), g.normal(0, 1e-3, 1000), g.normal(0, 300, 1000)])
    got = ck.bf16_round(x)
    for xi, gi in zip(x, got):
        t = int((np.array([xi], np.float32).view(np.uint32)[0] >> 16))   # truncation: a neighbour
        cands = [(t - 1) & 0xFFFF, t, (t + 1) & 0xFFFF]
        vals = [float(ck.bf16_decode(np.array([c], np.uint16))[0]) for c in cands]
        d = [abs(v - xi) for v in vals]
        best = min(d)
        win = [c for c, di in zip(cands, d) if di == best]
        want = win[0] if len(win) == 1 else [c for c in win if c % 2 == 0][0]
        assert int(gi) == want, (xi, hex(int(gi)), hex(want))


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_hand_worked_and_invariants():
    y = ck.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 1.0]), 0.0)
    r = np.sqrt((9 + 16) / 2)
    assert np.allclose(y, [3 / r, 4 / r], rtol=0, atol=1e-15)
    y = ck.rms_norm(np.array([3.0, 4.0]), np.array([2.0, 0.5]), 0.0)
    assert np.allclose(y, [6 / r, 2 / r], rtol=0, atol=1e-15)
    g = np.random.default_rng(1)
    x = g.normal(size=(5, 64))
    ones = np.ones(64)
    assert np.allclose(np.sqrt(np.mean(ck.rms_norm(x, ones, 0.0) ** 2, axis=-1)), 1.0, atol=1e-13)
    assert np.allclose(ck.rms_norm(7.5 * x, ones, 0.0), ck.rms_norm(x, ones, 0.0), atol=1e-13)
    # eps enters under the square root: a zero row stays zero, a tiny row is damped
    assert np.all(ck.rms_norm(np.zeros(8), np.ones(8), 1e-6) == 0)
    t = ck.rms_norm(np.full(4, 1e-4), np.ones(4), 1e-6)
    assert np.allclose(t, 1e-4 / np.sqrt(1e-8 + 1e-6), rtol=1e-12)


# ---------------------------------------------------------------- RoPE

def test_rope_hand_worked():
    # hd = 4, theta = 10000: inverse frequencies 1 and 0.01
    x = np.array([1.0, 2.0, 3.0, 4.0])
    y = ck.rope_rotate_half(x, 1, 10000.0)
    c0, s0, c1, s1 = np.cos(1.0), np.sin(1.0), np.cos(0.01), np.sin(0.01)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_rope_properties():
    g = np.random.default_rng(2)
    hd = 128
    q, k = g.normal(size=hd), g.normal(size=hd)
    assert np.array_equal(ck.rope_rotate_half(q, 0, 1e6), q)                 # position 0: identity
    for p in (1, 17, 4095, 32767):
        y = ck.rope_rotate_half(q, p, 1e6)
        half = hd // 2
        assert np.allclose(y[:half] ** 2 + y[half:] ** 2, q[:half] ** 2 + q[half:] ** 2, rtol=1e-12)
    # the score of two rotated vectors depends on the position difference only
    for m, n in ((5, 3), (1000, 998), (77, 75)):
        a = ck.rope_rotate_half(q, m, 1e6) @ ck.rope_rotate_half(k, n, 1e6)
        b = ck.rope_rotate_half(q, m - n, 1e6) @ k
        assert np.isclose(a, b, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- the fused projection

def test_fused_projection_equals_per_layer_projections():
    """The fused weight stacks every layer's K then V projection (the listing's
    view(num_ctx, L, 2, nkv, hd)): the oracle's split equals L separate K and V
    projections with the corresponding row blocks."""
    g = np.random.default_rng(4)
    n, H_in, H_d, L, nkv, hd = 5, 16, 8, 3, 2, 4
    kv = nkv * hd
    aux = _bits_of(g.normal(size=(n, H_in)))
    fc_w = _bits_of(g.normal(0, 0.3, size=(H_d, H_in)))
    hn = _bits_of(1 + 0.1 * g.normal(size=H_d))
    kv_w = _bits_of(g.normal(0, 0.3, size=(L * 2 * kv, H_d)))
    kv_b = _bits_of(0.1 * g.normal(size=L * 2 * kv))
    kn = _bits_of(1 + 0.1 * g.normal(size=(L, hd)))
    pos = np.arange(n) + 3
    out = ck.context_kv(aux, fc_w, None, hn, kv_w, kv_b, kn, pos, np.arange(n), L, nkv, hd, n, 1e-6, 1e6)
    normed = ck.bf16_decode(out["normed_bits"])
    W, b = ck.bf16_decode(kv_w), ck.bf16_decode(kv_b)
    for layer in range(L):
        rk = slice((2 * layer) * kv, (2 * layer + 1) * kv)
        rv = slice((2 * layer + 1) * kv, (2 * layer + 2) * kv)
        k_sep = (normed @ W[rk].T + b[rk]).reshape(n, nkv, hd)
        v_sep = (normed @ W[rv].T + b[rv]).reshape(n, nkv, hd)
        k_sep = ck.rms_norm(k_sep, ck.bf16_decode(kn)[layer], 1e-6)
        k_sep = ck.rope_rotate_half(k_sep, pos[:, None], 1e6)
        assert np.allclose(out["k_final"][:, layer], k_sep, rtol=1e-12, atol=1e-12)
        assert np.array_equal(out["v_cache"][layer], ck.bf16_round(v_sep))
        assert np.array_equal(out["k_cache"][layer], ck.bf16_round(k_sep))


def test_cache_slots_and_untouched_entries():
    g = np.random.default_rng(5)
    n, H, L, nkv, hd, S = 4, 8, 2, 1, 4, 11
    aux = _bits_of(g.normal(size=(n, H)))
    eye = _bits_of(np.eye(H))
    kv_w = _bits_of(g.normal(0, 0.4, size=(L * 2 * nkv * hd, H)))
    zero_b = np.zeros(L * 2 * nkv * hd, np.uint16)
    slots = np.array([9, 2, 5, 0])
    kc = np.full((L, S, nkv, hd), 0x1234, np.uint16)
    vc = np.full((L, S, nkv, hd), 0x4321, np.uint16)
    out = ck.context_kv(aux, eye, None, _bits_of(np.ones(H)), kv_w, zero_b, _bits_of(np.ones((L, hd))),
                        np.zeros(n, int), slots, L, nkv, hd, S, 1e-6, 1e6, k_cache=kc, v_cache=vc)
    untouched = [s for s in range(S) if s not in set(slots.tolist())]
    assert np.all(out["k_cache"][:, untouched] == 0x1234) and np.all(out["v_cache"][:, untouched] == 0x4321)
    # position 0: no rotation, so token m's K at its slot is the bf16 of its K-normed projection
    normed = ck.bf16_decode(out["normed_bits"])
    allkv = normed @ ck.bf16_decode(kv_w).T
    for m, s in enumerate(slots):
        for layer in range(L):
            k = allkv[m, (2 * layer) * hd:(2 * layer + 1) * hd]
            assert np.array_equal(out["k_cache"][layer, s, 0], ck.bf16_round(ck.rms_norm(k, np.ones(hd), 1e-6)))


def test_tiny_pipeline_by_hand():
    """H = 2, L = 1, nkv = 1, hd = 2, identity fc, K = V = the normalised state, unit norm
    weights, eps = 0: the cache holds [a, b] / rms and its rotation by the position."""
    aux = _bits_of([[3.0, 4.0]])
    eye = _bits_of(np.eye(2))
    kv_w = _bits_of([[1, 0], [0, 1], [1, 0], [0, 1]])
    out = ck.context_kv(aux, eye, None, _bits_of([1.0, 1.0]), kv_w, np.zeros(4, np.uint16), _bits_of([[1.0, 1.0]]),
                        np.array([2]), np.array([0]), 1, 1, 2, 1, 0.0, 10000.0)
    r = np.sqrt(12.5)
    a, b = float(ck.bf16_decode(ck.bf16_round(3 / r))), float(ck.bf16_decode(ck.bf16_round(4 / r)))
    assert np.array_equal(out["v_cache"][0, 0, 0], ck.bf16_round(np.array([a, b])))
    # K: the bf16 state renormalised (rms of [a, b]), then rotated by angle 2 (hd = 2: one pair, frequency 1)
    rk = np.sqrt((a * a + b * b) / 2)
    ka, kb = a / rk, b / rk
    want = [ka * np.cos(2.0) - kb * np.sin(2.0), kb * np.cos(2.0) + ka * np.sin(2.0)]
    assert np.array_equal(out["k_cache"][0, 0, 0], ck.bf16_round(np.array(want)))


def test_fc_bias_is_added_before_the_norm():
    aux = _bits_of([[1.0, 0.0]])
    eye = _bits_of(np.eye(2))
    kv_w = _bits_of([[1, 0], [0, 1], [1, 0], [0, 1]])
    out = ck.context_kv(aux, eye, _bits_of([0.0, 1.0]), _bits_of([1.0, 1.0]), kv_w, np.zeros(4, np.uint16),
                        _bits_of([[1.0, 1.0]]), np.array([0]), np.array([0]), 1, 1, 2, 1, 0.0, 1e6)
    assert np.allclose(out["context"], [[1.0, 1.0]])
    assert np.array_equal(ck.bf16_decode(out["normed_bits"]), [[1.0, 1.0]])
