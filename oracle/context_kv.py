"""Context-KV precompute, written plainly (test infrastructure, like the rest of oracle/).

Source: [P1] "DSpark 的实现和测评", section "Context KV 预计算" (the KV-injection step
DSpark inherits from DFlash; [P2] "推测解码：从零到DSpark" describes the same
injection).  Instead of running the target forward layer by layer to fill the draft's
KV cache, the target's intermediate hidden states are projected once:

  1. fc: aux hidden states [num_ctx, H_in] -> context states [num_ctx, H_d];
  2. the context states are normalised and one GEMM with the weights of every
     draft layer's K and V projections side by side gives all_kv [num_ctx, L*2*kv];
  3. all_kv is viewed as [num_ctx, L, 2, nkv, hd]; the K half of every layer is
     RMS-normalised over hd (per-layer weight) in one grouped pass;
  4. rotary position embedding is applied to every layer's K in one pass;
  5. K and V of each layer are written to that layer's cache at the token's slot.

Readings where the pages are silent (the GPU side takes the same):
  * the normalisation of step 2 is RMSNorm with a weight (the norm the draft model
    uses elsewhere), eps given; fc may carry a bias (NULL = none); the fused KV
    projection carries one (the listing passes a fused bias);
  * the model runs in bf16: every weight is bf16, the normalised context states
    are rounded to bf16 before the fused GEMM (its operand type), and the caches
    hold bf16; accumulation and the norms are in higher precision (fp64 here);
  * RoPE is the rotate-half form: for i < hd/2, the pair (x_i, x_{i+hd/2}) is
    rotated by the angle pos * theta^(-2i/hd);
  * V is neither normalised nor rotated;
  * cache layout [L, num_slots, nkv, hd], token m written at slot slots[m].

Every function is checked against hand-worked values, closed forms and properties in
tests/test_oracle_context_kv.py.
"""
from __future__ import annotations

import numpy as np


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as bit patterns.

    Done on the exact binary value: the 16 dropped bits of the float32 encoding decide,
    with the float64 remainder below float32 precision breaking an exact half-way case.
    Non-finite inputs are not expected here (inputs are finite by construction)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)                        # nearest float32 (ties to even)
    rem = x - f.astype(np.float64)                  # what float32 lost (exact in float64)
    u = f.view(np.uint32).astype(np.uint64)
    lo = u & 0xFFFF
    hi = u >> 16
    half = 0x8000
    # value above the bf16 below f: lo (+ the sign of rem in f's magnitude direction)
    mag_dir = np.where(f >= 0, 1.0, -1.0) * np.sign(rem)
    up = (lo > half) | ((lo == half) & ((mag_dir > 0) | ((mag_dir == 0) & ((hi & 1) == 1))))
    hi = hi + up.astype(np.uint64)
    return hi.astype(np.uint16)


def rms_norm(x, w, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, dtype=np.float64)


def rope_rotate_half(x, pos, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half form, over the last axis (length hd, even).

    x: [..., hd]; pos: positions broadcastable to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq          # [..., half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def context_kv(aux_bits, fc_w_bits, fc_b_bits, hnorm_w_bits, kv_w_bits, kv_b_bits, knorm_w_bits, positions,
               slots, L: int, nkv: int, hd: int, num_slots: int, eps: float, theta: float,
               k_cache=None, v_cache=None, normed_bits=None):
    """Steps 1-5 above.

    aux_bits [num_ctx, H_in], fc_w_bits [H_d, H_in], fc_b_bits [H_d] or None,
    hnorm_w_bits [H_d], kv_w_bits [L*2*nkv*hd, H_d], kv_b_bits [L*2*nkv*hd],
    knorm_w_bits [L, hd]: bf16 bit patterns.  positions [num_ctx] int, slots
    [num_ctx] int in [0, num_slots).  k_cache / v_cache: [L, num_slots, nkv, hd]
    uint16 arrays to write into (fresh zero arrays if None).  normed_bits: optional
    [num_ctx, H_d] bf16 operand of the fused GEMM to start from (steps 3-5 from
    another implementation's rounding of step 2); computed here if None.

    Returns dict(k_cache, v_cache, context, normed, normed_bits, all_kv, k_final): the caches
    (bf16 bits) and the float64 intermediates of each step."""
    aux = bf16_decode(aux_bits)
    fc_w = bf16_decode(fc_w_bits)
    ctx = aux @ fc_w.T                                                    # step 1
    if fc_b_bits is not None:
        ctx = ctx + bf16_decode(fc_b_bits)
    normed = rms_norm(ctx, bf16_decode(hnorm_w_bits), eps)               # step 2: bf16 operand
    if normed_bits is None:
        normed_bits = bf16_round(normed)
    all_kv = bf16_decode(normed_bits) @ bf16_decode(kv_w_bits).T + bf16_decode(kv_b_bits)
    n = aux.shape[0]
    kv = all_kv.reshape(n, L, 2, nkv, hd)
    k = kv[:, :, 0]                                                       # [num_ctx, L, nkv, hd]
    v = kv[:, :, 1]
    knorm = bf16_decode(knorm_w_bits).reshape(L, hd)
    k = rms_norm(k, knorm[None, :, None, :], eps)                         # step 3, every layer
    k = rope_rotate_half(k, np.asarray(positions)[:, None, None], theta)  # step 4, every layer
    if k_cache is None:
        k_cache = np.zeros((L, num_slots, nkv, hd), np.uint16)
    if v_cache is None:
        v_cache = np.zeros((L, num_slots, nkv, hd), np.uint16)
    kb, vb = bf16_round(k), bf16_round(v)
    for m in range(n):                                                    # step 5
        s = int(slots[m])
        for layer in range(L):
            k_cache[layer, s] = kb[m, layer]
            v_cache[layer, s] = vb[m, layer]
    return dict(k_cache=k_cache, v_cache=v_cache, context=ctx, normed=normed, normed_bits=normed_bits, all_kv=all_kv,
                k_final=k)
