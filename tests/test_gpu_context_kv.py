"""dspark_context_kv against the oracle (oracle/context_kv.py), in two checks split at the
method's one bf16 operand, the normalised context states (the fused GEMM's input):

  1. the GPU's normalised states (read from its workspace, where the library keeps
     them between the two products) are a correct bf16 rounding of a value within
     1e-5 x (the row's RMS) of the oracle's exact one: the float32 product over H_in
     terms carries an absolute error of a few 1e-6 at the row's scale; almost all
     elements equal the oracle's own rounding;
  2. the caches equal the oracle's steps 3-5 run from the GPU's own normalised states,
     within one bf16 step plus 1e-5 absolute (float32 accumulation, a cancelling
     rotated pair), and elements that differ at all are rare (<= 5 %).
A wrong sign, weight, eps, slot or position moves values by far more.
"""
import numpy as np
import pytest
import torch

import draft_sampling_lossless_amd as dsl
import synth
from oracle import context_kv as ck

from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(dspark_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _case(M, H_in, H_d, L, nkv, hd, S, seed, fc_bias=True):
    g = np.random.default_rng(seed)
    c = dict(
        aux=synth.bf16_bits(g.normal(0, 1, (M, H_in)).astype(np.float32)),
        fc_w=synth.bf16_bits(g.normal(0, 1 / np.sqrt(H_in), (H_d, H_in)).astype(np.float32)),
        fc_b=synth.bf16_bits(g.normal(0, 0.1, H_d).astype(np.float32)) if fc_bias else None,
        hnorm_w=synth.bf16_bits((1 + 0.1 * g.normal(size=H_d)).astype(np.float32)),
        kv_w=synth.bf16_bits(g.normal(0, 1 / np.sqrt(H_d), (L * 2 * nkv * hd, H_d)).astype(np.float32)),
        kv_b=synth.bf16_bits(g.normal(0, 0.1, L * 2 * nkv * hd).astype(np.float32)),
        knorm_w=synth.bf16_bits((1 + 0.1 * g.normal(size=(L, hd))).astype(np.float32)),
        positions=g.integers(0, 32768, M).astype(np.int32),
        slots=g.permutation(S)[:M].astype(np.int64),
    )
    c.update(M=M, H_in=H_in, H_d=H_d, L=L, nkv=nkv, hd=hd, S=S)
    return c


SENT_K, SENT_V = 0x7E7E, 0x3E3E   # sentinels of slots no token writes


def _run_gpu(c, eps=1e-6, theta=1e6):
    """Caches, plus the normalised states from the workspace (after the fc product's
    float32 output, 256-byte aligned, as the library lays it out)."""
    L, S, nkv, hd = c["L"], c["S"], c["nkv"], c["hd"]
    M, H_d = c["M"], c["H_d"]
    kc = torch.full((L, S, nkv, hd), SENT_K, dtype=torch.int16, device="cuda")
    vc = torch.full((L, S, nkv, hd), SENT_V, dtype=torch.int16, device="cuda")
    ws = torch.zeros(dsl.context_kv_workspace_size(M, H_d, L, nkv, hd), dtype=torch.uint8, device="cuda")
    dsl.context_kv(dev(c["aux"]), dev(c["fc_w"]), None if c["fc_b"] is None else dev(c["fc_b"]),
                   dev(c["hnorm_w"]), dev(c["kv_w"]), dev(c["kv_b"]), dev(c["knorm_w"]), dev(c["positions"]),
                   dev(c["slots"]), kc, vc, eps=eps, rope_theta=theta, workspace=ws)
    off = (M * H_d * 4 + 255) // 256 * 256
    normed = host(ws[off:off + M * H_d * 2]).view(np.uint16).reshape(M, H_d)
    return host(kc).view(np.uint16), host(vc).view(np.uint16), normed


def _run_oracle(c, rows=None, eps=1e-6, theta=1e6, normed_bits=None):
    rows = np.arange(c["M"]) if rows is None else np.asarray(rows)
    L, S, nkv, hd = c["L"], c["S"], c["nkv"], c["hd"]
    kc = np.full((L, S, nkv, hd), SENT_K, np.uint16)
    vc = np.full((L, S, nkv, hd), SENT_V, np.uint16)
    return ck.context_kv(c["aux"][rows], c["fc_w"], c["fc_b"], c["hnorm_w"], c["kv_w"], c["kv_b"], c["knorm_w"],
                         c["positions"][rows], c["slots"][rows], L, nkv, hd, S, eps, theta, k_cache=kc, v_cache=vc,
                         normed_bits=None if normed_bits is None else normed_bits[rows])


def _check_normed(gpu_bits, exact, window=1e-5):
    """Check 1: the GPU's bf16 normalised states against the oracle's exact values: each
    within half a bf16 step (at its magnitude) of a value within window x row RMS of the
    exact one."""
    rms = np.broadcast_to(np.sqrt(np.mean(exact * exact, axis=-1, keepdims=True)), exact.shape)
    g = ck.bf16_decode(gpu_bits)
    mag = np.maximum(np.abs(g), np.abs(exact))
    half_step = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 8), 0.0)
    bad = np.abs(g - exact) > half_step + window * rms
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"normalised states: {int(bad.sum())} elements off, e.g. {tuple(i)}: exact "
                             f"{exact[tuple(i)]!r}, gpu {g[tuple(i)]!r}")
    return int((gpu_bits != ck.bf16_round(exact)).sum())


def _within_tolerance(a_bits, b_bits, abs_tol=1e-5):
    """Elementwise: |a - b| <= one bf16 step at max(|a|, |b|) + abs_tol."""
    fa = ck.bf16_decode(a_bits)
    fb = ck.bf16_decode(b_bits)
    mag = np.maximum(np.abs(fa), np.abs(fb))
    step = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 7), 0.0)
    err = np.abs(fa - fb)
    return err <= step + abs_tol, a_bits != b_bits, err, fa, fb


def _compare(gpu, ref, label):
    ok, diff, err, fa, fb = _within_tolerance(gpu, ref)
    if not ok.all():
        i = np.unravel_index(np.argmax(np.where(ok, 0, err)), err.shape)
        raise AssertionError(f"{label}: {int((~ok).sum())} elements outside the bar; worst at {i}: gpu {fa[i]:.6g} "
                             f"oracle {fb[i]:.6g}")
    frac = diff.mean()
    assert frac <= 0.05, f"{label}: {frac:.3%} of elements one step off"
    return frac


@pytest.mark.parametrize("M,H_in,H_d,L,nkv,hd,S,bias", [
    (1, 256, 256, 1, 1, 64, 4, True),          # one token: the stream GEMM
    (7, 512, 256, 2, 2, 128, 16, True),        # ragged
    (130, 256, 512, 3, 4, 64, 200, True),      # big tiles for both products, ragged tail
    (300, 1024, 512, 5, 8, 128, 1024, False),  # L x 2 x kv = 10240 columns, no fc bias
    (33, 264, 136, 2, 2, 32, 64, True),        # H_in % 64 != 0: the tiled GEMM; small heads
    (20, 256, 256, 1, 2, 256, 32, True),       # hd = 256: two rotary pairs per lane
    (70, 512, 256, 2, 1, 2, 80, True),         # hd = 2: one pair per head
    (100, 256, 192, 2, 3, 128, 160, True),     # the fused K/V epilogue: ragged rows, tiles mixing K and V heads
    (65, 512, 128, 1, 1, 128, 65, False),      # fused at its smallest: 65 tokens, one layer, one head
])
def test_context_kv_parity(M, H_in, H_d, L, nkv, hd, S, bias):
    say(f"context_kv M={M} H_in={H_in} H_d={H_d} L={L} nkv={nkv} hd={hd} S={S} fc_bias={bias}")
    c = _case(M, H_in, H_d, L, nkv, hd, S, seed=M + H_in + hd, fc_bias=bias)
    gk, gv, gn = _run_gpu(c)
    ref = _run_oracle(c, normed_bits=gn)
    flips = _check_normed(gn, ref["normed"])
    fk = _compare(gk, ref["k_cache"], "K")
    fv = _compare(gv, ref["v_cache"], "V")
    # slots no token names keep their contents
    unused = np.setdiff1d(np.arange(S), c["slots"])
    assert np.all(gk[:, unused] == SENT_K) and np.all(gv[:, unused] == SENT_V)
    say(f"  normalised states: {flips} of {M * H_d} differ from the oracle's rounding; one-step differences: "
        f"K {fk:.3%}, V {fv:.3%}")


@pytest.mark.parametrize("M,hd,S", [(12, 64, 32), (90, 128, 96)])   # the finishing pass; the fused epilogue
def test_context_kv_slots_outside_the_cache_are_skipped(M, hd, S):
    c = _case(M, 256, 128, 2, 2, hd, S, seed=5)
    c["slots"][[2, 7]] = [-1, S]
    gk, gv, gn = _run_gpu(c)
    keep = [m for m in range(M) if m not in (2, 7)]
    ref = _run_oracle(c, rows=keep, normed_bits=gn)
    _compare(gk, ref["k_cache"], "K")
    _compare(gv, ref["v_cache"], "V")


def test_context_kv_full_size_sampled_tokens():
    """A prefill chunk of 8192 tokens at the Qwen3-8B widths (H_in = H_d = 4096), 5 layers
    of 8 KV heads x 128: the whole chunk on the GPU, a sample of tokens through the oracle
    (at their own slots; the oracle's caches start from the same sentinels)."""
    M, H, L, nkv, hd = 8192, 4096, 5, 8, 128
    S = M + 64
    c = _case(M, H, H, L, nkv, hd, S, seed=2026)
    gk, gv, gn = _run_gpu(c)
    g = np.random.default_rng(7)
    rows = np.unique(np.concatenate([g.integers(0, M, 6), [0, M - 1]]))
    ref = _run_oracle(c, rows=rows, normed_bits=gn)
    _check_normed(gn[rows], ref["normed"])
    sl = c["slots"][rows]
    fk = _compare(gk[:, sl], ref["k_cache"][:, sl], "K")
    fv = _compare(gv[:, sl], ref["v_cache"][:, sl], "V")
    say(f"  tokens {rows.tolist()}: one-step differences K {fk:.3%}, V {fv:.3%}")
