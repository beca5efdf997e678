"""Deferred draft rows: stage 2 keeps the base logits, stage 3 rebuilds only the rows it reads.

* dspark_markov_sample_deferred against dspark_markov_sample on the same per-step kernels
  (B > 16): the same tokens, log Z and confidence bit for bit, the base logits untouched,
  and win_logit equal to the stored processed logit at each drafted token;
* at few requests (B <= 16, where the stored path takes the few-request kernel) against
  the oracle, teacher-forced, with the near-tie rule of the other Markov tests;
* dspark_verify_deferred against dspark_verify on the stored processed logits: accepted
  counts and emitted tokens bit for bit, each request's first-rejection row rebuilt in
  place equal to the stored row, every other row left as it was; up to the admission
  workload's full size (B = 256, N = 16, V = 151936, r = 256).
"""
import numpy as np
import pytest
import torch

import draft_sampling_lossless_amd as dsl
import synth
from oracle import stages

from gpu_util import compare_verify, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(dspark_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _case(B, N, V, r, temps, seed, wstd=0.16):
    g = np.random.default_rng(seed)
    base = g.normal(0, 1.28, size=(B, N, V)).astype(np.float32)
    w1 = synth.bf16_bits(g.normal(0, wstd, size=(V, r)).astype(np.float32))
    w2 = synth.bf16_bits(g.normal(0, wstd, size=(V, r)).astype(np.float32))
    anchor = g.integers(0, V, size=B).astype(np.int32)
    temp = np.asarray(temps, np.float32)[g.integers(0, len(temps), size=B)]
    rid = (np.arange(B) * 7 + 3).astype(np.uint32)
    return dict(base=base, w1=w1, w2=w2, anchor=anchor, temp=temp, rid=rid, seed=seed & 0xFFFF)


def _dev_case(c):
    return {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in c.items()}


def _stored(d, conf=None):
    proc = d["base"].clone()
    out = dsl.markov_sample(proc, d["w1"], d["w2"], None, d["anchor"], d["temp"], d["rid"], d["seed"], conf=conf)
    return (proc,) + tuple(out)


def _deferred(d, conf=None):
    kept = d["base"].clone()
    out = dsl.markov_sample_deferred(kept, d["w1"], d["w2"], d["anchor"], d["temp"], d["rid"], d["seed"], conf=conf)
    return (kept,) + tuple(out)


@pytest.mark.parametrize("B,N,V,r,temps", [
    (70, 5, 2048, 64, (0.0, 0.7, 1.0)),
    (130, 2, 1024, 8, (1.0,)),
    (40, 3, 2048, 128, (0.7, 0.0)),
    (17, 4, 3000 // 4 * 4, 200, (1.0,)),
    (64, 3, 1024, 32, (0.0,)),
    (200, 6, 4096, 256, (0.0, 0.7, 1.0)),
])
def test_markov_deferred_bit_equal_to_stored(B, N, V, r, temps):
    say(f"markov deferred vs stored B={B} N={N} V={V} r={r} T={temps}")
    d = _dev_case(_case(B, N, V, r, temps, seed=B * 31 + N))
    proc, tok_s, lz_s = _stored(d)
    kept, tok_k, lz_k, win = _deferred(d)
    tok_s, lz_s, tok_k, lz_k, win = host(tok_s), host(lz_s), host(tok_k), host(lz_k), host(win)
    assert np.array_equal(tok_k, tok_s)
    assert np.array_equal(lz_k.view(np.uint32), lz_s.view(np.uint32))
    assert torch.equal(kept, d["base"]), "the base logits must be left untouched"
    at_tok = host(torch.gather(proc, 2, torch.as_tensor(tok_s, device="cuda").long().unsqueeze(2)).squeeze(2))
    assert np.array_equal(win.view(np.uint32), at_tok.view(np.uint32))
    say(f"  {B * N} positions: tokens, log Z and winner logits bit-equal; base untouched")


def test_markov_deferred_confidence_bit_equal():
    B, N, V, r, H = 64, 8, 4096, 64, 256
    say(f"markov deferred with the confidence head B={B} N={N} V={V} r={r}")
    c = _case(B, N, V, r, (0.0, 0.7, 1.0), seed=77)
    g = np.random.default_rng(78)
    h_dot = dev(g.normal(0, 1.0, size=B * N).astype(np.float32))
    w_e = dev(synth.bf16_bits(g.normal(0, 0.1, size=r).astype(np.float32)))
    tau = dev(np.linspace(0.8, 1.6, N).astype(np.float32))
    d = _dev_case(c)
    _, tok_s, lz_s, c_s = _stored(d, conf=(h_dot, w_e, 0.25, tau, None))
    kept, tok_k, lz_k, win, c_k = _deferred(d, conf=(h_dot, w_e, 0.25, tau, None))
    assert torch.equal(tok_s, tok_k) and torch.equal(lz_s, lz_k) and torch.equal(c_s, c_k)
    assert torch.equal(kept, d["base"])


@pytest.mark.parametrize("B,N,V,r,temps", [(1, 8, 2048, 64, (1.0,)), (3, 5, 4096, 256, (0.0, 0.7, 1.0)),
                                           (16, 4, 1024, 16, (0.7,))])
def test_markov_deferred_few_requests_against_oracle(B, N, V, r, temps):
    """B <= 16 (the stored path's few-request kernel is not the deferred path's kernel):
    against the oracle, teacher-forced on the GPU tokens.  A token may differ only at a
    near-tie of the oracle's keys; winner logits within 1e-5 relative of the oracle's
    processed logit at the GPU token."""
    say(f"markov deferred few requests B={B} N={N} V={V} r={r} T={temps}")
    c = _case(B, N, V, r, temps, seed=500 + B)
    d = _dev_case(c)
    kept, tok, lz, win = _deferred(d)
    tok, lz, win = host(tok), host(lz), host(win)
    assert torch.equal(kept, d["base"])
    ref = stages.markov_sample(c["base"], c["w1"], c["w2"], None, c["anchor"], c["temp"], c["rid"], c["seed"],
                               teacher=tok)
    near = 0
    for b in range(B):
        for i in range(N):
            p = ref["processed"][b, i].astype(np.float64)
            assert abs(float(win[b, i]) - p[tok[b, i]]) <= 1e-5 * max(1.0, abs(p[tok[b, i]])), (b, i)
            lz_r = float(ref["logZ"][b, i])
            assert abs(float(lz[b, i]) - lz_r) <= 2e-5 * max(1.0, abs(lz_r)), (b, i)
            if tok[b, i] != ref["tokens"][b, i]:
                assert ref["gap"][b, i] <= 1e-2 and ref["teacher_deficit"][b, i] <= 1e-2, (b, i)
                near += 1
    assert near <= max(1, B * N // 50)
    say(f"  {B * N} positions, {near} near-tie mismatches")


def _target_from(proc, B, N, V, seed):
    """Target logits near the processed draft rows (per-request noise level), so acceptance
    lengths spread over 0 .. N."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sigma = torch.rand((B, 1, 1), generator=g, device="cuda") * 1.5
    tgt = torch.randn((B, N + 1, V), generator=g, device="cuda")
    tgt[:, :N] = proc + sigma * tgt[:, :N]
    return tgt


@pytest.mark.parametrize("B,N,V,r,temps", [
    (70, 5, 2048, 64, (0.0, 0.7, 1.0)),
    (200, 6, 4096, 256, (0.0, 0.7, 1.0)),
    (33, 8, 1024, 16, (1.0,)),
    (256, 16, 151936, 256, (0.0, 0.7, 1.0)),
])
def test_verify_deferred_bit_equal_to_stored(B, N, V, r, temps):
    say(f"verify deferred vs stored B={B} N={N} V={V} r={r} T={temps}")
    d = _dev_case(_case(B, N, V, r, temps, seed=B + 3 * N))
    proc, tok, lz = _stored(d)
    kept, tok_k, lz_k, win = _deferred(d)
    assert torch.equal(tok, tok_k) and torch.equal(lz, lz_k)
    tgt = _target_from(proc, B, N, V, seed=B)
    g = np.random.default_rng(B)
    L = g.integers(0, N + 1, size=B).astype(np.int32)
    L[: max(1, B // 4)] = N
    Ld = dev(L)
    seed = 0xABCD
    acc_s, out_s = dsl.verify(dsl.INPUT_LOGITS, tgt, proc, lz, tok, None, Ld, d["temp"], d["rid"], seed)
    acc_k, out_k = dsl.verify_deferred(tgt, kept, lz_k, win, tok_k, d["anchor"], d["w1"], d["w2"], Ld, d["temp"],
                                       d["rid"], seed)
    acc_s, out_s, acc_k, out_k = host(acc_s), host(out_s), host(acc_k), host(out_k)
    assert np.array_equal(acc_k, acc_s)
    assert np.array_equal(out_k, out_s)
    # the rows rebuilt: each hot request's first rejection; every other row as it was
    temp = host(d["temp"])
    rebuilt = np.zeros((B, N), bool)
    for b in range(B):
        if temp[b] > 0 and acc_s[b] < L[b]:
            rebuilt[b, acc_s[b]] = True
    mask = torch.as_tensor(rebuilt, device="cuda")
    assert torch.equal(kept[mask], proc[mask]), "rebuilt rows differ from the stored processed rows"
    assert torch.equal(kept[~mask], d["base"][~mask]), "rows that are not read were changed"
    say(f"  accepted {acc_s[:12].tolist()}..., {int(rebuilt.sum())} rows rebuilt, mean accepted "
        f"{acc_s.mean():.2f}")


def test_verify_deferred_few_requests_against_oracle():
    """B = 3: the deferred pipeline against the oracle's verification of its own drafts (the
    oracle's processed logits, teacher-forced on the GPU tokens): equal except at a near-tie."""
    B, N, V, r = 3, 6, 2048, 64
    c = _case(B, N, V, r, (0.0, 0.7, 1.0), seed=901)
    d = _dev_case(c)
    kept, tok, lz, win = _deferred(d)
    ref_m = stages.markov_sample(c["base"], c["w1"], c["w2"], None, c["anchor"], c["temp"], c["rid"], c["seed"],
                                 teacher=host(tok))
    proc = ref_m["processed"].astype(np.float32)
    g = np.random.default_rng(902)
    tg = np.concatenate([proc + 0.5 * g.normal(size=proc.shape), g.normal(size=(B, 1, V))], axis=1).astype(np.float32)
    L = np.array([N, 2, 4], np.int32)
    seed = 0x77
    acc, out = dsl.verify_deferred(dev(tg), kept, lz, win, tok, d["anchor"], d["w1"], d["w2"], dev(L), d["temp"],
                                   d["rid"], seed)
    ref = stages.verify("logits", tg, proc, host(tok), None, L, c["temp"], c["rid"], seed)
    near = compare_verify(host(acc), host(out), ref, exact=False)
    assert near <= 1
    say(f"  accepted {host(acc).tolist()}, {near} near-tie")
