"""Verification at the full-size workloads (V = 151936), on sampled requests.

Verify never mixes requests, so the whole batch runs on the GPU in the shape the
bench uses while the oracle checks a sample of requests one by one.  The sampled
requests carry the seeded inputs the oracle regenerates; the others carry stand-in
values made on the device (never compared).

  * probability input, the exact domain: accepted counts and emitted tokens bit for
    bit, plus the acceptance probability 1 - TV, at one request and at 64;
  * the reduced-vocabulary workload (Vd = 32000 mapped into V by the d2t offsets,
    temperatures mixed over {0, 0.7, 1}) in both input kinds;
  * logits input on the admission workload's admitted prefixes (B = 256, N = 16,
    verify lengths from the GPU admission of K = 1024).
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


def _logz(row, T):
    y = np.asarray(row, np.float64)
    if T > 0:
        y = y / T
        return np.float32(y.max() + np.log(np.exp(y - y.max()).sum()))
    return np.float32(y.max())


def _case(name, reqs, seed):
    """Device inputs of the whole batch; exact seeded values at `reqs`."""
    w = synth.get(name)
    rp = synth.request_params(w)
    d2t = synth.d2t_offsets(w)
    inv = None if d2t is None else stages.build_inverse_map(d2t, w.Vd, w.V)
    t_of_j = np.arange(w.Vd) + (0 if d2t is None else d2t)
    B, N, V, Vd = w.B, w.N, w.V, w.Vd
    std = w.weight_std * w.H ** 0.5
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    proc = torch.randn((B, N, Vd), generator=gen, device="cuda") * std
    tgt = torch.randn((B, N + 1, V), generator=gen, device="cuda")
    # sampled requests: stand-in draft logits and the target built from them (the
    # workloads' recipe: target = draft logits scattered to target ids + sigma * noise)
    sb = synth.synthetic_base_logits(w, reqs)
    tg = synth.target_noise(w, reqs) * rp["sigma"][reqs][:, None, None]
    rows = list(range(N)) + [N - 1]
    tg[:, :, t_of_j] += sb[:, rows]
    tg = tg.astype(np.float32)
    ridx = torch.as_tensor(reqs, device="cuda")
    proc[ridx] = dev(sb)
    tgt[ridx] = dev(tg)
    # drafts: argmax rows for the stand-ins; draws from the tempered draft row (argmax
    # at T = 0) for the sampled requests
    tok_d = proc.argmax(dim=2).to(torch.int64)
    tok = torch.as_tensor(t_of_j, device="cuda")[tok_d].to(torch.int32)
    g = np.random.default_rng(seed)
    tok_s = np.empty((len(reqs), N), np.int32)
    for n, b in enumerate(reqs):
        T = float(rp["temperature"][b])
        for k in range(N):
            if T > 0:
                p = stages.probs_from_logits(sb[n, k], T).astype(np.float64)
                j = g.choice(Vd, p=p / p.sum())
            else:
                j = int(np.argmax(sb[n, k]))
            tok_s[n, k] = t_of_j[j]
    tok[ridx] = dev(tok_s)
    return dict(w=w, rp=rp, d2t=d2t, inv=inv, reqs=np.asarray(reqs), proc=proc, tgt=tgt, tok=tok, sb=sb, tg=tg,
                tok_s=tok_s)


def _probs_inputs(c):
    """p_t [B, N+1, V] and p_d [B, N, Vd] float32: the oracle's arrays at the sampled
    requests, a device softmax elsewhere (not compared)."""
    w, rp = c["w"], c["rp"]
    T = torch.as_tensor(rp["temperature"], device="cuda").clamp_min(1e-3).view(-1, 1, 1)
    p_t = torch.softmax(c["tgt"] / T, dim=2)
    p_d = torch.softmax(c["proc"] / T, dim=2)
    inv = c["inv"]
    for n, b in enumerate(c["reqs"]):
        Tb = float(rp["temperature"][b])
        pt = np.stack([stages.probs_from_logits(c["tg"][n, k], Tb) for k in range(w.N + 1)])
        pd = np.stack([stages.draft_probs(c["sb"][n, k], Tb,
                                          int(inv[c["tok_s"][n, k]]) if inv is not None else int(c["tok_s"][n, k]))
                       for k in range(w.N)])
        p_t[int(b)] = dev(pt)
        p_d[int(b)] = dev(pd)
    return p_t, p_d


def _alpha_ref(p_t, p_d, inv, L):
    N = p_d.shape[0]
    out = np.full(N, np.nan)
    for k in range(int(L)):
        pd_t = p_d[k] if inv is None else np.where(inv >= 0, p_d[k][np.maximum(inv, 0)], 0.0)
        out[k] = stages.accept_prob(p_t[k], pd_t)
    return out


def _check_probs(c, L, seed):
    w = c["w"]
    p_t, p_d = _probs_inputs(c)
    inv_d = None if c["inv"] is None else dev(c["inv"])
    acc, out, alpha = dsl.verify(dsl.INPUT_PROBS, p_t, p_d, None, c["tok"], inv_d, L, None,
                                 dev(c["rp"]["request_id"]), seed, with_accept_prob=True)
    acc, out, alpha = host(acc), host(out), host(alpha)
    Lh = host(L)
    reqs = c["reqs"]
    pt_s = host(p_t[torch.as_tensor(reqs, device="cuda")])
    pd_s = host(p_d[torch.as_tensor(reqs, device="cuda")])
    ref = stages.verify("probs", pt_s, pd_s, c["tok_s"], c["inv"], Lh, None, c["rp"]["request_id"], seed,
                        requests=reqs)
    compare_verify(acc[reqs], out[reqs], ref, exact=True)
    worst = 0.0
    for n, b in enumerate(reqs):
        a_ref = _alpha_ref(pt_s[n], pd_s[n], c["inv"], Lh[b])
        a_gpu = alpha[b].astype(np.float64)
        assert np.array_equal(np.isnan(a_gpu), np.isnan(a_ref))
        m = ~np.isnan(a_ref)
        if m.any():
            worst = max(worst, float(np.abs(a_gpu[m] - a_ref[m]).max()))
    assert worst <= 2e-5, f"accept_prob max abs err {worst:.3g}"
    say(f"  probs: {len(reqs)} requests bit-exact, accepted {acc[reqs].tolist()}, alpha err {worst:.2e}")


def _check_logits(c, L, seed):
    w, rp = c["w"], c["rp"]
    reqs = c["reqs"]
    T = torch.as_tensor(rp["temperature"], device="cuda")
    y = c["proc"] / T.clamp_min(1e-3).view(-1, 1, 1)
    logz = torch.where(T.view(-1, 1) > 0, torch.logsumexp(y, dim=2), c["proc"].amax(dim=2))
    lz_s = np.array([[_logz(c["sb"][n, k], float(rp["temperature"][b])) for k in range(w.N)]
                     for n, b in enumerate(reqs)], np.float32)
    logz[torch.as_tensor(reqs, device="cuda")] = dev(lz_s)
    inv_d = None if c["inv"] is None else dev(c["inv"])
    acc, out = dsl.verify(dsl.INPUT_LOGITS, c["tgt"], c["proc"], logz, c["tok"], inv_d, L, dev(rp["temperature"]),
                          dev(rp["request_id"]), seed)
    acc, out = host(acc), host(out)
    ref = stages.verify("logits", c["tg"], c["sb"], c["tok_s"], c["inv"], host(L), rp["temperature"],
                        rp["request_id"], seed, requests=reqs)
    near = compare_verify(acc[reqs], out[reqs], ref, exact=False)
    assert near <= max(1, len(reqs) // 50)
    say(f"  logits: {len(reqs)} requests, {near} near-tie, accepted {acc[reqs].tolist()}")


def _sample(B, k, seed):
    g = np.random.default_rng(seed)
    return np.array(sorted({0, B - 1, *g.integers(0, B, k).tolist()}))


def test_verify_probs_full_vocab_single_request():
    c = _case("qwen3_8b_single", np.array([0]), seed=101)
    say("verify probs, full vocabulary, B=1")
    L = torch.full((1,), c["w"].N, dtype=torch.int32, device="cuda")
    _check_probs(c, L, seed=0x3141)


def test_verify_probs_full_vocab_batched():
    w = synth.get("batched")
    reqs = _sample(w.B, 5, 3)
    c = _case("batched", reqs, seed=102)
    say(f"verify probs, full vocabulary, B={w.B}, requests {reqs.tolist()}")
    L = dev(np.random.default_rng(7).integers(0, w.N + 1, size=w.B).astype(np.int32))
    L[0] = w.N                   # one request verifies the whole block (the bonus row)
    _check_probs(c, L, seed=0x2718)


@pytest.mark.parametrize("kind", ["probs", "logits"])
def test_verify_reduced_vocab_full_size(kind):
    w = synth.get("reduced_vocab")
    reqs = _sample(w.B, 6, 5)
    c = _case("reduced_vocab", reqs, seed=103)
    say(f"verify {kind}, reduced vocabulary Vd={w.Vd} -> V={w.V}, B={w.B}, requests {reqs.tolist()}, "
        f"T {c['rp']['temperature'][reqs].tolist()}")
    L = dev(np.random.default_rng(9).integers(0, w.N + 1, size=w.B).astype(np.int32))
    if kind == "probs":
        _check_probs(c, L, seed=0x1618)
    else:
        _check_logits(c, L, seed=0x1618)


def test_verify_logits_on_admitted_prefixes():
    w = synth.get("admission")
    reqs = _sample(w.B, 5, 11)
    c = _case("admission", reqs, seed=104)
    conf = synth.confidence(w)
    _, L = dsl.admit(dev(conf), w.budget)
    Lh = host(L)
    assert np.array_equal(Lh, stages.admit(conf, w.budget)["admit_len"])
    say(f"verify logits on admitted prefixes, B={w.B} N={w.N} K={w.budget}: L of the sample "
        f"{Lh[reqs].tolist()}, sum {int(Lh.sum())}")
    _check_logits(c, L, seed=0x5EED)
