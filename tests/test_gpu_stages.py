"""GPU parity of each stage against the oracle, through the C ABI.

Small cases compare every output; the full Qwen3-8B-shaped workloads compare
sampled requests / entries (the stages never mix requests, except admission,
which is always compared in full).
"""
import math

import numpy as np
import pytest
import torch

import draft_sampling_lossless_amd as dsl
import synth
from oracle import philox, stages, variates

from gpu_util import compare_markov, compare_verify, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(dspark_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- random numbers

def test_philox_blocks_bit_exact():
    g = np.random.default_rng(0)
    ctr = g.integers(0, 2**32, size=(10_000, 4), dtype=np.uint64)
    ctr[0] = [0, 0, 0, 0]
    ctr[1] = [0xFFFFFFFF] * 4
    for seed in (0, 0xFFFFFFFFFFFFFFFF, 0x299F31D0A4093822, 12345):
        say(f"philox seed={seed:#x}")
        out = host(dsl.philox_blocks(dev(ctr.astype(np.uint32)), seed)).view(np.uint32)
        ref = philox.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], seed & 0xFFFFFFFF, seed >> 32)
        assert np.array_equal(out, np.stack(ref, axis=1).astype(np.uint32))


@pytest.mark.parametrize("n,pos,req,tag", [(1 << 16, 0, 0, 2), (151936, 7, 12345, 3), (37, 1, 2**32 - 1, 2)])
def test_race_exponentials_bit_exact(n, pos, req, tag):
    say(f"race_exponentials n={n}")
    out = host(dsl.race_exponentials(0xDEADBEEF12345678, pos, req, tag, n))
    ref = variates.race_exponentials(0xDEADBEEF12345678, n, pos, req, tag)
    assert out.dtype == np.float32 and np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- stage 1

@pytest.mark.parametrize("M,H,Vd", [(8, 256, 1024), (20, 264, 1000), (40, 256, 996), (1, 4096, 4096),
                                    (300, 200, 1004), (129, 4096, 640), (64, 64, 68),
                                    (8, 4096, 4100), (16, 512, 1000), (13, 1024, 72), (1, 2048, 65540),
                                    (8, 4096, 8), (257, 128, 1000), (520, 96, 300), (96, 32, 260), (300, 64, 500),
                                    (700, 4096, 2000),
                                    # H = 4096, a few 16-row blocks per workgroup and a partial last one
                                    (8, 4096, 20000), (3, 4096, 20004), (16, 4096, 12300),
                                    # the stream kernel's LDS output buffer exactly full (96 KB per
                                    # workgroup at 256 CUs), and one size past it (the skinny kernel)
                                    (16, 512, 393216), (16, 512, 400000),
                                    # big tiles with Vd % 4 = 1, 2, 3: rows of the output not
                                    # 16-byte aligned, the epilogue's scalar stores
                                    (130, 128, 1001), (260, 256, 1002), (333, 192, 771),
                                    # enough tiles for five LM-head fragments per wave (256 x 320
                                    # tiles): a partial last row tile and last column tile, with
                                    # and without 16-byte aligned output rows
                                    (600, 128, 100001), (600, 128, 100000)])
def test_draft_logits_small(M, H, Vd):
    say(f"draft_logits M={M} H={H} Vd={Vd}")
    g = np.random.default_rng(M * 7 + H)
    hid = synth.bf16_bits(g.normal(0, 1, size=(M, H)).astype(np.float32))
    W = synth.bf16_bits(g.normal(0, 0.02, size=(Vd, H)).astype(np.float32))
    out = host(dsl.draft_logits(dev(hid), dev(W)))
    ref = stages.draft_logits(hid, W)
    err = np.abs(out.astype(np.float64) - ref.astype(np.float64)).max()
    say(f"  max |err| = {err:.3g}")
    assert err <= 2e-2


@pytest.mark.parametrize("name", ["qwen3_8b_single", "batched", "reduced_vocab"])
def test_draft_logits_full_size_sampled(name):
    w = synth.get(name)
    say(f"draft_logits full size {name}: M={w.M} H={w.H} Vd={w.Vd}")
    hid = synth.hidden_bf16(w)
    W = synth.lm_head_bf16(w)
    out = dsl.draft_logits(dev(hid), dev(W))
    g = np.random.default_rng(1)
    cols = np.unique(np.concatenate([g.integers(0, w.Vd, 300), [0, w.Vd - 1]]))
    rows = np.unique(np.concatenate([g.integers(0, w.M, 16), [0, w.M - 1]]))
    got = host(out[torch.as_tensor(rows).cuda()][:, torch.as_tensor(cols).cuda()])
    ref = stages.draft_logits(hid[rows], synth.lm_head_bf16(w, rows=cols))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()
    say(f"  max |err| = {err:.3g}")
    assert err <= 2e-2


# ---------------------------------------------------------------- stage 2

def _markov_case(B, N, V, Vd, r, temps, seed=0, base=None, d2t=None, wstd=0.16):
    g = np.random.default_rng(B * 1000 + N * 10 + r)
    if base is None:
        base = (g.normal(0, 1.28, size=(B, N, Vd))).astype(np.float32)
    w1 = synth.bf16_bits(g.normal(0, wstd, size=(V, r)).astype(np.float32))
    w2 = synth.bf16_bits(g.normal(0, wstd, size=(Vd, r)).astype(np.float32))
    anchor = g.integers(0, V, size=B).astype(np.int32)
    temp = np.asarray(temps, np.float32)[g.integers(0, len(temps), size=B)]
    rid = (np.arange(B) * 7 + 3).astype(np.uint32)
    return dict(base=base, w1=w1, w2=w2, d2t=d2t, anchor=anchor, temp=temp, rid=rid, seed=seed, V=V)


def _run_markov_gpu(c):
    logits = dev(c["base"])
    tok, logz = dsl.markov_sample(logits, dev(c["w1"]), dev(c["w2"]),
                                  None if c["d2t"] is None else dev(c["d2t"]),
                                  dev(c["anchor"]), dev(c["temp"]), dev(c["rid"]), c["seed"])
    return host(tok), host(logits), host(logz)


@pytest.mark.parametrize("B,N,V,Vd,r,temps,reduced", [
    (1, 8, 1024, 1024, 16, (1.0,), False),
    (1, 8, 1024, 1024, 16, (0.0,), False),
    (70, 5, 2048, 2048, 64, (0.0, 0.7, 1.0), False),
    (33, 4, 4096, 1000, 32, (0.0, 0.7, 1.0), True),
    (20, 3, 3000, 3000, 256, (0.7,), False),
    (130, 2, 1024, 1024, 8, (1.0,), False),
    (16, 6, 2048, 2048, 64, (0.0, 0.7, 1.0), False),
    (5, 4, 4096, 1000, 64, (0.0, 1.0), True),
    (3, 3, 3000, 3000, 256, (0.7,), False),
    (2, 64, 1024, 1024, 16, (1.0,), False),
    (40, 3, 2048, 2048, 128, (0.7, 0.0), False),
    (24, 2, 3000, 1000, 200, (1.0,), True),
    (65, 2, 1024, 1000, 96, (0.0,), True),
])
def test_markov_small(B, N, V, Vd, r, temps, reduced):
    say(f"markov B={B} N={N} V={V} Vd={Vd} r={r} T={temps} reduced={reduced}")
    d2t = None
    if reduced:
        g = np.random.default_rng(5)
        d2t = (g.permutation(V)[:Vd] - np.arange(Vd)).astype(np.int64)
    c = _markov_case(B, N, V, Vd, r, temps, seed=0x1234, d2t=d2t)
    tok, proc, logz = _run_markov_gpu(c)
    ref = stages.markov_sample(c["base"], c["w1"], c["w2"], d2t, c["anchor"], c["temp"], c["rid"], c["seed"],
                               teacher=tok)
    checked, near = compare_markov(tok, proc, logz, ref, label=f"small B={B} N={N} Vd={Vd} r={r} T={temps}")
    say(f"  compared {checked} positions, {near} near-tie mismatches")
    if d2t is not None:
        image = set((np.arange(Vd) + d2t).tolist())
        assert all(int(t) in image for t in tok.ravel())


@pytest.mark.parametrize("B,N,V,Vd,r,temps,wstd", [
    (1, 8, 8192, 8192, 64, (1.0,), 0.02),       # few survivors: chain on rows staged in LDS
    (4, 5, 2048, 2048, 64, (0.7, 1.0), 0.15),    # wider margin, mixed temperatures
    (3, 4, 4096, 4096, 64, (0.0, 1.0), 1.0),     # margin too wide for the recorded entries: per-step pass
    (2, 6, 4096, 1000, 32, (1.0,), 1.0),         # the same with a reduced vocabulary
    (1, 20, 151936, 151936, 64, (1.0,), 0.02),   # recorded entries in several rounds; two 16-step tiles
    # one request (every workgroup runs the candidate phase itself): the per-step pass
    # from the first step, and greedy steps on rows staged in LDS
    (1, 6, 4096, 4096, 64, (1.0,), 1.0),
    (1, 5, 8192, 8192, 64, (0.0,), 0.02),
])
def test_markov_candidate_paths(B, N, V, Vd, r, temps, wstd):
    say(f"markov candidate paths B={B} N={N} V={V} Vd={Vd} r={r} std={wstd}")
    d2t = None
    if Vd != V:
        g = np.random.default_rng(7)
        d2t = (g.permutation(V)[:Vd] - np.arange(Vd)).astype(np.int64)
    c = _markov_case(B, N, V, Vd, r, temps, seed=0x777, d2t=d2t, wstd=wstd)
    tok, proc, logz = _run_markov_gpu(c)
    ref = stages.markov_sample(c["base"], c["w1"], c["w2"], d2t, c["anchor"], c["temp"], c["rid"], c["seed"],
                               teacher=tok)
    checked, near = compare_markov(tok, proc, logz, ref, label=f"candidate paths B={B} N={N} Vd={Vd} std={wstd}")
    say(f"  compared {checked} positions, {near} near-tie mismatches")


def test_markov_unstaged_chain():
    # one large base logit per 256-entry workgroup slice, the rest far below: every
    # slice's best entry survives the margin while its second one stays outside, so
    # the survivors (about 256 per step) exceed what fits in LDS and the chain reads
    # weight rows from global memory
    B, N, V, Vd, r = 1, 4, 65536, 65536, 64
    g = np.random.default_rng(11)
    base = np.full((B, N, Vd), -60.0, np.float32)
    pick = np.arange(0, Vd, 256) + g.integers(0, 256, size=Vd // 256)
    base[:, :, pick] = g.normal(0, 0.3, size=(B, N, pick.size)).astype(np.float32)
    say(f"markov unstaged chain B={B} N={N} V={V} r={r}")
    c = _markov_case(B, N, V, Vd, r, (1.0,), seed=0x99, base=base, wstd=0.33)
    tok, proc, logz = _run_markov_gpu(c)
    ref = stages.markov_sample(c["base"], c["w1"], c["w2"], None, c["anchor"], c["temp"], c["rid"], c["seed"],
                               teacher=tok)
    checked, near = compare_markov(tok, proc, logz, ref, label="unstaged chain")
    say(f"  compared {checked} positions, {near} near-tie mismatches")
    assert set(tok.ravel().tolist()) <= set(pick.tolist())


@pytest.mark.parametrize("B,N,V,Vd,r,temps,wstd", [
    (2, 5, 8192, 8192, 64, (1.0,), 0.02),   # survivors: the staged chain
    (3, 4, 4096, 4096, 64, (0.0, 1.0), 1.0),  # the per-step pass
])
def test_markov_few_solo(B, N, V, Vd, r, temps, wstd):
    # the few-request kernel with every slice run by one workgroup (what it does when
    # not all of its workgroups become resident): same results as the oracle
    say(f"markov few solo B={B} N={N} V={V} r={r} std={wstd}")
    c = _markov_case(B, N, V, Vd, r, temps, seed=0x51, wstd=wstd)
    dsl.markov_test_mode(1)
    try:
        tok, proc, logz = _run_markov_gpu(c)
    finally:
        dsl.markov_test_mode(0)
    dsl.markov_check()
    ref = stages.markov_sample(c["base"], c["w1"], c["w2"], None, c["anchor"], c["temp"], c["rid"], c["seed"],
                               teacher=tok)
    checked, near = compare_markov(tok, proc, logz, ref, label=f"few solo B={B} std={wstd}")
    say(f"  compared {checked} positions, {near} near-tie mismatches")


def test_markov_deterministic():
    # same inputs twice (few requests: the cooperative kernel; many: the per-step kernels)
    for B in (1, 40):
        c = _markov_case(B, 6, 2048, 2048, 64, (0.0, 1.0), seed=3)
        a = _run_markov_gpu(c)
        b = _run_markov_gpu(c)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y)


def test_markov_few_counter_sets_reused():
    """The few-request kernel's barrier counters live in a ring of counter sets that each
    launch leaves cleared.  Well over two rounds of the ring, alternating normal and
    single-workgroup launches (which clear the counters on different paths), give the
    first launch's outputs bit for bit."""
    c = _markov_case(2, 5, 4096, 4096, 64, (0.0, 1.0), seed=11)
    say("markov few: 150 launches over the counter sets")
    ref = _run_markov_gpu(c)
    for i in range(150):
        dsl.markov_test_mode(1 if i % 3 == 2 else 0)
        try:
            got = _run_markov_gpu(c)
        finally:
            dsl.markov_test_mode(0)
        for x, y in zip(ref, got):
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y), f"launch {i}"


@pytest.mark.parametrize("B,N,V,r,wstd,temps", [
    (2, 5, 8192, 64, 0.02, (0.0, 1.0)),   # several requests: a barrier after phase C
    (3, 4, 4096, 64, 1.0, (0.0, 1.0)),    # the per-step pass: a barrier per step
    (1, 6, 4096, 64, 1.0, (1.0,))])       # one request, margin too wide: the per-step pass from step 0
def test_markov_few_barrier_give_up_is_reported(B, N, V, r, wstd, temps):
    """A grid barrier that gives up (forced from the host: every barrier reports a give-up
    after completing) never leaves valid-looking outputs: every token is -1, log Z is NaN,
    and the check raises.  After the check the next launch is correct again."""
    c = _markov_case(B, N, V, V, r, temps, seed=0x61, wstd=wstd)
    say(f"markov few forced give-up B={B} N={N} V={V} std={wstd}")
    dsl.markov_check()                                   # nothing pending
    dsl.markov_test_mode(2)
    try:
        tok, _, logz = _run_markov_gpu(c)
    finally:
        dsl.markov_test_mode(0)
    with pytest.raises(dsl.DSparkError, match="gave up"):
        dsl.markov_check()
    assert (tok == -1).all() and np.isnan(logz).all()
    tok, proc, logz = _run_markov_gpu(c)
    dsl.markov_check()
    ref = stages.markov_sample(c["base"], c["w1"], c["w2"], None, c["anchor"], c["temp"], c["rid"], c["seed"],
                               teacher=tok)
    compare_markov(tok, proc, logz, ref, label=f"after give-up B={B}")


@pytest.mark.parametrize("name,nsample", [("qwen3_8b_single", 1), ("batched", 4), ("admission", 3),
                                          ("reduced_vocab", 6)])
def test_markov_full_size_sampled(name, nsample):
    w = synth.get(name)
    say(f"markov full size {name}: B={w.B} N={w.N} Vd={w.Vd} r={w.r}")
    rp = synth.request_params(w)
    d2t = synth.d2t_offsets(w)
    g = np.random.default_rng(2)
    reqs = np.array(sorted({0, w.B - 1, *g.integers(0, w.B, nsample).tolist()}))
    # every request gets stand-in base logits on the device; the sampled ones the seeded values
    base = torch.randn((w.B, w.N, w.Vd), device="cuda", dtype=torch.float32) * (w.weight_std * w.H ** 0.5)
    sb = synth.synthetic_base_logits(w, reqs)
    base[torch.as_tensor(reqs).cuda()] = dev(sb)
    w1, w2 = synth.markov_w1_bf16(w), synth.markov_w2_bf16(w)
    tok, logz = dsl.markov_sample(base, dev(w1), dev(w2), None if d2t is None else dev(d2t), dev(rp["anchor"]),
                                  dev(rp["temperature"]), dev(rp["request_id"]), w.philox_seed)
    tok, logz = host(tok)[reqs], host(logz)[reqs]
    proc = host(base[torch.as_tensor(reqs).cuda()])
    ref = stages.markov_sample(sb, w1, w2, d2t, rp["anchor"], rp["temperature"], rp["request_id"],
                               w.philox_seed, requests=reqs, teacher=tok)
    checked, near = compare_markov(tok, proc, logz, ref, label=f"full size {name} requests {reqs.tolist()}")
    say(f"  requests {reqs.tolist()}: compared {checked} positions, {near} near-tie mismatches")


# ---------------------------------------------------------------- stage 3

def _verify_inputs(B, N, V, Vd, temps, seed, reduced=False, sigma=1.0):
    g = np.random.default_rng(seed)
    d2t = inv = None
    if reduced:
        d2t = (g.permutation(V)[:Vd] - np.arange(Vd)).astype(np.int64)
        inv = stages.build_inverse_map(d2t, Vd, V)
    proc = g.normal(0, 1.28, size=(B, N, Vd)).astype(np.float32)
    tgt = g.normal(0, sigma, size=(B, N + 1, V))
    t_of_j = np.arange(Vd) + (0 if d2t is None else d2t)
    tgt[:, :N, t_of_j] += proc
    tgt[:, N, t_of_j] += proc[:, N - 1]
    tgt = tgt.astype(np.float32)
    temp = np.asarray(temps, np.float32)[g.integers(0, len(temps), size=B)]
    # drafts: the target id of a draw from the tempered draft row (argmax at T = 0)
    tok = np.empty((B, N), np.int32)
    for b in range(B):
        for k in range(N):
            if temp[b] > 0:
                p = stages.probs_from_logits(proc[b, k], float(temp[b])).astype(np.float64)
                j = g.choice(Vd, p=p / p.sum())
            else:
                j = int(np.argmax(proc[b, k]))
            tok[b, k] = t_of_j[j]
    L = g.integers(0, N + 1, size=B).astype(np.int32)
    rid = (np.arange(B) * 3 + 11).astype(np.uint32)
    return dict(proc=proc, tgt=tgt, temp=temp, tok=tok, L=L, rid=rid, d2t=d2t, inv=inv)


@pytest.mark.parametrize("B,N,V,Vd,reduced", [(200, 6, 1024, 1024, False), (64, 8, 2048, 1000, True),
                                              (3, 1, 64, 64, False), (3, 64, 256, 256, False)])
def test_verify_probs_bit_exact(B, N, V, Vd, reduced):
    say(f"verify probs B={B} N={N} V={V} Vd={Vd}")
    c = _verify_inputs(B, N, V, Vd, (0.7, 1.0), seed=B + N, reduced=reduced)
    p_t = np.stack([[stages.probs_from_logits(c["tgt"][b, k], float(c["temp"][b])) for k in range(N + 1)]
                    for b in range(B)])
    p_d = np.stack([[stages.probs_from_logits(c["proc"][b, k], float(c["temp"][b])) for k in range(N)]
                    for b in range(B)])
    seed = 0xABCDEF0123
    acc, out = dsl.verify(dsl.INPUT_PROBS, dev(p_t), dev(p_d), None, dev(c["tok"]),
                          None if c["inv"] is None else dev(c["inv"]), dev(c["L"]), None, dev(c["rid"]), seed)
    ref = stages.verify("probs", p_t, p_d, c["tok"], c["inv"], c["L"], None, c["rid"], seed)
    compare_verify(host(acc), host(out), ref, exact=True)
    say(f"  accepted mean {host(acc).mean():.2f}")


@pytest.mark.parametrize("B,N,V,Vd,temps,reduced", [(200, 6, 1024, 1024, (0.0, 0.7, 1.0), False),
                                                    (64, 8, 2048, 1000, (0.0, 1.0), True),
                                                    (16, 4, 4096, 4096, (0.0,), False),
                                                    # more than 24 target rows: several passes of the
                                                    # acceptance kernel's statistics merge
                                                    (6, 40, 1024, 1024, (0.7, 1.0), False),
                                                    (4, 64, 512, 512, (0.0, 1.0), False),
                                                    # more than 16 requests: statistics and acceptance in
                                                    # separate launches, lazy rows from N = 2 on
                                                    (300, 2, 256, 256, (0.0, 1.0), False),
                                                    (17, 2, 2048, 2048, (0.0, 0.7, 1.0), False),
                                                    (40, 1, 1024, 1024, (0.7, 1.0), False),   # N = 1: not lazy
                                                    # one full-vocabulary request; a few with mixed temperatures
                                                    (1, 8, 151936, 151936, (1.0,), False),
                                                    (37, 5, 4096, 4096, (0.0, 0.7, 1.0), False)])
def test_verify_logits_parity(B, N, V, Vd, temps, reduced):
    say(f"verify logits B={B} N={N} V={V} Vd={Vd} T={temps}")
    c = _verify_inputs(B, N, V, Vd, temps, seed=B * N + 1, reduced=reduced)
    # draft log Z of the processed rows (the oracle's values; stage 2 emits the same quantity)
    logz = np.empty((B, N), np.float32)
    for b in range(B):
        for k in range(N):
            T = float(c["temp"][b])
            y = c["proc"][b, k].astype(np.float64)
            logz[b, k] = (np.log(np.exp(y / T - (y / T).max()).sum()) + (y / T).max()) if T > 0 else y.max()
    seed = 77
    acc, out = dsl.verify(dsl.INPUT_LOGITS, dev(c["tgt"]), dev(c["proc"]), dev(logz), dev(c["tok"]),
                          None if c["inv"] is None else dev(c["inv"]), dev(c["L"]), dev(c["temp"]), dev(c["rid"]),
                          seed)
    ref = stages.verify("logits", c["tgt"], c["proc"], c["tok"], c["inv"], c["L"], c["temp"], c["rid"], seed)
    near = compare_verify(host(acc), host(out), ref, exact=False)
    say(f"  {near} near-tie requests of {B}")
    assert near <= max(1, B // 50)


@pytest.mark.parametrize("B,N,temps", [(48, 6, (0.0, 0.7, 1.0)), (20, 3, (1.0,))])
def test_verify_logits_lazy_rows(B, N, temps):
    """Target rows close to the draft rows (small noise), so many requests accept two
    positions or more and the second statistics pass decides them: equal to the oracle
    except at a near-tie."""
    V = 2048
    say(f"verify logits, lazy rows B={B} N={N} V={V} T={temps}")
    c = _verify_inputs(B, N, V, V, temps, seed=4 * B + N, sigma=0.05)
    logz = np.empty((B, N), np.float32)
    for b in range(B):
        for k in range(N):
            T = float(c["temp"][b])
            y = c["proc"][b, k].astype(np.float64)
            logz[b, k] = (np.log(np.exp(y / T - (y / T).max()).sum()) + (y / T).max()) if T > 0 else y.max()
    seed = 91
    acc, out = dsl.verify(dsl.INPUT_LOGITS, dev(c["tgt"]), dev(c["proc"]), dev(logz), dev(c["tok"]), None,
                          dev(c["L"]), dev(c["temp"]), dev(c["rid"]), seed)
    ref = stages.verify("logits", c["tgt"], c["proc"], c["tok"], None, c["L"], c["temp"], c["rid"], seed)
    near = compare_verify(host(acc), host(out), ref, exact=False)
    assert near <= max(1, B // 50)
    assert (ref["accepted"] >= 2).sum() >= 3, "the second statistics pass must have requests to decide"
    say(f"  accepted {host(acc).tolist()}, {near} near-tie")


def _alpha_ref(p_t, p_d, inv, L):
    """Oracle alpha_k = sum_v min(p_t, p_d) for k < L (p_d mapped to target ids), NaN after."""
    B, N = p_d.shape[:2]
    out = np.full((B, N), np.nan)
    for b in range(B):
        for k in range(int(L[b])):
            pd_t = p_d[b, k] if inv is None else np.where(inv >= 0, p_d[b, k][np.maximum(inv, 0)], 0.0)
            out[b, k] = stages.accept_prob(p_t[b, k], pd_t)
    return out


def _check_alpha(gpu, ref, tol):
    assert np.array_equal(np.isnan(gpu), np.isnan(ref)), "alpha: NaN pattern (positions past verify_len)"
    m = ~np.isnan(ref)
    err = np.abs(gpu[m].astype(np.float64) - ref[m])
    assert err.max(initial=0.0) <= tol, f"alpha: max abs err {err.max():.3g}"
    return err.max(initial=0.0)


@pytest.mark.parametrize("mode,B,N,V,Vd,temps,reduced", [
    ("probs", 40, 6, 1024, 1024, (0.7, 1.0), False),
    ("probs", 9, 8, 2048, 1000, (1.0,), True),
    ("logits", 33, 5, 4096, 4096, (0.0, 0.7, 1.0), False),
    ("logits", 12, 8, 2048, 1000, (0.0, 1.0), True),
    ("logits", 1, 8, 151936, 151936, (1.0,), False),
])
def test_verify_accept_prob(mode, B, N, V, Vd, temps, reduced):
    say(f"verify accept_prob {mode} B={B} N={N} V={V} Vd={Vd} T={temps}")
    c = _verify_inputs(B, N, V, Vd, temps, seed=B * 7 + N, reduced=reduced)
    temp = c["temp"]
    p_t = np.stack([[stages.probs_from_logits(c["tgt"][b, k], float(temp[b])) for k in range(N + 1)]
                    for b in range(B)])
    p_d = np.stack([[stages.draft_probs(c["proc"][b, k], float(temp[b]),
                                        int(c["inv"][c["tok"][b, k]]) if c["inv"] is not None else int(c["tok"][b, k]))
                     for k in range(N)] for b in range(B)])
    seed = 991
    inv = None if c["inv"] is None else dev(c["inv"])
    if mode == "probs":
        args = (dsl.INPUT_PROBS, dev(p_t), dev(p_d), None, dev(c["tok"]), inv, dev(c["L"]), None, dev(c["rid"]), seed)
    else:
        logz = np.empty((B, N), np.float32)
        for b in range(B):
            for k in range(N):
                T = float(temp[b])
                y = c["proc"][b, k].astype(np.float64)
                logz[b, k] = (np.log(np.exp(y / T - (y / T).max()).sum()) + (y / T).max()) if T > 0 else y.max()
        args = (dsl.INPUT_LOGITS, dev(c["tgt"]), dev(c["proc"]), dev(logz), dev(c["tok"]), inv, dev(c["L"]),
                dev(temp), dev(c["rid"]), seed)
    acc0, out0 = dsl.verify(*args)
    acc1, out1, alpha = dsl.verify(*args, with_accept_prob=True)
    # the optional output does not change the sampled result
    assert np.array_equal(host(acc0), host(acc1)) and np.array_equal(host(out0), host(out1))
    ref = _alpha_ref(p_t, p_d, c["inv"], c["L"])
    err = _check_alpha(host(alpha), ref, 2e-5)
    say(f"  alpha max abs err {err:.2e}")


def test_verify_greedy_is_longest_argmax_prefix():
    B, N, V = 100, 6, 1024
    c = _verify_inputs(B, N, V, V, (0.0,), seed=9, sigma=0.3)
    L = np.full(B, N, np.int32)
    logz = c["proc"].max(axis=2).astype(np.float32)
    acc, out = dsl.verify(dsl.INPUT_LOGITS, dev(c["tgt"]), dev(c["proc"]), dev(logz), dev(c["tok"]), None,
                          dev(L), dev(c["temp"]), dev(c["rid"]), 5)
    acc, out = host(acc), host(out)
    am = c["tgt"].argmax(axis=2)
    for b in range(B):
        a = 0
        while a < N and c["tok"][b, a] == am[b, a]:
            a += 1
        assert acc[b] == a and out[b, a] == am[b, a]
        assert np.array_equal(out[b, :a], c["tok"][b, :a]) and (out[b, a + 1:] == -1).all()


# ---------------------------------------------------------------- stage 4

@pytest.mark.parametrize("B,N,K", [(256, 16, 1024), (1, 8, 3), (100, 7, 0), (100, 7, 700), (100, 7, 5000),
                                   (1024, 16, 9000), (7, 64, 100), (64, 8, 1)])
def test_admit_bit_exact(B, N, K):
    say(f"admit B={B} N={N} K={K}")
    w = synth.get("admission", B=B, N=N)
    c = synth.confidence(w)
    if B >= 64:
        c[:8] = c[8:16]          # exact survival ties across requests
    surv, L = dsl.admit(dev(c), K)
    ref = stages.admit(c, K)
    assert np.array_equal(host(surv).view(np.uint32), ref["survival"].view(np.uint32))
    assert np.array_equal(host(L), ref["admit_len"])


# ---------------------------------------------------------------- next rows: coupled verify

def _compare_coupled(acc, out, ref, gap_tol=1e-4):
    """Identical results, except where the oracle's decisive row was a near-tie."""
    near = 0
    for b in range(len(acc)):
        if acc[b] == ref["accepted"][b] and np.array_equal(out[b], ref["out_tokens"][b]):
            continue
        k = min(int(acc[b]), int(ref["accepted"][b]))   # the first row the two read differently
        assert ref["gap"][b, k] <= gap_tol, (
            f"request {b}: gpu accepted={acc[b]} out={out[b].tolist()} vs oracle accepted={ref['accepted'][b]} "
            f"out={ref['out_tokens'][b].tolist()} (row {k} gap {ref['gap'][b, k]:.3g})")
        near += 1
    return near


@pytest.mark.parametrize("B,N,V,Vd,temps", [(64, 6, 1024, 1024, (0.0, 0.7, 1.0)), (40, 8, 2048, 1000, (0.0, 1.0)),
                                            (4, 8, 151936, 151936, (1.0,)), (3, 1, 64, 64, (0.8,))])
def test_verify_coupled_parity(B, N, V, Vd, temps):
    say(f"verify coupled B={B} N={N} V={V} Vd={Vd} T={temps}")
    c = _verify_inputs(B, N, V, Vd, temps, seed=B + 3 * N, reduced=Vd != V)
    seed = 0x5EED
    acc, out = dsl.verify_coupled(dev(c["tgt"]), dev(c["tok"]), None if c["inv"] is None else dev(c["inv"]),
                                  dev(c["L"]), dev(c["temp"]), dev(c["rid"]), seed, Vd=Vd)
    ref = stages.verify_coupled(c["tgt"], c["tok"], c["inv"], c["L"], c["temp"], c["rid"], seed)
    near = _compare_coupled(host(acc), host(out), ref)
    say(f"  {near} near-tie requests of {B}, accepted mean {host(acc).mean():.2f}")
    assert near <= max(1, B // 50)


def test_verify_coupled_lazy_rows_full_vocab():
    """More than 16 requests at V = 151936: rows 0-1 first, the rest for the undecided
    requests.  Each request's drafts are the target's own coupled draws (from the
    oracle's noise) for a random prefix, so accepted counts spread over 0 .. L and the
    second pass has work; results equal the oracle's except at a near-tie."""
    B, N, V = 20, 6, 151936
    say(f"verify coupled, lazy rows, B={B} N={N} V={V}")
    c = _verify_inputs(B, N, V, V, (0.0, 0.7, 1.0), seed=77)
    seed = 0x5EED
    g = np.random.default_rng(78)
    for b in range(B):
        T = float(c["temp"][b])
        m = int(g.integers(0, N + 1))
        for k in range(m):
            l = c["tgt"][b, k].astype(np.float64)
            key = (l / T + stages.coupled_noise(seed, k, int(c["rid"][b]), V, None)) if T > 0 else l
            c["tok"][b, k] = int(np.argmax(key))
    acc, out = dsl.verify_coupled(dev(c["tgt"]), dev(c["tok"]), None, dev(c["L"]), dev(c["temp"]), dev(c["rid"]),
                                  seed, Vd=V)
    ref = stages.verify_coupled(c["tgt"], c["tok"], None, c["L"], c["temp"], c["rid"], seed)
    near = _compare_coupled(host(acc), host(out), ref)
    assert near <= 1
    assert (ref["accepted"] >= 2).sum() >= 3, "the second pass must have requests to decide"
    say(f"  accepted {host(acc).tolist()}, {near} near-tie")


@pytest.mark.parametrize("Vd", [2048, 1000])
def test_verify_coupled_accepts_stage2_drafts(Vd):
    # drafts from the GPU Markov sampler, target rows equal to its processed logits:
    # under the shared noise the target draws the drafted tokens
    B, N, V, r = 24, 6, 2048, 64
    d2t = None
    if Vd != V:
        g = np.random.default_rng(4)
        d2t = (g.permutation(V)[:Vd] - np.arange(Vd)).astype(np.int64)
    c = _markov_case(B, N, V, Vd, r, (0.7, 1.0), seed=0x77, d2t=d2t)
    tok, proc, logz = _run_markov_gpu(c)
    t_of_j = np.arange(Vd) + (0 if d2t is None else d2t)
    tgt = np.full((B, N + 1, V), -np.inf, np.float32)
    tgt[:, :N, t_of_j] = proc
    tgt[:, N] = np.random.default_rng(5).normal(size=(B, V)).astype(np.float32)
    inv = None if d2t is None else stages.build_inverse_map(d2t, Vd, V)
    acc, out = dsl.verify_coupled(dev(tgt), dev(tok), None if inv is None else dev(inv), None, dev(c["temp"]),
                                  dev(c["rid"]), c["seed"], Vd=Vd)
    acc = host(acc)
    say(f"  accepted {np.count_nonzero(acc == N)} of {B} requests in full")
    assert (acc == N).all()


# ---------------------------------------------------------------- next rows: verification budget

@pytest.mark.parametrize("B,N,knee", [(1, 8, 4), (64, 8, 256), (256, 16, 1024), (1024, 16, 4096), (3, 5, 8)])
def test_choose_k_parity(B, N, knee):
    say(f"choose_k B={B} N={N} knee={knee}")
    g = np.random.default_rng(B * 31 + N)
    c = (1.0 / (1.0 + np.exp(-g.normal(1.5, 1.0, size=(B, N))))).astype(np.float32)
    surv = stages.admit(np.minimum.accumulate(c, axis=1), 0)["survival"]
    sps = synth.sps_table(B * N + B + 64, seed=B, tile=max(1, knee // 4), knee=knee)
    k, obj = dsl.choose_k(dev(surv), dev(sps))
    k, obj = int(host(k)[0]), float(host(obj)[0])
    ref = stages.choose_k(surv, sps)
    objs = ref["objectives"]
    say(f"  gpu K={k} oracle K={ref['k']} objective {obj:.6g}")
    assert abs(objs[k] - ref["objective"]) <= 1e-12 * ref["objective"]   # an optimal K (near-ties aside)
    assert abs(obj - objs[k]) <= 1e-12 * objs[k]
    assert k == ref["k"] or abs(objs[k] - objs[ref["k"]]) <= 1e-12 * objs[k]


def test_choose_k_scans_past_a_local_maximum_on_gpu():
    s = np.full((4, 8), 0.9, np.float32)
    n = np.arange(64)
    sps = np.where(n <= 12, 1.0, 0.5).astype(np.float32)
    sps[20:37] = 0.9
    k, _ = dsl.choose_k(dev(s), dev(sps))
    assert int(host(k)[0]) == stages.choose_k(s, sps)["k"] == 32


# ---------------------------------------------------------------- next rows: confidence head

@pytest.mark.parametrize("B,N,H,V,Vd,r", [
    (1, 8, 4096, 151936, 151936, 64),    # one request: the stream GEMM, the few-request Markov kernel
    (64, 8, 4096, 32000, 32000, 256),    # the big-tile GEMM, the per-step Markov kernel
    (5, 3, 264, 100, 100, 8),            # H not a multiple of 64: the tiled GEMM
    (256, 16, 4096, 4096, 4096, 64),     # Vd a multiple of 256: the extra row opens a new column tile
    (40, 4, 512, 8192, 2048, 32),        # reduced vocabulary, skinny GEMM
    (12, 2, 4096, 1024, 1024, 16),       # several requests in the few-request kernel
    (64, 8, 256, 151936, 151936, 16),    # 256 x 320 tiles with and without the extra row
    (256, 16, 256, 38400, 38400, 16)])   # Vd a multiple of 320: the extra row alone in a last 320-wide tile
def test_confidence_fused_parity(B, N, H, V, Vd, r):
    """The confidence head inside stages 1 and 2: w_h as one more LM-head row (h_dot), the
    embedding part and the sigmoid inside the Markov loop.  Against the oracle's head on the
    GPU's own draft tokens; the logits, tokens and log Z equal the plain calls' bit for bit."""
    say(f"confidence fused B={B} N={N} H={H} V={V} Vd={Vd} r={r}")
    g = np.random.default_rng(B + N + H + Vd)
    hid = synth.bf16_bits(g.normal(size=(B * N, H)).astype(np.float32))
    W = synth.bf16_bits(g.normal(0, 0.02, size=(Vd, H)).astype(np.float32))
    w1 = synth.bf16_bits(g.normal(0, 0.3, size=(V, r)).astype(np.float32))
    w2 = synth.bf16_bits(g.normal(0, 0.3, size=(Vd, r)).astype(np.float32))
    wconf = synth.bf16_bits(g.normal(0, 1.0 / math.sqrt(H + r), size=H + r).astype(np.float32))
    d2t = None if Vd == V else (g.permutation(V)[:Vd] - np.arange(Vd)).astype(np.int64)
    anc = g.integers(0, V, size=B).astype(np.int32)
    temp = np.asarray([0.0, 0.7, 1.0], np.float32)[g.integers(0, 3, size=B)]
    rid = np.arange(B, dtype=np.uint32)
    tau = g.uniform(0.7, 1.5, size=N).astype(np.float32)
    args = (dev(w1), dev(w2), None if d2t is None else dev(d2t), dev(anc), dev(temp), dev(rid), 99)
    plain = dsl.draft_logits(dev(hid), dev(W))
    logits, h_dot = dsl.draft_logits(dev(hid), dev(W), w_h=dev(wconf[:H].copy()))
    assert torch.equal(plain, logits), "the extra LM-head row changed the logits"
    plain = plain.view(B, N, Vd)
    tok0, lz0 = dsl.markov_sample(plain, *args)
    tok, lz, c = dsl.markov_sample(logits.view(B, N, Vd), *args,
                                   conf=(h_dot, dev(wconf[H:].copy()), 0.3, dev(tau), None))
    assert torch.equal(tok0, tok) and torch.equal(lz0, lz) and torch.equal(plain, logits.view(B, N, Vd))
    dsl.markov_check()
    ref = stages.confidence_head(hid, w1, host(tok), anc, wconf, 0.3, tau)
    err = np.abs(host(c).astype(np.float64) - ref).max()
    hd_ref = stages.bf16_decode(hid) @ stages.bf16_decode(wconf[:H])
    hd_err = np.abs(host(h_dot).astype(np.float64) - hd_ref).max()
    say(f"  c max abs err {err:.2e} (h_dot {hd_err:.2e}), c in [{ref.min():.3f}, {ref.max():.3f}]")
    assert hd_err <= 2e-2
    assert err <= 1e-6


# ---------------------------------------------------------------- end of a round

def test_advance_parity():
    B, N = 300, 7
    g = np.random.default_rng(17)
    acc = g.integers(0, N + 1, size=B).astype(np.int32)
    out = g.integers(0, 151936, size=(B, N + 1)).astype(np.int32)
    anchor = np.zeros(B, np.int32)
    emitted = g.integers(0, 1000, size=B).astype(np.int64)
    a_d, e_d = dev(anchor), dev(emitted)
    dsl.advance(dev(acc), dev(out), a_d, e_d)
    ra, re = stages.advance(acc, out, anchor, emitted)
    assert np.array_equal(host(a_d), ra) and np.array_equal(host(e_d), re)


@pytest.mark.parametrize("name,over", [("tiny", {}), ("batched", dict(B=24, H=512, V=4096, Vd=4096, r=32))])
def test_multi_round_graph(name, over):
    """R rounds chained by advance (each drafting from the last emitted token, its own seed),
    captured in one HIP graph: every replay equals the same rounds run eagerly, bit for bit
    (each stage's parity against the oracle is tested on its own); every round's anchor is the
    previous round's last emitted token; tau lies in [1, N + 1]."""
    import bench
    w = synth.get(name, **over)
    R = 4
    path = bench.Path(w, torch, dsl, synth, "rejection", False)
    anchor0 = path.anchor.clone()
    path.advance = True
    eager = []
    for q in range(R):
        path.round_seed = q + 1
        path.step()
        eager.append((path.tokens.clone(), path.accepted.clone(), path.out_tokens.clone(), path.anchor.clone()))
    em_eager = path.emitted.clone()
    graph = torch.cuda.CUDAGraph()
    path.anchor.copy_(anchor0)
    path.emitted.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for q in range(R):
            path.round_seed = q + 1
            path.step()
    for rep in range(2):
        path.anchor.copy_(anchor0)
        path.emitted.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(path.anchor, eager[-1][3]) and torch.equal(path.emitted, em_eager), f"replay {rep}"
        assert torch.equal(path.out_tokens, eager[-1][2]) and torch.equal(path.accepted, eager[-1][1])
    # the anchors follow the verified tokens: each round's anchor is the previous round's last emitted token
    for q in range(1, R):
        prev_acc, prev_out = host(eager[q - 1][1]), host(eager[q - 1][2])
        assert np.array_equal(host(eager[q - 1][3]), prev_out[np.arange(w.B), prev_acc])
    tau = host(em_eager).sum() / (w.B * R)
    say(f"  tau {tau:.3f} over {R} rounds")
    assert 1.0 <= tau <= w.N + 1


# ------------------------------------------------------------------ whole round in a HIP graph
def _round_outputs(path):
    outs = [path.tokens, path.logz, path.logits, path.survival, path.admit_len, path.accepted, path.out_tokens]
    if path.deferred:
        outs.append(path.win)
    return [t.detach().clone() for t in outs]


@pytest.mark.gpu
@pytest.mark.parametrize("name,over,coupled,rows", [
    ("tiny", {}, False, "stored"),                                                # few-request Markov kernel
    ("batched", dict(B=20, H=256, V=4096, Vd=4096, r=32), False, "deferred"),     # deferred rows, 20 requests
    ("batched", dict(B=8, H=256, V=8192, Vd=8192, r=64), False, "stored"),        # few-request, several requests
    ("batched", dict(B=40, H=256, V=8192, Vd=8192, r=64), False, "deferred"),     # deferred rows, replay in the graph
    ("reduced_vocab", dict(B=40, H=256, V=8192, Vd=2048, r=64, K=200), False, "deferred"),  # target map: stored
    ("batched", dict(B=24, H=512, V=4096, Vd=4096, r=32), True, "deferred"),      # coupled verification
])
def test_graph_replay_round(name, over, coupled, rows):
    """A whole round (stages 1-4) captured once in a HIP graph and replayed: every replay,
    with eager work and synchronisations between replays, gives the eager round's outputs
    bit for bit (the library allocates nothing and clears its counters with kernels)."""
    import bench
    import draft_sampling_lossless_amd as dsl
    w = synth.get(name, **over)
    say(f"graph replay {name} {over} coupled={coupled} draft rows {rows}")
    path = bench.Path(w, torch, dsl, synth, "coupled" if coupled else "rejection", False, rows)
    path.step()
    torch.cuda.synchronize()
    ref = _round_outputs(path)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path.step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (path.tokens, path.logz, path.logits, path.out_tokens, path.win):
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _round_outputs(path)
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager round"
        # eager work between replays
        path.step()
        x = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(x)
