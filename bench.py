"""Benchmark of the DSpark draft-sample-verify path on one MI355X.

One step = one round of the whole hot path over one batch of synthetic input:
  stage 1 draft_logits -> stage 2 markov_sample -> stage 4 admit -> stage 3 verify
(verify on the admitted prefixes, logits input).  All inputs are resident in
HBM before the timed region; the target logits are the step's own base logits
plus seeded noise, made once before timing.

Metric: draft+verify positions per second (B * N per step).  The default
workload is the largest single-GPU one at V = 151936: B = 256 requests, N = 16
draft positions, rank 256, K = 1024 admitted.  Beside it: the roofline of the
dominant kernel (the draft-logit GEMM, MFMA-bound at that size) and the HBM
fractions of the Markov loop and of verify, each from HIP events recorded on the
stream the kernels run on inside the timed steps; the same stages timed cold
(a 1 GiB read-write scrub before each stage evicts the 256 MB last-level cache);
and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="admission",
                   help="tiny | qwen3_8b_single | batched | admission | reduced_vocab")
    p.add_argument("--graph", action="store_true", help="replay each step as one captured HIP graph")
    p.add_argument("--verify", default="rejection", choices=("rejection", "coupled"),
                   help="stage 3 rule: rejection sampling on p_t, p_d (default) or Gumbel-coupled verification")
    p.add_argument("--draft-rows", default="deferred", choices=("deferred", "stored"),
                   help="deferred (default where it applies: no target map, rejection verification, more "
                        "than 16 requests): stage 2 keeps the base logits and stage 3 rebuilds only the draft rows "
                        "it reads; stored: stage 2 writes every processed draft row")
    p.add_argument("--round", default="path", choices=("path", "full"),
                   help="path: stages 1-4 with the workload's synthetic confidences and fixed K (default); "
                        "full: also the confidence head (its output feeds admission) and the throughput-optimal "
                        "K, computed from this round's survival and used two rounds later")
    p.add_argument("--context-kv", type=int, default=8192, metavar="NCTX",
                   help="also time the context-KV precompute (the step before the path) on one prefill chunk of "
                        "NCTX tokens at H_in = H_d = 4096, 5 layers of 8 KV heads x 128 (0: skip); reported beside "
                        "the headline, not in it")
    p.add_argument("--rounds", type=int, default=8,
                   help="multi-round driver: R consecutive rounds (each drafting from the previous round's last "
                        "emitted token, with its own seed) captured in one HIP graph and replayed; reports tau and "
                        "the time per emitted token (0: skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache stage timings")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB five times (reference for the "
                        "HBM byte counters) and exit")
    return p.parse_args()


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


class Path:
    """Device buffers and the four C-ABI calls of one round."""

    def __init__(self, w, torch, dsl, synth, verify_mode="rejection", full_round=False, draft_rows="deferred"):
        self.w, self.torch, self.dsl = w, torch, dsl
        self.coupled = verify_mode == "coupled"
        self.full = full_round
        # deferred draft rows need the identity vocabulary map and rejection verification, and
        # take the per-step Markov kernels: at 16 requests or fewer the few-request kernel,
        # which stores the rows, is faster (one request: 0.28 against 0.37 ms per round)
        self.deferred = draft_rows == "deferred" and not self.coupled and w.Vd == w.V and w.B > 16
        # which kernels a stage launches: counter records apply only to the same variant
        self.variant = "/".join(("deferred" if self.deferred else "stored", verify_mode,
                                 "full" if full_round else "path"))
        dev = torch.device("cuda:0")
        rp = synth.request_params(w)

        def up(x):
            x = np.ascontiguousarray(x)
            if x.dtype == np.uint16:
                x = x.view(np.int16)
            if x.dtype == np.uint32:
                x = x.view(np.int32)
            return torch.from_numpy(x).to(dev)

        t0 = time.time()
        self.hidden = up(synth.hidden_bf16(w))
        self.lm_head = up(synth.lm_head_bf16(w))
        self.w1 = up(synth.markov_w1_bf16(w))
        self.w2 = up(synth.markov_w2_bf16(w))
        d2t = synth.d2t_offsets(w)
        self.d2t = None if d2t is None else up(d2t)
        self.inv = None if d2t is None else dsl.build_inverse_map(self.d2t, w.V)
        self.anchor = up(rp["anchor"])
        self.temp = up(rp["temperature"])
        self.rid = up(rp["request_id"])
        self.sigma = up(rp["sigma"])
        self.conf = up(synth.confidence(w))
        self.K = w.budget
        self.seed = w.philox_seed
        self.logits = torch.empty((w.B, w.N, w.Vd), dtype=torch.float32, device=dev)
        self.tokens = torch.empty((w.B, w.N), dtype=torch.int32, device=dev)
        self.logz = torch.empty((w.B, w.N), dtype=torch.float32, device=dev)
        self.survival = torch.empty((w.B, w.N), dtype=torch.float32, device=dev)
        self.admit_len = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.accepted = torch.empty(w.B, dtype=torch.int32, device=dev)
        self.out_tokens = torch.empty((w.B, w.N + 1), dtype=torch.int32, device=dev)
        self.ws_markov = torch.empty(max(16, dsl.markov_workspace_size(w.B, w.N, w.Vd, w.r)),
                                     dtype=torch.uint8, device=dev)
        vws = dsl.verify_coupled_workspace_size(w.B, w.N, w.V) if self.coupled else \
            dsl.verify_deferred_workspace_size(w.B, w.N, w.V) if self.deferred else \
            dsl.verify_workspace_size(w.B, w.N, w.V)
        self.win = torch.empty((w.B, w.N), dtype=torch.float32, device=dev)
        self.ws_verify = torch.empty(max(16, vws), dtype=torch.uint8, device=dev)
        # target logits [B, N+1, V]: this batch's base logits (row N repeats row N-1),
        # scattered to target ids, plus N(0, sigma_b) noise -- made once, untimed
        dsl.draft_logits(self.hidden, self.lm_head, out=self.logits.view(w.M, w.Vd))
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed)
        self.target = torch.randn((w.B, w.N + 1, w.V), generator=gen, device=dev, dtype=torch.float32)
        self.target.mul_(self.sigma.view(-1, 1, 1))
        rows = list(range(w.N)) + [w.N - 1]
        if self.d2t is None:
            self.target.add_(self.logits[:, rows])
        else:
            tids = torch.arange(w.Vd, device=dev, dtype=torch.int64) + self.d2t
            self.target[:, :, tids] += self.logits[:, rows]
        if self.full:
            # confidence head weights (random, like every weight here): w ~ N(0, 1/(H + r)),
            # bias 1.5 and per-position temperatures; an SPS table of the target engine
            g = np.random.default_rng([w.seed, 91])
            wconf = synth.bf16_bits(g.normal(0, 1.0 / np.sqrt(w.H + w.r), size=w.H + w.r).astype(np.float32))
            self.w_h, self.w_e = up(wconf[:w.H].copy()), up(wconf[w.H:].copy())
            self.h_dot = torch.empty(w.M, dtype=torch.float32, device=dev)
            self.cbias = 1.5
            self.tau = up(np.linspace(1.0, 1.6, w.N).astype(np.float32))
            self.sps = up(synth.sps_table(w.B * w.N + w.B + 64, seed=w.seed, tile=64, knee=max(64, w.B * 4)))
            self.c_model = torch.empty((w.B, w.N), dtype=torch.float32, device=dev)
            self.k_dev = torch.empty(1, dtype=torch.int32, device=dev)
            self.k_obj = torch.empty(1, dtype=torch.float64, device=dev)
            self.k_host = torch.empty(3, dtype=torch.int32, pin_memory=True)
            self.k_ready = [torch.cuda.Event() for _ in range(3)]
            self.round = 0
            self.K_used = []
        # multi-round driving (off by default): anchor <- last emitted token, emitted count
        self.advance = False
        self.round_seed = 0
        self.emitted = torch.zeros(w.B, dtype=torch.int64, device=dev)
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    def budget(self):
        """K for this round: fixed, or (full round) the K chosen two rounds ago."""
        if not self.full or self.round < 2:
            return self.K
        slot = (self.round - 2) % 3
        self.k_ready[slot].synchronize()        # long done: the GPU is at most a round behind
        return int(self.k_host[slot])

    def step(self, timer=None, scrub=None):
        """One round.  timer: optional StageTimer that brackets each stage with HIP
        events on the launch stream.  scrub: optional callable run before each stage,
        outside its events (cold-cache timing)."""
        w, dsl = self.w, self.dsl

        def stage(name, fn):
            if scrub is not None:
                scrub()
            if timer is not None:
                timer.begin(name)
            fn()
            if timer is not None:
                timer.end(name)

        seed = self.seed + self.round_seed
        if self.full:
            # the confidence head rides along: w_h as one more LM-head row, the rest in stage 2
            stage("draft_logits", lambda: dsl.draft_logits(self.hidden, self.lm_head, out=self.logits.view(w.M, w.Vd),
                                                           w_h=self.w_h, h_dot=self.h_dot))
            cargs = (self.h_dot, self.w_e, self.cbias, self.tau, self.c_model)
            if self.deferred:
                stage("markov_sample", lambda: dsl.markov_sample_deferred(
                    self.logits, self.w1, self.w2, self.anchor, self.temp, self.rid, seed, draft_tokens=self.tokens,
                    log_z=self.logz, win_logit=self.win, workspace=self.ws_markov, conf=cargs))
            else:
                stage("markov_sample", lambda: dsl.markov_sample(
                    self.logits, self.w1, self.w2, self.d2t, self.anchor, self.temp, self.rid, seed,
                    draft_tokens=self.tokens, log_z=self.logz, workspace=self.ws_markov, conf=cargs))
            conf = self.c_model
        else:
            stage("draft_logits", lambda: dsl.draft_logits(self.hidden, self.lm_head,
                                                           out=self.logits.view(w.M, w.Vd)))
            if self.deferred:
                stage("markov_sample", lambda: dsl.markov_sample_deferred(
                    self.logits, self.w1, self.w2, self.anchor, self.temp, self.rid, seed, draft_tokens=self.tokens,
                    log_z=self.logz, win_logit=self.win, workspace=self.ws_markov))
            else:
                stage("markov_sample", lambda: dsl.markov_sample(
                    self.logits, self.w1, self.w2, self.d2t, self.anchor, self.temp, self.rid, seed,
                    draft_tokens=self.tokens, log_z=self.logz, workspace=self.ws_markov))
            conf = self.conf
        K = self.budget()
        if self.full:
            self.K_used.append(K)
        stage("admit", lambda: dsl.admit(conf, K, survival=self.survival, admit_len=self.admit_len))
        if self.coupled:
            stage("verify", lambda: dsl.verify_coupled(
                self.target, self.tokens, self.inv, self.admit_len, self.temp, self.rid, seed, Vd=w.Vd,
                accepted=self.accepted, out_tokens=self.out_tokens, workspace=self.ws_verify))
        elif self.deferred:
            # (stage 2's anchor: advance runs after this stage)
            stage("verify", lambda: dsl.verify_deferred(
                self.target, self.logits, self.logz, self.win, self.tokens, self.anchor, self.w1, self.w2,
                self.admit_len, self.temp, self.rid, seed, accepted=self.accepted, out_tokens=self.out_tokens,
                workspace=self.ws_verify))
        else:
            stage("verify", lambda: dsl.verify(
                dsl.INPUT_LOGITS, self.target, self.logits, self.logz, self.tokens, self.inv, self.admit_len,
                self.temp, self.rid, seed, accepted=self.accepted, out_tokens=self.out_tokens,
                workspace=self.ws_verify))
        if self.advance:
            # the next round drafts from this round's last emitted token
            stage("advance", lambda: dsl.advance(self.accepted, self.out_tokens, self.anchor, self.emitted))
        if self.full:
            def budget_ahead():
                # the budget of two rounds ahead, from this round's survival
                dsl.choose_k(self.survival, self.sps, k_out=self.k_dev, objective_out=self.k_obj)
                slot = self.round % 3
                self.k_host[slot:slot + 1].copy_(self.k_dev, non_blocking=True)
                self.k_ready[slot].record()
            stage("choose_k", budget_ahead)
            self.round += 1


class StageTimer:
    """HIP event pairs around each stage, recorded on torch's current stream (the
    stream the binding launches on); durations are read after a synchronisation."""

    def __init__(self, torch, only=None):
        self.torch = torch
        self.only = only        # stage names to time (None: every stage)
        self.pairs = {}
        self.open = {}

    def begin(self, name):
        if self.only is not None and name not in self.only:
            return
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.open[name] = e

    def end(self, name):
        if name not in self.open:
            return
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append((self.open.pop(name), e))

    def mean_ms(self):
        return {k: float(np.mean([b.elapsed_time(e) for b, e in v])) for k, v in self.pairs.items()}


def stage_bytes(w, accepted, coupled, deferred=False):
    """Compulsory HBM bytes of stage 2 and stage 3 per step.
    Stage 2: base logits read and processed logits written (8 B per entry), W2
    once, one W1 row per position; with deferred draft rows only the read (4 B).
    Stage 3: the target rows k <= a_b (4 V each), a_b = the accepted count: the
    rows of the accepted positions and the decisive one (the first rejection, or
    the bonus row); verification stops there, so rows past it are not part of the
    method's work.  Rejection sampling also reads one target and one draft row to
    sample from (deferred: the base row and W2 once)."""
    per_entry = 4 if deferred else 8
    k2 = per_entry * w.B * w.N * w.Vd + 2 * w.r * w.Vd + 2 * w.r * w.B * w.N
    k3 = 4 * w.V * int((np.asarray(accepted, dtype=np.int64) + 1).sum())
    if not coupled:
        k3 += w.B * (4 * w.V + 4 * w.Vd)
    if deferred:
        k3 += 2 * w.r * w.Vd
    return k2, k3


def k1_work(w):
    """Algorithmic work of one draft-logit GEMM launch: bytes and flops."""
    bytes_ = 2 * w.Vd * w.H + 2 * w.M * w.H + 4 * w.M * w.Vd
    flops = 2 * w.M * w.H * w.Vd
    return bytes_, flops


def k1_roofline(w, k1_ms, variant):
    bytes_, flops = k1_work(w)
    # arithmetic intensity vs the ridge of the chip decides the bound
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / bytes_ < ridge:
        ach = bytes_ / (k1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = flops / (k1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFS, 4)}
    if w.M <= 16 and w.H % 512 == 0 and w.H <= 4096:
        roof["kernel"] = "draft_logits (k1_stream)"
    else:
        roof["kernel"] = ("draft_logits (k1_skinny)" if w.M <= 64 else
                          "draft_logits (k1_tiled)" if w.H % 64 else "draft_logits (k1_pingpong)")
    roof["traffic"] = measured_traffic("draft_logits", w, variant)
    if roof["traffic"]:
        roof["traffic_gbs"] = round(roof["traffic"] / (k1_ms * 1e-3) / 1e9, 1)
    return roof


def measured_traffic(stage, w, variant):
    """HBM bytes (FETCH + WRITE, calibrated) per call of a stage from the committed
    rocprofv3 counter summary profiles/<stage>_<workload>_traffic.json, if it was
    taken on the same path variant (draft rows / verify rule / round) and on the
    current sources of the kernel files it names; else null."""
    path = os.path.join(PROFILES, f"{stage}_{w.name}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        if d.get("variant") != variant:
            return None
        # every kernel source the stage's launches come from (older files name one)
        files = d.get("source_files") or {d["source_file"]: d["source_sha256_16"]}
        for f, h in files.items():
            if h != src_hash(os.path.join(ROOT, f)):
                return None
        return d.get("bytes_per_call")
    except Exception:
        return None


def hbm_roofline(name, bytes_, ms, w, variant, cold_ms=None):
    ach = bytes_ / (ms * 1e-3) / 1e9
    out = {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(bytes_),
           "traffic": measured_traffic(name.split(" ")[0], w, variant)}
    if out["traffic"]:
        # the counted HBM bytes over the same time: how hard the stage drives the memory
        out["traffic_gbs"] = round(out["traffic"] / (ms * 1e-3) / 1e9, 1)
        out["traffic_frac"] = round(out["traffic_gbs"] / HBM_PEAK_GBS, 4)
    if cold_ms:
        cold = bytes_ / (cold_ms * 1e-3) / 1e9
        out["achieved_cold"] = round(cold, 1)
        out["frac_cold"] = round(cold / HBM_PEAK_GBS, 4)
    return out


def context_kv_bench(torch, dsl, n_ctx, H=4096, L=5, nkv=8, hd=128, reps=10):
    """dspark_context_kv on one prefill chunk: seeded synthetic bf16 weights and hidden
    states made on the device, positions 0 .. n_ctx-1 at slots 0 .. n_ctx-1.  Time per
    call from HIP events on the launch stream, warm; flops of the two products."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4242)

    def bf(shape, std, mean=0.0):
        return (torch.randn(shape, generator=g, device=dev) * std + mean).to(torch.bfloat16)

    kvr = L * 2 * nkv * hd
    args = dict(aux=bf((n_ctx, H), 1.0), fc_w=bf((H, H), H ** -0.5), fc_b=bf((H,), 0.1), hnorm_w=bf((H,), 0.1, 1.0),
                kv_w=bf((kvr, H), H ** -0.5), kv_b=bf((kvr,), 0.1), knorm_w=bf((L, hd), 0.1, 1.0),
                positions=torch.arange(n_ctx, dtype=torch.int32, device=dev),
                slots=torch.arange(n_ctx, dtype=torch.int64, device=dev),
                k_cache=torch.empty((L, n_ctx, nkv, hd), dtype=torch.bfloat16, device=dev),
                v_cache=torch.empty((L, n_ctx, nkv, hd), dtype=torch.bfloat16, device=dev))
    ws = torch.empty(dsl.context_kv_workspace_size(n_ctx, H, L, nkv, hd), dtype=torch.uint8, device=dev)

    def call():
        dsl.context_kv(args["aux"], args["fc_w"], args["fc_b"], args["hnorm_w"], args["kv_w"], args["kv_b"],
                       args["knorm_w"], args["positions"], args["slots"], args["k_cache"], args["v_cache"],
                       workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * n_ctx * H * (H + kvr)
    tfs = flops / (ms * 1e-3) / 1e12
    out = {"num_ctx": n_ctx, "H_in": H, "H_d": H, "L": L, "nkv": nkv, "hd": hd, "ms": round(ms, 4),
           "tokens_per_s": round(n_ctx / (ms * 1e-3), 1), "achieved_tflops": round(tfs, 1),
           "peak_tflops": MFMA_BF16_PEAK_TFS, "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
           "note": "fc and fused K/V products (MFMA) plus the norm, RoPE and cache-write passes; flops of the "
                   "products; synthetic seeded weights"}
    del args, ws
    torch.cuda.synchronize()
    return out


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on a bounded sample of the workload: whole rounds
    of the first request (all N positions, full vocabulary), repeated while the
    budget lasts (at least once)."""
    import synth
    from oracle import stages
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    reqs = [0]
    ws = synth.get(w.name, B=1, K=None if w.K is None else max(1, w.K // w.B))
    rp = synth.request_params(w)
    hid = synth.hidden_bf16(w, rows=list(range(w.N)))
    lm = synth.lm_head_bf16(w)
    w1, w2 = synth.markov_w1_bf16(w), synth.markov_w2_bf16(w)
    d2t = synth.d2t_offsets(w)
    inv = None if d2t is None else stages.build_inverse_map(d2t, w.Vd, w.V)
    conf = synth.confidence(w)[:1]
    noise = synth.target_noise(w, reqs)
    t_of_j = np.arange(w.Vd) + (0 if d2t is None else d2t)
    runs, t_total = 0, 0.0
    while runs == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        base = stages.draft_logits(hid, lm).reshape(1, w.N, w.Vd)
        mk = stages.markov_sample(base, w1, w2, d2t, rp["anchor"], rp["temperature"], rp["request_id"],
                                  w.philox_seed, requests=reqs)
        ad = stages.admit(conf, ws.budget)
        tgt = noise * rp["sigma"][0]
        tgt[:, :, t_of_j] += base[:, list(range(w.N)) + [w.N - 1]]
        stages.verify("logits", tgt.astype(np.float32), mk["processed"], mk["tokens"], inv, ad["admit_len"],
                      rp["temperature"], rp["request_id"], w.philox_seed, requests=reqs)
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total > budget_s:
            break
    pos = runs * w.N
    return {"value": round(pos / t_total, 3), "unit": "positions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} round(s) of request 0 of {w.name} (N={w.N} positions, V={w.V}, full stage 1-4 "
                      f"oracle incl. the {w.Vd}x{w.H} fp64 draft-logit product), {t_total:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import draft_sampling_lossless_amd as dsl
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return
    if not os.path.exists(dsl.LIB_PATH):
        from draft_sampling_lossless_amd import build
        build.build()
    if args.graph and args.round == "full":
        print(json.dumps({"error": "--round full chooses K on the host two rounds ahead; it cannot be "
                                   "replayed as one captured graph"}))
        sys.exit(2)
    w = synth.get(args.workload)
    path = Path(w, torch, dsl, synth, args.verify, args.round == "full", args.draft_rows)
    result = run(args, w, path, torch)
    # release the graph and every device buffer, synchronised, before the interpreter
    # (and any profiler attached to it) tears the HIP runtime down
    torch.cuda.synchronize()
    del path
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def multi_round(w, path, torch, R, reps=5):
    """R consecutive rounds captured in one HIP graph: round q drafts from the previous
    round's last emitted token (dspark_advance) with seed base + q.  The hidden states
    and target logits stay those of the synthetic batch (no backbone or target model
    runs here).  tau = tokens emitted per request per round; time per emitted token =
    round time / tau, i.e. (T_draft + T_verify) / tau."""
    anchor0 = path.anchor.clone()
    path.advance = True
    for q in range(R):                      # warm-up of the same rounds, eager
        path.round_seed = q + 1
        path.step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for q in range(R):
            path.round_seed = q + 1        # (each captured launch keeps its own seed)
            path.step()
    path.round_seed = 0
    times = []
    for _ in range(reps):
        path.anchor.copy_(anchor0)
        path.emitted.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    emitted = int(path.emitted.sum().item())
    ms = float(np.median(times))
    tau = emitted / (w.B * R)
    path.advance = False
    path.anchor.copy_(anchor0)
    del graph
    return {"rounds": R, "graph": True, "tau": round(tau, 4), "ms_per_round": round(ms / R, 4),
            "round_ms_per_token": round(ms / R / tau, 4), "emitted_tokens_per_s": round(emitted / (ms * 1e-3), 1),
            "note": "tau = tokens emitted per request per round (accepted drafts + 1); round_ms_per_token = "
                    "(T_draft + T_verify) / tau"}


def run(args, w, path, torch):
    graph = None
    if args.graph:
        for _ in range(2):
            path.step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            path.step()
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        if graph is not None:
            graph.replay()
        else:
            path.step()
    torch.cuda.synchronize()

    # timed region: K steps; eager steps carry one HIP event pair, around the dominant
    # kernel (the draft-logit product) -- events around every stage would add their own
    # cost to a round that lasts a fraction of a millisecond
    live = StageTimer(torch, only={"draft_logits"}) if graph is None else None
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            path.step(live)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # every stage's time from eager rounds after the timed region
    timer = StageTimer(torch)
    for _ in range(max(5, min(args.steps, 50))):
        path.step(timer)
    torch.cuda.synchronize()
    stage_ms = timer.mean_ms()
    if live is not None:
        stage_ms["draft_logits_live"] = live.mean_ms()["draft_logits"]

    cold_ms = None
    if not args.no_cold:
        # a 1 GiB read-modify-write before each stage: 2 GiB of traffic evicts the 256 MB MALL
        scrub_buf = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        cold = StageTimer(torch)
        for _ in range(5):
            path.step(cold, scrub=lambda: scrub_buf.add_(1.0))
        torch.cuda.synchronize()
        cold_ms = cold.mean_ms()
        del scrub_buf

    positions = w.B * w.N
    value = positions / (ms_per_step * 1e-3)
    k2_bytes, k3_bytes = stage_bytes(w, path.accepted.cpu().numpy(), path.coupled, path.deferred)
    roof = k1_roofline(w, stage_ms.get("draft_logits_live", stage_ms["draft_logits"]), path.variant)
    if cold_ms:
        _, flops = k1_work(w)
        roof["frac_cold"] = round(flops / (cold_ms["draft_logits"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4) \
            if roof["bound"] == "mfma" else round(k1_work(w)[0] / (cold_ms["draft_logits"] * 1e-3) / 1e9
                                                  / HBM_PEAK_GBS, 4)
    roof["stages"] = [
        hbm_roofline("markov_sample", k2_bytes, stage_ms["markov_sample"], w, path.variant,
                     cold_ms and cold_ms["markov_sample"]),
        hbm_roofline("verify", k3_bytes, stage_ms["verify"], w, path.variant, cold_ms and cold_ms["verify"]),
    ]
    result = {
        "metric": "draft+verify positions/sec (B*N) and achieved HBM GB/s at V=151936",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "V": w.V, "Vd": w.Vd, "r": w.r,
                   "K": w.budget, "graph": graph is not None,
                   "draft_rows": "deferred" if path.deferred else "stored"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roof,
    }
    if cold_ms:
        result["stage_ms_cold"] = {k: round(v, 4) for k, v in cold_ms.items()}
    if path.coupled:
        result["config"]["verify"] = "coupled"
    if path.full:
        result["config"]["round"] = "full"
        result["budget_K"] = {"first": path.K_used[2] if len(path.K_used) > 2 else None,
                              "last": path.K_used[-1], "of": w.B * w.N}
    if graph is not None:
        del graph
    if args.rounds > 0 and not path.full:
        result["multi_round"] = multi_round(w, path, torch, args.rounds)
    if args.context_kv > 0:
        result["context_kv"] = context_kv_bench(torch, path.dsl, args.context_kv)
    return result


if __name__ == "__main__":
    main()
