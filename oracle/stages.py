"""The four stages of the DSpark draft-sample-verify path, written plainly.

Sources (the pages this follows):
  [P1] "DSpark 的实现和测评" (vLLM's DSpark speculator walked through)
  [P2] "推测解码：从零到DSpark" (summary of the DSpark paper)
  [P3] "xserv/docs/25-speculative-methods-comparison.md"

Stage 1  draft_logits    [P1 §2.2, §4 step 2]: base logits for all N draft
                         positions at once, one dense product of the backbone
                         hidden states with the LM head.
Stage 2  markov_sample   [P1 §2.2, §3, §5; P2 §4]: left-to-right loop; step i
                         adds the low-rank bigram bias W2 . W1[prev] to the base
                         logits of position i and draws x_i by Gumbel-max;
                         prev starts at the anchor token (which is itself a
                         prediction position, P1 §2.1).
Stage 3  verify          [P2 §2; greedy case P3 §2]: accept x_k with
                         probability min(1, p_t(x_k)/p_d(x_k)) left to right;
                         at the first rejection draw from the normalised
                         positive part of p_t - p_d; if all are accepted draw
                         a bonus token from the next target row.
Stage 4  admit           [P2 §6, §7]: survival = running product of the
                         conditional acceptances; all B*N candidates pooled,
                         ordered by survival, the first K admitted.
Next rows:
  verify_coupled         [P1 §5]: the target verifies with the same Gumbel seed
                         the draft sampled with: y_k = Gumbel-max sample of the
                         target row under the draft's noise; accept while y_k ==
                         x_k; the first mismatch (or the bonus row) emits y.
  choose_k               [P2 §6, §7]: the verification budget K that maximises
                         expected tokens per batch times the engine's steps per
                         second at that batch size, by a full scan.
  confidence_head        [P2 §6]: a linear projection of the backbone hidden
                         state and the Markov embedding of the previous token,
                         temperature-scaled per position, through a sigmoid:
                         each position's conditional acceptance probability.

Readings where the pages are silent (the same readings hold on the GPU side):
  * temperature T > 0 divides the logits; T = 0 means greedy (argmax, no
    noise, point-mass distributions);
  * the Markov bias is added in draft-vocabulary space, before the map to
    target ids; W1 is indexed by a target id, W2 has one row per draft token;
  * the Gumbel noise of stage 2 is keyed on the draft-vocabulary index j; ties
    of the argmax go to the smaller target id t(j) = j + d2t[j];
  * processed logits are stored untempered (base + bias, fp32);
  * row statistic of a processed row: logZ = log sum_j exp(l_j / T) (natural
    log); for T = 0 it is max_j l_j;
  * in verify, at T = 0 the draft distribution at position k is the point mass
    on the drafted token x_k;
  * if the residual max(0, p_t - p_d) is zero everywhere (only rounding can do
    that), the resample uses p_t itself, with the same uniforms;
  * admission order: survival descending, then position ascending, then
    request ascending; K counts draft positions only.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

from . import philox
from .variates import gumbel, race_argmax, race_exponentials, race_top2_margin


# ---------------------------------------------------------------- helpers

def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _target_ids(Vd: int, d2t: Optional[np.ndarray]) -> np.ndarray:
    j = np.arange(Vd, dtype=np.int64)
    return j if d2t is None else j + np.asarray(d2t, dtype=np.int64)


def key_top2_gap(key) -> float:
    """Distance of the winning Gumbel-max key from the runner-up, in key units
    (natural-log units for keys l/T + G).  0 when the largest key is shared by
    several entries, +inf when there is only one entry (no other can win).

    This is what decides whether a disagreement between two implementations of the
    same sampler is a rounding-order near-tie.
    Pins: hand-worked keys (unique maximum, exact tie, single entry, -inf entries);
    markov_sample's greedy gap on a hand-worked row; the Gumbel gap of a row with one
    dominant logit lies in that logit's margin / T plus or minus the Gumbel range.
    """
    k = np.asarray(key, dtype=np.float64).ravel()
    if k.size < 2:
        return math.inf
    best = k.max()
    if np.count_nonzero(k == best) > 1:
        return 0.0
    return float(best - k[k < best].max())


def build_inverse_map(d2t: Optional[np.ndarray], Vd: int, V: int) -> np.ndarray:
    """inv[v] = j if v = j + d2t[j], else -1 [P3 §3.2: target id = draft id + d2t].

    Pins: round trip inv[t(j)] == j on random injective maps; -1 count == V - Vd.
    """
    t = _target_ids(Vd, d2t)
    if t.min() < 0 or t.max() >= V or np.unique(t).size != Vd:
        raise ValueError("d2t does not map the draft vocabulary injectively into [0, V)")
    inv = np.full(V, -1, dtype=np.int32)
    inv[t] = np.arange(Vd, dtype=np.int32)
    return inv


# ---------------------------------------------------------------- stage 1

def draft_logits(hidden_bits, lm_head_bits, chunk: int = 16384) -> np.ndarray:
    """base[m, j] = sum_h h[m, h] * W[j, h], fp64 accumulation, stored fp32.

    hidden_bits [M, H] and lm_head_bits [Vd, H] are bf16 bit patterns.  The
    vocabulary is processed in slices of ``chunk`` rows only to bound memory;
    every output is the same single dot product.
    Pins: one-hot hidden states select LM-head entries exactly; linearity;
    bf16 decoding of known bit patterns.
    """
    h = bf16_decode(hidden_bits)
    lm = np.asarray(lm_head_bits)
    Vd = lm.shape[0]
    out = np.empty((h.shape[0], Vd), dtype=np.float32)
    for lo in range(0, Vd, chunk):
        W = bf16_decode(lm[lo:lo + chunk])
        out[:, lo:lo + W.shape[0]] = (h @ W.T).astype(np.float32)
    return out


# ---------------------------------------------------------------- stage 2

def markov_sample(base, w1_bits, w2_bits, d2t, anchor, temperature, request_id,
                  seed: int, requests: Optional[Sequence[int]] = None,
                  teacher: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Sequential low-rank Markov sampling [P1 §2.2, §3; P2 §4].

    base:        [B, N, Vd] fp32 base logits (rows of ``requests`` if given)
    w1_bits:     [V, r] bf16 bits    (embedding of the previous target token)
    w2_bits:     [Vd, r] bf16 bits   (projection rank -> draft vocabulary)
    d2t:         [Vd] int64 offsets or None (draft vocabulary == target vocabulary)
    anchor, temperature, request_id: per request [B]
    requests:    which requests' rows ``base`` holds (default: all, in order)
    teacher:     optional [.., N] target ids of another run of the same sampler.
                 Teacher forcing: step i then takes prev = teacher[.., i-1] (the
                 anchor at i = 0) instead of its own previous draw, so every step
                 can be compared with that run's step even after the two have drawn
                 different tokens; the output adds ``teacher_deficit``.

    Step i of request b:  e = W1[prev];  bias_j = sum_k W2[j,k] e_k;
    l_j = base[b,i,j] + bias_j;  key_j = l_j / T + G_j (T > 0) or l_j (T = 0);
    x = t(argmax key), ties to the smaller t(j);  prev = x.

    Returns processed [.., N, Vd] fp32 (= base + bias), tokens [.., N] int32
    (target ids), logZ [.., N] fp32, gap [.., N] fp64 (key_top2_gap of the step's
    keys, natural-log units); with a teacher also teacher_deficit [.., N] fp64: the
    best key minus the key of the teacher's token at that step (0 when the teacher
    drew the same token; +inf when its token is outside the draft vocabulary).
    Pins: equals an explicit V x Vd bigram table lookup on tiny V; W1 = 0 gives
    independent per-position sampling; the anchor only changes step 0's bias;
    chi-square of samples against softmax(l/T); T = 0 gives the argmax.
    """
    base = np.asarray(base, dtype=np.float32)
    nb, N, Vd = base.shape
    reqs = np.arange(nb) if requests is None else np.asarray(requests, dtype=np.int64)
    W2 = bf16_decode(w2_bits)                      # [Vd, r]
    w1 = np.asarray(w1_bits)
    t_of_j = _target_ids(Vd, d2t)
    j_all = np.arange(Vd, dtype=np.uint64)
    processed = np.empty_like(base)
    tokens = np.empty((nb, N), dtype=np.int32)
    logZ = np.empty((nb, N), dtype=np.float32)
    gap = np.empty((nb, N), dtype=np.float64)
    deficit = np.full((nb, N), np.nan)
    if teacher is not None:
        teacher = np.asarray(teacher, dtype=np.int64)
        j_of_t = {int(t): j for j, t in enumerate(t_of_j)}
    for n, b in enumerate(reqs):
        prev = int(anchor[b])
        T = float(np.float32(temperature[b]))
        req = int(request_id[b])
        for i in range(N):
            e = bf16_decode(w1[prev])              # [r]
            bias = W2 @ e                          # [Vd]
            l = base[n, i].astype(np.float64) + bias
            processed[n, i] = l.astype(np.float32)
            if T > 0.0:
                u = philox.uniforms(seed, j_all, i, req, philox.TAG_DRAFT)
                key = l / T + gumbel(u)
                y = l / T
                ymax = y.max()
                logZ[n, i] = np.float32(ymax + math.log(np.exp(y - ymax).sum()))
            else:
                key = l
                logZ[n, i] = np.float32(l.max())
            best = key.max()
            x = int(t_of_j[key == best].min())
            gap[n, i] = key_top2_gap(key)
            tokens[n, i] = x
            if teacher is None:
                prev = x
            else:
                jt = j_of_t.get(int(teacher[n, i]))
                deficit[n, i] = math.inf if jt is None else float(best - key[jt])
                prev = int(teacher[n, i])
    out = {"processed": processed, "tokens": tokens, "logZ": logZ, "gap": gap}
    if teacher is not None:
        out["teacher_deficit"] = deficit
    return out


# ---------------------------------------------------------------- stage 3

def probs_from_logits(logits_row, T: float) -> np.ndarray:
    """fp32(softmax(l / T)) computed in fp64; T = 0: one-hot at the argmax
    (ties to the smaller index).  Parity unpinned beyond the softmax definition
    (pinned indirectly: the acceptance and losslessness tests use it)."""
    l = np.asarray(logits_row, dtype=np.float64)
    if T > 0.0:
        y = l / T
        p = np.exp(y - y.max())
        return (p / p.sum()).astype(np.float32)
    p = np.zeros(l.shape, dtype=np.float32)
    p[int(np.argmax(l))] = 1.0                     # argmax returns the first max
    return p


def draft_probs(processed_row, T: float, drafted_draft_index: int) -> np.ndarray:
    """Draft distribution over the draft vocabulary for one position.

    T > 0: fp32(softmax(l / T)); T = 0: point mass on the drafted token.
    """
    if T > 0.0:
        return probs_from_logits(processed_row, T)
    p = np.zeros(np.asarray(processed_row).shape, dtype=np.float32)
    p[int(drafted_draft_index)] = 1.0
    return p


def _verify_one(pt_rows, pd_rows, x, inv, L: int, req: int, seed: int):
    """Exact rejection loop of one request on fp32 probability rows.

    pt_rows(k) -> target probabilities [V] at position k (k <= L)
    pd_rows(k) -> draft probabilities [Vd] at position k (k < L)
    """
    margins = []
    for k in range(L):
        xk = int(x[k])
        jk = int(inv[xk]) if inv is not None else xk
        pt = pt_rows(k)
        pdk = pd_rows(k)
        p_t = np.float64(pt[xk])
        p_d = np.float64(pdk[jk]) if jk >= 0 else 0.0
        u = np.float64(philox.uniforms(seed, 0, k, req, philox.TAG_ACCEPT))
        lhs = u * p_d
        margins.append(abs(lhs - p_t) / p_t if p_t > 0 else math.inf)
        if lhs < p_t:
            continue
        # first rejection: residual max(0, p_t - p_d) over the target vocabulary
        if inv is None:
            pd_t = pdk
        else:
            pd_t = np.where(inv >= 0, pdk[np.maximum(inv, 0)], np.float32(0.0)).astype(np.float32)
        resid = np.maximum(np.float32(0.0), (pt - pd_t).astype(np.float32)).astype(np.float32)
        if not resid.any():
            resid = np.asarray(pt, dtype=np.float32)
        E = race_exponentials(seed, resid.size, k, req, philox.TAG_RESID)
        y = race_argmax(resid, E)
        return k, y, margins, race_top2_margin(resid, E)
    pt = pt_rows(L)
    E = race_exponentials(seed, pt.size, L, req, philox.TAG_BONUS)
    y = race_argmax(pt, E)
    return L, y, margins, race_top2_margin(pt, E)


def verify(mode: str, target, draft, draft_tokens, inv_map, verify_len, temperature,
           request_id, seed: int, requests: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Lossless rejection-sampling verification [P2 §2; greedy case P3 §2].

    mode "probs":  target = p_t [B, N+1, V] fp32, draft = p_d [B, N, Vd] fp32;
                   temperature is not used.
    mode "logits": target = target logits [B, N+1, V], draft = processed draft
                   logits [B, N, Vd]; p_t = fp32(softmax(l/T)), p_d likewise
                   (T = 0: point masses on the target argmax / the drafted token).
    draft_tokens [B, N] target ids; inv_map [V] int32 (-1 = not in the draft
    vocabulary) or None when Vd == V; verify_len [B] (None -> N).

    Per request b with L = verify_len[b]: for k < L accept x_k iff
    u_k * p_d(x_k) < p_t(x_k) (fp64 of fp32 values, exact), u_k the uniform of
    (seed, index 0, position k, request, tag 1).  At the first rejection k the
    output token is the exponential-race sample (tag 2, position k) of
    max(0, fp32(p_t - p_d)); with every position accepted it is the race sample
    (tag 3, position L) of p_t at row L.

    Returns accepted [B] int32, out_tokens [B, N+1] int32 (x_0..x_{a-1}, y,
    then -1), and per-request near-tie margins (relative distance of each
    acceptance test from its threshold, relative top-2 gap of the race).
    Pins: T = 0 gives the longest prefix matching the target argmaxes plus the
    target argmax after it (P3 §2); p_t == p_d accepts every position; emitted
    tokens follow p_t (chi-square); acceptance rate at position 0 equals
    sum min(p_t, p_d) = 1 - TV (P2 §2).
    """
    nb = np.asarray(draft_tokens).shape[0]
    N = np.asarray(draft_tokens).shape[1]
    reqs = np.arange(nb) if requests is None else np.asarray(requests, dtype=np.int64)
    inv = None if inv_map is None else np.asarray(inv_map, dtype=np.int64)
    accepted = np.empty(nb, dtype=np.int32)
    out = np.full((nb, N + 1), -1, dtype=np.int32)
    acc_margins, race_margins = [], []
    for n, b in enumerate(reqs):
        L = N if verify_len is None else int(verify_len[b])
        x = np.asarray(draft_tokens[n], dtype=np.int64)
        req = int(request_id[b])
        if mode == "probs":
            def pt_rows(k, n=n):
                return np.asarray(target[n, k], dtype=np.float32)

            def pd_rows(k, n=n):
                return np.asarray(draft[n, k], dtype=np.float32)
        elif mode == "logits":
            T = float(np.float32(temperature[b]))

            def pt_rows(k, n=n, T=T):
                return probs_from_logits(target[n, k], T)

            def pd_rows(k, n=n, T=T, x=x):
                jk = int(inv[x[k]]) if inv is not None else int(x[k])
                return draft_probs(draft[n, k], T, jk)
        else:
            raise ValueError(mode)
        a, y, m_acc, m_race = _verify_one(pt_rows, pd_rows, x, inv, L, req, seed)
        accepted[n] = a
        out[n, :a] = x[:a]
        out[n, a] = y
        acc_margins.append(m_acc)
        race_margins.append(m_race)
    return {"accepted": accepted, "out_tokens": out,
            "accept_margins": acc_margins, "race_margin": race_margins}


def accept_prob(p_t_row, p_d_row_target_space) -> float:
    """Per-position acceptance probability sum_v min(p_t, p_d) = 1 - TV [P2 §2].

    Pin: empirical acceptance frequency of ``verify`` at position 0.
    """
    a = np.asarray(p_t_row, dtype=np.float64)
    b = np.asarray(p_d_row_target_space, dtype=np.float64)
    return float(np.minimum(a, b).sum())


def coupled_noise(seed: int, position: int, req: int, V: int, inv) -> np.ndarray:
    """Gumbel noise G(v) of target row ``position`` for Gumbel-coupled verification.

    A target id v that is draft entry j (inv[v] = j, or j = v without a reduced
    vocabulary) gets the very noise stage 2 drew for j at that position (tag 0,
    keyed on j); an id outside the draft vocabulary gets its own draw (tag 4,
    keyed on v).  So the G(v) are independent standard Gumbels over v.
    """
    v_all = np.arange(V, dtype=np.int64)
    if inv is None:
        j = v_all
        own = np.zeros(V, dtype=bool)
    else:
        inv = np.asarray(inv, dtype=np.int64)
        own = inv < 0
        j = np.where(own, v_all, inv)
    u_draft = philox.uniforms(seed, j.astype(np.uint64), position, req, philox.TAG_DRAFT)
    u_own = philox.uniforms(seed, v_all.astype(np.uint64), position, req, philox.TAG_TARGET)
    return gumbel(np.where(own, u_own, u_draft))


def verify_coupled(target_logits, draft_tokens, inv_map, verify_len, temperature, request_id,
                   seed: int, requests: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Gumbel-coupled verification [P1 §5: the target verifies with the same
    Gumbel seed as the draft, and the output distribution is unchanged].

    target_logits [B, N+1, V] fp32; draft_tokens [B, N] target ids drawn by
    stage 2 with the same seed and request ids; inv_map [V] or None.
    Row k of request b: y_k = argmax_v l_t[k](v) / T + G_k(v) (coupled_noise;
    T = 0: argmax l_t[k]), ties to the smaller v, keys in fp64.  With L the
    verify length, a = the first k < L with y_k != x_k (else L); the output is
    x_0 .. x_{a-1}, y_a, then -1.  Every emitted token is a y, a Gumbel-max draw
    from p_t, so the output follows the target; a draft token is accepted exactly
    when the target's own draw under the same noise picks it.

    Returns accepted [B], out_tokens [B, N+1], and gap [B, N+1]: the top-2 key
    margin of each row k <= L (NaN beyond), for near-tie tolerance.
    Pins: T = 0 equals greedy verification; a target equal to the draft's
    processed logits accepts every stage-2 draft; the emitted first token follows
    softmax(l_t/T) (chi-square); acceptance at position 0 is at most 1 - TV.
    """
    x_all = np.asarray(draft_tokens, dtype=np.int64)
    nb, N = x_all.shape
    reqs = np.arange(nb) if requests is None else np.asarray(requests, dtype=np.int64)
    inv = None if inv_map is None else np.asarray(inv_map, dtype=np.int64)
    accepted = np.empty(nb, dtype=np.int32)
    out = np.full((nb, N + 1), -1, dtype=np.int32)
    gap = np.full((nb, N + 1), np.nan)
    for n, b in enumerate(reqs):
        L = N if verify_len is None else int(verify_len[b])
        T = float(np.float32(temperature[b]))
        req = int(request_id[b])
        a, y_a = L, None
        for k in range(L + 1):
            l = np.asarray(target_logits[n, k], dtype=np.float64)
            key = (l / T + coupled_noise(seed, k, req, l.size, inv)) if T > 0.0 else l
            y = int(np.argmax(key))                 # the first maximum: the smaller v
            top2 = np.partition(key, -2)[-2:] if key.size > 1 else np.array([-np.inf, key[0]])
            gap[n, k] = float(top2[1] - top2[0])
            if k == L or y != x_all[n, k]:
                a, y_a = k, y
                break
        accepted[n] = a
        out[n, :a] = x_all[n, :a]
        out[n, a] = y_a
    return {"accepted": accepted, "out_tokens": out, "gap": gap}


# ---------------------------------------------------------------- stage 4

def admit(cond_accept, K: int) -> Dict[str, np.ndarray]:
    """Confidence-scheduled admission [P2 §6, §7].

    survival[b, 0] = c[b, 0];  survival[b, k] = fp32(survival[b, k-1] * c[b, k]).
    All B*N (b, k) are ordered by survival descending, then k ascending, then b
    ascending; the first min(K, B*N) are admitted; admit_len[b] counts the
    admitted positions of request b.  With c <= 1 survival never increases
    along k, so each request's admitted set is a prefix, and whether (b, k) is
    admitted does not depend on c[b, j] for j > k.
    Pins: prefix closure; sum admit_len == min(K, B*N); K = 0 and K >= B*N;
    non-anticipation (re-drawing c[b, j > k] leaves (b, k) unchanged); a
    hand-worked example in tests/golden.
    """
    c = np.asarray(cond_accept, dtype=np.float32)
    B, N = c.shape
    s = np.empty_like(c)
    s[:, 0] = c[:, 0]
    for k in range(1, N):
        s[:, k] = (s[:, k - 1] * c[:, k]).astype(np.float32)
    bb, kk = np.meshgrid(np.arange(B), np.arange(N), indexing="ij")
    order = np.lexsort((bb.ravel(), kk.ravel(), -s.ravel().astype(np.float64)))
    take = order[: max(0, min(int(K), B * N))]
    admitted = np.zeros(B * N, dtype=bool)
    admitted[take] = True
    admit_len = admitted.reshape(B, N).sum(axis=1).astype(np.int32)
    return {"survival": s, "admit_len": admit_len, "admitted": admitted.reshape(B, N)}


# ---------------------------------------------------------------- end of a round

def advance(accepted, out_tokens, anchor, emitted=None):
    """The next round's anchors [P1 §2.1: the anchor of a request is the token its
    previous step verified]: anchor[b] = out_tokens[b, accepted[b]] (the correction or
    bonus token verify emitted last); emitted[b] += accepted[b] + 1.  Returns the new
    (anchor, emitted) arrays.
    Pins: a hand-worked round (a rejection and a full acceptance); chaining verify's
    greedy outputs reproduces the greedy decode of the target argmaxes.
    """
    acc = np.asarray(accepted, dtype=np.int64)
    out = np.asarray(out_tokens, dtype=np.int64)
    new_anchor = out[np.arange(acc.size), acc].astype(np.int32)
    new_emitted = None if emitted is None else (np.asarray(emitted, dtype=np.int64) + acc + 1)
    return new_anchor, new_emitted


# ---------------------------------------------------------------- next rows: budget K

def choose_k(survival, sps, B: Optional[int] = None) -> Dict[str, object]:
    """Throughput-optimal verification budget [P2 §6: maximise expected tokens per
    batch times SPS at that batch size; pool every request's candidates and admit
    by survival; P2 §7: the SPS curve is jagged, so the search does not stop early].

    survival [B, N] fp32 (stage 4's running products: non-increasing along k);
    sps [S] steps per second of the target engine at a batch of n tokens, n = 0..S-1.
    Readings: admitting the K best candidates costs a batch of B + K tokens (every
    request verifies its current position plus its admitted drafts) and yields
    B + (sum of their survival) expected tokens (every request emits one token
    beyond its accepted drafts; a draft's survival is the probability it is
    accepted).  objective(K) = (B + S_K) * sps[B + K] with S_K the sum of the K
    largest survivals (fp64, sequential over the sorted values); K ranges over
    0 .. min(B*N, S - 1 - B); the smallest K of the largest objective wins.

    Returns k (int), objective (fp64), objectives [fp64 per K].
    Pins: brute force over all prefix-closed admission sets on tiny inputs; a flat
    SPS admits every candidate; an SPS that is zero past a capacity never exceeds
    it; a jagged SPS whose first local maximum is not the global one.
    """
    s = np.asarray(survival, dtype=np.float32).astype(np.float64)
    Bq = s.shape[0] if B is None else int(B)
    flat = np.sort(s.ravel())[::-1]
    sps = np.asarray(sps, dtype=np.float64)
    kmax = min(flat.size, sps.size - 1 - Bq)
    if kmax < 0:
        raise ValueError("the SPS table does not reach the batch of B tokens")
    prefix = 0.0
    obj = np.empty(kmax + 1)
    for K in range(kmax + 1):
        if K > 0:
            prefix += flat[K - 1]
        obj[K] = (Bq + prefix) * sps[Bq + K]
    k = int(np.argmax(obj))                        # the first maximum: the smallest K
    return {"k": k, "objective": float(obj[k]), "objectives": obj}


# ---------------------------------------------------------------- next rows: confidence head

def confidence_head(hidden_bits, w1_bits, draft_tokens, anchor, w_bits, bias: float, tau) -> np.ndarray:
    """Per-position conditional acceptance probability [P2 §6: a linear projection
    of the backbone hidden state plus the Markov embedding, calibrated by a
    per-position temperature].

    hidden_bits [B*N, H] bf16 (row b*N + k, the stage-1 input); w1_bits [V, r] bf16;
    draft_tokens [B, N] target ids; anchor [B]; w_bits [H + r] bf16 (the first H
    weights act on the hidden state, the last r on the embedding); bias fp32;
    tau [N] fp32 > 0.  Position k of request b uses the embedding of its previous
    token (k = 0: the anchor, the same token stage 2 starts from):
        z = w[:H] . h[b*N + k] + w[H:] . W1[x_{k-1}] + bias        (fp64)
        c[b, k] = fp32(1 / (1 + exp(-z / tau[k])))
    Pins: w = 0 gives sigmoid(bias / tau) (0.5 at bias 0); logit(c) * tau does not
    depend on tau; x_k moves c[k+1] only and the anchor c[0] only; the logit is
    affine in h.
    """
    h = bf16_decode(hidden_bits)
    w = bf16_decode(w_bits)
    x = np.asarray(draft_tokens, dtype=np.int64)
    B, N = x.shape
    H = h.shape[1]
    w1 = np.asarray(w1_bits)
    tau = np.asarray(tau, dtype=np.float32).astype(np.float64)
    c = np.empty((B, N), dtype=np.float32)
    for b in range(B):
        for k in range(N):
            prev = int(anchor[b]) if k == 0 else int(x[b, k - 1])
            e = bf16_decode(w1[prev])
            z = float(w[:H] @ h[b * N + k]) + float(w[H:] @ e) + float(np.float32(bias))
            c[b, k] = np.float32(1.0 / (1.0 + math.exp(-z / tau[k])))
    return c
