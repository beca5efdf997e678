"""Helpers for the GPU parity tests: device upload and the comparison rules.

Comparison rules (the parity bar of each stage):
  * integer / index outputs (tokens, accepted counts, admission): bit-exact,
    except a stochastic decision taken at a near-tie, which is counted and must
    be rare (see compare_markov / compare_verify);
  * float outputs: an explicit tolerance, written at the call.
"""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> device tensor (bf16 bit patterns and uint32 travel as int16 / int32)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    elif x.dtype == np.uint32:
        x = x.view(np.int32)
    t = torch.from_numpy(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


# every Markov comparison of the session: (label, positions compared, near-tie mismatches);
# written out at the end of the session (tests/conftest.py) as the residual mismatch rate
MARKOV_RECORD = []


def compare_markov(gpu_tok, gpu_proc, gpu_logz, ref, gap_tol=1e-2, proc_rtol=1e-5, logz_rtol=2e-5, label=""):
    """Compare stage-2 outputs position by position, teacher-forced.

    ``ref`` must be the oracle run with teacher=gpu_tok: its step i then starts from
    the GPU's token i-1, so every position stays comparable after a disagreement.
    Processed logits and log Z must match at every position.  A token may differ only
    at a near-tie of the oracle's keys: the oracle's top-2 gap is <= gap_tol AND the
    GPU's token has an oracle key within gap_tol of the best one (it was one of the
    near-tied candidates).  Such mismatches are counted; at most max(1, checked // 50)
    are allowed.  Returns (checked, near_ties).
    """
    assert "teacher_deficit" in ref, "compare_markov needs the oracle run teacher-forced on the GPU tokens"
    checked, near = 0, 0
    B, N = ref["tokens"].shape
    for b in range(B):
        for i in range(N):
            p_ref = ref["processed"][b, i].astype(np.float64)
            p_gpu = gpu_proc[b, i].astype(np.float64)
            err = np.abs(p_gpu - p_ref) / np.maximum(1.0, np.abs(p_ref))
            assert err.max() <= proc_rtol, f"processed logits b={b} i={i}: rel err {err.max():.3g}"
            lz_r, lz_g = float(ref["logZ"][b, i]), float(gpu_logz[b, i])
            assert abs(lz_g - lz_r) <= logz_rtol * max(1.0, abs(lz_r)), f"log Z b={b} i={i}: {lz_g} vs {lz_r}"
            checked += 1
            if gpu_tok[b, i] != ref["tokens"][b, i]:
                gap, deficit = ref["gap"][b, i], ref["teacher_deficit"][b, i]
                assert gap <= gap_tol and deficit <= gap_tol, (
                    f"token mismatch b={b} i={i}: gpu {gpu_tok[b, i]} oracle {ref['tokens'][b, i]} "
                    f"(oracle top-2 gap {gap:.4g}, gpu token {deficit:.4g} below the best key)")
                near += 1
    assert near <= max(1, checked // 50), f"{near} near-tie mismatches in {checked} positions"
    MARKOV_RECORD.append((label, checked, near))
    return checked, near


def compare_verify(gpu_acc, gpu_out, ref, exact: bool, margin_tol=1e-5):
    """Compare stage-3 outputs.  exact=True: bit-for-bit.  Otherwise a request
    may differ only if one of its acceptance tests or its race was a near-tie
    (relative margin <= margin_tol).  Returns the number of near-tie requests."""
    near = 0
    for b in range(len(gpu_acc)):
        same = gpu_acc[b] == ref["accepted"][b] and np.array_equal(gpu_out[b], ref["out_tokens"][b])
        if same:
            continue
        assert not exact, (f"request {b}: gpu accepted={gpu_acc[b]} out={gpu_out[b].tolist()} vs oracle "
                           f"accepted={ref['accepted'][b]} out={ref['out_tokens'][b].tolist()}")
        m_acc = ref["accept_margins"][b]
        worst = min(m_acc) if m_acc else np.inf
        assert min(worst, ref["race_margin"][b]) <= margin_tol, (
            f"request {b} differs without a near-tie: gpu {gpu_acc[b]} {gpu_out[b].tolist()} vs oracle "
            f"{ref['accepted'][b]} {ref['out_tokens'][b].tolist()} (margins {m_acc}, race {ref['race_margin'][b]})")
        near += 1
    return near
