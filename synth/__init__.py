"""Seeded synthetic inputs for the DSpark draft-sample-verify path.

This module only draws random numbers and quantises them to the input dtypes
(bf16 bit patterns, fp32, int32, int64).  It holds none of the method's
arithmetic: no logits, no sampling, no probabilities.  Both the CPU oracle
side (tests, cpu baseline) and the GPU side (tests, bench) take their inputs
from here, so that they see identical values.

Every large array is generated in row blocks, each block from its own
``numpy.random.default_rng([seed, tag, block])`` stream.  A test can therefore
regenerate any subset of rows (say, the handful of requests it checks against
the oracle at full vocabulary size) without drawing the rest.

Workload shapes follow the Qwen3-8B setting the pages describe (hidden 4096,
vocabulary 151936, Markov rank 64 or 256, N = 8 or 16 draft positions; a
32000-entry reduced draft vocabulary mapped by an int64 offset table).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "bf16_bits", "bf16_to_f32",
    "rows_normal_bf16", "rows_normal_f32", "hidden_bf16", "lm_head_bf16",
    "markov_w1_bf16", "markov_w2_bf16", "request_params", "target_noise",
    "synthetic_base_logits", "d2t_offsets", "confidence", "generate",
]

# stream tags: one per array kind, so streams never overlap
_TAG = {
    "hidden": 1, "lm_head": 2, "w1": 3, "w2": 4, "req": 5, "noise": 6,
    "base": 7, "d2t": 8, "conf": 9,
}
_BLOCK_ROWS = 1024


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes plus the per-request value recipe."""

    name: str
    B: int                 # requests
    N: int                 # draft positions per request
    H: int                 # backbone hidden size
    V: int                 # target vocabulary
    Vd: int                # draft vocabulary (== V unless reduced)
    r: int                 # Markov rank
    temperatures: Tuple[float, ...]   # per-request choice set
    sigmas: Tuple[float, ...]         # per-request target-noise std choice set
    K: Optional[int] = None           # admission budget (None -> B*N)
    weight_std: float = 0.02
    seed: int = 1000                  # input generator seed
    philox_seed: int = 0              # sampling RNG seed
    note: str = ""

    @property
    def M(self) -> int:
        return self.B * self.N

    @property
    def budget(self) -> int:
        return self.B * self.N if self.K is None else self.K


WORKLOADS: Dict[str, Workload] = {
    # tiny CPU-checkable case; "fp32" inputs are drawn in fp32 and rounded to
    # bf16 so both sides see the same values
    "tiny": Workload("tiny", B=1, N=8, H=256, V=1024, Vd=1024, r=16,
                     temperatures=(1.0,), sigmas=(1.0,), seed=1000,
                     note="B=1 N=8 H=256 V=1024 r=16, T=1 (and T=0 run)"),
    "qwen3_8b_single": Workload(
        "qwen3_8b_single", B=1, N=8, H=4096, V=151936, Vd=151936, r=64,
        temperatures=(1.0,), sigmas=(1.0,), seed=1001,
        note="Qwen3-8B-shaped single request, B=1 N=8 r=64, T=1, sigma=1"),
    "batched": Workload(
        "batched", B=64, N=8, H=4096, V=151936, Vd=151936, r=256,
        temperatures=(0.7,), sigmas=(0.5, 1.0, 2.0), seed=1002,
        note="B=64 N=8 r=256, T=0.7, sigma per request from {0.5,1,2}"),
    "admission": Workload(
        "admission", B=256, N=16, H=4096, V=151936, Vd=151936, r=256,
        temperatures=(1.0,), sigmas=(1.0,), K=1024, seed=1003,
        note="B=256 N=16 r=256, K=1024 pooled admission, T=1, sigma=1"),
    "reduced_vocab": Workload(
        "reduced_vocab", B=512, N=8, H=4096, V=151936, Vd=32000, r=64,
        temperatures=(0.0, 0.7, 1.0), sigmas=(1.0,), seed=1004,
        note="B=512 N=8 Vd=32000 -> V=151936 via d2t, r=64, T from {0,0.7,1}"),
}


def get(name: str, **overrides) -> Workload:
    """Workload by name, optionally with fields replaced (e.g. a smaller B)."""
    w = WORKLOADS[name]
    if overrides:
        d = dict(w.__dict__)
        d.update(overrides)
        w = Workload(**d)
    return w


# ---------------------------------------------------------------- quantising

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- row-block streams

def _rng(seed: int, tag: str, block: int) -> np.random.Generator:
    return np.random.default_rng([seed, _TAG[tag], block])


def rows_normal_f32(seed: int, tag: str, n_rows: int, n_cols: int, std: float,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """N(0, std) fp32 matrix [n_rows, n_cols], drawn in blocks of 1024 rows.

    With ``rows`` given, only those rows are returned (same values as in the
    full matrix); only the blocks that hold them are drawn.
    """
    want = np.arange(n_rows) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(want), n_cols), dtype=np.float32)
    blocks = np.unique(want // _BLOCK_ROWS)
    for blk in blocks:
        lo = int(blk) * _BLOCK_ROWS
        hi = min(n_rows, lo + _BLOCK_ROWS)
        g = _rng(seed, tag, int(blk))
        vals = g.standard_normal((hi - lo, n_cols), dtype=np.float32)
        if std != 1.0:
            vals *= np.float32(std)
        sel = np.nonzero((want >= lo) & (want < hi))[0]
        out[sel] = vals[want[sel] - lo]
    return out


def rows_normal_bf16(seed: int, tag: str, n_rows: int, n_cols: int, std: float,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    return bf16_bits(rows_normal_f32(seed, tag, n_rows, n_cols, std, rows))


# ---------------------------------------------------------------- arrays

def hidden_bf16(w: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Backbone hidden states h ~ N(0,1), [B*N, H] bf16 bits; row m = b*N + i."""
    return rows_normal_bf16(w.seed, "hidden", w.M, w.H, 1.0, rows)


def lm_head_bf16(w: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Draft LM head W ~ N(0, 0.02), [Vd, H] bf16 bits (one row per draft token)."""
    return rows_normal_bf16(w.seed, "lm_head", w.Vd, w.H, w.weight_std, rows)


def markov_w1_bf16(w: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Markov embedding W1 ~ N(0, 0.02), [V, r] bf16 bits (indexed by target id)."""
    return rows_normal_bf16(w.seed, "w1", w.V, w.r, w.weight_std, rows)


def markov_w2_bf16(w: Workload, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Markov projection W2 ~ N(0, 0.02), [Vd, r] bf16 bits (one row per draft token)."""
    return rows_normal_bf16(w.seed, "w2", w.Vd, w.r, w.weight_std, rows)


def request_params(w: Workload) -> Dict[str, np.ndarray]:
    """Per-request scalars: anchor token, temperature, target-noise sigma, id."""
    g = _rng(w.seed, "req", 0)
    anchor = g.integers(0, w.V, size=w.B, dtype=np.int64).astype(np.int32)
    temps = np.asarray(w.temperatures, dtype=np.float32)
    sig = np.asarray(w.sigmas, dtype=np.float32)
    temperature = temps[g.integers(0, len(temps), size=w.B)]
    sigma = sig[g.integers(0, len(sig), size=w.B)]
    return {
        "anchor": anchor,
        "temperature": temperature.astype(np.float32),
        "sigma": sigma.astype(np.float32),
        "request_id": np.arange(w.B, dtype=np.uint32),
    }


def target_noise(w: Workload, requests: Optional[Sequence[int]] = None) -> np.ndarray:
    """Standard-normal noise eps [len(requests), N+1, V] fp32, one stream per request."""
    reqs = np.arange(w.B) if requests is None else np.asarray(requests, dtype=np.int64)
    out = np.empty((len(reqs), w.N + 1, w.V), dtype=np.float32)
    for n, b in enumerate(reqs):
        out[n] = _rng(w.seed, "noise", int(b)).standard_normal((w.N + 1, w.V), dtype=np.float32)
    return out


def synthetic_base_logits(w: Workload, requests: Optional[Sequence[int]] = None) -> np.ndarray:
    """Stand-in draft base logits [len(requests), N, Vd] fp32, one stream per request.

    Drawn N(0, std * sqrt(H)) -- the spread that N(0,1) hidden states times an
    N(0, std) LM head give -- so that the sampling stages can be checked at full
    vocabulary size without the dense contraction in front of them.
    """
    reqs = np.arange(w.B) if requests is None else np.asarray(requests, dtype=np.int64)
    s = np.float32(w.weight_std * np.sqrt(w.H))
    out = np.empty((len(reqs), w.N, w.Vd), dtype=np.float32)
    for n, b in enumerate(reqs):
        out[n] = _rng(w.seed, "base", int(b)).standard_normal((w.N, w.Vd), dtype=np.float32) * s
    return out


def d2t_offsets(w: Workload) -> Optional[np.ndarray]:
    """Reduced-vocab offset table d2t [Vd] int64 (target id = j + d2t[j]).

    A random injective map: the first Vd entries of a random permutation of the
    target vocabulary.  None when the draft vocabulary is the target vocabulary.
    """
    if w.Vd == w.V:
        return None
    g = _rng(w.seed, "d2t", 0)
    image = g.permutation(w.V)[: w.Vd].astype(np.int64)
    return image - np.arange(w.Vd, dtype=np.int64)


def confidence(w: Workload) -> np.ndarray:
    """Per-position conditional acceptance c [B, N] fp32 in (0, 1).

    sigmoid(N(1.5, 1)) made monotone non-increasing along the block by a
    running minimum.
    """
    g = _rng(w.seed, "conf", 0)
    z = g.normal(1.5, 1.0, size=(w.B, w.N))
    c = 1.0 / (1.0 + np.exp(-z))
    c = np.minimum.accumulate(c, axis=1)
    return c.astype(np.float32)


def sps_table(max_tokens: int, seed: int = 0, tile: int = 64, knee: int = 256) -> np.ndarray:
    """Synthetic steps-per-second curve of a target engine, sps[n] for a batch of n
    tokens (n = 0 .. max_tokens).  The pages give no table, only its shape: flat
    while the forward pass is bandwidth-bound, then falling once it is
    compute-bound, jagged at kernel tile boundaries.  Step time here: 10 ms up to
    the knee, then +1.2 ms per extra tile of `tile` tokens, times a seeded +-3%
    ripple per tile.  Returned as float32."""
    n = np.arange(max_tokens + 1)
    tiles = np.maximum(0, np.ceil(n / tile) * tile - knee) / tile
    ripple = 1.0 + 0.03 * np.random.default_rng([seed, 77]).uniform(-1, 1, size=int(np.ceil((max_tokens + 1) / tile)) + 1)
    step_ms = (10.0 + 1.2 * tiles) * ripple[n // tile]
    return (1000.0 / step_ms).astype(np.float32)


def generate(w: Workload, big: bool = True) -> Dict[str, object]:
    """All inputs of a workload (weights included when ``big``)."""
    out: Dict[str, object] = {"workload": w}
    out.update(request_params(w))
    out["d2t"] = d2t_offsets(w)
    out["confidence"] = confidence(w)
    out["K"] = w.budget
    if big:
        out["hidden"] = hidden_bf16(w)
        out["lm_head"] = lm_head_bf16(w)
        out["w1"] = markov_w1_bf16(w)
        out["w2"] = markov_w2_bf16(w)
    return out
