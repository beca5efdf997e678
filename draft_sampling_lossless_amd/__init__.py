"""Python binding of libdspark.so, the MI355X DSpark draft-sample-verify path.

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity of torch tensors, then passes raw device pointers and the current
HIP stream to the C ABI (include/dspark.h).  All computation happens in the
library's HIP kernels.  PyTorch supplies device memory and streams; the
library itself never allocates.  If the library has not been built, every call
raises: there is no fallback.

Stages (names follow the C ABI):
  draft_logits    stage 1, base logits of every draft position
  markov_sample   stage 2, N-step low-rank Markov Gumbel-max loop (in place)
  admit           stage 4, survival by chain rule + pooled top-K admission
  verify          stage 3, lossless rejection-sampling verification
plus build_inverse_map (reduced vocabulary), philox_blocks and
race_exponentials (bit-exact access to the random numbers).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "load", "abi_version", "INPUT_LOGITS", "INPUT_PROBS", "DSparkError",
    "philox_blocks", "race_exponentials", "draft_logits", "markov_sample",
    "markov_workspace_size", "build_inverse_map", "verify", "verify_workspace_size", "verify_noalloc", "admit",
    "markov_sample_deferred", "verify_deferred", "verify_deferred_workspace_size",
    "context_kv", "context_kv_workspace_size",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspark.so")
INPUT_LOGITS, INPUT_PROBS = 0, 1
_STATUS = {0: "OK", 1: "INVALID", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}

_c_void_p, _c_int, _c_size, _c_u64, _c_u32, _c_i64 = (
    ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64)

_SIGS = {
    "dspark_abi_version": (_c_int, []),
    "dspark_last_error": (ctypes.c_char_p, []),
    "dspark_philox_blocks": (_c_int, [_c_void_p, _c_u64, _c_void_p, _c_i64, _c_void_p]),
    "dspark_race_exponentials": (_c_int, [_c_u64, _c_u32, _c_u32, _c_u32, _c_void_p, _c_i64, _c_void_p]),
    "dspark_draft_logits": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "dspark_markov_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "dspark_markov_sample": (_c_int, [_c_void_p] * 7 + [_c_u64, _c_void_p, _c_void_p] + [_c_int] * 5
                             + [_c_void_p, _c_size, _c_void_p]),
    "dspark_markov_check": (_c_int, [_c_void_p]),
    "dspark_markov_test_mode": (_c_int, [_c_int]),
    "dspark_build_inverse_map": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_void_p]),
    "dspark_verify_workspace_size": (_c_size, [_c_int, _c_int, _c_int]),
    "dspark_verify": (_c_int, [_c_int] + [_c_void_p] * 8 + [_c_u64, _c_void_p, _c_void_p, _c_void_p] + [_c_int] * 4
                      + [_c_void_p, _c_size, _c_void_p]),
    "dspark_verify_noalloc_max_bytes": (_c_size, []),
    "dspark_verify_noalloc": (_c_int, [_c_int] + [_c_void_p] * 8 + [_c_u64, _c_void_p, _c_void_p, _c_void_p]
                              + [_c_int] * 4 + [_c_void_p]),
    "dspark_verify_coupled_workspace_size": (_c_size, [_c_int, _c_int, _c_int]),
    "dspark_verify_coupled": (_c_int, [_c_void_p] * 6 + [_c_u64, _c_void_p, _c_void_p] + [_c_int] * 4
                              + [_c_void_p, _c_size, _c_void_p]),
    "dspark_draft_logits_conf": (_c_int, [_c_void_p] * 5 + [_c_int] * 3 + [_c_void_p]),
    "dspark_markov_sample_conf": (_c_int, [_c_void_p] * 7 + [_c_u64] + [_c_void_p] * 4 + [ctypes.c_float]
                                  + [_c_void_p] * 2 + [_c_int] * 5 + [_c_void_p, _c_size, _c_void_p]),
    "dspark_advance": (_c_int, [_c_void_p] * 4 + [_c_int] * 2 + [_c_void_p]),
    "dspark_markov_sample_deferred": (_c_int, [_c_void_p] * 6 + [_c_u64] + [_c_void_p] * 5 + [ctypes.c_float]
                                      + [_c_void_p] * 2 + [_c_int] * 5 + [_c_void_p, _c_size, _c_void_p]),
    "dspark_verify_deferred_workspace_size": (_c_size, [_c_int, _c_int, _c_int]),
    "dspark_context_kv_workspace_size": (_c_size, [_c_int] * 5),
    "dspark_context_kv": (_c_int, [_c_void_p] * 11 + [_c_int] * 6 + [_c_i64, ctypes.c_float, ctypes.c_float]
                          + [_c_void_p, _c_size, _c_void_p]),
    "dspark_verify_deferred": (_c_int, [_c_void_p] * 8 + [_c_int] + [_c_void_p] * 3 + [_c_u64, _c_void_p, _c_void_p]
                               + [_c_int] * 3 + [_c_void_p, _c_size, _c_void_p]),
    "dspark_choose_k": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "dspark_admit": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
}

_lib = None


class DSparkError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: DSPARK_ERR_{_STATUS.get(status, status)}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libdspark.so (built by ``python -m draft_sampling_lossless_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m draft_sampling_lossless_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def abi_version() -> int:
    return load().dspark_abi_version()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DSparkError(fn, status, load().dspark_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor], name: str, dtypes, device=None, shape=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_U32 = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)
_I64 = (torch.int64,)


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.numel() < need:
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {need} bytes")
    return ws


# ---------------------------------------------------------------- random numbers

def philox_blocks(counters: torch.Tensor, seed: int) -> torch.Tensor:
    """Philox4x32-10 of each [n, 4] counter row (int32 tensors holding uint32 bits)."""
    n = counters.shape[0]
    out = torch.empty((n, 4), dtype=counters.dtype, device=counters.device)
    _check("dspark_philox_blocks", load().dspark_philox_blocks(
        _ptr(counters, "counters", _U32, shape=(n, 4)), seed, out.data_ptr(), n, _stream(counters)))
    return out


def race_exponentials(seed: int, position: int, request_id: int, tag: int, n: int,
                      device="cuda") -> torch.Tensor:
    out = torch.empty(n, dtype=torch.float32, device=device)
    _check("dspark_race_exponentials", load().dspark_race_exponentials(
        seed, position, request_id, tag, out.data_ptr(), n, _stream(out)))
    return out


# ---------------------------------------------------------------- stage 1

def draft_logits(hidden: torch.Tensor, lm_head: torch.Tensor,
                 out: Optional[torch.Tensor] = None, w_h: Optional[torch.Tensor] = None,
                 h_dot: Optional[torch.Tensor] = None):
    """logits[m, j] = sum_h hidden[m, h] * lm_head[j, h]; hidden [M, H], lm_head [Vd, H] bf16.
    With w_h [H] bf16 (the confidence head's hidden-state weights, dspark_draft_logits_conf)
    also h_dot[m] = w_h . hidden[m]; returns (logits, h_dot) then."""
    M, H = hidden.shape
    Vd = lm_head.shape[0]
    dev = hidden.device
    if out is None:
        out = torch.empty((M, Vd), dtype=torch.float32, device=dev)
    if w_h is None:
        _check("dspark_draft_logits", load().dspark_draft_logits(
            _ptr(hidden, "hidden", _BF16, dev), _ptr(lm_head, "lm_head", _BF16, dev, (Vd, H)),
            _ptr(out, "out", _F32, dev, (M, Vd)), M, H, Vd, _stream(hidden)))
        return out
    if h_dot is None:
        h_dot = torch.empty(M, dtype=torch.float32, device=dev)
    _check("dspark_draft_logits_conf", load().dspark_draft_logits_conf(
        _ptr(hidden, "hidden", _BF16, dev), _ptr(lm_head, "lm_head", _BF16, dev, (Vd, H)),
        _ptr(w_h, "w_h", _BF16, dev, (H,)), _ptr(out, "out", _F32, dev, (M, Vd)),
        _ptr(h_dot, "h_dot", _F32, dev, (M,)), M, H, Vd, _stream(hidden)))
    return out, h_dot


# ---------------------------------------------------------------- stage 2

def markov_workspace_size(B: int, N: int, Vd: int, r: int) -> int:
    return int(load().dspark_markov_workspace_size(B, N, Vd, r))


def markov_sample(logits: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, d2t: Optional[torch.Tensor],
                  anchor: torch.Tensor, temperature: torch.Tensor, request_id: torch.Tensor, seed: int,
                  draft_tokens: Optional[torch.Tensor] = None, log_z: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, conf=None):
    """Stage 2 on logits [B, N, Vd] (base in, processed out, in place).  Returns (tokens, log_z).
    conf = (h_dot [B*N], w_e [r] bf16, bias, tau [N], c_out [B, N] or None): the fused
    confidence head (dspark_markov_sample_conf); returns (tokens, log_z, c) then."""
    B, N, Vd = logits.shape
    V, r = w1.shape
    dev = logits.device
    if draft_tokens is None:
        draft_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if log_z is None:
        log_z = torch.empty((B, N), dtype=torch.float32, device=dev)
    ws = _workspace(workspace, markov_workspace_size(B, N, Vd, r), dev)
    if conf is not None:
        h_dot, w_e, cbias, tau, c_out = conf
        if c_out is None:
            c_out = torch.empty((B, N), dtype=torch.float32, device=dev)
        _check("dspark_markov_sample_conf", load().dspark_markov_sample_conf(
            _ptr(logits, "logits", _F32, dev), _ptr(w1, "w1", _BF16, dev),
            _ptr(w2, "w2", _BF16, dev, (Vd, r)), _ptr(d2t, "d2t", _I64, dev, (Vd,)),
            _ptr(anchor, "anchor", _I32, dev, (B,)), _ptr(temperature, "temperature", _F32, dev, (B,)),
            _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
            _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)), _ptr(log_z, "log_z", _F32, dev, (B, N)),
            _ptr(h_dot, "h_dot", _F32, dev, (B * N,)), _ptr(w_e, "w_e", _BF16, dev, (r,)), float(cbias),
            _ptr(tau, "tau", _F32, dev, (N,)), _ptr(c_out, "c_out", _F32, dev, (B, N)),
            B, N, V, Vd, r, ws.data_ptr(), ws.numel(), _stream(logits)))
        return draft_tokens, log_z, c_out
    _check("dspark_markov_sample", load().dspark_markov_sample(
        _ptr(logits, "logits", _F32, dev), _ptr(w1, "w1", _BF16, dev),
        _ptr(w2, "w2", _BF16, dev, (Vd, r)), _ptr(d2t, "d2t", _I64, dev, (Vd,)),
        _ptr(anchor, "anchor", _I32, dev, (B,)), _ptr(temperature, "temperature", _F32, dev, (B,)),
        _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
        _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)), _ptr(log_z, "log_z", _F32, dev, (B, N)),
        B, N, V, Vd, r, ws.data_ptr(), ws.numel(), _stream(logits)))
    return draft_tokens, log_z


def markov_sample_deferred(logits: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, anchor: torch.Tensor,
                           temperature: torch.Tensor, request_id: torch.Tensor, seed: int,
                           draft_tokens: Optional[torch.Tensor] = None, log_z: Optional[torch.Tensor] = None,
                           win_logit: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           conf=None):
    """Stage 2 keeping the base logits (dspark_markov_sample_deferred): logits [B, N, V] are
    only read.  Returns (tokens, log_z, win_logit), plus c when conf = (h_dot, w_e, bias,
    tau, c_out or None) is given."""
    B, N, Vd = logits.shape
    V, r = w1.shape
    dev = logits.device
    if draft_tokens is None:
        draft_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if log_z is None:
        log_z = torch.empty((B, N), dtype=torch.float32, device=dev)
    if win_logit is None:
        win_logit = torch.empty((B, N), dtype=torch.float32, device=dev)
    ws = _workspace(workspace, markov_workspace_size(B, N, Vd, r), dev)
    h_dot = w_e = tau = c_out = None
    cbias = 0.0
    if conf is not None:
        h_dot, w_e, cbias, tau, c_out = conf
        if c_out is None:
            c_out = torch.empty((B, N), dtype=torch.float32, device=dev)
    _check("dspark_markov_sample_deferred", load().dspark_markov_sample_deferred(
        _ptr(logits, "logits", _F32, dev), _ptr(w1, "w1", _BF16, dev), _ptr(w2, "w2", _BF16, dev, (Vd, r)),
        _ptr(anchor, "anchor", _I32, dev, (B,)), _ptr(temperature, "temperature", _F32, dev, (B,)),
        _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
        _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)), _ptr(log_z, "log_z", _F32, dev, (B, N)),
        _ptr(win_logit, "win_logit", _F32, dev, (B, N)),
        _ptr(h_dot, "h_dot", _F32, dev, (B * N,)), _ptr(w_e, "w_e", _BF16, dev, (r,)), float(cbias),
        _ptr(tau, "tau", _F32, dev, (N,)), _ptr(c_out, "c_out", _F32, dev, (B, N)),
        B, N, V, Vd, r, ws.data_ptr(), ws.numel(), _stream(logits)))
    if conf is not None:
        return draft_tokens, log_z, win_logit, c_out
    return draft_tokens, log_z, win_logit


def markov_check() -> None:
    """Synchronise the current stream and raise DSparkError if a few-request Markov
    launch since the last check gave up on a grid barrier (its outputs are -1 / NaN)."""
    _check("dspark_markov_check", load().dspark_markov_check(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))


def markov_test_mode(mode: int) -> None:
    """Test hook: 0 normal, 1 single-workgroup few-request kernel, 2 forced barrier give-up."""
    _check("dspark_markov_test_mode", load().dspark_markov_test_mode(int(mode)))


def build_inverse_map(d2t: torch.Tensor, V: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    Vd = d2t.shape[0]
    if out is None:
        out = torch.empty(V, dtype=torch.int32, device=d2t.device)
    _check("dspark_build_inverse_map", load().dspark_build_inverse_map(
        _ptr(d2t, "d2t", _I64, shape=(Vd,)), Vd, V, _ptr(out, "inv_map", _I32, d2t.device, (V,)),
        _stream(d2t)))
    return out


# ---------------------------------------------------------------- stage 3

def verify_workspace_size(B: int, N: int, V: int) -> int:
    return int(load().dspark_verify_workspace_size(B, N, V))


def verify(input_kind: int, target: torch.Tensor, draft: torch.Tensor, draft_log_z: Optional[torch.Tensor],
           draft_tokens: torch.Tensor, inv_map: Optional[torch.Tensor], verify_len: Optional[torch.Tensor],
           temperature: Optional[torch.Tensor], request_id: torch.Tensor, seed: int,
           accepted: Optional[torch.Tensor] = None, out_tokens: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, accept_prob: Optional[torch.Tensor] = None,
           with_accept_prob: bool = False):
    """Stage 3.  target [B, N+1, V], draft [B, N, Vd].  Returns (accepted [B], out_tokens [B, N+1]),
    plus accept_prob [B, N] (NaN past verify_len) when it is passed or with_accept_prob is set."""
    B, N, Vd = draft.shape
    V = target.shape[2]
    dev = target.device
    if accepted is None:
        accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    if accept_prob is None and with_accept_prob:
        accept_prob = torch.empty((B, N), dtype=torch.float32, device=dev)
    ws = _workspace(workspace, verify_workspace_size(B, N, V), dev)
    _check("dspark_verify", load().dspark_verify(
        input_kind, _ptr(target, "target", _F32, dev, (B, N + 1, V)), _ptr(draft, "draft", _F32, dev),
        _ptr(draft_log_z, "draft_log_z", _F32, dev, (B, N)),
        _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)), _ptr(inv_map, "inv_map", _I32, dev, (V,)),
        _ptr(verify_len, "verify_len", _I32, dev, (B,)), _ptr(temperature, "temperature", _F32, dev, (B,)),
        _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
        _ptr(accepted, "accepted", _I32, dev, (B,)), _ptr(out_tokens, "out_tokens", _I32, dev, (B, N + 1)),
        _ptr(accept_prob, "accept_prob", _F32, dev, (B, N)),
        B, N, V, Vd, ws.data_ptr(), ws.numel(), _stream(target)))
    if accept_prob is not None:
        return accepted, out_tokens, accept_prob
    return accepted, out_tokens


def verify_deferred_workspace_size(B: int, N: int, V: int) -> int:
    return int(load().dspark_verify_deferred_workspace_size(B, N, V))


def verify_deferred(target: torch.Tensor, draft_base: torch.Tensor, draft_log_z: torch.Tensor,
                    win_logit: torch.Tensor, draft_tokens: torch.Tensor, anchor: torch.Tensor, w1: torch.Tensor,
                    w2: torch.Tensor, verify_len: Optional[torch.Tensor], temperature: torch.Tensor,
                    request_id: torch.Tensor, seed: int, accepted: Optional[torch.Tensor] = None,
                    out_tokens: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Stage 3 on kept base logits (dspark_verify_deferred).  draft_base [B, N, V]: each
    request's first-rejection row is recomputed in place.  Returns (accepted, out_tokens)."""
    B, N, V = draft_base.shape
    r = w1.shape[1]
    dev = target.device
    if accepted is None:
        accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    ws = _workspace(workspace, verify_deferred_workspace_size(B, N, V), dev)
    _check("dspark_verify_deferred", load().dspark_verify_deferred(
        _ptr(target, "target", _F32, dev, (B, N + 1, V)), _ptr(draft_base, "draft_base", _F32, dev, (B, N, V)),
        _ptr(draft_log_z, "draft_log_z", _F32, dev, (B, N)), _ptr(win_logit, "win_logit", _F32, dev, (B, N)),
        _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)), _ptr(anchor, "anchor", _I32, dev, (B,)),
        _ptr(w1, "w1", _BF16, dev), _ptr(w2, "w2", _BF16, dev, (V, r)), r,
        _ptr(verify_len, "verify_len", _I32, dev, (B,)), _ptr(temperature, "temperature", _F32, dev, (B,)),
        _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
        _ptr(accepted, "accepted", _I32, dev, (B,)), _ptr(out_tokens, "out_tokens", _I32, dev, (B, N + 1)),
        B, N, V, ws.data_ptr(), ws.numel(), _stream(target)))
    return accepted, out_tokens


# ---------------------------------------------------------------- context-KV precompute

def context_kv_workspace_size(num_ctx: int, H_d: int, L: int, nkv: int, hd: int) -> int:
    return int(load().dspark_context_kv_workspace_size(num_ctx, H_d, L, nkv, hd))


def context_kv(aux: torch.Tensor, fc_w: torch.Tensor, fc_b: Optional[torch.Tensor], hnorm_w: torch.Tensor,
               kv_w: torch.Tensor, kv_b: torch.Tensor, knorm_w: torch.Tensor, positions: torch.Tensor,
               slots: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, eps: float = 1e-6,
               rope_theta: float = 1e6, workspace: Optional[torch.Tensor] = None) -> None:
    """dspark_context_kv: writes the K/V of the M context tokens into k_cache / v_cache
    [L, num_slots, nkv, hd] (bf16) at their slots.  Weights are bf16 (or int16 bit
    patterns); positions int32 [M], slots int64 [M]."""
    M, H_in = aux.shape
    H_d = fc_w.shape[0]
    L, num_slots, nkv, hd = k_cache.shape
    dev = aux.device
    ws = _workspace(workspace, context_kv_workspace_size(M, H_d, L, nkv, hd), dev)
    kvr = L * 2 * nkv * hd
    _check("dspark_context_kv", load().dspark_context_kv(
        _ptr(aux, "aux", _BF16, dev, (M, H_in)), _ptr(fc_w, "fc_w", _BF16, dev, (H_d, H_in)),
        _ptr(fc_b, "fc_b", _BF16, dev, (H_d,)), _ptr(hnorm_w, "hnorm_w", _BF16, dev, (H_d,)),
        _ptr(kv_w, "kv_w", _BF16, dev, (kvr, H_d)), _ptr(kv_b, "kv_b", _BF16, dev, (kvr,)),
        _ptr(knorm_w, "knorm_w", _BF16, dev, (L, hd)), _ptr(positions, "positions", _I32, dev, (M,)),
        _ptr(slots, "slots", _I64, dev, (M,)), _ptr(k_cache, "k_cache", _BF16, dev),
        _ptr(v_cache, "v_cache", _BF16, dev, tuple(k_cache.shape)), M, H_in, H_d, L, nkv, hd, num_slots,
        float(eps), float(rope_theta), ws.data_ptr(), ws.numel(), _stream(aux)))


def verify_noalloc(input_kind: int, target: torch.Tensor, draft: torch.Tensor, draft_log_z: Optional[torch.Tensor],
                   draft_tokens: torch.Tensor, inv_map: Optional[torch.Tensor], verify_len: Optional[torch.Tensor],
                   temperature: Optional[torch.Tensor], request_id: torch.Tensor, seed: int,
                   accepted: torch.Tensor, out_tokens: torch.Tensor, accept_prob: Optional[torch.Tensor] = None):
    """verify() on the library's static scratch (dspark_verify_noalloc): the outputs must be
    passed in, nothing is allocated.  Calls that overlap on one device race."""
    B, N, Vd = draft.shape
    V = target.shape[2]
    dev = target.device
    _check("dspark_verify_noalloc", load().dspark_verify_noalloc(
        input_kind, _ptr(target, "target", _F32, dev, (B, N + 1, V)), _ptr(draft, "draft", _F32, dev),
        _ptr(draft_log_z, "draft_log_z", _F32, dev, (B, N)),
        _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)), _ptr(inv_map, "inv_map", _I32, dev, (V,)),
        _ptr(verify_len, "verify_len", _I32, dev, (B,)), _ptr(temperature, "temperature", _F32, dev, (B,)),
        _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
        _ptr(accepted, "accepted", _I32, dev, (B,)), _ptr(out_tokens, "out_tokens", _I32, dev, (B, N + 1)),
        _ptr(accept_prob, "accept_prob", _F32, dev, (B, N)), B, N, V, Vd, _stream(target)))


def verify_coupled_workspace_size(B: int, N: int, V: int) -> int:
    return int(load().dspark_verify_coupled_workspace_size(B, N, V))


def verify_coupled(target: torch.Tensor, draft_tokens: torch.Tensor, inv_map: Optional[torch.Tensor],
                   verify_len: Optional[torch.Tensor], temperature: torch.Tensor, request_id: torch.Tensor, seed: int,
                   Vd: Optional[int] = None, accepted: Optional[torch.Tensor] = None,
                   out_tokens: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gumbel-coupled verification.  target [B, N+1, V] logits.  Returns (accepted [B], out_tokens [B, N+1])."""
    B, N1, V = target.shape
    N = N1 - 1
    Vd = V if Vd is None else Vd
    dev = target.device
    if accepted is None:
        accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    ws = _workspace(workspace, verify_coupled_workspace_size(B, N, V), dev)
    _check("dspark_verify_coupled", load().dspark_verify_coupled(
        _ptr(target, "target", _F32, dev, (B, N + 1, V)), _ptr(draft_tokens, "draft_tokens", _I32, dev, (B, N)),
        _ptr(inv_map, "inv_map", _I32, dev, (V,)), _ptr(verify_len, "verify_len", _I32, dev, (B,)),
        _ptr(temperature, "temperature", _F32, dev, (B,)), _ptr(request_id, "request_id", _U32, dev, (B,)), seed,
        _ptr(accepted, "accepted", _I32, dev, (B,)), _ptr(out_tokens, "out_tokens", _I32, dev, (B, N + 1)),
        B, N, V, Vd, ws.data_ptr(), ws.numel(), _stream(target)))
    return accepted, out_tokens


def advance(accepted: torch.Tensor, out_tokens: torch.Tensor, anchor: torch.Tensor,
            emitted: Optional[torch.Tensor] = None) -> None:
    """End of a round: anchor[b] = out_tokens[b, accepted[b]]; emitted[b] += accepted[b] + 1."""
    B, N1 = out_tokens.shape
    dev = out_tokens.device
    _check("dspark_advance", load().dspark_advance(
        _ptr(accepted, "accepted", _I32, dev, (B,)), _ptr(out_tokens, "out_tokens", _I32, dev, (B, N1)),
        _ptr(anchor, "anchor", _I32, dev, (B,)), _ptr(emitted, "emitted", (torch.int64,), dev, (B,)),
        B, N1 - 1, _stream(out_tokens)))


def choose_k(survival: torch.Tensor, sps: torch.Tensor, k_out: Optional[torch.Tensor] = None,
             objective_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Throughput-optimal budget.  survival [B, N] float32, sps [S] float32.
    Returns (K [1] int32, objective [1] float64), both on the device."""
    B, N = survival.shape
    dev = survival.device
    if k_out is None:
        k_out = torch.empty(1, dtype=torch.int32, device=dev)
    if objective_out is None:
        objective_out = torch.empty(1, dtype=torch.float64, device=dev)
    _check("dspark_choose_k", load().dspark_choose_k(
        _ptr(survival, "survival", _F32, dev, (B, N)), B, N, _ptr(sps, "sps", _F32, dev), sps.numel(),
        _ptr(k_out, "k_out", _I32, dev, (1,)), _ptr(objective_out, "objective_out", (torch.float64,), dev, (1,)),
        _stream(survival)))
    return k_out, objective_out


# ---------------------------------------------------------------- stage 4

def admit(cond_accept: torch.Tensor, K: int, survival: Optional[torch.Tensor] = None,
          admit_len: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stage 4.  cond_accept [B, N] float32.  Returns (survival [B, N], admit_len [B])."""
    B, N = cond_accept.shape
    dev = cond_accept.device
    if survival is None:
        survival = torch.empty((B, N), dtype=torch.float32, device=dev)
    if admit_len is None:
        admit_len = torch.empty(B, dtype=torch.int32, device=dev)
    _check("dspark_admit", load().dspark_admit(
        _ptr(cond_accept, "cond_accept", _F32, dev), B, N, K, _ptr(survival, "survival", _F32, dev, (B, N)),
        _ptr(admit_len, "admit_len", _I32, dev, (B,)), _stream(cond_accept)))
    return survival, admit_len
