"""The C-ABI library loads, exports every declared symbol and validates its
arguments on the host (no GPU needed: every call here fails validation before
any kernel is launched)."""
import ctypes
import os
import re

import pytest

import draft_sampling_lossless_amd as dsl

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dspark.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x100000          # 16-byte aligned non-null address; never dereferenced here
FAKE_ODD = 0x100004      # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dspark_status|size_t|int|const char\s*\*)\s*(dspark_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_four_stages():
    names = declared_functions()
    for stage in ("dspark_draft_logits", "dspark_markov_sample", "dspark_verify", "dspark_admit"):
        assert stage in names


def test_library_exports_every_declared_symbol(dspark_lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(dspark_lib, name), name


def test_abi_version(dspark_lib):
    assert dsl.abi_version() == 6


def _err():
    return dsl.load().dspark_last_error().decode()


def test_admit_validation(dspark_lib):
    L = dsl.load()
    assert L.dspark_admit(None, 4, 4, 3, FAKE, FAKE, None) == INVALID and "cond_accept" in _err()
    assert L.dspark_admit(FAKE, 0, 4, 3, FAKE, FAKE, None) == INVALID
    assert L.dspark_admit(FAKE, 4, 65, 3, FAKE, FAKE, None) == UNSUPPORTED
    assert L.dspark_admit(FAKE, 1024, 64, 3, FAKE, FAKE, None) == UNSUPPORTED   # B*N > 16384
    assert L.dspark_admit(FAKE, 4, 4, -1, FAKE, FAKE, None) == INVALID


def _markov(**kw):
    a = dict(logits=FAKE, w1=FAKE, w2=FAKE, d2t=None, anchor=FAKE, temperature=FAKE, request_id=FAKE, seed=0,
             draft_tokens=FAKE, log_z=FAKE, B=4, N=8, V=1024, Vd=1024, r=16, workspace=FAKE,
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return dsl.load().dspark_markov_sample(*a.values())


def test_markov_validation(dspark_lib):
    assert _markov(B=0) == INVALID
    assert _markov(N=65) == UNSUPPORTED
    assert _markov(r=12) == INVALID
    assert _markov(r=264) == UNSUPPORTED
    assert _markov(V=1026, Vd=1026) == INVALID
    assert _markov(Vd=2048) == INVALID                        # Vd > V
    assert _markov(Vd=512) == INVALID and "d2t" in _err()     # reduced vocab needs d2t
    assert _markov(logits=FAKE_ODD) == INVALID and "aligned" in _err()
    assert _markov(workspace=None) == WORKSPACE
    need = dsl.markov_workspace_size(4, 8, 1024, 16)
    assert need > 0
    assert _markov(workspace_bytes=need - 1) == WORKSPACE and "too small" in _err()


def _verify(**kw):
    a = dict(kind=0, target=FAKE, draft=FAKE, draft_log_z=FAKE, draft_tokens=FAKE, inv_map=None, verify_len=None,
             temperature=FAKE, request_id=FAKE, seed=0, accepted=FAKE, out_tokens=FAKE, accept_prob=None, B=2, N=8, V=1024,
             Vd=1024, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return dsl.load().dspark_verify(*a.values())


def test_verify_validation(dspark_lib):
    assert _verify(kind=7) == INVALID
    assert _verify(B=70000) == UNSUPPORTED
    assert _verify(draft_log_z=None) == INVALID and "draft_log_z" in _err()
    assert _verify(Vd=512) == INVALID and "inv_map" in _err()
    assert _verify(target=FAKE_ODD) == INVALID
    need = dsl.verify_workspace_size(2, 8, 1024)
    assert need > 0
    assert _verify(workspace_bytes=need - 1) == WORKSPACE


def _markov_deferred(**kw):
    a = dict(logits=FAKE, w1=FAKE, w2=FAKE, anchor=FAKE, temperature=FAKE, request_id=FAKE, seed=0,
             draft_tokens=FAKE, log_z=FAKE, win_logit=FAKE, h_dot=None, w_e=None, conf_bias=0.0, tau=None,
             c_out=None, B=4, N=8, V=1024, Vd=1024, r=16, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return dsl.load().dspark_markov_sample_deferred(*a.values())


def _verify_deferred(**kw):
    a = dict(target=FAKE, draft_base=FAKE, draft_log_z=FAKE, win_logit=FAKE, draft_tokens=FAKE, anchor=FAKE,
             w1=FAKE, w2=FAKE, r=16, verify_len=None, temperature=FAKE, request_id=FAKE, seed=0, accepted=FAKE,
             out_tokens=FAKE, B=2, N=8, V=1024, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return dsl.load().dspark_verify_deferred(*a.values())


def test_deferred_validation(dspark_lib):
    assert _markov_deferred(Vd=512) == UNSUPPORTED and "target map" in _err()
    assert _markov_deferred(win_logit=None) == INVALID and "win_logit" in _err()
    assert _markov_deferred(h_dot=FAKE) == INVALID and "all given or all NULL" in _err()
    assert _markov_deferred(B=0) == INVALID
    assert _markov_deferred(workspace=None) == WORKSPACE
    assert _verify_deferred(win_logit=None) == INVALID and "win_logit" in _err()
    assert _verify_deferred(anchor=None) == INVALID and "anchor" in _err()
    assert _verify_deferred(r=12) == INVALID
    assert _verify_deferred(draft_log_z=None) == INVALID and "draft_log_z" in _err()
    need = dsl.verify_deferred_workspace_size(2, 8, 1024)
    assert need > dsl.verify_workspace_size(2, 8, 1024)
    assert _verify_deferred(workspace_bytes=need - 1) == WORKSPACE


def _context_kv(**kw):
    a = dict(aux=FAKE, fc_w=FAKE, fc_b=None, hnorm_w=FAKE, kv_w=FAKE, kv_b=FAKE, knorm_w=FAKE, positions=FAKE,
             slots=FAKE, k_cache=FAKE, v_cache=FAKE, num_ctx=16, H_in=256, H_d=128, L=2, nkv=2, hd=64,
             num_slots=64, eps=1e-6, theta=1e6, workspace=FAKE, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return dsl.load().dspark_context_kv(*a.values())


def test_context_kv_validation(dspark_lib):
    assert _context_kv(H_in=12) == INVALID
    assert _context_kv(hd=63) == INVALID
    assert _context_kv(hd=512) == UNSUPPORTED
    assert _context_kv(eps=-1.0) == INVALID
    assert _context_kv(theta=0.0) == INVALID
    assert _context_kv(num_ctx=0) == OK                     # empty: nothing enqueued
    assert _context_kv(slots=None) == INVALID and "slots" in _err()
    assert _context_kv(aux=FAKE_ODD) == INVALID and "aligned" in _err()
    assert _context_kv(workspace=None) == WORKSPACE
    need = dsl.context_kv_workspace_size(16, 128, 2, 2, 64)
    assert need > 0 and _context_kv(workspace_bytes=need - 1) == WORKSPACE


def test_draft_logits_and_rng_validation(dspark_lib):
    L = dsl.load()
    assert L.dspark_draft_logits(FAKE, FAKE, FAKE, 8, 12, 1024, None) == INVALID   # H % 8
    assert L.dspark_draft_logits(FAKE, FAKE, FAKE, -1, 16, 1024, None) == INVALID
    assert L.dspark_draft_logits(FAKE, FAKE, FAKE, 0, 16, 1024, None) == OK        # empty: nothing enqueued
    assert L.dspark_draft_logits(None, FAKE, FAKE, 8, 16, 1024, None) == INVALID
    assert L.dspark_philox_blocks(FAKE, 0, FAKE, -1, None) == INVALID
    assert L.dspark_philox_blocks(FAKE, 0, FAKE, 0, None) == OK
    assert L.dspark_race_exponentials(0, 0, 0, 0, None, 5, None) == INVALID
    assert L.dspark_build_inverse_map(FAKE, 10, 5, FAKE, None) == INVALID


def test_workspace_sizes_at_full_shapes(dspark_lib):
    # the batched shapes of the pages' Qwen3-8B setting
    assert 0 < dsl.markov_workspace_size(256, 16, 151936, 256) < 64 << 20
    assert 0 < dsl.verify_workspace_size(256, 16, 151936) < 64 << 20
    assert dsl.markov_workspace_size(0, 8, 1024, 16) == 0
