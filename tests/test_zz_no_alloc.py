"""dspark_verify_noalloc (static scratch, no allocation) against dspark_verify (caller's
workspace): identical outputs, called through the C ABI, on two calls in a row with the
second one smaller (the scratch keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import draft_sampling_lossless_amd as dsl
from oracle import stages

from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _case(B, N, V, T, seed):
    g = np.random.default_rng(seed)
    proc = g.normal(0, 1.28, size=(B, N, V)).astype(np.float32)
    tgt = np.concatenate([proc, proc[:, -1:]], axis=1) + g.normal(0, 1.0, size=(B, N + 1, V))
    tgt = tgt.astype(np.float32)
    temp = np.full(B, T, np.float32)
    y = proc.astype(np.float64) / T
    m = y.max(axis=2)
    logz = (m + np.log(np.exp(y - m[..., None]).sum(axis=2))).astype(np.float32)
    tok = g.integers(0, V, size=(B, N)).astype(np.int32)
    tok[:, ::2] = proc[:, ::2].argmax(axis=2)          # some likely drafts, so some are accepted
    L = g.integers(0, N + 1, size=B).astype(np.int32)
    rid = np.arange(B, dtype=np.uint32) * 5 + 1
    return [dev(x) for x in (tgt, proc, logz, tok, L, temp, rid)]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.fixture(scope="module", autouse=True)
def _gpu(dspark_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_matches_workspace_entry_point():
    lib = dsl.load()
    assert lib.dspark_verify_noalloc_max_bytes() == 4 << 20
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # the second call is smaller, and a different batch: the scratch holds the first call's data
    for (B, N, V, T, seed) in [(200, 8, 8192, 1.0, 1), (3, 5, 4096, 0.7, 2)]:
        assert dsl.verify_workspace_size(B, N, V) <= (4 << 20)
        say(f"verify_noalloc B={B} N={N} V={V}")
        tgt, proc, logz, tok, L, temp, rid = _case(B, N, V, T, seed)
        outs = []
        for noalloc in (False, True):
            acc = torch.full((B,), -5, dtype=torch.int32, device="cuda")
            out = torch.full((B, N + 1), -5, dtype=torch.int32, device="cuda")
            alpha = torch.full((B, N), -5.0, dtype=torch.float32, device="cuda")
            common = [dsl.INPUT_LOGITS, _ptr(tgt), _ptr(proc), _ptr(logz), _ptr(tok), None, _ptr(L), _ptr(temp),
                      _ptr(rid), ctypes.c_uint64(0x1234), _ptr(acc), _ptr(out), _ptr(alpha), B, N, V, V]
            if noalloc:
                st = lib.dspark_verify_noalloc(*common, stream)
            else:
                ws = torch.empty(dsl.verify_workspace_size(B, N, V), dtype=torch.uint8, device="cuda")
                st = lib.dspark_verify(*common, _ptr(ws), ctypes.c_size_t(ws.numel()), stream)
            assert st == 0, lib.dspark_last_error().decode()
            outs.append((host(acc), host(out), host(alpha)))
        (a0, o0, p0), (a1, o1, p1) = outs
        assert np.array_equal(a0, a1) and np.array_equal(o0, o1)
        assert np.array_equal(p0.view(np.uint32), p1.view(np.uint32))
        assert (a0 >= 0).all() and (a0 <= host(L)).all()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = dsl.load()
    B, N, V = 4096, 16, 151936
    need = dsl.verify_workspace_size(B, N, V)
    assert need > (4 << 20)
    fake = ctypes.c_void_p(0x100000)
    st = lib.dspark_verify_noalloc(dsl.INPUT_LOGITS, fake, fake, fake, fake, None, None, fake, fake,
                                   ctypes.c_uint64(0), fake, fake, None, B, N, V, V, None)
    assert st == 2 and "scratch" in lib.dspark_last_error().decode()
