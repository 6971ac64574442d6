"""GPU check of indexer_topk_noalloc, the entry point that allocates
nothing (its scratch is a static device array): called through the C ABI, it
must give exactly what indexer_topk gives with a caller workspace, on two
calls in a row, the second smaller than the first (the scratch keeps the
first call's contents), and refuse a problem larger than its scratch before
launching anything."""
import ctypes

import numpy as np
import pytest

import synth
from util import dev, host

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")


def _case(seed, B, T, N, k, HI=64, dI=128, m=4):
    g = synth.rng(seed)
    qc, qs = csk.mxfp4_quantize(dev(synth.normal(g, (B, T, HI, dI))))
    kc, ks = csk.mxfp4_quantize(dev(synth.normal(g, (B, N, dI))))
    w = dev(synth.normal(g, (B, T, HI), 1.0 / HI))
    q_pos = dev(np.full((B, T), m * N - 1, np.int32) - g.integers(0, 9, (B, T)).astype(np.int32))
    ne = dev(np.full(B, N, np.int32))
    return dict(q=qc, q_scale=qs, w=w, kk=kc, k_scale=ks, q_pos=q_pos, n_entries=ne, m=m, k=k)


def _noalloc_c(c):
    """indexer_topk_noalloc called directly through the C ABI."""
    L = csk.lib()
    B, T, HI = c["w"].shape
    k = c["k"]
    idx = torch.full((B, T, k), -9, dtype=torch.int32, device="cuda")
    sc = torch.full((B, T, k), 7.0, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.indexer_topk_noalloc(p(c["q"]), p(c["q_scale"]), p(c["w"]), p(c["kk"]), p(c["k_scale"]), p(c["q_pos"]),
                                p(c["n_entries"]), B, T, HI, c["q"].shape[-1] * 2, c["kk"].shape[1], c["m"], k,
                                csk.CSK_MXFP4, csk.CSK_F32, p(idx), p(sc),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.csk_last_error().decode()
    return idx, sc


def test_noalloc_matches_workspace_call_twice():
    # a long filtered decode problem, then a smaller one of short rows
    for seed, B, T, N, k in ((901, 4, 1, 100000, 2048), (902, 2, 5, 5000, 256)):
        c = _case(seed, B, T, N, k)
        want_idx, want_sc = csk.indexer_topk(c["q"], c["w"], c["kk"], c["q_pos"], c["n_entries"], c["m"], k,
                                             q_scale=c["q_scale"], k_scale=c["k_scale"])
        got_idx, got_sc = _noalloc_c(c)
        torch.cuda.synchronize()
        assert torch.equal(got_idx, want_idx), (seed, "idx")
        assert torch.equal(got_sc.view(torch.int32), want_sc.view(torch.int32)), (seed, "scores")
        assert int((host(got_idx) >= 0).sum()) == B * T * k


def test_noalloc_refuses_a_problem_past_its_scratch():
    L = csk.lib()
    B, T, HI, dI, N, k = 64, 1, 64, 128, 262144, 2048
    need = L.indexer_topk_workspace_size(B, T, HI, dI, N, k, csk.CSK_MXFP4)
    assert need > (32 << 20)
    fake = ctypes.c_void_p(4096)
    rc = L.indexer_topk_noalloc(fake, fake, fake, fake, fake, fake, fake, B, T, HI, dI, N, 4, k, csk.CSK_MXFP4,
                                csk.CSK_F32, fake, fake, None)
    assert rc == -3 and b"scratch" in L.csk_last_error()
