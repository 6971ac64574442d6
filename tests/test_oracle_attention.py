"""Pins for the oracle's sparse (CSA) and dense (HCA) attention."""
import numpy as np
import pytest

import oracle
import synth


def _rope_complex(x, pos, d_rope, base=10000.0):
    x = np.asarray(x, np.float64).copy()
    D = x.shape[-1]
    j = np.arange(d_rope // 2)
    ang = np.asarray(pos, np.float64)[..., None] * np.power(base, -2.0 * j / d_rope)
    z = (x[..., D - d_rope::2] + 1j * x[..., D - d_rope + 1::2]) * np.exp(1j * ang)
    x[..., D - d_rope::2], x[..., D - d_rope + 1::2] = z.real, z.imag
    return x


def test_hca_m1_no_window_is_textbook_causal_attention():
    # With m' = 1, no window and no sink, compress + dense attention is plain
    # causal softmax attention with RoPE on q and k, here computed by a naive
    # O(S^2) numpy routine with its own RoPE.
    g = synth.rng(41)
    S, H, D, dr = 37, 3, 32, 16
    c, z = synth.normal(g, (1, S, D)), synth.normal(g, (1, S, D))
    q = synth.normal(g, (1, S, H, D))
    kv = oracle.hca_compress(c, z, synth.normal(g, (1, D), 0.1), 1, d_rope=dr)
    kv32 = oracle.round_f32(kv)
    scale = 1.0 / np.sqrt(D)
    out, lse = oracle.dense_attn(q, np.arange(S, dtype=np.int32)[None], kv32, np.array([S], np.int32), 1,
                                 None, None, 0, None, D, dr, scale)
    K = _rope_complex(c[0].astype(np.float64), np.arange(S), dr)
    np.testing.assert_allclose(kv[0], K, atol=1e-12)
    Kf = kv32[0].astype(np.float64)
    for h in range(H):
        Q = _rope_complex(q[0, :, h].astype(np.float64), np.arange(S), dr)
        L = (Q @ Kf.T) * scale
        L[np.triu_indices(S, 1)] = -np.inf
        P = np.exp(L - L.max(axis=1, keepdims=True))
        ref = (P / P.sum(axis=1, keepdims=True)) @ Kf
        np.testing.assert_allclose(out[:, h], ref, atol=1e-12)
        ref_lse = L.max(axis=1) + np.log(P.sum(axis=1))
        np.testing.assert_allclose(lse[:, h], ref_lse, atol=1e-12)


def _problem(seed, B=2, T=5, H=4, D=32, N=30, S_w=16, dr=8):
    g = synth.rng(seed)
    q = synth.normal(g, (B, T, H, D))
    kv_c = synth.normal(g, (B, N, D))
    kv_w = synth.normal(g, (B, S_w, D))
    q_pos = np.stack([np.array([3, 40, 60, 100, 119], np.int32)] * B)[:, :T]
    w_pos0 = np.array([104, 100], np.int32)[:B]
    sink = synth.normal(g, (H,))
    return g, q, kv_c, kv_w, q_pos, w_pos0, sink


def test_sparse_with_all_visible_equals_dense():
    # CSA with k >= #visible selects every visible entry: identical to dense
    # attention over the same compressed cache.
    g, q, kv_c, kv_w, q_pos, w_pos0, sink = _problem(42)
    B, T, H, D = q.shape
    N, m, k = kv_c.shape[1], 4, 40
    n_entries = np.array([N, 21], np.int32)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            vis = [i for i in range(n_entries[b]) if m * (i + 1) - 1 <= q_pos[b, t]]
            idx[b, t, :len(vis)] = vis
    a = oracle.sparse_attn(q, q_pos, kv_c, idx, kv_w, w_pos0, 8, sink, 24, 8, 0.2)
    d = oracle.dense_attn(q, q_pos, kv_c, n_entries, m, kv_w, w_pos0, 8, sink, 24, 8, 0.2)
    np.testing.assert_allclose(a[0], d[0], atol=1e-12)
    np.testing.assert_allclose(a[1], d[1], atol=1e-12)
    # the order of idx does not matter
    perm = idx[..., ::-1].copy()
    p = oracle.sparse_attn(q, q_pos, kv_c, perm, kv_w, w_pos0, 8, sink, 24, 8, 0.2)
    np.testing.assert_allclose(p[0], a[0], atol=1e-12)


def test_zero_query_and_single_candidate_closed_forms():
    g, q, kv_c, kv_w, q_pos, w_pos0, sink = _problem(43, B=1, T=1)
    D = q.shape[-1]
    q0 = np.zeros_like(q)
    idx = np.array([[[2, 5, 7, -1]]], np.int32)
    q_pos = np.array([[1000]], np.int32)
    out, lse = oracle.sparse_attn(q0, q_pos, kv_c, idx, None, None, 0, sink, D, 8, 0.3)
    V = kv_c[0, [2, 5, 7]].astype(np.float64)
    for h in range(q.shape[2]):
        ref = V.sum(axis=0) / (3 + np.exp(np.float64(sink[h])))          # q = 0: all logits 0
        np.testing.assert_allclose(out[0, h], ref, atol=1e-13)
        assert abs(lse[0, h] - np.log(3 + np.exp(np.float64(sink[h])))) < 1e-13
    idx1 = np.array([[[5]]], np.int32)
    out, lse = oracle.sparse_attn(q, q_pos, kv_c, idx1, None, None, 0, sink, D, 8, 0.3)
    for h in range(q.shape[2]):
        l = 0.3 * (_rope_complex(q[0, 0, h], 1000, 8) @ kv_c[0, 5].astype(np.float64))
        p = np.exp(l) / (np.exp(l) + np.exp(np.float64(sink[h])))
        np.testing.assert_allclose(out[0, h], p * kv_c[0, 5].astype(np.float64), atol=1e-13)
    # no candidate and no sink: output 0, lse -inf
    out, lse = oracle.sparse_attn(q, q_pos, kv_c, np.full((1, 1, 2), -1, np.int32), None, None, 0, None, D, 8, 0.3)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_window_membership_and_sink_limit():
    # The window holds tokens [p-W+1, p] present in the buffer; a sink of
    # -1e30 is no sink at all.
    g, q, kv_c, kv_w, q_pos, w_pos0, sink = _problem(44, B=1, T=1)
    B, T, H, D = q.shape
    q_pos = np.array([[110]], np.int32)              # buffer holds positions 104..119
    W = 4                                            # -> tokens 107..110 = rows 3..6
    empty = np.full((1, 1, 1), -1, np.int32)
    out, _ = oracle.sparse_attn(q, q_pos, kv_c, empty, kv_w, w_pos0, W, None, D, 8, 0.25)
    for h in range(H):
        Q = _rope_complex(q[0, 0, h], 110, 8)
        K = kv_w[0, 3:7].astype(np.float64)
        l = 0.25 * (K @ Q)
        p = np.exp(l - l.max()); p /= p.sum()
        np.testing.assert_allclose(out[0, h], p @ K, atol=1e-13)
    a = oracle.sparse_attn(q, q_pos, kv_c, empty, kv_w, w_pos0, W, np.full(H, -1e30, np.float32), D, 8, 0.25)
    np.testing.assert_allclose(a[0], out, atol=1e-13)


def test_decode_equals_last_prefill_row():
    g, q, kv_c, kv_w, q_pos, w_pos0, sink = _problem(45, B=1, T=5)
    n_entries = np.array([30], np.int32)
    full, lse = oracle.dense_attn(q, q_pos, kv_c, n_entries, 4, kv_w, w_pos0, 16, sink, 32, 8, 0.2)
    last, lse1 = oracle.dense_attn(q[:, -1:], q_pos[:, -1:], kv_c, n_entries, 4, kv_w, w_pos0, 16, sink, 32, 8, 0.2)
    assert np.array_equal(full[-1:], last) and np.array_equal(lse[-1:], lse1)
    sub, _ = oracle.dense_attn(q, q_pos, kv_c, n_entries, 4, kv_w, w_pos0, 16, sink, 32, 8, 0.2,
                               rows=[(0, 4), (0, 1)])
    assert np.array_equal(sub[0], full[4]) and np.array_equal(sub[1], full[1])


def test_lse_matches_logsumexp():
    scipy_special = pytest.importorskip("scipy.special")
    g, q, kv_c, kv_w, q_pos, w_pos0, sink = _problem(46, B=1, T=1)
    D = q.shape[-1]
    idx = np.array([[[0, 3, 9, 11, 29]]], np.int32)
    q_pos = np.array([[500]], np.int32)
    out, lse = oracle.sparse_attn(q, q_pos, kv_c, idx, None, None, 0, sink, D, 8, 0.17)
    for h in range(q.shape[2]):
        Q = _rope_complex(q[0, 0, h], 500, 8)
        l = 0.17 * (kv_c[0, [0, 3, 9, 11, 29]].astype(np.float64) @ Q)
        assert abs(lse[0, h] - scipy_special.logsumexp(np.append(l, np.float64(sink[h])))) < 1e-12


def test_value_slice_is_the_leading_dv_dims():
    # With dv < D (the 512 + 64 latent layout: keys span all D dims, values
    # are the first dv of them) the closed forms pin which dims are values:
    # a single candidate gives p * K[:dv] and q = 0 gives sum K[:dv] / (n +
    # e^sink). The trailing dims differ from the leading ones here, so taking
    # the last dv dims, or all D, fails both.
    g, q, kv_c, kv_w, q_pos, w_pos0, sink = _problem(47, B=1, T=1, D=32)
    D, dv, dr = q.shape[-1], 20, 8
    q_pos = np.array([[900]], np.int32)
    idx1 = np.array([[[6]]], np.int32)
    out, lse = oracle.sparse_attn(q, q_pos, kv_c, idx1, None, None, 0, sink, dv, dr, 0.3)
    assert out.shape[-1] == dv
    K = kv_c[0, 6].astype(np.float64)
    assert np.abs(K[:dv] - K[D - dv:]).max() > 0.1
    for h in range(q.shape[2]):
        l = 0.3 * (_rope_complex(q[0, 0, h], 900, dr) @ K)
        p = np.exp(l) / (np.exp(l) + np.exp(np.float64(sink[h])))
        np.testing.assert_allclose(out[0, h], p * K[:dv], atol=1e-13)
        assert abs(lse[0, h] - np.logaddexp(l, np.float64(sink[h]))) < 1e-12
    idx = np.array([[[1, 4, 11, 17]]], np.int32)
    out, lse = oracle.sparse_attn(np.zeros_like(q), q_pos, kv_c, idx, None, None, 0, sink, dv, dr, 0.3)
    V = kv_c[0, [1, 4, 11, 17]].astype(np.float64)
    for h in range(q.shape[2]):
        ref = V[:, :dv].sum(axis=0) / (4 + np.exp(np.float64(sink[h])))
        np.testing.assert_allclose(out[0, h], ref, atol=1e-13)
    # dense attention slices the same way: one visible entry, no window
    dout, _ = oracle.dense_attn(np.zeros_like(q), np.array([[3]], np.int32), kv_c, np.array([30], np.int32), 4,
                                None, None, 0, None, dv, dr, 0.3)
    np.testing.assert_allclose(dout[0], np.broadcast_to(kv_c[0, 0, :dv].astype(np.float64), dout[0].shape),
                               atol=1e-13)
