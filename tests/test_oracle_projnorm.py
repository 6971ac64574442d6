"""Pins of the oracle's QK RMSNorm and projection-then-compression (the
series computed from hidden states by learned projections, DeepSeek-V4
technical report page, «CSA: сжать в 4 раза и выбрать top-k», step 1;
queries and KV entries normalised by RMSNorm, same page, «Muon и борьба с
нестабильностью»). Readings pinned here: the norm covers all D dims of a
vector, y = x * gamma / sqrt(mean(x^2) + eps), and an entry is normalised
after pooling and before its RoPE rotation."""
import numpy as np
import pytest

import oracle


def test_rmsnorm_alternating_signs_closed_form():
    # |x_c| = a for every c: mean(x^2) = a^2, so with eps = 0 the output is
    # sign(x_c) * gamma_c whatever a is
    D = 64
    s = np.where(np.arange(D) % 3 == 0, -1.0, 1.0).astype(np.float32)
    gamma = np.linspace(0.5, 2.0, D).astype(np.float32)
    for a in (3.5, 1e-3, 1024.0):
        y = oracle.rmsnorm((a * s)[None], gamma, eps=0.0)
        assert np.allclose(y[0], s * gamma.astype(np.float64), rtol=1e-15, atol=0)


def test_rmsnorm_one_hot_closed_form():
    # x = a e_j: mean(x^2) = a^2 / D, y_j = sign(a) sqrt(D) gamma_j, others 0
    D, j = 576, 77
    x = np.zeros((2, D), np.float32)
    x[0, j], x[1, j] = 5.0, -0.25
    gamma = np.full(D, 1.5, np.float32)
    y = oracle.rmsnorm(x, gamma, eps=0.0)
    assert np.allclose(y[:, j], [np.sqrt(D) * 1.5, -np.sqrt(D) * 1.5], rtol=1e-15, atol=0)
    assert np.count_nonzero(y) == 2


def test_rmsnorm_mean_square_invariant():
    # gamma = 1: mean(y^2) = mean(x^2) / (mean(x^2) + eps)
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 576)).astype(np.float32) * np.array([[1e-4], [1e-3], [1], [10], [1e3]], np.float32)
    y = oracle.rmsnorm(x, np.ones(576, np.float32), eps=1e-6)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean(y ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-12, atol=0)


def _int_case(csa, seed, B=2, S=24, hidden=8, D=64, m=4):
    # small integers: every projected value is an exact small integer
    g = np.random.default_rng(seed)
    x = g.integers(-2, 3, (B, S, hidden)).astype(np.float32)
    w = g.integers(-1, 2, (4 if csa else 2, D, hidden)).astype(np.float32)
    ba = g.standard_normal((m, D)).astype(np.float32)
    bb = g.standard_normal((m, D)).astype(np.float32)
    series = [np.einsum("bsh,dh->bsd", x.astype(np.float64), w[i].astype(np.float64)) for i in range(len(w))]
    assert all(np.abs(s_).max() < 2 ** 24 for s_ in series)
    return x, w, ba, bb, [s_.astype(np.float32) for s_ in series]


@pytest.mark.parametrize("d_rope", [0, 32])
def test_projection_then_csa_pooling(d_rope):
    # the series X W_s^T (exact here) fed to the CSA pooling give the same
    # entries as the fused definition, bit for bit
    x, w, ba, bb, (ca, za, cb, zb) = _int_case(True, 11)
    got = oracle.project_compress(x, w, ba, bb, 4, d_rope=d_rope)
    want = oracle.csa_compress(ca, za, cb, zb, ba, bb, 4, d_rope=d_rope)
    assert np.array_equal(got, want)


def test_projection_then_hca_pooling():
    x, w, ba, _, (c, z) = _int_case(False, 12, S=32, m=8)
    got = oracle.project_compress(x, w, ba, None, 8, d_rope=16)
    assert np.array_equal(got, oracle.hca_compress(c, z, ba, 8, d_rope=16))


def test_identity_projection_reduces_to_compression():
    # hidden = D, W_c = I and W_z = 0: the series are the hidden states
    # themselves with uniform weights
    g = np.random.default_rng(13)
    B, S, D = 1, 16, 32
    x = g.standard_normal((B, S, D)).astype(np.float32)
    eye, zero = np.eye(D, dtype=np.float32), np.zeros((D, D), np.float32)
    ba = np.zeros((4, D), np.float32)
    got = oracle.project_compress(x, np.stack([eye, zero, eye, zero]), ba, ba, 4)
    # uniform softmax: entry i = mean of tokens 4(i-1) .. 4i+3 (entry 0: of 0..3)
    want = np.stack([x[0, max(0, 4 * i - 4):4 * i + 4].astype(np.float64).mean(axis=0) for i in range(S // 4)])
    assert np.allclose(got[0], want, rtol=1e-14, atol=1e-15)


def test_entry_norm_before_rope():
    # with a non-uniform gamma the order matters: the fused definition is
    # RMSNorm of the pooled entry, then the rotation of its last dims
    x, w, ba, bb, _ = _int_case(True, 14)
    gamma = np.linspace(0.25, 4.0, 64).astype(np.float32)
    plain = oracle.project_compress(x, w, ba, bb, 4)
    normed = oracle.project_compress(x, w, ba, bb, 4, gamma=gamma)
    assert np.allclose(normed, oracle.rmsnorm(plain.astype(np.float32), gamma), rtol=1e-6, atol=1e-7)
    roped = oracle.project_compress(x, w, ba, bb, 4, gamma=gamma, d_rope=32)
    N = plain.shape[1]
    want = np.stack([np.stack([oracle.rope(normed[b, i], 4 * i, 32) for i in range(N)]) for b in range(2)])
    assert np.allclose(roped, want, rtol=1e-12, atol=1e-12)
    # rotating before normalising would differ
    pre = np.stack([np.stack([oracle.rope(plain[b, i], 4 * i, 32) for i in range(N)]) for b in range(2)])
    assert not np.allclose(roped, oracle.rmsnorm(pre.astype(np.float32), gamma), rtol=1e-3, atol=1e-3)
