"""Pins for the oracle's lightning-indexer scores and top-k selection."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from exact import f32_round, fmaf


def _mx(x):
    return oracle.mxfp4_encode(x)


def test_single_head_reduces_to_relu_dot():
    # H_I = 1, w = 1: the score is ReLU of the exact q.k of the decoded MXFP4
    # operands. numpy's float64 dot of decoded values is exact here (products
    # of small dyadic numbers), so rounding it to float32 gives the reference.
    g = synth.rng(31)
    B, T, N, dI = 1, 3, 50, 128
    qc, qs = _mx(synth.normal(g, (B, T, 1, dI)))
    kc, ks = _mx(synth.normal(g, (B, N, dI)))
    w = np.ones((B, T, 1), np.float32)
    q_pos = np.array([[4 * N - 1, 7, 4 * N + 9]], np.int32)
    s, nv = oracle.indexer_scores(qc, w, kc, q_pos, np.array([N], np.int32), 4, q_scale=qs, k_scale=ks)
    qd = oracle.mxfp4_decode(qc, qs).astype(np.float64)
    kd = oracle.mxfp4_decode(kc, ks).astype(np.float64)
    assert nv.tolist() == [N, 2, N]
    for r in range(T):
        ref = np.maximum(np.float32(kd[0] @ qd[0, r, 0]), np.float32(0))
        assert np.array_equal(s[r, :nv[r]], ref[:nv[r]].astype(np.float32))
        assert np.all(np.isneginf(s[r, nv[r]:]))


def test_exact_dot_with_wide_scale_spread():
    # Tiles whose scales differ by ~40 binades: the oracle still returns the
    # exact sum rounded once; the reference is exact rational arithmetic.
    g = synth.rng(32)
    dI = 128
    for trial in range(30):
        q = synth.normal(g, (1, 1, 1, dI))
        k = synth.normal(g, (1, 1, dI))
        for t in range(4):
            q[..., 32 * t:32 * t + 32] *= np.float32(2.0 ** int(g.integers(-20, 20)))
            k[..., 32 * t:32 * t + 32] *= np.float32(2.0 ** int(g.integers(-20, 20)))
        qc, qs = _mx(q)
        kc, ks = _mx(k)
        s, _ = oracle.indexer_scores(qc, np.ones((1, 1, 1), np.float32), kc, np.array([[3]], np.int32),
                                     np.array([1], np.int32), 4, q_scale=qs, k_scale=ks)
        qd = oracle.mxfp4_decode(qc, qs)[0, 0, 0]
        kd = oracle.mxfp4_decode(kc, ks)[0, 0]
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qd, kd))
        ref = f32_round(exact)
        assert s[0, 0] == max(ref, np.float32(0.0)), trial


def test_head_sum_is_ascending_fma_chain():
    # The weighted ReLU head sum, checked with exact single-rounding fma
    # emulation over heads in ascending order; the fp32 path's per-head dot
    # is itself an fma chain over channels.
    g = synth.rng(33)
    B, T, HI, dI, N = 1, 2, 5, 16, 6
    q = synth.normal(g, (B, T, HI, dI))
    k = synth.normal(g, (B, N, dI))
    w = synth.normal(g, (B, T, HI))
    s, nv = oracle.indexer_scores(q, w, k, np.array([[23, 9]], np.int32), np.array([N], np.int32), 4)
    assert nv.tolist() == [6, 2]
    for t in range(T):
        for j in range(nv[t]):
            acc = np.float32(0.0)
            for h in range(HI):
                d = np.float32(0.0)
                for i in range(dI):
                    d = fmaf(q[0, t, h, i], k[0, j, i], d)
                acc = fmaf(w[0, t, h], max(d, np.float32(0.0)), acc)
            assert s[t, j] == acc


def test_visibility_counts():
    # An entry is visible once its last source token is in the past; at the
    # decode position ctx-1 all ctx/m entries are visible (131072 -> 32768).
    N = 40
    kf = np.zeros((1, N, 32), np.float32)
    qf = np.zeros((1, 6, 1, 32), np.float32)
    w = np.ones((1, 6, 1), np.float32)
    q_pos = np.array([[0, 2, 3, 4, 7, 159]], np.int32)
    _, nv = oracle.indexer_scores(qf, w, kf, q_pos, np.array([N], np.int32), 4)
    assert nv.tolist() == [0, 0, 1, 1, 2, 40]
    _, nv = oracle.indexer_scores(qf, w, kf, q_pos, np.array([25], np.int32), 4)
    assert nv.tolist() == [0, 0, 1, 1, 2, 25]
    ctx = 131072
    kf = np.zeros((1, ctx // 4, 32), np.float32)
    _, nv = oracle.indexer_scores(qf[:, :1], w[:, :1], kf, np.array([[ctx - 1]], np.int32),
                                  np.array([ctx // 4], np.int32), 4)
    assert nv.tolist() == [32768]


def test_topk_brute_force():
    g = synth.rng(34)
    for trial in range(40):
        N = int(g.integers(1, 300))
        k = int(g.integers(1, 64))
        sc = np.round(synth.normal(g, (1, N)) * 4) / 4      # many exact ties
        nv = np.array([int(g.integers(0, N + 1))], np.int32)
        idx, out = oracle.topk(sc.astype(np.float32), nv, k)
        n = nv[0]
        order = np.lexsort((np.arange(n), -sc[0, :n].astype(np.float64)))   # score desc, index asc
        sel = np.sort(order[:min(k, n)])
        assert idx[0, :len(sel)].tolist() == sel.tolist()
        assert np.all(idx[0, len(sel):] == -1)
        assert np.array_equal(out[0, :len(sel)], sc[0, sel].astype(np.float32))
        assert np.all(np.isneginf(out[0, len(sel):]))


def test_topk_degenerate_cases():
    # all equal: the lowest indices win; k >= n selects everything
    idx, _ = oracle.topk(np.zeros((1, 10), np.float32), np.array([10], np.int32), 4)
    assert idx.tolist() == [[0, 1, 2, 3]]
    idx, _ = oracle.topk(np.arange(5, dtype=np.float32)[None], np.array([5], np.int32), 8)
    assert idx.tolist() == [[0, 1, 2, 3, 4, -1, -1, -1]]
    idx, _ = oracle.topk(np.array([[1.0, -0.0, 0.0, 2.0]], np.float32), np.array([4], np.int32), 3)
    assert idx.tolist() == [[0, 1, 3]]                      # -0 ties +0: lower index wins
    idx, _ = oracle.topk(np.ones((1, 4), np.float32), np.array([0], np.int32), 2)
    assert idx.tolist() == [[-1, -1]]


def test_bf16_scores_round_like_a_library_cast():
    # The BF16-score step rounds each fp32 score once to the nearest bf16,
    # ties to even: the same bits as torch's float32 -> bfloat16 cast, on
    # random magnitudes over 80 binades, exact halfway cases, zeros, -inf
    # and subnormals.
    torch = pytest.importorskip("torch")
    g = synth.rng(36)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-28, 28, 20000))).astype(np.float32)
    j = np.arange(-300, 300, dtype=np.int64)
    mant = 128 + np.abs(j) % 127                    # a bf16 significand (8 bits)
    halfway = ((mant + 0.5) * 2.0 ** (j % 40 - 27) * np.sign(j + 0.5)).astype(np.float32)
    special = np.array([0.0, -0.0, -np.inf, 1e-40, -3e-39, 2.0 ** -126, 3.3895314e38], np.float32)
    allx = np.concatenate([x, halfway, special])
    got = oracle.scores_bf16(allx)
    want = torch.from_numpy(allx.copy()).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # halfway cases go to the even neighbour: the low mantissa bit is 0
    hb = got[len(x):len(x) + len(halfway)].view(np.uint32) >> 16
    assert np.all((hb & 1) == 0)


def test_bf16_scores_topk_ties_and_validity():
    # Scores that differ only below bf16 precision become ties: the lower
    # index wins. The bf16 selection is a valid top-k of the fp32 scores
    # within twice the rounding error (|s - bf16(s)| <= 2^-9 |s|).
    s = np.array([[1.0, 1.0 + 2 ** -12, 1.0 + 2 ** -11, 0.5, 1.0 + 2 ** -6, 2.0]], np.float32)
    nv = np.array([6], np.int32)
    idx32, _ = oracle.topk(s, nv, 3)
    idxbf, scbf = oracle.topk(oracle.scores_bf16(s), nv, 3)
    assert idx32.tolist() == [[2, 4, 5]]
    assert idxbf.tolist() == [[0, 4, 5]]          # 1, 1+2^-12, 1+2^-11 all round to 1.0: 0 wins
    assert scbf.tolist() == [[1.0, 1.015625, 2.0]]
    g = synth.rng(37)
    B, T, N, HI, dI, k = 1, 4, 3000, 8, 128, 200
    qc, qs = _mx(synth.normal(g, (B, T, HI, dI)))
    kc, ks = _mx(synth.normal(g, (B, N, dI)))
    w = synth.normal(g, (B, T, HI), 1.0 / HI)
    q_pos = np.full((B, T), 4 * N - 1, np.int32)
    sc, nv = oracle.indexer_scores(qc, w, kc, q_pos, np.array([N], np.int32), 4, q_scale=qs, k_scale=ks)
    ib, _ = oracle.indexer_topk(qc, w, kc, q_pos, np.array([N], np.int32), 4, k, q_scale=qs, k_scale=ks,
                                score_dtype=oracle.BF16)
    for r in range(T):
        s64 = sc[r].astype(np.float64)
        kth = np.sort(s64)[::-1][k - 1]
        eps = 2.0 ** -8 * np.abs(s64).max()
        sel = np.zeros(N, bool)
        sel[ib[r]] = True
        assert s64[sel].min() >= kth - eps and s64[~sel].max() <= kth + eps
