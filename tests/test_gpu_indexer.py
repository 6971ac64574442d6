"""GPU parity: lightning-indexer scores and top-k. Bit-exact bar: given
identical input bytes, the selected indices and their scores must equal the
oracle's exactly (exact MXFP4 dot products, fp32 fma head chain in
ascending order, ties to the lower index)."""
import numpy as np
import pytest

import oracle
import synth
from mx_regime import assert_in_regime, pair_spread_exact
from util import dev, host

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")


def _mx_both(x):
    """Quantise on both sides and require identical bytes."""
    gc, gs = csk.mxfp4_quantize(dev(x))
    rc, rs = oracle.mxfp4_encode(x)
    assert np.array_equal(host(gc), rc) and np.array_equal(host(gs), rs)
    return (gc, gs), (rc, rs)


def _run_mx(qI, kI, w, q_pos, n_entries, m, k):
    (gqc, gqs), (rqc, rqs) = _mx_both(qI)
    (gkc, gks), (rkc, rks) = _mx_both(kI)
    assert_in_regime(rqc, rqs, rkc, rks)
    idx, sc = csk.indexer_topk(gqc, dev(w), gkc, dev(q_pos), dev(n_entries), m, k, q_scale=gqs, k_scale=gks)
    ridx, rsc = oracle.indexer_topk(rqc, w, rkc, q_pos, n_entries, m, k, q_scale=rqs, k_scale=rks)
    B, T = q_pos.shape
    return host(idx).reshape(B * T, k), host(sc).reshape(B * T, k), ridx, rsc


def _assert_same(gi, gs, ri, rs):
    bad = np.where(np.any(gi != ri, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))


def test_fp32_path_tiny_prefill():
    g = synth.rng(501)
    B, T, HI, dI, N, m, k = 1, 256, 2, 32, 64, 4, 8
    q = synth.normal(g, (B, T, HI, dI))
    kk = synth.normal(g, (B, N, dI))
    w = synth.normal(g, (B, T, HI))
    q_pos = np.arange(T, dtype=np.int32)[None]
    ne = np.array([N], np.int32)
    idx, sc = csk.indexer_topk(dev(q), dev(w), dev(kk), dev(q_pos), dev(ne), m, k)
    ridx, rsc = oracle.indexer_topk(q, w, kk, q_pos, ne, m, k)
    _assert_same(host(idx).reshape(-1, k), host(sc).reshape(-1, k), ridx, rsc)
    assert np.all(host(idx)[0, :3] == -1)          # rows 0..2 see no entry


@pytest.mark.parametrize("HI,dI", [(64, 128), (32, 128), (64, 256), (32, 256), (48, 128), (16, 256), (8, 64)])
def test_mxfp4_short_rows(HI, dI):
    g = synth.rng(502 + HI + dI)
    B, T, N, m, k = 2, 37, 1000, 4, 64
    qI = synth.normal(g, (B, T, HI, dI))
    kI = synth.normal(g, (B, N, dI))
    w = synth.normal(g, (B, T, HI), 1.0 / HI)
    q_pos = g.integers(-3, 4 * N + 40, (B, T)).astype(np.int32)
    q_pos[0, :4] = [0, 3, 4 * k - 1, 4 * k + 3]      # none, 1, k, k+1 visible
    ne = np.array([N, 700], np.int32)
    gi, gs, ri, rs = _run_mx(qI, kI, w, q_pos, ne, m, k)
    _assert_same(gi, gs, ri, rs)


@pytest.mark.parametrize("N,k", [(40000, 2048), (20000, 512)])
def test_mxfp4_long_rows_filtered(N, k):
    g = synth.rng(503 + N)
    B, T, HI, dI, m = 2, 1, 64, 128, 4
    qI = synth.normal(g, (B, T, HI, dI))
    kI = synth.normal(g, (B, N, dI))
    w = synth.normal(g, (B, T, HI), 1.0 / HI)
    q_pos = np.array([[4 * N - 1], [4 * 31000 + 2]], np.int32)
    ne = np.array([N, N], np.int32)
    gi, gs, ri, rs = _run_mx(qI, kI, w, q_pos, ne, m, k)
    _assert_same(gi, gs, ri, rs)


@pytest.mark.parametrize("HI,dI", [(64, 128), (32, 256)])
def test_mxfp4_prefill_rows_filtered(HI, dI):
    # several queries per sequence over a cache longer than the in-LDS
    # select (the prefill indexer form with its group maxima), causal
    # positions from none to every entry visible
    g = synth.rng(505 + HI + dI)
    B, T, N, m, k = 2, 5, 40000, 4, 2048
    qI = synth.normal(g, (B, T, HI, dI))
    kI = synth.normal(g, (B, N, dI))
    w = synth.normal(g, (B, T, HI), 1.0 / HI)
    q_pos = np.array([[2, 4 * k + 5, 4 * 20000 + 1, 4 * 33333 + 3, 4 * N - 1],
                      [4 * N + 9, 4 * 16384, 4 * 1000, 4 * 39999 + 2, 0]], np.int32)
    ne = np.array([N, 37001], np.int32)
    gi, gs, ri, rs = _run_mx(qI, kI, w, q_pos, ne, m, k)
    _assert_same(gi, gs, ri, rs)


@pytest.mark.parametrize("N", [3000, 40000])
def test_ties_go_to_lower_index(N):
    # w = 0 makes every score +0: the lowest k indices win. Repeated keys
    # with w > 0 give exact ties among different indices.
    g = synth.rng(504)
    B, T, HI, dI, m, k = 1, 2, 64, 128, 4, 2048
    qI = synth.normal(g, (B, T, HI, dI))
    base = synth.normal(g, (B, 50, dI))
    kI = base[:, g.integers(0, 50, N)]
    w = np.abs(synth.normal(g, (B, T, HI), 1.0 / HI))
    w[0, 0] = 0.0
    q_pos = np.full((B, T), 4 * N - 1, np.int32)
    ne = np.array([N], np.int32)
    gi, gs, ri, rs = _run_mx(qI, kI, w, q_pos, ne, m, k)
    _assert_same(gi, gs, ri, rs)
    assert gi[0].tolist() == list(range(k))


def test_invalid_arguments_raise():
    g = synth.rng(505)
    q = dev(synth.normal(g, (1, 1, 2, 32)))
    with pytest.raises(csk.CskError):
        csk.indexer_topk(q, dev(np.ones((1, 1, 2), np.float32)), dev(synth.normal(g, (1, 4, 32))),
                         dev(np.zeros((1, 1), np.int32)), dev(np.ones(1, np.int32)), 0, 4)


@pytest.mark.parametrize("spread", [6, 8, 9])
def test_mxfp4_bit_exact_at_exponent_spread(spread):
    # Operands built byte by byte so that the four tile exponents of a
    # (query head, key) pair span up to `spread` binades, the edge of the
    # exactness regime at 9, with the largest tile products where the
    # exponent is highest (tile 1 of both operands all +-6). Every score of
    # every row is returned (k = N) and must equal the oracle's bit for bit.
    g = synth.rng(530 + spread)
    B, T, HI, dI, N, m = 1, 3, 64, 128, 512, 4
    G = dI // 32
    qc = g.integers(0, 256, (B, T, HI, dI // 2), dtype=np.uint8)
    kc = g.integers(0, 256, (B, N, dI // 2), dtype=np.uint8)
    qc[..., 16:32] = 0x77                                        # +6, +6
    kc[..., 16:32] = np.where(g.random((B, N, 1)) < 0.5, 0x77, 0xFF).astype(np.uint8)  # +-6
    aq_max = spread // 2
    aq = g.integers(0, aq_max + 1, (B, T, HI))
    aq[..., 0] = aq_max
    ak = g.integers(0, spread - aq_max + 1, (B, N))
    ak[..., 0] = spread - aq_max
    qs = np.empty((B, T, HI, G), np.int64)
    ks = np.empty((B, N, G), np.int64)
    qs[..., 0], qs[..., 1] = 124, 124 + aq
    ks[..., 0], ks[..., 1] = 125, 125 + ak
    for t in (2, 3):
        qs[..., t] = 124 + (g.random((B, T, HI)) * (aq + 1)).astype(np.int64)
        ks[..., t] = 125 + (g.random((B, N)) * (ak + 1)).astype(np.int64)
    qs, ks = qs.astype(np.uint8), ks.astype(np.uint8)
    assert pair_spread_exact(qc, qs, kc, ks) == spread
    assert_in_regime(qc, qs, kc, ks)
    w = synth.normal(g, (B, T, HI), 1.0 / HI)
    q_pos = np.full((B, T), 4 * N - 1, np.int32)
    ne = np.array([N], np.int32)
    idx, sc = csk.indexer_topk(dev(qc), dev(w), dev(kc), dev(q_pos), dev(ne), m, N, q_scale=dev(qs),
                               k_scale=dev(ks))
    ridx, rsc = oracle.indexer_topk(qc, w, kc, q_pos, ne, m, N, q_scale=qs, k_scale=ks)
    _assert_same(host(idx).reshape(B * T, N), host(sc).reshape(B * T, N), ridx, rsc)
    assert np.all(ridx == np.arange(N)[None])


@pytest.mark.parametrize("B,T,N,k", [(2, 37, 1000, 64), (2, 1, 40000, 2048), (4, 1, 262144, 2048)])
def test_bf16_scores_bit_exact(B, T, N, k):
    # BF16 scores for the top-k: every score rounded once to bf16 before the
    # selection, on both sides; the selection (many more ties) and the
    # returned bf16 scores must be bit-exact. The recall of the fp32
    # selection is reported.
    g = synth.rng(540 + N)
    HI, dI, m = 64, 128, 4
    qI = synth.normal(g, (B, T, HI, dI))
    kI = synth.normal(g, (B, N, dI))
    w = synth.normal(g, (B, T, HI), 1.0 / HI)
    q_pos = np.full((B, T), 4 * N - 1, np.int32) - g.integers(0, 3, (B, T)).astype(np.int32)
    ne = np.array([N] * B, np.int32)
    (gqc, gqs), (rqc, rqs) = _mx_both(qI)
    (gkc, gks), (rkc, rks) = _mx_both(kI)
    assert_in_regime(rqc, rqs, rkc, rks)
    idx, sc = csk.indexer_topk(gqc, dev(w), gkc, dev(q_pos), dev(ne), m, k, q_scale=gqs, k_scale=gks,
                               score_dtype=csk.CSK_BF16)
    ridx, rsc = oracle.indexer_topk(rqc, w, rkc, q_pos, ne, m, k, q_scale=rqs, k_scale=rks,
                                    score_dtype=oracle.BF16)
    _assert_same(host(idx).reshape(B * T, k), host(sc).reshape(B * T, k), ridx, rsc)
    assert np.all(host(sc).view(np.uint32)[host(idx) >= 0] & 0xffff == 0)   # bf16 values
    i32, _ = csk.indexer_topk(gqc, dev(w), gkc, dev(q_pos), dev(ne), m, k, q_scale=gqs, k_scale=gks)
    a, b = host(i32).reshape(B * T, k), host(idx).reshape(B * T, k)
    rec = np.mean([len(set(a[r][a[r] >= 0]) & set(b[r][b[r] >= 0])) / max(1, (a[r] >= 0).sum())
                   for r in range(B * T)])
    print(f"[recall] bf16 scores, N={N}, k={k}: {rec:.4f} of the fp32 selection")
