"""GPU parity of FP8 KV entries (E4M3 non-RoPE dims with a power-of-two
scale per 32, BF16 RoPE dims): the compress epilogue's bytes against the
oracle's encoder, the attention kernels' dequantisation bit for bit, and
sparse / dense attention over FP8 caches against the oracle's attention over
the decoded entries (bf16 bars: max-abs <= 2e-2, rel-L2 <= 1e-2)."""
import numpy as np
import pytest

import oracle
import synth
from util import check_bf16_attention, check_f32, dev, host

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")

D, DR, DV, H = 576, 64, 512, 64


def _fp8_cache(g, shape):
    """Random N(0,1) entries as FP8 KV bytes (oracle encoder) and their exact
    decoded values."""
    x = synth.normal(g, shape + (D,))
    e = oracle.fp8kv_encode(x, DR)
    return e, oracle.fp8kv_decode(e, D, DR)


def test_compress_fp8kv_bytes():
    # CSA and HCA compression with FP8 KV output: the bytes are the oracle's
    # encoding of the GPU's own fp32 pooled (and rotated) values, which are
    # within 1e-5 of the oracle's fp64 pooling
    g = synth.rng(801)
    B, S = 2, 512
    ca, za, cb, zb = (synth.to_bf16(synth.normal(g, (B, S, D))) for _ in range(4))
    ba, bb = synth.normal(g, (4, D), 0.1), synth.normal(g, (4, D), 0.1)
    t = [dev(x) for x in (ca, za, cb, zb, ba, bb)]
    e8 = csk.csa_compress(*t, 4, d_rope=DR, out_dtype=csk.CSK_FP8KV)
    f32 = csk.csa_compress(*t, 4, d_rope=DR, out_dtype=csk.CSK_F32)
    assert e8.shape == (B, S // 4, 656)
    assert np.array_equal(host(e8), oracle.fp8kv_encode(host(f32), DR))
    r64 = oracle.csa_compress(ca, za, cb, zb, ba, bb, 4, d_rope=DR)
    check_f32(host(f32), r64, 1e-5, "csa pool")
    c, z = synth.to_bf16(synth.normal(g, (B, 1024, D))), synth.to_bf16(synth.normal(g, (B, 1024, D)))
    bh = synth.normal(g, (128, D), 0.1)
    h8 = csk.hca_compress(dev(c), dev(z), dev(bh), 128, d_rope=DR, out_dtype=csk.CSK_FP8KV)
    h32 = csk.hca_compress(dev(c), dev(z), dev(bh), 128, d_rope=DR, out_dtype=csk.CSK_F32)
    assert np.array_equal(host(h8), oracle.fp8kv_encode(host(h32), DR))
    # the batched launch (decode: the newest entry into a larger cache)
    cache = torch.zeros((B, 10, 656), dtype=torch.uint8, device="cuda")
    job = csk.csa_job(t[0][:, 4:8], t[1][:, 4:8], t[2][:, 4:8], t[3][:, 4:8], t[4], t[5], 4, d_rope=DR,
                      entry0=9, src_bstride=S, out_dtype=csk.CSK_FP8KV, out=cache[:, 9:], dst_bstride=10, S=4, B=B)
    csk.compress_batch([job])
    one32 = csk.csa_compress(t[0][:, 4:8], t[1][:, 4:8], t[2][:, 4:8], t[3][:, 4:8], t[4], t[5], 4, d_rope=DR,
                             entry0=9, src_bstride=S, out_dtype=csk.CSK_F32, S=4, B=B)
    assert np.array_equal(host(cache[:, 9]), oracle.fp8kv_encode(host(one32)[:, 0], DR))
    assert not host(cache[:, :9]).any()


@pytest.mark.parametrize("dense", [False, True])
def test_fp8kv_dequant_is_exact(dense):
    # one candidate and no sink: the softmax weight is exactly 1, so every
    # output is the entry's value, which bf16 holds exactly: the outputs must
    # equal the oracle's decoded entries bit for bit (per row, value dims)
    g = synth.rng(802 + dense)
    B, T, N = 3, 2, 40
    e, x = _fp8_cache(g, (B, N))
    q = synth.to_bf16(synth.normal(g, (B, T, H, D)))
    if dense:
        # entry 0 visible only (m = 4, positions 3 and 6)
        q_pos = np.array([[3, 6]] * B, np.int32)
        out, _ = csk.dense_compressed_attn(dev(q), dev(q_pos), dev(e), dev(np.full(B, N, np.int32)), 4, None, None,
                                           0, None, DV, DR, 0.04)
        want = np.broadcast_to(x[:, None, None, 0, :DV], (B, T, H, DV))
    else:
        sel = g.integers(0, N, (B, T))
        idx = np.full((B, T, 8), -1, np.int32)
        idx[:, :, 3] = sel
        q_pos = np.full((B, T), 4 * N, np.int32)
        out, _ = csk.sparse_attn(dev(q), dev(q_pos), dev(e), dev(idx), None, None, 0, None, DV, DR, 0.04)
        want = np.stack([np.stack([np.broadcast_to(x[b, sel[b, t], :DV], (H, DV)) for t in range(T)]) for b in range(B)])
    got = host(out)
    assert np.array_equal(got.astype(np.float32).view(np.uint32), want.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("B,T,N,k,S_w,W,decode,cap", [
    (3, 1, 5000, 2048, 128, 128, True, 0),     # decode: rows split over workgroups, merged
    (4, 1, 5000, 2048, 128, 128, True, 40),    # decode under a workgroup cap (runs of several tiles)
    (2, 90, 700, 150, 200, 40, False, 0),      # prefill: rows kept whole, ragged tiles, empty slots
])
def test_fp8kv_sparse_attention(B, T, N, k, S_w, W, decode, cap):
    g = synth.rng(810 + T + cap)
    e, x = _fp8_cache(g, (B, N))
    ew, xw = _fp8_cache(g, (B, S_w))
    q = synth.to_bf16(synth.normal(g, (B, T, H, D)))
    if decode:
        q_pos = np.full((B, T), 4 * N - 1, np.int32)
        w_pos0 = np.full(B, 4 * N - S_w, np.int32)
    else:
        q_pos = np.sort(g.integers(0, S_w, (B, T)), axis=1).astype(np.int32)
        w_pos0 = np.zeros(B, np.int32)
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            nsel = int(g.integers(0, k + 1))
            idx[b, t, :nsel] = np.sort(g.choice(N, nsel, replace=False))
    sk = synth.normal(g, (H,))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = csk.sparse_attn(dev(q), dev(q_pos), dev(e), dev(idx), dev(ew), dev(w_pos0), W, dev(sk), DV, DR, scale,
                               max_workgroups=cap)
    rout, rlse = oracle.sparse_attn(q, q_pos, x, idx, xw, w_pos0, W, sk, DV, DR, scale)
    check_bf16_attention(host(out).reshape(-1, H, DV), rout, "fp8 sparse out")
    check_f32(host(lse).reshape(-1, H), rlse, 2e-2, "fp8 sparse lse")


@pytest.mark.parametrize("B,N,cap", [(4, 3000, 0), (4, 3000, 8), (2, 8192, 64)])
def test_fp8kv_dense_attention_decode(B, N, cap):
    g = synth.rng(820 + N + cap)
    e, x = _fp8_cache(g, (B, N))
    ew, xw = _fp8_cache(g, (B, 128))
    q = synth.to_bf16(synth.normal(g, (B, 1, H, D)))
    q_pos = np.full((B, 1), 128 * N - 1, np.int32)
    w_pos0 = np.full(B, 128 * N - 128, np.int32)
    ne = np.array([N] + [N - 7] * (B - 1), np.int32)
    sk = synth.normal(g, (H,))
    out, lse = csk.dense_compressed_attn(dev(q), dev(q_pos), dev(e), dev(ne), 128, dev(ew), dev(w_pos0), 128, dev(sk),
                                         DV, DR, 1 / 24, max_workgroups=cap)
    rout, rlse = oracle.dense_attn(q, q_pos, x, ne, 128, xw, w_pos0, 128, sk, DV, DR, 1 / 24)
    check_bf16_attention(host(out).reshape(-1, H, DV), rout, "fp8 dense out")
    check_f32(host(lse).reshape(-1, H), rlse, 2e-2, "fp8 dense lse")


def test_fp8kv_unsupported_shape_raises():
    g = synth.rng(830)
    e, _ = _fp8_cache(g, (1, 10))
    q = dev(synth.to_bf16(synth.normal(g, (1, 1, 16, D))))
    with pytest.raises(csk.CskError):
        csk.sparse_attn(q, dev(np.array([[40]], np.int32)), dev(e), dev(np.zeros((1, 1, 4), np.int32)), None, None, 0,
                        None, DV, DR, 0.04)


def test_fp8kv_dense_attention_prefill_rows():
    # many query rows kept whole (the streamed-row kernel in dense mode over
    # FP8 entries): causal visibility of 4-token entries, window 32, sink
    g = synth.rng(840)
    B, T, N, m, S_w, W = 2, 70, 300, 4, 280, 32
    e, x = _fp8_cache(g, (B, N))
    ew, xw = _fp8_cache(g, (B, S_w))
    q = synth.to_bf16(synth.normal(g, (B, T, H, D)))
    q_pos = np.sort(g.integers(0, S_w, (B, T)), axis=1).astype(np.int32)
    w_pos0 = np.zeros(B, np.int32)
    ne = np.array([N, N - 50], np.int32)
    sk = synth.normal(g, (H,))
    out, lse = csk.dense_compressed_attn(dev(q), dev(q_pos), dev(e), dev(ne), m, dev(ew), dev(w_pos0), W, dev(sk),
                                         DV, DR, 1 / 24)
    rout, rlse = oracle.dense_attn(q, q_pos, x, ne, m, xw, w_pos0, W, sk, DV, DR, 1 / 24)
    check_bf16_attention(host(out).reshape(-1, H, DV), rout, "fp8 dense prefill out")
    check_f32(host(lse).reshape(-1, H), rlse, 2e-2, "fp8 dense prefill lse")
