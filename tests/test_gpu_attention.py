"""GPU parity: CSA sparse and HCA dense attention with window, sink and
partial RoPE. bf16 bar: max-abs <= 2e-2 and relative L2 <= 1e-2; fp32 bar:
max-abs <= 1e-5 (lse checked with the same bars)."""
import numpy as np
import pytest

import oracle
import synth
from util import check_bf16_attention, check_f32, dev, host

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")


def _inputs(g, B, T, H, D, N, S_w, bf16):
    cast = synth.to_bf16 if bf16 else (lambda x: x)
    q = cast(synth.normal(g, (B, T, H, D)))
    kv_c = cast(synth.normal(g, (B, N, D)))
    kv_w = cast(synth.normal(g, (B, S_w, D)))
    return q, kv_c, kv_w


def _check(got, ref, bf16, what):
    if bf16:
        check_bf16_attention(got, ref, what)
    else:
        check_f32(got, ref, 1e-5, what)


def _sparse_case(seed, B, T, H, D, dv, N, k, S_w, W, bf16, d_rope, sink=True, decode=False, max_workgroups=0):
    g = synth.rng(seed)
    q, kv_c, kv_w = _inputs(g, B, T, H, D, N, S_w, bf16)
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
    idx[0, 0, 0] = N + 5                      # out of range: skipped on both sides
    sk = synth.normal(g, (H,)) if sink else None
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = csk.sparse_attn(dev(q), dev(q_pos), dev(kv_c), dev(idx), dev(kv_w), dev(w_pos0), W,
                               None if sk is None else dev(sk), dv, d_rope, scale, max_workgroups=max_workgroups)
    rout, rlse = oracle.sparse_attn(q, q_pos, kv_c, idx, kv_w, w_pos0, W, sk, dv, d_rope, scale)
    _check(host(out).reshape(-1, H, dv), rout, bf16, "out")
    check_f32(host(lse).reshape(-1, H), rlse, 2e-2 if bf16 else 1e-5, "lse")


@pytest.mark.parametrize("bf16", [True, False])
def test_sparse_prefill_small(bf16):
    _sparse_case(601, B=2, T=19, H=64, D=576, dv=512, N=300, k=40, S_w=300, W=16, bf16=bf16, d_rope=64)


@pytest.mark.parametrize("B,k", [(16, 1000), (32, 480)])
def test_sparse_decode_batched_split(B, k):
    # batched decode rows split over at most 16 workgroups each (16 and 8
    # here): the one-wave-per-(row, head) merge of the bf16 partials
    _sparse_case(630 + B, B=B, T=1, H=64, D=576, dv=512, N=2500, k=k, S_w=128, W=100, bf16=True,
                 d_rope=64, decode=True)


def test_sparse_fp32_tiny_shapes():
    _sparse_case(602, B=1, T=256, H=4, D=64, dv=64, N=64, k=8, S_w=256, W=32, bf16=False, d_rope=32)


@pytest.mark.parametrize("H,D,dv", [(64, 576, 512), (16, 128, 128), (32, 576, 576), (64, 64, 64), (8, 96, 80),
                                    (64, 256, 256), (64, 128, 128)])
def test_sparse_decode_split(H, D, dv):
    # decode rows: long candidate lists split across workgroups and merged
    _sparse_case(603 + H + D, B=3, T=1, H=H, D=D, dv=dv, N=5000, k=2048, S_w=128, W=128, bf16=True,
                 d_rope=min(64, D // 2), decode=True)


@pytest.mark.parametrize("cap", [4, 40])
def test_sparse_decode_workgroup_cap(cap):
    # the sparse split capped: 4 workgroups over 4 rows (each row whole in
    # one workgroup, no merge) and 40 (ten runs of three or four tiles a
    # row, merged)
    _sparse_case(770 + cap, B=4, T=1, H=64, D=576, dv=512, N=5000, k=2048, S_w=128, W=128, bf16=True,
                 d_rope=64, decode=True, max_workgroups=cap)


@pytest.mark.parametrize("D,dv", [(576, 512), (256, 256), (128, 128), (64, 64)])
def test_sparse_prefill_whole_rows(D, dv):
    # 320 rows of up to 150 selected entries + 40 window tokens: rows stay
    # whole, three 64-row tiles with a ragged last one, rows with padding
    _sparse_case(610 + D, B=2, T=160, H=64, D=D, dv=dv, N=700, k=150, S_w=200, W=40, bf16=True,
                 d_rope=min(64, D // 2))


def test_sparse_no_sink_no_window_and_empty():
    g = synth.rng(604)
    B, T, H, D, N = 1, 3, 64, 576, 50
    q, kv_c, _ = _inputs(g, B, T, H, D, N, 1, True)
    idx = np.full((B, T, 8), -1, np.int32)
    idx[0, 1, :3] = [4, 9, 7]
    q_pos = np.array([[10, 20, 30]], np.int32)
    out, lse = csk.sparse_attn(dev(q), dev(q_pos), dev(kv_c), dev(idx), None, None, 0, None, 512, 64, 0.05)
    rout, rlse = oracle.sparse_attn(q, q_pos, kv_c, idx, None, None, 0, None, 512, 64, 0.05)
    check_bf16_attention(host(out).reshape(-1, H, 512), rout, "out")
    o = host(out)
    assert np.all(o[0, 0] == 0) and np.all(np.isneginf(host(lse)[0, 0]))   # no candidate, no sink


def _dense_case(seed, B, T, H, D, dv, N, m, S_w, W, bf16, d_rope, decode, q_pos=None, max_workgroups=0):
    g = synth.rng(seed)
    q, kv_c, kv_w = _inputs(g, B, T, H, D, N, S_w, bf16)
    if q_pos is not None:
        w_pos0 = np.zeros(B, np.int32)
    elif decode:
        q_pos = np.full((B, T), m * N - 1, np.int32)
        w_pos0 = np.full(B, m * N - S_w, np.int32)
    else:
        q_pos = np.arange(T, dtype=np.int32)[None].repeat(B, 0) + g.integers(0, 3, (B, 1)).astype(np.int32)
        w_pos0 = np.zeros(B, np.int32)
    ne = np.array([N] + [max(1, N - 7)] * (B - 1), np.int32)
    sk = synth.normal(g, (H,))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = csk.dense_compressed_attn(dev(q), dev(q_pos), dev(kv_c), dev(ne), m, dev(kv_w), dev(w_pos0), W,
                                         dev(sk), dv, d_rope, scale, max_workgroups=max_workgroups)
    rows = None
    if B * T > 600:
        rows = [(b, t) for b in range(B) for t in list(range(0, T, 37)) + [T - 1]]
    rout, rlse = oracle.dense_attn(q, q_pos, kv_c, ne, m, kv_w, w_pos0, W, sk, dv, d_rope, scale, rows=rows)
    go, gl = host(out), host(lse)
    if rows is not None:
        go = np.stack([go[b, t] for b, t in rows])
        gl = np.stack([gl[b, t] for b, t in rows])
    _check(go.reshape(-1, H, dv), rout, bf16, "out")
    check_f32(gl.reshape(-1, H), rlse, 2e-2 if bf16 else 1e-5, "lse")


def test_dense_prefill_hca_shape():
    # 16 heads x dim 128, m' = 128, window 128: the HCA prefill layer shape
    _dense_case(701, B=1, T=2048, H=16, D=128, dv=128, N=16, m=128, S_w=2048, W=128, bf16=True, d_rope=64,
                decode=False)


@pytest.mark.parametrize("B,T,H,D,N,m,S_w,W", [
    (2, 100, 32, 128, 30, 4, 100, 16),      # rows per tile not dividing T, two head groups
    (1, 1200, 16, 128, 300, 4, 1200, 128),  # candidate union staged in LDS twice
    (2, 40, 64, 64, 12, 4, 40, 8),          # four head groups, two rows per tile
    (1, 70, 16, 256, 20, 4, 70, 32),        # one column tile per wave
])
def test_dense_prefill_query_tiles(B, T, H, D, N, m, S_w, W):
    _dense_case(720 + T + H, B=B, T=T, H=H, D=D, dv=D, N=N, m=m, S_w=S_w, W=W, bf16=True,
                d_rope=min(64, D // 2), decode=False)


@pytest.mark.parametrize("T", [48, 96])
def test_dense_prefill_unordered_positions(T):
    # query rows at scattered positions: a tile's candidate union spans
    # several windows and its rows keep different subsets of it (at 96 rows
    # a workgroup takes four query groups, and their union exceeds what it
    # can stage at once)
    g = synth.rng(731 + T)
    q_pos = np.stack([np.sort(g.permutation(400)[:T]), g.permutation(400)[:T]]).astype(np.int32)
    _dense_case(732 + T, B=2, T=T, H=16, D=128, dv=128, N=100, m=4, S_w=400, W=24, bf16=True, d_rope=64,
                decode=False, q_pos=q_pos)


def test_dense_decode_split():
    _dense_case(702, B=4, T=1, H=64, D=576, dv=512, N=3000, m=128, S_w=128, W=128, bf16=True, d_rope=64,
                decode=True)


@pytest.mark.parametrize("D", [256, 128, 64])
def test_dense_decode_split_shapes(D):
    # 64 heads at the other streamed-row shapes: rows split over runs of
    # 64-row tiles (a ragged last tile, shorter visible lists on rows 1..)
    _dense_case(740 + D, B=3, T=1, H=64, D=D, dv=D, N=1500, m=128, S_w=128, W=128, bf16=True,
                d_rope=min(64, D // 2), decode=True)


def test_dense_many_rows_kept_whole():
    # more rows than CUs: each row stays in one workgroup, which writes the
    # normalised output itself (no partials, no merge)
    _dense_case(750, B=260, T=1, H=64, D=128, dv=128, N=40, m=4, S_w=160, W=32, bf16=True, d_rope=64,
                decode=True)


def test_dense_few_query_rows():
    # a short run of query rows per sequence (below the query-tile path):
    # each row has its own visible count and window
    _dense_case(751, B=2, T=9, H=64, D=576, dv=512, N=300, m=4, S_w=1300, W=64, bf16=True, d_rope=64,
                decode=False, q_pos=np.array([[1190 + 3 * t for t in range(9)]] * 2, np.int32))


def test_dense_decode_workgroup_cap():
    # the split capped at 8 workgroups: two runs of about 25 tiles per row
    _dense_case(760, B=4, T=1, H=64, D=576, dv=512, N=3000, m=128, S_w=128, W=128, bf16=True, d_rope=64,
                decode=True, max_workgroups=8)


@pytest.mark.parametrize("B,N", [(2, 16384), (4, 8192)])
def test_dense_decode_extra_rows(B, N):
    # rows of 16512 / 8320 candidates (the 1M-context HCA shape): each row
    # split over 64 or 128 workgroups of two or three 64-row tiles, bf16
    # partials merged
    _dense_case(705 + B, B=B, T=1, H=64, D=576, dv=512, N=N, m=128, S_w=128, W=128, bf16=True, d_rope=64,
                decode=True)


def test_dense_fp32():
    _dense_case(703, B=2, T=70, H=4, D=64, dv=64, N=20, m=4, S_w=70, W=8, bf16=False, d_rope=32, decode=False)


def test_sparse_all_visible_equals_dense():
    # CSA with k >= #visible selects every visible entry: same as HCA attention
    g = synth.rng(704)
    B, T, H, D, N, m = 1, 1, 64, 576, 700, 4
    q, kv_c, kv_w = _inputs(g, B, T, H, D, N, 128, True)
    q_pos = np.array([[4 * N - 1]], np.int32)
    w_pos0 = np.array([4 * N - 128], np.int32)
    idx = np.arange(N, dtype=np.int32)[None, None]
    sk = np.zeros(H, np.float32)
    a, al = csk.sparse_attn(dev(q), dev(q_pos), dev(kv_c), dev(idx), dev(kv_w), dev(w_pos0), 128, dev(sk),
                            512, 64, 1 / 24)
    d, dl = csk.dense_compressed_attn(dev(q), dev(q_pos), dev(kv_c), dev(np.array([N], np.int32)), m, dev(kv_w),
                                      dev(w_pos0), 128, dev(sk), 512, 64, 1 / 24)
    check_bf16_attention(host(a), host(d), "sparse vs dense")


def _launches(kernel, fn):
    """Runs fn() with the library's launch timer armed for `kernel` and
    returns how many launches of that kernel it made."""
    tm = csk.KernelTimer(kernel, 16)
    try:
        fn()
        torch.cuda.synchronize()
        return tm.count()
    finally:
        tm.disarm()


@pytest.mark.parametrize("H,D,dv", [(16, 128, 128), (32, 576, 512), (48, 576, 576)])
def test_sparse_whole_rows_stream_kernel(H, D, dv):
    # fewer than 64 heads with short candidate lists over 300 rows: rows stay
    # whole in one workgroup of the streamed-tile kernel (attn_bf16_stream);
    # the launch timer confirms which kernel ran
    n = _launches("attn_bf16_stream", lambda: _sparse_case(
        780 + H, B=2, T=150, H=H, D=D, dv=dv, N=400, k=96, S_w=200, W=24, bf16=True, d_rope=64))
    assert n == 1


@pytest.mark.parametrize("H,D,T", [(16, 128, 8), (32, 576, 20)])
def test_dense_few_rows_stream_kernel(H, D, T):
    # dense rows the query-tile kernel does not take (fewer than 16 rows, or
    # D = 576 with fewer than 64 heads) over many sequences: whole rows in the
    # streamed-tile kernel
    dv = 128 if D == 128 else 512
    n = _launches("attn_bf16_stream", lambda: _dense_case(
        790 + H, B=40, T=T, H=H, D=D, dv=dv, N=60, m=4, S_w=240, W=32, bf16=True, d_rope=64, decode=False))
    assert n == 1
