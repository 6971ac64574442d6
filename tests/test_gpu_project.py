"""GPU parity of the fused projection-then-compression (the series X W^T
computed on the matrix cores and pooled in registers; DeepSeek-V4 technical
report page, CSA section, step 1, and the HCA section), the entry RMSNorm
and the standalone query RMSNorm (same page, the section on Muon: queries
and KV entries normalised by RMSNorm).

Bars: the fp32 bar of the method, max-abs 1e-5, for fp32 entries against
the oracle's fp64 ones. Each projected value is an fp32 sum of `hidden`
exact bf16 products; with x N(0,1) and w N(0,1/hidden) the series are about
N(0,1) and the matrix core adds K-steps of 16 products into one fp32
accumulator, so the sum's error is of order sqrt(hidden/16) 2^-24 (about
1e-6 at hidden 4096); pooling, the norm (values of order 1-2 after it) and
RoPE add a few fp32 roundings. bf16 entries: one bf16 ulp more; MXFP4 and
FP8 KV bytes must equal the oracle's encoding of the GPU's own fp32
entries."""
import numpy as np
import pytest

import oracle
import synth
from util import bf16_ulp, check_f32, dev, host

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")

BAR = 1e-5


def _inputs(seed, B, S, hidden, D, csa, m):
    d = synth.projection(seed, B, S, hidden, D, csa, m)
    return d, {k: dev(v) for k, v in d.items()}


@pytest.mark.parametrize("B,S,hidden,D,d_rope,norm", [
    (2, 520, 256, 576, 64, True),    # two full tiles and a ragged one, nine channel blocks
    (1, 256, 128, 128, 0, False),    # one tile, indexer-key width, no rotation
    (3, 60, 64, 64, 32, True),       # a short ragged tile, one channel block
])
def test_csa_fused_matches_oracle(B, S, hidden, D, d_rope, norm):
    d, t = _inputs(1100 + S, B, S, hidden, D, True, 4)
    g = t["gamma"] if norm else None
    got = csk.project_compress(t["x"], t["w"], t["bias_a"], t["bias_b"], 4, gamma=g, d_rope=d_rope,
                               out_dtype=csk.CSK_F32)
    want = oracle.project_compress(d["x"], d["w"], d["bias_a"], d["bias_b"], 4,
                                   gamma=d["gamma"] if norm else None, d_rope=d_rope)
    check_f32(host(got), want, BAR, "csa fused fp32")
    g16 = csk.project_compress(t["x"], t["w"], t["bias_a"], t["bias_b"], 4, gamma=g, d_rope=d_rope)
    assert np.all(np.abs(host(g16) - want) <= bf16_ulp(want) + BAR)


@pytest.mark.parametrize("B,S,hidden,D,norm", [(1, 300, 128, 576, True), (2, 512, 256, 128, False)])
def test_hca_fused_matches_oracle(B, S, hidden, D, norm):
    # 128-token blocks: two per tile, a ragged tail that makes no entry;
    # 576 channels = four full 128-channel blocks and a half one
    d, t = _inputs(1200 + S, B, S, hidden, D, False, 128)
    g = t["gamma"] if norm else None
    got = csk.project_compress(t["x"], t["w"], t["bias_a"], None, 128, gamma=g, d_rope=64,
                               out_dtype=csk.CSK_F32)
    want = oracle.project_compress(d["x"], d["w"], d["bias_a"], None, 128, gamma=d["gamma"] if norm else None,
                                   d_rope=64)
    check_f32(host(got), want, BAR, "hca fused fp32")


def test_encoded_outputs_are_the_oracle_encoding_of_the_fp32_entries():
    d, t = _inputs(1300, 2, 264, 128, 576, True, 4)
    args = (t["x"], t["w"], t["bias_a"], t["bias_b"], 4)
    f32 = host(csk.project_compress(*args, gamma=t["gamma"], d_rope=64, out_dtype=csk.CSK_F32))
    e8 = host(csk.project_compress(*args, gamma=t["gamma"], d_rope=64, out_dtype=csk.CSK_FP8KV))
    assert np.array_equal(e8, oracle.fp8kv_encode(f32, 64))
    dk, tk = _inputs(1301, 2, 264, 128, 128, True, 4)
    argk = (tk["x"], tk["w"], tk["bias_a"], tk["bias_b"], 4)
    k32 = host(csk.project_compress(*argk, out_dtype=csk.CSK_F32))
    kc, ks = csk.project_compress(*argk, out_dtype=csk.CSK_MXFP4)
    rc, rs = oracle.mxfp4_encode(k32)
    assert np.array_equal(host(kc), rc) and np.array_equal(host(ks), rs)


def test_incremental_equals_one_shot():
    # a decode-style call: the tokens of entries 5 and 6 of a sequence, the
    # previous block in memory before them; bit-identical to those entries
    # of a one-shot call (same products, same order)
    d, t = _inputs(1400, 2, 64, 128, 576, True, 4)
    args = (t["bias_a"], t["bias_b"], 4)
    full = host(csk.project_compress(t["x"], t["w"], *args, gamma=t["gamma"], d_rope=64, out_dtype=csk.CSK_F32))
    inc = csk.project_compress(t["x"][:, 20:], t["w"], *args, gamma=t["gamma"], d_rope=64, out_dtype=csk.CSK_F32,
                               entry0=5, src_bstride=64, S=8, B=2)
    assert np.array_equal(host(inc), full[:, 5:7])


def test_prefill_64k_shape_sampled_entries():
    # the 64K CSA prefill layer's projection (hidden 4096, KV 512 + 64),
    # one launch over 65536 tokens; the oracle recomputes sampled entries
    # from their own tokens (a window starting one block earlier)
    S, hidden, D = 65536, 4096, 576
    gen = synth.rng(1500)
    x = synth.to_bf16(synth.normal(gen, (1, S, hidden)))
    w = synth.to_bf16(synth.normal(gen, (4, D, hidden), 1.0 / hidden))
    ba, bb = synth.normal(gen, (4, D), 0.1), synth.normal(gen, (4, D), 0.1)
    gamma = (1.0 + synth.normal(gen, (D,), 0.01)).astype(np.float32)
    got = host(csk.project_compress(dev(x), dev(w), dev(ba), dev(bb), 4, gamma=dev(gamma), d_rope=64,
                                    out_dtype=csk.CSK_F32))
    worst = 0.0
    for e in (0, 1, 63, 64, 65, 4095, 4096, 9999, 16383):
        lo = max(e - 1, 0)
        xs = x[:, 4 * lo: 4 * e + 4]
        pos = np.arange(lo, e + 1, dtype=np.int32)[None] * 4
        want = oracle.project_compress(xs, w, ba, bb, 4, gamma=gamma, d_rope=64, entry_pos=pos)[0, -1]
        worst = max(worst, check_f32(got[0, e], want, BAR, f"entry {e}"))
    print(f"[margin] csa projection+compression 64K (hidden 4096): max-abs {worst:.3e} (bar {BAR:g})", flush=True)


def test_query_rmsnorm():
    gen = synth.rng(1600)
    q = synth.to_bf16(synth.normal(gen, (2, 3, 64, 576)))
    gamma = (1.0 + synth.normal(gen, (576,), 0.01)).astype(np.float32)
    want = oracle.rmsnorm(q.reshape(-1, 576), gamma).reshape(q.shape)
    got32 = host(csk.rmsnorm(dev(q), dev(gamma), out_dtype=csk.CSK_F32))
    check_f32(got32, want, 1e-5, "rmsnorm fp32")
    got16 = host(csk.rmsnorm(dev(q), dev(gamma)))
    assert np.all(np.abs(got16 - want) <= 0.5 * bf16_ulp(want) + 1e-5)
    # in place
    tq = dev(q)
    csk.rmsnorm(tq, dev(gamma), out=tq)
    assert np.array_equal(host(tq), got16)


def test_project_compress_errors():
    d, t = _inputs(1700, 1, 64, 64, 64, True, 4)
    with pytest.raises(csk.CskError):
        csk.project_compress(t["x"], t["w"], t["bias_a"], t["bias_b"], 8)     # CSA needs m = 4
    with pytest.raises(csk.CskError):
        csk.project_compress(t["x"][:, :, :32], t["w"][:, :, :32], t["bias_a"], t["bias_b"], 4)  # hidden 32


@pytest.mark.parametrize("csa", [True, False])
def test_strides_and_entry_positions(csa):
    # batch strides on both sides (sources inside a longer buffer, entries
    # into a larger cache), explicit entry positions, a ragged tail
    m = 4 if csa else 128
    B, S, S_buf, hidden, D = 2, 4 * 67 + 3 if csa else 2 * 128 + 40, 600, 128, 576
    d, t = _inputs(1800 + csa, B, S_buf, hidden, D, csa, m)
    N = S // m
    gen = synth.rng(1810)
    pos = np.sort(gen.integers(0, 1 << 20, (B, N)), axis=1).astype(np.int32)
    cache = torch.zeros((B, N + 5, D), dtype=torch.float32, device="cuda")
    csk.project_compress(t["x"], t["w"], t["bias_a"], t["bias_b"] if csa else None, m, gamma=t["gamma"], d_rope=64,
                         entry_pos=dev(pos), out_dtype=csk.CSK_F32, src_bstride=S_buf, out=cache, dst_bstride=N + 5,
                         S=S, B=B)
    want = oracle.project_compress(d["x"][:, :S], d["w"], d["bias_a"], d["bias_b"] if csa else None, m,
                                   gamma=d["gamma"], d_rope=64, entry_pos=pos)
    got = host(cache)
    check_f32(got[:, :N], want, BAR, "strided fused fp32")
    assert not got[:, N:].any()
