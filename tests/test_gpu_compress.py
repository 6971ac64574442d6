"""GPU parity: compression (CSA / HCA), partial RoPE, MXFP4 quantisation.

The oracle computes in fp64 and rounds once; the GPU computes in fp32.
fp32 outputs: max-abs <= 1e-5. bf16 outputs: within one bf16 ulp of the
oracle's value plus the fp32 bar (the fp32 pooling and rotation error is
about 1e-7 absolute, more than one bf16 ulp of an output near zero).
MXFP4 quantisation of identical fp32 inputs: bit-exact. MXFP4 output of the
compressor: the codes equal the oracle encoder applied to the GPU's own fp32
pooled values (the decision is taken on the same fp32 value on both sides),
and those fp32 values meet the fp32 bar.
"""
import numpy as np
import pytest

import oracle
import synth
from util import bf16_ulp, check_f32, dev, host


def _bf16_ok(got, ref):
    return np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-5)

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")


def _series(g, B, S, D, bf16):
    xs = [synth.normal(g, (B, S, D)) for _ in range(4)]
    return [synth.to_bf16(x) for x in xs] if bf16 else xs


@pytest.mark.parametrize("rows,cols,seed", [(1, 32, 1), (37, 128, 2), (1000, 576, 3), (5, 64, 4)])
def test_mxfp4_quantize_bit_exact(rows, cols, seed):
    g = synth.rng(100 + seed)
    x = synth.normal(g, (rows, cols)) * np.float32(2.0) ** g.integers(-20, 20, (rows, 1)).astype(np.float32)
    x[0, :32] = 0.0                                     # all-zero tile
    if cols >= 64:
        x[0, 32:64] = np.float32(1.5) * np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6] * 4, np.float32)
    codes, scales = csk.mxfp4_quantize(dev(x))
    rc, rs = oracle.mxfp4_encode(x)
    assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)
    xb = synth.to_bf16(x)                               # bf16 input path
    codes, scales = csk.mxfp4_quantize(dev(xb))
    rc, rs = oracle.mxfp4_encode(oracle.bf16_to_f32(xb))
    assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)


@pytest.mark.parametrize("bf16_in", [False, True])
def test_mxfp4_quantize_unaligned_input(bf16_in):
    # an input 4 bytes past a 16-byte boundary takes the per-pair kernel,
    # an aligned one the sixteen-values-per-lane kernel: both give the
    # oracle's bytes
    g = synth.rng(150)
    rows, cols = 300, 160
    x = synth.normal(g, (rows, cols))
    xh = synth.to_bf16(x) if bf16_in else x
    ref_in = oracle.bf16_to_f32(xh) if bf16_in else x
    rc, rs = oracle.mxfp4_encode(ref_in)
    flat = np.concatenate([np.zeros(2 if bf16_in else 1, xh.dtype), xh.reshape(-1)])
    buf = dev(flat)
    view = buf[2 if bf16_in else 1:].view(rows, cols)
    assert view.data_ptr() % 16 != 0
    for t in (view, dev(xh)):
        codes, scales = csk.mxfp4_quantize(t)
        assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)


@pytest.mark.parametrize("bf16_in", [False, True])
@pytest.mark.parametrize("B,S,D,m,d_rope", [(1, 64, 64, 4, 32), (3, 203, 576, 4, 64), (2, 40, 128, 8, 0)])
def test_csa_compress(bf16_in, B, S, D, m, d_rope):
    g = synth.rng(200 + S + D)
    ca, za, cb, zb = _series(g, B, S, D, bf16_in)
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    ref = oracle.csa_compress(ca, za, cb, zb, ba, bb, m, d_rope=d_rope)
    args = [dev(x) for x in (ca, za, cb, zb, ba, bb)]
    out32 = host(csk.csa_compress(*args, m, d_rope=d_rope, out_dtype=csk.CSK_F32))
    assert out32.shape == ref.shape
    check_f32(out32, ref, 1e-5, "csa fp32 out")
    outb = host(csk.csa_compress(*args, m, d_rope=d_rope, out_dtype=csk.CSK_BF16))
    assert _bf16_ok(outb, ref), np.abs(outb - ref).max()
    if D % 32 == 0 and d_rope == 0:
        codes, scales = csk.csa_compress(*args, m, out_dtype=csk.CSK_MXFP4)
        rc, rs = oracle.mxfp4_encode(out32)
        assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)


@pytest.mark.parametrize("bf16_in", [False, True])
@pytest.mark.parametrize("B,S,D,m,d_rope", [(1, 512, 128, 128, 64), (2, 300, 576, 128, 64), (1, 64, 64, 1, 32)])
def test_hca_compress(bf16_in, B, S, D, m, d_rope):
    g = synth.rng(300 + S + D + m)
    c, z, _, _ = _series(g, B, S, D, bf16_in)
    bias = synth.normal(g, (m, D), 0.1)
    ref = oracle.hca_compress(c, z, bias, m, d_rope=d_rope)
    out32 = host(csk.hca_compress(dev(c), dev(z), dev(bias), m, d_rope=d_rope, out_dtype=csk.CSK_F32))
    check_f32(out32, ref, 1e-5, "hca fp32 out")
    outb = host(csk.hca_compress(dev(c), dev(z), dev(bias), m, d_rope=d_rope, out_dtype=csk.CSK_BF16))
    assert _bf16_ok(outb, ref)


def test_entry_positions_and_constant_pooling():
    g = synth.rng(401)
    B, S, D, m = 2, 64, 128, 4
    ca, za, cb, zb = _series(g, B, S, D, True)
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    pos = g.integers(0, 1 << 20, (B, S // m)).astype(np.int32)
    ref = oracle.csa_compress(ca, za, cb, zb, ba, bb, m, d_rope=64, entry_pos=pos)
    out = host(csk.csa_compress(*[dev(x) for x in (ca, za, cb, zb, ba, bb)], m, d_rope=64,
                                entry_pos=dev(pos), out_dtype=csk.CSK_F32))
    check_f32(out, ref, 1e-5, "entry_pos")
    # a constant source pools to itself (pooling weights sum to 1)
    v = synth.to_bf16(np.full((B, S, D), 0.8125, np.float32))
    out = host(csk.csa_compress(*[dev(x) for x in (v, za, v, zb, ba, bb)], m, out_dtype=csk.CSK_BF16))
    assert np.all(out == np.float32(0.8125))


def test_incremental_equals_one_shot():
    # Appending entries with entry0 > 0 (previous block read from the rows
    # before the first a-block) reproduces one-shot compression, written in
    # place into the full cache through the batch strides.
    g = synth.rng(402)
    B, S, D, m = 3, 96, 576, 4
    ca, za, cb, zb = _series(g, B, S, D, True)
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    t = [dev(x) for x in (ca, za, cb, zb, ba, bb)]
    full = csk.csa_compress(*t, m, d_rope=64)
    cache = torch.zeros_like(full)
    csk.csa_compress(*t, m, d_rope=64, out=cache, S=40, src_bstride=S, dst_bstride=S // m)  # entries 0..9
    off = 40
    tail = [x[:, off:] for x in t[:4]]
    csk.csa_compress(*tail, t[4], t[5], m, d_rope=64, entry0=off // m, src_bstride=S,
                     out=cache[:, off // m:], dst_bstride=S // m, S=S - off)  # entries 10..23
    assert torch.equal(cache.view(torch.int16), full.view(torch.int16))
    # single newest entry (the decode-time append)
    last = torch.zeros_like(full[:, -1:])
    csk.csa_compress(*[x[:, S - m:] for x in t[:4]], t[4], t[5], m, d_rope=64, entry0=S // m - 1,
                     src_bstride=S, out=last, S=m)
    assert torch.equal(last.view(torch.int16), full[:, -1:].view(torch.int16))


def test_ragged_and_empty():
    g = synth.rng(403)
    ca, za, cb, zb = _series(g, 1, 10, 64, False)
    ba, bb = synth.normal(g, (4, 64), 0.1), synth.normal(g, (4, 64), 0.1)
    out = csk.csa_compress(*[dev(x) for x in (ca, za, cb, zb, ba, bb)], 4, out_dtype=csk.CSK_F32)
    assert out.shape == (1, 2, 64)
    check_f32(host(out), oracle.csa_compress(ca, za, cb, zb, ba, bb, 4), 1e-5)
    out = csk.csa_compress(*[dev(x[:, :3]) for x in (ca, za, cb, zb)], dev(ba), dev(bb), 4)
    assert out.shape == (1, 0, 64)
    with pytest.raises(csk.CskError):
        csk.csa_compress(*[dev(x) for x in (ca, za, cb, zb, ba, bb)], 4, d_rope=3)


def _batch_case(g, B, bf16_in):
    """Decode-step jobs (the newest entry of an 8-token window written into
    row N-1 of a cache, its MXFP4 indexer key, the MXFP4 query encode) and a
    whole-sequence compression with a ragged tail and the generic m path."""
    N = 10
    cvt = (lambda a: synth.to_bf16(a)) if bf16_in else (lambda a: a)
    kv_src = [dev(cvt(synth.normal(g, (B, 8, 576)))) for _ in range(4)]
    ik_src = [dev(cvt(synth.normal(g, (B, 8, 128)))) for _ in range(4)]
    seq = [dev(cvt(synth.normal(g, (B, 50, 64)))) for _ in range(4)]
    bias = {k: dev(synth.normal(g, (m, dd), 0.1)) for k, m, dd in
            (("kv_a", 4, 576), ("kv_b", 4, 576), ("ik_a", 4, 128), ("ik_b", 4, 128), ("s_a", 3, 64),
             ("s_b", 3, 64))}
    q = dev(cvt(synth.normal(g, (B, 1, 64, 128)) * np.float32(4.0)))
    pos = dev(np.arange(B, dtype=np.int32).reshape(B, 1) * 7 + 1000)

    def jobs(outs):
        kvc, kc, ks, qc, qs, so = outs
        return [
            ("csa", dict(args=[x[:, 4:] for x in ik_src] + [bias["ik_a"], bias["ik_b"], 4],
                         kw=dict(entry0=N - 1, src_bstride=8, out_dtype=csk.CSK_MXFP4, out=kc[:, N - 1:],
                                 out_scale=ks[:, N - 1:], dst_bstride=N, S=4, B=B))),
            ("mx", dict(args=[q], kw=dict(codes=qc, scales=qs))),
            ("csa", dict(args=[x[:, 4:] for x in kv_src] + [bias["kv_a"], bias["kv_b"], 4],
                         kw=dict(d_rope=64, entry0=N - 1, src_bstride=8, entry_pos=pos, out=kvc[:, N - 1:],
                                 dst_bstride=N, S=4, B=B, out_dtype=csk.CSK_BF16))),
            ("csa", dict(args=seq + [bias["s_a"], bias["s_b"], 3],
                         kw=dict(d_rope=32, out_dtype=csk.CSK_F32, out=so))),
        ]

    def outs():
        return [torch.zeros((B, N, 576), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((B, N, 64), dtype=torch.uint8, device="cuda"),
                torch.zeros((B, N, 4), dtype=torch.uint8, device="cuda"),
                torch.zeros((B, 1, 64, 64), dtype=torch.uint8, device="cuda"),
                torch.zeros((B, 1, 64, 4), dtype=torch.uint8, device="cuda"),
                torch.zeros((B, 16, 64), dtype=torch.float32, device="cuda")]

    return jobs, outs, q, seq, bias


def _same_bytes(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("bf16_in", [False, True])
def test_compress_batch_matches_own_calls(bf16_in):
    # each batched job writes exactly the bytes of its own call (whole
    # buffers are compared, so stray writes would show), twice in a row with
    # the second batch smaller, and in job subsets of every size
    for B, seed in ((4, 1), (1, 2)):
        g = synth.rng(700 + 10 * seed + bf16_in)
        jobs, outs, q, seq, bias = _batch_case(g, B, bf16_in)
        own, bat = outs(), outs()
        for kind, j in jobs(own):
            if kind == "csa":
                csk.csa_compress(*j["args"], **j["kw"])
            else:
                csk.mxfp4_quantize(*j["args"], **j["kw"])
        recs = [csk.csa_job(*j["args"], **j["kw"]) if kind == "csa" else csk.mxfp4_job(*j["args"], **j["kw"])
                for kind, j in jobs(bat)]
        csk.compress_batch(recs)
        torch.cuda.synchronize()
        for a, b in zip(own, bat):
            assert _same_bytes(a, b)
        # the batch against the oracle directly: the encode bit-exact, the
        # fp32 compression within the fp32 bar
        rc, rs = oracle.mxfp4_encode(host(q))  # bf16 inputs come back as their fp32 values
        assert np.array_equal(host(bat[3]), rc) and np.array_equal(host(bat[4]), rs)
        ref = oracle.csa_compress(*[host(x) for x in seq], host(bias["s_a"]), host(bias["s_b"]), 3, d_rope=32)
        check_f32(host(bat[5]), ref, 1e-5, "batched csa fp32 out")
    # one job alone, and a batch whose every job is empty
    jobs, outs, *_ = _batch_case(synth.rng(799), 2, bf16_in)
    own, bat = outs(), outs()
    kind, j = jobs(own)[2]
    csk.csa_compress(*j["args"], **j["kw"])
    kind, j = jobs(bat)[2]
    csk.compress_batch([csk.csa_job(*j["args"], **j["kw"])])
    # fewer source rows than the ratio: no entry, nothing launched or written
    csk.compress_batch([csk.csa_job(*j["args"], **dict(j["kw"], S=3))])
    torch.cuda.synchronize()
    assert _same_bytes(own[0], bat[0])
