"""GPU parity on the five workloads at their stated sizes.

Each workload runs through the same entry points and launch configuration
as bench.py. Where the oracle is too slow for every output, it checks
sampled rows (first, last and boundary positions). Top-k is compared
bit-exactly whenever both sides see identical input bytes; a whole-pipeline
comparison (each side with its own compressed keys) accepts a differing row
only if the GPU's selection is a valid top-k under the oracle's scores up to
the fp32-vs-fp64 compression difference."""
import numpy as np
import pytest

import oracle
import synth
from util import check_bf16_attention, check_f32, dev, host

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")


def _valid_topk(gi, scores_row, nv, k, eps):
    """gi is a valid top-k of scores_row[:nv] if every selected score is >= the
    k-th best score - eps and every unselected one <= it + eps."""
    sel = gi[gi >= 0]
    if len(sel) != min(k, nv) or len(set(sel.tolist())) != len(sel) or np.any(sel >= nv):
        return False
    s = scores_row[:nv].astype(np.float64)
    if nv <= k:
        return True
    kth = np.sort(s)[::-1][k - 1]
    mask = np.zeros(nv, bool)
    mask[sel] = True
    return s[mask].min() >= kth - eps and (s[~mask].max() if (~mask).any() else -np.inf) <= kth + eps


def test_tiny_csa_prefill_fp32():
    d = synth.make("tiny_csa_prefill")
    m, k, W, dr, sc = d["m"], d["k"], d["W"], d["d_rope"], d["scale"]
    t = {n: dev(d[n]) for n in d if isinstance(d[n], np.ndarray)}
    # GPU pipeline
    kv = csk.csa_compress(t["ca"], t["za"], t["cb"], t["zb"], t["bias_a"], t["bias_b"], m, d_rope=dr)
    keys = csk.csa_compress(t["ia"], t["iza"], t["ib"], t["izb"], t["ibias_a"], t["ibias_b"], m)
    ne = np.array([kv.shape[1]], np.int32)
    gidx, gsc = csk.indexer_topk(t["qI"], t["w"], keys, t["q_pos"], dev(ne), m, k)
    gout, glse = csk.sparse_attn(t["q"], t["q_pos"], kv, gidx, t["kv_w"], t["w_pos0"], W, t["sink"], d["dv"], dr, sc)
    # oracle pipeline
    rkv = oracle.round_f32(oracle.csa_compress(d["ca"], d["za"], d["cb"], d["zb"], d["bias_a"], d["bias_b"], m,
                                               d_rope=dr))
    rkeys = oracle.round_f32(oracle.csa_compress(d["ia"], d["iza"], d["ib"], d["izb"], d["ibias_a"],
                                                 d["ibias_b"], m))
    check_f32(host(kv), rkv, 1e-5, "kv")
    check_f32(host(keys), rkeys, 1e-5, "keys")
    ridx, rsc = oracle.indexer_topk(d["qI"], d["w"], rkeys, d["q_pos"], ne, m, k)
    # identical inputs: bit-exact
    eidx, esc = csk.indexer_topk(t["qI"], t["w"], dev(rkeys), t["q_pos"], dev(ne), m, k)
    assert np.array_equal(host(eidx).reshape(-1, k), ridx)
    assert np.array_equal(host(esc).reshape(-1, k).view(np.uint32), rsc.view(np.uint32))
    # whole pipeline: rows may differ only on near-ties
    rs_full, nv = oracle.indexer_scores(d["qI"], d["w"], rkeys, d["q_pos"], ne, m)
    gi = host(gidx).reshape(-1, k)
    same = np.all(gi == ridx, axis=1)
    for r in np.where(~same)[0]:
        assert _valid_topk(gi[r], rs_full[r], nv[r], k, 1e-4), f"row {r} is not a valid top-k"
    assert same.mean() >= 0.97
    rout, rlse = oracle.sparse_attn(d["q"], d["q_pos"], rkv, ridx[None], d["kv_w"], d["w_pos0"], W, d["sink"],
                                    d["dv"], dr, sc)
    go = host(gout).reshape(-1, d["H"], d["dv"])
    check_f32(go[same], rout[same], 1e-5, "attention")
    check_f32(host(glse).reshape(-1, d["H"])[same], rlse[same], 1e-5, "lse")


def test_hca_prefill_16k():
    d = synth.make("hca_prefill_16k")
    m, W, dr, sc, H, D = d["m"], d["W"], d["d_rope"], d["scale"], d["H"], d["D"]
    S = d["q"].shape[1]
    kv = csk.hca_compress(dev(d["c"]), dev(d["z"]), dev(d["bias"]), m, d_rope=dr)
    rkv64 = oracle.hca_compress(d["c"], d["z"], d["bias"], m, d_rope=dr)
    from util import bf16_ulp
    assert np.all(np.abs(host(kv) - rkv64) <= bf16_ulp(rkv64) + 1e-5)
    rkv = oracle.round_bf16(rkv64)
    ne = np.array([kv.shape[1]], np.int32)
    out, lse = csk.dense_compressed_attn(dev(d["q"]), dev(d["q_pos"]), kv, dev(ne), m, dev(d["kv_w"]),
                                         dev(d["w_pos0"]), W, dev(d["sink"]), D, dr, sc)
    ts = sorted(set([0, 1, 126, 127, 128, 129, 255, 256, 4095, 4096, 8191, 12000, S - 129, S - 128, S - 1]
                    + list(range(17, S, 997))))
    rout, rlse = oracle.dense_attn(d["q"][:, ts], d["q_pos"][:, ts], rkv, ne, m, d["kv_w"], d["w_pos0"], W,
                                   d["sink"], D, dr, sc)
    go = host(out)[0, ts]
    check_bf16_attention(go, rout, "hca prefill")
    check_f32(host(lse)[0, ts], rlse, 2e-2, "lse")


def _decode_parity(name, overrides=None):
    import bench

    wl = bench.DecodeWorkload(name, copies=1, overrides=overrides)
    wl.step(0)
    torch.cuda.synchronize()
    rows = list(range(wl.B))
    ref = wl.oracle_step(rows)
    st = wl.copies[0]
    N = wl.N
    # appended entries
    from util import bf16_ulp
    got_kv = host(st["kv_c"][:, N - 1])
    want_kv = oracle.bf16_to_f32(ref["kv_new"])
    assert np.all(np.abs(got_kv - want_kv) <= 2 * bf16_ulp(want_kv) + 1e-5)
    kn_c, kn_s = ref["key_new"]
    assert np.array_equal(host(st["kc"][:, N - 1]), kn_c) and np.array_equal(host(st["ks"][:, N - 1]), kn_s), \
        "newest MXFP4 key differs (fp32 vs fp64 rounding decision)"
    assert np.array_equal(host(wl.qc), ref["qc"]) and np.array_equal(host(wl.qs), ref["qs"])
    # the key cache was quantised on each side from the same fp32 values: the
    # bytes are identical, so top-k must match bit-exactly
    assert np.array_equal(host(st["kc"]), ref["kc"]) and np.array_equal(host(st["ks"]), ref["ks"])
    gi = host(wl.idx).reshape(wl.B, -1)
    assert np.array_equal(gi, ref["idx"])
    assert np.array_equal(host(wl.score).reshape(wl.B, -1).view(np.uint32), ref["score"].view(np.uint32))
    check_bf16_attention(host(wl.out).reshape(ref["out"].shape), ref["out"], "csa attention")
    check_f32(host(wl.lse).reshape(ref["lse"].shape), ref["lse"], 2e-2, "csa lse")
    if wl.pair:
        check_bf16_attention(host(wl.out_h).reshape(ref["out_h"].shape), ref["out_h"], "hca attention")
        check_f32(host(wl.lse_h).reshape(ref["lse_h"].shape), ref["lse_h"], 2e-2, "hca lse")
    return wl


def test_csa_decode_128k():
    _decode_parity("csa_decode_128k")


def test_decode_1m_pair():
    wl = _decode_parity("decode_1m_pair")
    # graph replays reproduce the eager step bit for bit, with eager work and
    # synchronisation between the replays
    eager = (wl.idx.clone(), wl.out.clone(), wl.out_h.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        wl.step(0)
    for rep in range(3):
        wl.idx.fill_(-7)
        wl.out.zero_()
        wl.out_h.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(wl.idx, eager[0]), rep
        assert torch.equal(wl.out.view(torch.int16), eager[1].view(torch.int16)), rep
        assert torch.equal(wl.out_h.view(torch.int16), eager[2].view(torch.int16)), rep


def test_csa_prefill_64k_sampled():
    d = synth.make("csa_prefill_64k")
    m, k, W, dr, sc, H, D, dv = d["m"], d["k"], d["W"], d["d_rope"], d["scale"], d["H"], d["D"], d["dv"]
    S = d["q_pos"].shape[1]
    # compression: GPU vs oracle
    t4 = [dev(d[n]) for n in ("ca", "za", "cb", "zb", "bias_a", "bias_b")]
    kv = csk.csa_compress(*t4, m, d_rope=dr)
    kv32 = csk.csa_compress(*t4, m, d_rope=dr, out_dtype=csk.CSK_F32)
    rkv64 = oracle.csa_compress(*(d[n] for n in ("ca", "za", "cb", "zb", "bias_a", "bias_b")), m, d_rope=dr)
    check_f32(host(kv32), rkv64, 1e-5, "kv fp32")
    del kv32
    rkv = oracle.round_bf16(rkv64)
    del rkv64
    ti = [dev(d[n]) for n in ("ia", "iza", "ib", "izb", "ibias_a", "ibias_b")]
    kc, ks = csk.csa_compress(*ti, m, out_dtype=csk.CSK_MXFP4)
    k32 = host(csk.csa_compress(*ti, m, out_dtype=csk.CSK_F32))
    gc_from_gpu32, gs_from_gpu32 = oracle.mxfp4_encode(k32)
    assert np.array_equal(host(kc), gc_from_gpu32) and np.array_equal(host(ks), gs_from_gpu32)
    rk64 = oracle.csa_compress(*(d[n] for n in ("ia", "iza", "ib", "izb", "ibias_a", "ibias_b")), m)
    check_f32(k32, rk64, 1e-5, "keys fp32")
    rkc, rks = oracle.mxfp4_encode(oracle.round_f32(rk64))
    # queries
    qc, qs = csk.mxfp4_quantize(dev(d["qI"]))
    ts = sorted(set([0, 3, 4, 7, 8191, 8192, 8195, 30000, S - 5, S - 1] + list(range(101, S, 7919))))
    rqc, rqs = oracle.mxfp4_encode(d["qI"][:, ts])
    assert np.array_equal(host(qc)[:, ts], rqc) and np.array_equal(host(qs)[:, ts], rqs)
    ne = np.array([rkc.shape[1]], np.int32)
    q_pos = dev(d["q_pos"])
    # indexer on identical bytes (the oracle's keys), full launch over all rows
    eidx, esc = csk.indexer_topk(qc, dev(d["w"]), dev(rkc), q_pos, dev(ne), m, k, q_scale=qs, k_scale=dev(rks))
    ridx, rsc = oracle.indexer_topk(rqc, d["w"][:, ts], rkc, d["q_pos"][:, ts], ne, m, k, q_scale=rqs,
                                    k_scale=rks)
    assert np.array_equal(host(eidx)[0, ts], ridx)
    assert np.array_equal(host(esc)[0, ts].view(np.uint32), rsc.view(np.uint32))
    del eidx, esc
    # whole GPU pipeline with its own keys and cache
    gidx, _ = csk.indexer_topk(qc, dev(d["w"]), kc, q_pos, dev(ne), m, k, q_scale=qs, k_scale=ks, with_score=False)
    out, lse = csk.sparse_attn(dev(d["q"]), q_pos, kv, gidx, dev(d["kv_w"]), dev(d["w_pos0"]), W, dev(d["sink"]),
                               dv, dr, sc, want_lse=True)
    gi = host(gidx)[0, ts]
    same = np.all(gi == ridx, axis=1)
    assert same.mean() >= 0.9, same
    rout, rlse = oracle.sparse_attn(d["q"][:, ts], d["q_pos"][:, ts], rkv, ridx[None], d["kv_w"], d["w_pos0"], W,
                                    d["sink"], dv, dr, sc)
    go = host(out)[0, ts]
    check_bf16_attention(go[same], rout[same], "csa prefill attention")
    check_f32(host(lse)[0, ts][same], rlse[same], 2e-2, "lse")
