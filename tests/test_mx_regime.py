"""CPU checks of the MXFP4 exactness regime (tests/mx_regime.py) and of the
synthetic workloads' place in it."""
import itertools

import numpy as np

import oracle
import synth
from mx_regime import SPREAD_MAX, assert_in_regime, pair_spread_bound, pair_spread_exact


def _orders_of_tile_sum(P, e):
    """All results of adding the tile terms P_g * 2^e_g in fp32, one per order
    (every partial sum rounded to fp32), and the exact sum."""
    terms = [np.float32(np.ldexp(float(p), int(x))) for p, x in zip(P, e)]
    assert all(float(t) == float(np.ldexp(float(p), int(x))) for t, p, x in zip(terms, P, e))
    res = set()
    for perm in itertools.permutations(range(len(terms))):
        acc = np.float32(0.0)
        for i in perm:
            acc = np.float32(acc + terms[i])
        res.add(float(acc))
    exact = sum(float(np.ldexp(float(p), int(x))) for p, x in zip(P, e))
    return res, exact


def test_regime_bound_is_tight():
    # The worst tile terms (|P_g| = 4608, and odd terms that need the lowest
    # bit) at a spread of 9 binades: every fp32 summation order gives the
    # exact sum. At 12 binades some order does not, so the bound cannot be
    # widened to there.
    for spread, P in ((9, [4608, 4608, 4608, 4607]), (9, [4607, -4608, 4608, 1]), (6, [4608, 3, 4608, 4607])):
        res, exact = _orders_of_tile_sum(P, [spread, spread, spread, 0][:len(P)])
        assert res == {exact}, (spread, P, res, exact)
    res, exact = _orders_of_tile_sum([4608, 4608, 4608, 4607], [12, 12, 12, 0])
    assert res != {exact}


def test_spread_of_crafted_pairs():
    # one query head and one key, four tiles: codes all nonzero
    qc = np.full((1, 64), 0x22, np.uint8)
    kc = np.full((1, 64), 0x22, np.uint8)
    qs = np.array([[127, 130, 127, 127]], np.uint8)
    ks = np.array([[127, 127, 133, 127]], np.uint8)
    assert pair_spread_exact(qc, qs, kc, ks) == 6 and pair_spread_bound(qc, qs, kc, ks) == 9
    ks2 = np.array([[127, 127, 134, 120]], np.uint8)
    assert pair_spread_exact(qc, qs, kc, ks2) == 14
    try:
        assert_in_regime(qc, qs, kc, ks2)
        raise RuntimeError("a 14-binade pair passed")
    except AssertionError:
        pass
    # an all-zero tile adds nothing: its exponent does not count
    kz = kc.copy()
    kz[0, 48:64] = 0
    assert pair_spread_exact(qc, qs, kz, ks2) == 7


def test_decode_workload_inputs_lie_in_regime():
    # the decode workloads' N(0,1) indexer queries and keys, quantised by the
    # method's encoder: tile exponents fall in a 4-binade band, so every pair
    # spans at most 6 binades (sizes shrunk; the distributions are the same)
    d = synth.make("decode_1m_pair", B=2, ctx=65536)
    qc, qs = oracle.mxfp4_encode(d["qI"])
    kc, ks = oracle.mxfp4_encode(d["kI"])
    assert pair_spread_bound(qc, qs, kc, ks) <= 6
    assert assert_in_regime(qc, qs, kc, ks) <= SPREAD_MAX


def test_prefill_workload_inputs_lie_in_regime():
    # CSA prefill: keys are the pooled indexer series (narrower than N(0,1)),
    # queries N(0,1)
    d = synth.make("csa_prefill_64k", S=4096)
    keys = oracle.round_f32(oracle.csa_compress(*(d[n] for n in ("ia", "iza", "ib", "izb", "ibias_a", "ibias_b")),
                                                d["m"]))
    kc, ks = oracle.mxfp4_encode(keys)
    qc, qs = oracle.mxfp4_encode(d["qI"][:, ::16])
    assert assert_in_regime(qc, qs, kc, ks) <= SPREAD_MAX
