"""Pins for the oracle's compression (CSA / HCA pooling) and partial RoPE.

Each test checks the oracle against something other than itself: a closed
form, an invariant the pages imply, a count the pages state, or an
independent numpy computation.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def _series(g, B, S, D, n=4):
    return [synth.normal(g, (B, S, D)) for _ in range(n)]


def test_constant_kv_pools_to_itself():
    # Pooling weights are a softmax: a constant source pools to that constant,
    # whatever the gate logits and biases (weights sum to 1 per entry/channel).
    g = synth.rng(11)
    B, S, D, m = 2, 40, 16, 4
    _, za, _, zb = _series(g, B, S, D)
    v = np.float32(0.3721)
    c = np.full((B, S, D), v, np.float32)
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    out = oracle.csa_compress(c, za * 5, c, zb * 5, ba, bb, m)
    assert np.all(oracle.round_f32(out) == v)
    ones = np.ones((B, S, D), np.float32)
    out1 = oracle.csa_compress(ones, za, ones, zb, ba, bb, m)
    assert np.all(oracle.round_f32(out1) == np.float32(1.0))
    outh = oracle.hca_compress(c, za, synth.normal(g, (8, D), 0.1), 8)
    assert np.all(oracle.round_f32(outh) == v)


def test_equal_gates_give_window_mean():
    # Exercise 2 ("compare with a plain window average"): with equal gate
    # logits and zero biases every softmax weight is equal, so each entry is
    # the mean of its 2m sources (m for entry 0, which has no previous block).
    g = synth.rng(12)
    B, S, D, m = 1, 32, 8, 4
    ca, _, cb, _ = _series(g, B, S, D)
    z = np.zeros((B, S, D), np.float32)
    zero = np.zeros((m, D), np.float32)
    out = oracle.csa_compress(ca, z, cb, z, zero, zero, m)
    N = S // m
    for i in range(N):
        srcs = [ca[0, m * i:m * i + m]]
        if i > 0:
            srcs.append(cb[0, m * (i - 1):m * i])
        mean = np.concatenate(srcs).astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[0, i], mean, rtol=0, atol=1e-12)
    outh = oracle.hca_compress(ca, z, np.zeros((16, D), np.float32), 16)
    np.testing.assert_allclose(outh[0], ca[0].astype(np.float64).reshape(2, 16, D).mean(axis=1), atol=1e-12)


def test_worked_example_rational_weights():
    # m = 2, one channel. Entry 1 pools a-slots {z=0, z=ln 3} and b-slots
    # {z=ln 2, z=ln 2} with biases 0: weights 1:3:2:2 over 8 -> closed form.
    l3, l2 = np.float32(math.log(3.0)), np.float32(math.log(2.0))
    ca = np.array([[[10.0], [20.0], [1.0], [5.0]]], np.float32)
    za = np.array([[[0.0], [0.0], [0.0], [l3]]], np.float32)
    cb = np.array([[[7.0], [-3.0], [0.0], [0.0]]], np.float32)
    zb = np.array([[[l2], [l2], [0.0], [0.0]]], np.float32)
    zero = np.zeros((2, 1), np.float32)
    out = oracle.csa_compress(ca, za, cb, zb, zero, zero, 2)
    assert out.shape == (1, 2, 1)
    assert abs(out[0, 0, 0] - 15.0) < 1e-12                     # entry 0: mean of 10, 20
    expect = (1 * 1.0 + 3 * 5.0 + 2 * 7.0 + 2 * (-3.0)) / 8.0     # = 3.0
    assert abs(out[0, 1, 0] - expect) < 1e-6


def test_gate_shift_invariance_and_one_hot():
    g = synth.rng(13)
    B, S, D, m = 1, 24, 8, 4
    ca, za, cb, zb = _series(g, B, S, D)
    za, zb = np.round(za * 1024) / 1024, np.round(zb * 1024) / 1024   # so that z + 3 is exact
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    o1 = oracle.csa_compress(ca, za, cb, zb, ba, bb, m)
    o2 = oracle.csa_compress(ca, za + 3.0, cb, zb + 3.0, ba, bb, m)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    # a dominant logit selects its source
    za2, zb2 = np.zeros_like(za), np.zeros_like(zb)
    za2[0, 4 * 2 + 1, :] = 200.0   # entry 2, a-slot 1
    o3 = oracle.csa_compress(ca, za2, cb, zb2, np.zeros((m, D), np.float32), np.zeros((m, D), np.float32), m)
    np.testing.assert_allclose(o3[0, 2], ca[0, 9].astype(np.float64), atol=1e-12)
    zb3 = np.zeros_like(zb)
    zb3[0, 4 * 1 + 3, :] = 200.0   # b-slot 3 of entry 2 is token 7
    o4 = oracle.csa_compress(ca, np.zeros_like(za), cb, zb3, np.zeros((m, D), np.float32),
                             np.zeros((m, D), np.float32), m)
    np.testing.assert_allclose(o4[0, 2], cb[0, 7].astype(np.float64), atol=1e-12)


def test_overlap_geometry_by_perturbation():
    # Entry i draws on 2m sources with stride m: a-series token j feeds only
    # entry j//m; b-series token j feeds only entry j//m + 1.
    g = synth.rng(14)
    B, S, D, m = 1, 32, 4, 4
    ca, za, cb, zb = _series(g, B, S, D)
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    base = oracle.csa_compress(ca, za, cb, zb, ba, bb, m)
    for j in (0, 5, 14, 31):
        ca2 = ca.copy(); ca2[0, j] += 1.0
        changed = np.where(np.any(oracle.csa_compress(ca2, za, cb, zb, ba, bb, m) != base, axis=(0, 2)))[0]
        assert changed.tolist() == [j // m]
        cb2 = cb.copy(); cb2[0, j] += 1.0
        changed = np.where(np.any(oracle.csa_compress(ca, za, cb2, zb, ba, bb, m) != base, axis=(0, 2)))[0]
        assert changed.tolist() == ([j // m + 1] if j // m + 1 < S // m else [])


def test_hca_m1_is_identity_and_prefix_causal():
    g = synth.rng(15)
    B, S, D = 2, 20, 8
    c, z = synth.normal(g, (B, S, D)), synth.normal(g, (B, S, D))
    out = oracle.hca_compress(c, z, synth.normal(g, (1, D), 0.1), 1)
    assert np.all(out == c.astype(np.float64))
    # prefix compression equals the first entries of the full compression
    ca, za, cb, zb = _series(g, B, 64, D)
    ba, bb = synth.normal(g, (4, D), 0.1), synth.normal(g, (4, D), 0.1)
    full = oracle.csa_compress(ca, za, cb, zb, ba, bb, 4, d_rope=4)
    pre = oracle.csa_compress(ca[:, :36], za[:, :36], cb[:, :36], zb[:, :36], ba, bb, 4, d_rope=4)
    assert np.array_equal(full[:, :9], pre)


def test_entry_counts_match_pages():
    # Exercise 1: entries left at 1M tokens for m = 4 and m' = 128; the
    # CSA decode workload: 131072 -> 32768.
    for S, m, key in ((1 << 20, 4, "entries_at_1M_csa"), (1 << 17, 4, "entries_at_128K_csa")):
        x = np.zeros((1, S, 1), np.float32)
        out = oracle.csa_compress(x, x, x, x, np.zeros((m, 1), np.float32), np.zeros((m, 1), np.float32), m)
        assert out.shape[1] == GOLDEN[key]["value"]
    x = np.zeros((1, 1 << 20, 1), np.float32)
    out = oracle.hca_compress(x, x, np.zeros((128, 1), np.float32), 128)
    assert out.shape[1] == GOLDEN["entries_at_1M_hca"]["value"]
    # a ragged tail produces no entry
    x = np.zeros((1, 4 * 5 + 3, 2), np.float32)
    assert oracle.csa_compress(x, x, x, x, np.zeros((4, 2), np.float32), np.zeros((4, 2), np.float32), 4).shape[1] == 5


# ------------------------------------------------------------------ RoPE

def _rope_complex(x, pos, d_rope, base):
    """Independent RoPE: interleaved pairs as complex numbers times e^{i a}."""
    x = np.asarray(x, np.float64).copy()
    D = x.shape[-1]
    j = np.arange(d_rope // 2)
    ang = pos * np.power(float(base), -2.0 * j / d_rope)
    z = x[D - d_rope::2] + 1j * x[D - d_rope + 1::2]
    z = z * np.exp(1j * ang)
    x[D - d_rope::2], x[D - d_rope + 1::2] = z.real, z.imag
    return x


def test_rope_invariants():
    g = synth.rng(16)
    D, dr = 48, 16
    x = synth.normal(g, (D,)).astype(np.float64)
    y = synth.normal(g, (D,)).astype(np.float64)
    assert np.array_equal(oracle.rope(x, 0, dr), x)                     # position 0 is the identity
    r = oracle.rope(x, 12345, dr)
    assert np.array_equal(r[:D - dr], x[:D - dr])                       # only the last d_rope dims turn
    pn = lambda v: np.hypot(v[D - dr::2], v[D - dr + 1::2])
    np.testing.assert_allclose(pn(r), pn(x), rtol=1e-13)               # pair norms preserved
    for p1, p2 in ((100, 40), (1000060, 1000000)):                      # q.k depends on p1 - p2 only
        a = oracle.rope(x, p1, dr) @ oracle.rope(y, p2, dr)
        b = oracle.rope(x, p1 - p2, dr) @ oracle.rope(y, 0, dr)
        assert abs(a - b) < 1e-9 * (1 + abs(a))
    np.testing.assert_allclose(oracle.rope(x, 777, dr), _rope_complex(x, 777, dr, 10000.0), atol=1e-12)
    e = np.zeros(D); e[D - dr] = 1.0                                    # pair 0 turns by exactly pos radians
    r = oracle.rope(e, 1.0, dr)
    assert abs(r[D - dr] - math.cos(1.0)) < 1e-15 and abs(r[D - dr + 1] - math.sin(1.0)) < 1e-15


def test_compress_rope_applied_at_entry_position():
    g = synth.rng(17)
    B, S, D, m, dr = 1, 32, 16, 4, 8
    ca, za, cb, zb = _series(g, B, S, D)
    ba, bb = synth.normal(g, (m, D), 0.1), synth.normal(g, (m, D), 0.1)
    plain = oracle.csa_compress(ca, za, cb, zb, ba, bb, m)
    rot = oracle.csa_compress(ca, za, cb, zb, ba, bb, m, d_rope=dr)
    pos = np.array([[5, 1000, 3, 77, 8, 9, 10, 1048575]], np.int32)
    rot2 = oracle.csa_compress(ca, za, cb, zb, ba, bb, m, d_rope=dr, entry_pos=pos)
    for i in range(S // m):
        np.testing.assert_allclose(rot[0, i], _rope_complex(plain[0, i], m * i, dr, 1e4), atol=1e-12)
        np.testing.assert_allclose(rot2[0, i], _rope_complex(plain[0, i], pos[0, i], dr, 1e4), atol=1e-12)


# -------------------------------------------------------------- rounding

def test_round_bf16_matches_torch_and_nearest():
    torch = pytest.importorskip("torch")
    g = synth.rng(18)
    x32 = np.concatenate([synth.normal(g, (5000,)) * 10.0 ** g.integers(-30, 30, 5000).astype(np.float32),
                          np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5e-39, 3.3895e38], np.float32)])
    ours = oracle.round_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # doubles off the float32 grid: the result is a nearest bf16 neighbour
    xd = synth.normal(g, (2000,)).astype(np.float64) * (1 + 1e-12)
    got = oracle.bf16_to_f32(oracle.round_bf16(xd)).astype(np.float64)
    err = np.abs(got - xd)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(xd))) - 7)
    assert np.all(err <= ulp / 2)
