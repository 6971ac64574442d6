"""Pins of the oracle's grouped output projection (the heads' outputs split
into g groups, each projected to an intermediate width, the intermediates
projected to the hidden size; DeepSeek-V4 technical report page, «CSA:
сжать в 4 раза и выбрать top-k», step 4). Reading pinned here: the
intermediate is rounded once to bf16 before the second projection."""
import numpy as np
import scipy.linalg

import oracle


def test_hand_worked_two_groups():
    # heads (1, 2 | 3, 4), one value each, two heads per group:
    # u = (1 + 2, 2*3 - 4) = (3, 2); y = 3 + 10*2 = 23
    o = np.array([[1, 2, 3, 4]], np.float32)
    w1 = np.array([[[1, 1]], [[2, -1]]], np.float32)
    w2 = np.array([[1, 10]], np.float32)
    y, u = oracle.grouped_out_proj(o, w1, w2)
    assert u.tolist() == [[3.0, 2.0]]
    assert y.tolist() == [[23.0]]


def test_intermediate_rounded_once_to_bf16():
    # bf16 spacing is 2 on [256, 512): 257 is a tie (to even: 256), 257.5
    # rounds to 258, 259 is a tie (to even: 260)
    w1 = np.array([[[1, 1]], [[0, 0]]], np.float32)
    w2 = np.array([[1, 1]], np.float32)
    for a, want in ((1.0, 256.0), (1.5, 258.0), (3.0, 260.0)):
        y, u = oracle.grouped_out_proj(np.array([[256, a, 7, 7]], np.float32), w1, w2)
        assert u[0, 0] == want and u[0, 1] == 0.0
        assert y[0, 0] == want


def test_equals_block_diagonal_projection():
    # small integers: every sum is exact and the intermediates are exact in
    # bf16, so the grouped form must equal one projection by the
    # block-diagonal matrix of the group matrices, then the second one
    g = np.random.default_rng(7)
    R, H, dv, G, dg, d = 7, 8, 3, 4, 5, 6
    K1 = H // G * dv
    o = g.integers(-3, 4, (R, H * dv)).astype(np.float32)
    w1 = g.integers(-2, 3, (G, dg, K1)).astype(np.float32)
    w2 = g.integers(-2, 3, (d, G * dg)).astype(np.float32)
    y, u = oracle.grouped_out_proj(o, w1, w2)
    bd = scipy.linalg.block_diag(*[w1[i].astype(np.float64) for i in range(G)])   # [G*dg, H*dv]
    u_ref = o.astype(np.float64) @ bd.T
    assert np.abs(u_ref).max() <= 256
    assert np.array_equal(u, u_ref)
    assert np.array_equal(y, u_ref @ w2.astype(np.float64).T)


def test_groups_are_independent():
    # changing the heads of one group changes only that group's intermediates
    g = np.random.default_rng(8)
    R, G, dg, K1, d = 3, 4, 6, 10, 5
    o = g.standard_normal((R, G * K1)).astype(np.float32)
    w1 = g.standard_normal((G, dg, K1)).astype(np.float32)
    w2 = g.standard_normal((d, G * dg)).astype(np.float32)
    _, u0 = oracle.grouped_out_proj(o, w1, w2)
    o2 = o.copy()
    o2[:, 2 * K1:3 * K1] += 1.0
    _, u1 = oracle.grouped_out_proj(o2, w1, w2)
    changed = np.any(u0 != u1, axis=0).reshape(G, dg).any(axis=1)
    assert changed.tolist() == [False, False, True, False]
