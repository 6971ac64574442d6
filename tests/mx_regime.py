"""The exactness regime of MXFP4 dot products on the matrix cores.

An MXFP4 dot product over dI = 32*G elements is a sum of G tile terms
P_g * 2^(e_g), where P_g is an integer (the tile's sum of doubled-code
products, |P_g| <= 32 * 12 * 12 = 4608) and e_g = sq_g + sk_g (the two tiles'
E8M0 exponents, up to a constant). When the e_g of a (query head, key) pair
span at most SPREAD_MAX binades, every partial sum of the G terms, in any
order, is an integer multiple of 2^(min e_g) below 4 * 4608 * 2^9 < 2^24 of
them, so it is exact in fp32: whatever order the matrix core adds the tile
terms in, the result is the exact dot product, which is what the oracle
rounds once. Outside that regime the two may round differently, so every
test that demands bit-exact MXFP4 scores first checks that its inputs lie
inside it.

Tiles whose codes are all zero add nothing and are left out.
"""
import numpy as np

SPREAD_MAX = 9


def _tile_exponents(codes, scales):
    """Per-tile exponents (int) with nonzero tiles marked, flattened to
    [rows, G]."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    G = scales.shape[-1]
    c = codes.reshape(-1, G, 16)
    nonzero = np.any(((c & 0x7) != 0) | (((c >> 4) & 0x7) != 0), axis=-1)
    return scales.reshape(-1, G).astype(np.int64), nonzero


def _spread(e, nz):
    hi = np.where(nz, e, -10**6).max(axis=-1)
    lo = np.where(nz, e, 10**6).min(axis=-1)
    return np.where(nz.any(axis=-1), hi - lo, 0)


def pair_spread_bound(q_codes, q_scales, k_codes, k_scales):
    """An upper bound of the combined tile-exponent spread over every (query
    row and head, key) pair: spread(q) + spread(k) >= max_g(eq+ek) -
    min_g(eq+ek) for each pair."""
    eq, nq = _tile_exponents(q_codes, q_scales)
    ek, nk = _tile_exponents(k_codes, k_scales)
    return int(_spread(eq, nq).max(initial=0) + _spread(ek, nk).max(initial=0))


def pair_spread_exact(q_codes, q_scales, k_codes, k_scales):
    """The largest combined spread over every pair (small inputs only)."""
    eq, nq = _tile_exponents(q_codes, q_scales)
    ek, nk = _tile_exponents(k_codes, k_scales)
    e = eq[:, None, :] + ek[None, :, :]
    nz = nq[:, None, :] & nk[None, :, :]
    return int(_spread(e, nz).max(initial=0))


def assert_in_regime(q_codes, q_scales, k_codes, k_scales):
    """Every (query head, key) pair lies in the exactness regime."""
    b = pair_spread_bound(q_codes, q_scales, k_codes, k_scales)
    if b <= SPREAD_MAX:
        return b
    nq = np.asarray(q_scales).size // np.asarray(q_scales).shape[-1]
    nk = np.asarray(k_scales).size // np.asarray(k_scales).shape[-1]
    assert nq * nk <= 1 << 24, f"tile-exponent spread bound {b} > {SPREAD_MAX} on a large input"
    s = pair_spread_exact(q_codes, q_scales, k_codes, k_scales)
    assert s <= SPREAD_MAX, f"a (query head, key) pair spans {s} > {SPREAD_MAX} binades"
    return s
