"""Pins for the oracle's MXFP4 encoder/decoder (E2M1 elements, one
power-of-two scale per 1x32 tile): brute force over every code and scale,
every rounding tie, saturation, zero handling and packing order."""
import numpy as np

import oracle
import synth

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _tile(vals):
    x = np.zeros(32, np.float32)
    x[:len(vals)] = vals
    return x


def _codes_of(codes_bytes):
    b = np.asarray(codes_bytes).reshape(-1)
    out = np.empty(b.size * 2, np.uint8)
    out[0::2] = b & 15
    out[1::2] = b >> 4
    return out


def test_all_codes_all_scales_roundtrip():
    # Every representable value survives encode -> decode exactly, for every
    # scale: a tile holding +-6*2^s pins the shared scale to s.
    for s in range(-127, 128, 7):
        for code in range(16):
            v = (-1 if code & 8 else 1) * GRID[code & 7] * 2.0 ** s
            x = _tile([6.0 * 2.0 ** s, -6.0 * 2.0 ** s, v])
            if not np.all(np.isfinite(x)) or (2.0 ** s * 6.0) < 1e-44:
                continue
            c, sc = oracle.mxfp4_encode(x[None])
            assert sc[0, 0] == s + 127
            codes = _codes_of(c)
            expect = code if (code & 7) != 0 else 0        # -0 encodes as +0
            assert codes[2] == expect, (s, code)
            y = oracle.mxfp4_decode(c, sc)[0]
            assert y[2] == np.float32(v if (code & 7) else 0.0)


def test_ties_to_even_and_saturation():
    # scale 0 (amax in [4, 8)); halfway points go to the even-mantissa code
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             0.2500001: 0.5, 0.7499999: 0.5, 1.2500001: 1.5, 4.9999995: 4.0, 5.0000005: 6.0,
             6.0: 6.0, 7.99: 6.0, 0.1: 0.0}
    for v, expect in cases.items():
        for sign in (1.0, -1.0):
            x = _tile([7.0, sign * v])
            c, sc = oracle.mxfp4_encode(x[None])
            assert sc[0, 0] == 127
            y = oracle.mxfp4_decode(c, sc)[0, 1]
            assert y == np.float32(sign * expect) or (expect == 0.0 and y == 0.0), (v, sign, y)
            if expect == 0.0:
                assert _codes_of(c)[1] == 0          # zero is always the +0 code


def test_scale_choice_and_zero_tile():
    for amax, s in ((4.0, 0), (7.999, 0), (8.0, 1), (3.99, -1), (1.0, -2), (0.75, -3), (2.0 ** -130, -127),
                    (1e30, 97)):
        c, sc = oracle.mxfp4_encode(_tile([amax])[None])
        assert int(sc[0, 0]) - 127 == s, (amax, sc)
    c, sc = oracle.mxfp4_encode(np.zeros((3, 64), np.float32))
    assert np.all(sc == 127) and np.all(c == 0)
    c, sc = oracle.mxfp4_encode(np.full((1, 32), -0.0, np.float32))
    assert np.all(c == 0)


def test_nearest_value_brute_force_and_packing():
    # Random tiles: each decoded element is a nearest grid point of x/2^s
    # (saturated at 6), found here by brute force over the 8 magnitudes.
    g = synth.rng(21)
    x = synth.normal(g, (200, 64)) * np.float32(3.0)
    c, sc = oracle.mxfp4_encode(x)
    y = oracle.mxfp4_decode(c, sc).astype(np.float64)
    s = sc.astype(np.int64) - 127
    for r in range(x.shape[0]):
        for t in range(2):
            amax = np.max(np.abs(x[r, 32 * t:32 * t + 32]).astype(np.float64))
            assert s[r, t] == np.floor(np.log2(amax)) - 2
            q = np.abs(x[r, 32 * t:32 * t + 32].astype(np.float64)) / 2.0 ** s[r, t]
            dist = np.abs(q[:, None] - GRID[None, :])
            best = dist.min(axis=1)
            got = np.abs(y[r, 32 * t:32 * t + 32]) / 2.0 ** s[r, t]
            assert np.all(np.abs(np.abs(got - q) - best) == 0)
    # packing: element 2j in the low nibble of byte j
    xx = _tile([6.0, 1.0, -0.5, 3.0])
    c, sc = oracle.mxfp4_encode(xx[None])
    assert c[0, 0] == (7 | (2 << 4)) and c[0, 1] == ((1 | 8) | (5 << 4))
