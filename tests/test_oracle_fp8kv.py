"""Pins for the oracle's FP8 KV entries: E4M3 codes with a power-of-two scale
per 32 non-RoPE dims, the RoPE dims in bf16 (an entry of D = 576, d_rope = 64
is 656 bytes)."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def _e4m3(codes):
    """A library's E4M3 decode (torch float8_e4m3fn) of uint8 codes."""
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _block(vals, anchor=200.0):
    """One entry (D = 32 + 2, d_rope = 2) whose non-RoPE block holds `vals`
    (up to 31) and one element `anchor` that fixes the block's scale."""
    x = np.zeros(34, np.float32)
    x[0] = anchor
    x[1:1 + len(vals)] = vals
    return x


def test_entry_layout_and_sizes():
    assert oracle.fp8kv_entry_bytes(576, 64) == 656           # 512 codes + 128 rope bytes + 16 scales
    assert oracle.fp8kv_entry_bytes(64, 32) == 112            # 32 + 64 + 1 = 97 -> 112
    g = synth.rng(61)
    x = synth.normal(g, (2, 576))
    e = oracle.fp8kv_encode(x, 64)
    assert e.shape == (2, 656)
    # the RoPE dims are the bf16 (RNE) bits of the values, little endian, at 512..639
    rope = torch.from_numpy(x[:, 512:].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(e[:, 512:640].view(np.uint16), rope)


def test_decode_matches_a_library_e4m3_for_every_code():
    # a block whose scale byte is 127 (2^0): decode(code) is the E4M3 value
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)
    for start in range(0, len(codes), 32):
        blk = codes[start:start + 32]
        e = np.zeros((1, oracle.fp8kv_entry_bytes(34, 2)), np.uint8)
        e[0, :len(blk)] = blk
        e[0, 32 + 4] = 127
        got = oracle.fp8kv_decode(e, 34, 2)[0, :len(blk)]
        assert np.array_equal(got.view(np.uint32), _e4m3(blk).view(np.uint32)) or \
            np.array_equal(got, _e4m3(blk))                  # +-0 compare equal


def test_encode_is_nearest_e4m3_ties_to_even():
    # scale fixed at 2^0 by an anchor in [128, 256): the codes must be the
    # library's round-to-nearest-even E4M3 casts, including every midpoint
    # between adjacent representable values and the subnormal range
    reps = np.unique(np.abs(_e4m3(np.arange(0, 0x78, dtype=np.uint8))))   # the values below 256
    mids = (reps[:-1] + reps[1:]) / 2
    g = synth.rng(62)
    vals = np.concatenate([mids, -mids, g.uniform(-255, 255, 600), g.uniform(-0.02, 0.02, 200)]).astype(np.float32)
    for start in range(0, len(vals), 31):
        v = vals[start:start + 31]
        e = oracle.fp8kv_encode(_block(v)[None], 2)[0]
        assert e[32 + 4] == 127
        want = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        want = np.where((want & 0x7f) == 0, 0, want)          # the +0 code for zero
        assert np.array_equal(e[1:1 + len(v)], want), start


def test_scale_choice_and_zero_blocks():
    # amax in [2^e, 2^(e+1)) gives scale byte 127 + e - 7, so the largest
    # code lies in [128, 256); an all-zero block gets byte 127 and +0 codes
    for e in (-20, -3, 0, 4, 19):
        for f in (1.0, 1.5, 1.999):
            x = _block([0.25 * 2.0 ** e, -0.75 * 2.0 ** e], anchor=-f * 2.0 ** e)
            ent = oracle.fp8kv_encode(x[None], 2)[0]
            assert ent[32 + 4] == 127 + e - 7
            assert 128 <= abs(_e4m3(ent[:1])[0]) <= 256
    z = oracle.fp8kv_encode(np.zeros((1, 34), np.float32), 2)[0]
    assert z[32 + 4] == 127 and not z[:32].any()


def test_round_trip_of_representable_values():
    # values already on the grid (an E4M3 value times the block's scale)
    # come back exactly; arbitrary values within half an E4M3 step
    g = synth.rng(63)
    codes = g.integers(0, 0x78, (4, 512)).astype(np.uint8) | (g.integers(0, 2, (4, 512)) * 0x80).astype(np.uint8)
    codes[:, ::32] = 0x70                                    # a code of 128 fixes each block's scale at 2^s
    s = g.integers(-10, 10, (4, 16))
    x = np.zeros((4, 576), np.float32)
    x[:, :512] = _e4m3(codes) * np.repeat(2.0 ** s, 32, axis=1)
    x[:, 512:] = synth.to_bf16(synth.normal(g, (4, 64))).astype(np.uint32).__lshift__(16).view(np.float32)
    y = oracle.fp8kv_decode(oracle.fp8kv_encode(x, 64), 576, 64)
    assert np.array_equal(y, x)
    r = synth.normal(g, (8, 576))
    yr = oracle.fp8kv_decode(oracle.fp8kv_encode(r, 64), 576, 64)
    step = np.repeat(np.abs(r[:, :512]).reshape(8, 16, 32).max(axis=2), 32, axis=1) * 2.0 ** -10
    assert np.all(np.abs(yr[:, :512] - r[:, :512]) <= np.maximum(np.abs(r[:, :512]) * 2.0 ** -4, step) + 1e-30)
