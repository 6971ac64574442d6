"""GPU parity of the grouped output projection (heads split into g groups,
each projected to an intermediate width, then all intermediates to the
hidden size; DeepSeek-V4 technical report page, CSA section, step 4).

Bars, from the arithmetic: the intermediate u is an fp32 sum rounded once to
bf16 on both sides, the oracle's from an exact (fp64) sum, so each u value
is within one bf16 ulp of the oracle's plus the fp32 sum's error bound
((K-1) 2^-24 sum|o w|, which matters only where the sum cancels), and
almost all are equal. With
y is then held, element by element, to the error bound that follows from
the GPU's own intermediates: their differences from the oracle's times
|w2|, plus the fp32 sum's bound (and half a bf16 ulp for bf16 y); bf16 y
also meets the bf16 bar (max-abs 2e-2, rel-L2 1e-2)."""
import numpy as np
import pytest

import oracle
import synth
from util import bf16_ulp, check_bf16_attention, dev, host, report_margin

pytestmark = pytest.mark.gpu

csk = pytest.importorskip("compressed_sparse_kv_amd")
torch = pytest.importorskip("torch")


def _case(seed, R, H, dv, g, dg, d, rows=None):
    x = synth.out_proj(seed, R, H, dv, g, dg, d)
    o, w1, w2 = dev(x["o"]), dev(x["w1"]), dev(x["w2"])
    y16, u = csk.grouped_out_proj(o, w1, w2)
    u = host(u).copy() if u is not None else None
    y32, u2 = csk.grouped_out_proj(o, w1, w2, y_dtype=csk.CSK_F32)
    assert np.array_equal(host(u2), u)
    rows = np.arange(R) if rows is None else np.asarray(rows)
    ry, ru = oracle.grouped_out_proj(x["o"][rows], x["w1"], x["w2"])
    gu = u[rows]
    # |fp32 sum - exact sum| <= (K-1) 2^-24 sum|o w| (any summation order),
    # plus half a bf16 ulp of rounding on each side
    K1 = x["w1"].shape[2]
    oa = np.abs(synth.bf16_to_f32(x["o"][rows]).astype(np.float64)).reshape(len(rows), g, K1)
    wa = np.abs(synth.bf16_to_f32(x["w1"]).astype(np.float64))
    delta = (K1 - 1) * 2.0 ** -24 * np.einsum("rgk,gnk->rgn", oa, wa).reshape(len(rows), -1)
    bound = bf16_ulp(np.maximum(np.abs(ru), np.abs(gu))) + delta
    excess = np.abs(gu - ru) / bound
    assert excess.max() <= 1.0, f"intermediate off by {excess.max():.3f} of its bound"
    same = np.mean(gu == ru)
    assert same >= 0.99, f"only {same:.4f} of the intermediates equal the oracle's"
    # y from the GPU's own intermediates: |y32 - ry| <= sum|gu - ru||w2|
    # (the intermediates' differences) + (K2-1) 2^-24 sum|gu||w2| (the fp32
    # sum), bf16 y half an ulp more
    K2 = x["w2"].shape[1]
    w2a = np.abs(synth.bf16_to_f32(x["w2"]).astype(np.float64))
    gu64 = gu.astype(np.float64)
    ybound = np.abs(gu64 - ru) @ w2a.T + (K2 - 1) * 2.0 ** -24 * (np.abs(gu64) @ w2a.T) + 1e-12
    g32, g16 = host(y32)[rows].astype(np.float64), host(y16)[rows].astype(np.float64)
    x32 = np.abs(g32 - ry) / ybound
    assert x32.max() <= 1.0, f"fp32 y off by {x32.max():.3f} of its bound"
    x16 = np.abs(g16 - ry) / (ybound + 0.5 * bf16_ulp(np.maximum(np.abs(g16), np.abs(ry))))
    assert x16.max() <= 1.0, f"bf16 y off by {x16.max():.3f} of its bound"
    e32 = np.abs(g32 - ry).max()
    m16 = check_bf16_attention(g16, ry, "y bf16")
    return e32, m16, same


@pytest.mark.parametrize("R,H,dv,g,dg,d", [
    (37, 16, 64, 4, 64, 96),      # one ragged 256x256 tile per product
    (300, 8, 128, 2, 96, 200),    # ragged tiles in both dims, two groups
    (600, 64, 64, 8, 128, 264),   # several tiles per product, 8 groups
    (33, 4, 64, 1, 64, 64),       # one group (a plain two-step projection)
])
def test_many_rows(R, H, dv, g, dg, d):
    _case(900 + R, R, H, dv, g, dg, d)


@pytest.mark.parametrize("R", [1, 4, 32])
def test_few_rows(R):
    # at most 32 rows: the weight-streaming kernel
    _case(950 + R, R, 16, 64, 4, 128, 136)


def test_decode_1m_shape():
    # a decode step's 4 rows at the 64-head, 512-value layout: 8 groups of 8
    # heads to 1024 each, then 8192 -> 4096
    e32, m16, same = _case(960, 4, 64, 512, 8, 1024, 4096)
    report_margin("out_proj decode (4 rows) y bf16", *m16)
    print(f"[margin] out_proj decode y fp32: max-abs {e32:.3e}; intermediates equal {same:.5f}", flush=True)


def test_prefill_shape_sampled_rows():
    # 4096 rows of the 64-head prefill layout (the full 65536-row launch
    # shape per tile); the oracle checks 48 sampled rows across tiles
    R = 4096
    rows = sorted(set([0, 1, 255, 256, 257, 2047, 4095] + list(range(13, R, 97))))
    e32, m16, same = _case(961, R, 64, 512, 8, 1024, 4096, rows=rows)
    report_margin("out_proj prefill (4096 rows, sampled) y bf16", *m16)


def test_zero_rows_and_errors():
    x = synth.out_proj(962, 4, 8, 64, 2, 64, 64)
    o, w1, w2 = dev(x["o"]), dev(x["w1"]), dev(x["w2"])
    y, u = csk.grouped_out_proj(o[:0], w1, w2)
    assert y.shape == (0, 64) and u is None
    with pytest.raises(csk.CskError):
        # (H/g)*dv = 4*40 is not a multiple of 64
        csk.grouped_out_proj(dev(np.zeros((4, 8 * 40), np.uint16)), dev(np.zeros((2, 64, 160), np.uint16)), w2)
