"""Plain CPU oracle for hybrid compressed attention (CSA + HCA).

TEST INFRASTRUCTURE ONLY. This package is the slow reference that the GPU
library is checked against; only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it. It shares no code with the GPU
library. Every function takes and returns numpy arrays; bf16 data is passed
as uint16 bit patterns and widened exactly to float32 before the call.

Each wrapper mirrors one C function in csk_oracle.c, which carries the
citations of the page passages it follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

F32 = 0
BF16 = 1
MXFP4 = 2

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def lib():
    """Load the oracle library, building it only if no built copy exists."""
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.csk_ref_rope.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.csk_ref_rope.restype = None
        L.csk_ref_csa_compress.argtypes = [_f32p] * 6 + [ctypes.c_int] * 5 + [ctypes.c_double, _i32p, _f64p]
        L.csk_ref_hca_compress.argtypes = [_f32p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_double, _i32p, _f64p]
        L.csk_ref_round_bf16.argtypes = [_f64p, _u16p, ctypes.c_int64]
        L.csk_ref_round_bf16.restype = None
        L.csk_ref_round_f32.argtypes = [_f64p, _f32p, ctypes.c_int64]
        L.csk_ref_round_f32.restype = None
        L.csk_ref_mxfp4_encode.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int, _u8p, _u8p]
        L.csk_ref_mxfp4_decode.argtypes = [_u8p, _u8p, ctypes.c_int64, ctypes.c_int, _f32p]
        L.csk_ref_indexer_scores.argtypes = ([_f32p, _u8p, _u8p, _f32p, _f32p, _u8p, _u8p, _i32p, _i32p]
                                             + [ctypes.c_int] * 7 + [_i32p, ctypes.c_int, _f32p, _i32p])
        L.csk_ref_topk.argtypes = [_f32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _f32p]
        L.csk_ref_scores_bf16.argtypes = [_f32p, ctypes.c_int64]
        L.csk_ref_scores_bf16.restype = None
        L.csk_ref_fp8kv_entry_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.csk_ref_fp8kv_encode.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _u8p]
        L.csk_ref_fp8kv_decode.argtypes = [_u8p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _f32p]
        L.csk_ref_grouped_out_proj.argtypes = [_f32p, _f32p, _f32p] + [ctypes.c_int] * 6 + [_f32p, _f64p]
        L.csk_ref_rmsnorm.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, _f64p]
        L.csk_ref_project_compress.argtypes = ([_f32p] * 5 + [ctypes.c_double] + [ctypes.c_int] * 7
                                               + [ctypes.c_double, _i32p, _f64p])
        attn_tail = ([_f32p, _i32p, ctypes.c_int, ctypes.c_int, _f32p] + [ctypes.c_int] * 6
                     + [ctypes.c_double, ctypes.c_double, _i32p, ctypes.c_int, _f64p, _f64p])
        L.csk_ref_sparse_attn.argtypes = [_f32p, _i32p, _f32p, ctypes.c_int, _i32p, ctypes.c_int] + attn_tail
        L.csk_ref_dense_attn.argtypes = [_f32p, _i32p, _f32p, ctypes.c_int, _i32p, ctypes.c_int] + attn_tail
        L.csk_ref_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _f32(a):
    """float32 contiguous view; uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads():
    return lib().csk_ref_num_threads()


def rope(x, pos, d_rope, base=10000.0):
    """Partial RoPE of one vector (double), returns a new array."""
    y = np.array(x, dtype=np.float64, copy=True)
    lib().csk_ref_rope(_p(y, ctypes.c_double), y.shape[-1], d_rope, float(pos), float(base))
    return y


def csa_compress(ca, za, cb, zb, bias_a, bias_b, m, d_rope=0, rope_base=10000.0, entry_pos=None):
    """[B,S,D] x4 -> [B,S//m,D] float64 (unrounded)."""
    ca, za, cb, zb = (_f32(a) for a in (ca, za, cb, zb))
    B, S, D = ca.shape
    out = np.empty((B, S // m, D), np.float64)
    ba, bb = _f32(bias_a), _f32(bias_b)
    ep = _i32(entry_pos)
    rc = lib().csk_ref_csa_compress(_p(ca, ctypes.c_float), _p(za, ctypes.c_float), _p(cb, ctypes.c_float),
                                    _p(zb, ctypes.c_float), _p(ba, ctypes.c_float), _p(bb, ctypes.c_float),
                                    B, S, D, m, d_rope, float(rope_base), _p(ep, ctypes.c_int32),
                                    _p(out, ctypes.c_double))
    _check(rc, "csa_compress")
    return out


def hca_compress(c, z, bias, m, d_rope=0, rope_base=10000.0, entry_pos=None):
    c, z = _f32(c), _f32(z)
    B, S, D = c.shape
    out = np.empty((B, S // m, D), np.float64)
    bs = _f32(bias)
    ep = _i32(entry_pos)
    rc = lib().csk_ref_hca_compress(_p(c, ctypes.c_float), _p(z, ctypes.c_float), _p(bs, ctypes.c_float),
                                    B, S, D, m, d_rope, float(rope_base), _p(ep, ctypes.c_int32),
                                    _p(out, ctypes.c_double))
    _check(rc, "hca_compress")
    return out


def round_bf16(x):
    """float64 -> bf16 bit patterns (uint16), one RNE rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, np.uint16)
    lib().csk_ref_round_bf16(_p(x, ctypes.c_double), _p(y, ctypes.c_uint16), x.size)
    return y


def round_f32(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, np.float32)
    lib().csk_ref_round_f32(_p(x, ctypes.c_double), _p(y, ctypes.c_float), x.size)
    return y


def bf16_to_f32(bits):
    return _f32(np.asarray(bits, dtype=np.uint16))


def mxfp4_encode(x):
    """x [..., cols] -> (codes [..., cols//2] uint8, scales [..., cols//32] uint8)."""
    x = _f32(x)
    cols = x.shape[-1]
    rows = x.size // cols
    codes = np.empty(x.shape[:-1] + (cols // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (cols // 32,), np.uint8)
    rc = lib().csk_ref_mxfp4_encode(_p(x, ctypes.c_float), rows, cols, _p(codes, ctypes.c_uint8),
                                    _p(scales, ctypes.c_uint8))
    _check(rc, "mxfp4_encode")
    return codes, scales


def mxfp4_decode(codes, scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    cols = codes.shape[-1] * 2
    rows = codes.size // codes.shape[-1]
    x = np.empty(codes.shape[:-1] + (cols,), np.float32)
    rc = lib().csk_ref_mxfp4_decode(_p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), rows, cols,
                                    _p(x, ctypes.c_float))
    _check(rc, "mxfp4_decode")
    return x


def _rows(rows, B, T):
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(T)]
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))


def indexer_scores(q, w, k, q_pos, n_entries, m, q_scale=None, k_scale=None, rows=None):
    """Scores [n_rows, Nmax] (float32, -inf past the visible count) and n_vis.

    fp32 path: q [B,T,HI,dI] float, k [B,Nmax,dI] float.
    MXFP4 path: q codes [B,T,HI,dI/2] + q_scale, k codes [B,Nmax,dI/2] + k_scale.
    """
    w = _f32(w)
    B, T, HI = w.shape
    if q_scale is None:
        qf, kf = _f32(q), _f32(k)
        dI = qf.shape[-1]
        Nmax = kf.shape[1]
        qc = qs = kc = ks = None
        dtype = F32
    else:
        qc = np.ascontiguousarray(q, np.uint8)
        qs = np.ascontiguousarray(q_scale, np.uint8)
        kc = np.ascontiguousarray(k, np.uint8)
        ks = np.ascontiguousarray(k_scale, np.uint8)
        dI = qc.shape[-1] * 2
        Nmax = kc.shape[1]
        qf = kf = None
        dtype = MXFP4
    rows = _rows(rows, B, T)
    scores = np.empty((rows.shape[0], Nmax), np.float32)
    n_vis = np.empty(rows.shape[0], np.int32)
    rc = lib().csk_ref_indexer_scores(_p(qf, ctypes.c_float), _p(qc, ctypes.c_uint8), _p(qs, ctypes.c_uint8),
                                      _p(w, ctypes.c_float), _p(kf, ctypes.c_float), _p(kc, ctypes.c_uint8),
                                      _p(ks, ctypes.c_uint8), _p(_i32(q_pos), ctypes.c_int32),
                                      _p(_i32(n_entries), ctypes.c_int32), B, T, HI, dI, Nmax, m, dtype,
                                      _p(rows, ctypes.c_int32), rows.shape[0], _p(scores, ctypes.c_float),
                                      _p(n_vis, ctypes.c_int32))
    _check(rc, "indexer_scores")
    return scores, n_vis


def topk(scores, n_vis, k):
    scores = np.ascontiguousarray(scores, np.float32)
    n_rows, Nmax = scores.shape
    idx = np.empty((n_rows, k), np.int32)
    out = np.empty((n_rows, k), np.float32)
    rc = lib().csk_ref_topk(_p(scores, ctypes.c_float), _p(_i32(n_vis), ctypes.c_int32), n_rows, Nmax, k,
                            _p(idx, ctypes.c_int32), _p(out, ctypes.c_float))
    _check(rc, "topk")
    return idx, out


def fp8kv_entry_bytes(D, d_rope):
    return lib().csk_ref_fp8kv_entry_bytes(D, d_rope)


def fp8kv_encode(x, d_rope):
    """x [..., D] (fp32 values; bf16 bit patterns accepted) -> FP8 KV entries
    [..., entry_bytes] uint8."""
    x = _f32(x)
    D = x.shape[-1]
    rows = x.size // D
    out = np.empty(x.shape[:-1] + (fp8kv_entry_bytes(D, d_rope),), np.uint8)
    _check(lib().csk_ref_fp8kv_encode(_p(x, ctypes.c_float), rows, D, d_rope, _p(out, ctypes.c_uint8)),
           "fp8kv_encode")
    return out


def fp8kv_decode(entries, D, d_rope):
    """FP8 KV entries [..., entry_bytes] -> exact fp32 values [..., D]."""
    e = np.ascontiguousarray(entries, dtype=np.uint8)
    rows = e.size // e.shape[-1]
    x = np.empty(e.shape[:-1] + (D,), np.float32)
    _check(lib().csk_ref_fp8kv_decode(_p(e, ctypes.c_uint8), rows, D, d_rope, _p(x, ctypes.c_float)),
           "fp8kv_decode")
    return x


def scores_bf16(scores):
    """Indexer scores rounded once to bf16 (RNE), as float32 (a new array)."""
    y = np.array(scores, dtype=np.float32, copy=True, order="C")
    lib().csk_ref_scores_bf16(_p(y, ctypes.c_float), y.size)
    return y


def indexer_topk(q, w, k_cache, q_pos, n_entries, m, topk_k, q_scale=None, k_scale=None, rows=None,
                 score_dtype=F32):
    """Scores, then (score_dtype BF16) their bf16 rounding, then top-k."""
    s, nv = indexer_scores(q, w, k_cache, q_pos, n_entries, m, q_scale, k_scale, rows)
    if score_dtype == BF16:
        s = scores_bf16(s)
    return topk(s, nv, topk_k)


def _attn_common(q, kv_w, w_pos0, sink):
    qf = _f32(q)
    B, T, H, D = qf.shape
    kvw = _f32(kv_w) if kv_w is not None else np.zeros((B, 0, D), np.float32)
    S_w = kvw.shape[1]
    wp = _i32(w_pos0 if w_pos0 is not None else np.zeros(B, np.int32))
    sk = _f32(sink) if sink is not None else None
    return qf, kvw, S_w, wp, sk, (B, T, H, D)


def sparse_attn(q, q_pos, kv_c, idx, kv_w, w_pos0, W, sink, dv, d_rope, scale, rope_base=10000.0, rows=None):
    """Returns (out [n_rows,H,dv] float64, lse [n_rows,H] float64)."""
    qf, kvw, S_w, wp, sk, (B, T, H, D) = _attn_common(q, kv_w, w_pos0, sink)
    kvc = _f32(kv_c)
    Nmax = kvc.shape[1]
    idx = _i32(idx)
    k = idx.shape[-1]
    rows = _rows(rows, B, T)
    out = np.empty((rows.shape[0], H, dv), np.float64)
    lse = np.empty((rows.shape[0], H), np.float64)
    rc = lib().csk_ref_sparse_attn(_p(qf, ctypes.c_float), _p(_i32(q_pos), ctypes.c_int32), _p(kvc, ctypes.c_float),
                                   Nmax, _p(idx, ctypes.c_int32), k, _p(kvw, ctypes.c_float), _p(wp, ctypes.c_int32),
                                   S_w, W, _p(sk, ctypes.c_float), B, T, H, D, dv, d_rope, float(rope_base),
                                   float(scale), _p(rows, ctypes.c_int32), rows.shape[0],
                                   _p(out, ctypes.c_double), _p(lse, ctypes.c_double))
    _check(rc, "sparse_attn")
    return out, lse


def dense_attn(q, q_pos, kv_c, n_entries, m, kv_w, w_pos0, W, sink, dv, d_rope, scale, rope_base=10000.0,
               rows=None):
    qf, kvw, S_w, wp, sk, (B, T, H, D) = _attn_common(q, kv_w, w_pos0, sink)
    kvc = _f32(kv_c)
    Nmax = kvc.shape[1]
    rows = _rows(rows, B, T)
    out = np.empty((rows.shape[0], H, dv), np.float64)
    lse = np.empty((rows.shape[0], H), np.float64)
    rc = lib().csk_ref_dense_attn(_p(qf, ctypes.c_float), _p(_i32(q_pos), ctypes.c_int32), _p(kvc, ctypes.c_float),
                                  Nmax, _p(_i32(n_entries), ctypes.c_int32), m, _p(kvw, ctypes.c_float),
                                  _p(wp, ctypes.c_int32), S_w, W, _p(sk, ctypes.c_float), B, T, H, D, dv, d_rope,
                                  float(rope_base), float(scale), _p(rows, ctypes.c_int32), rows.shape[0],
                                  _p(out, ctypes.c_double), _p(lse, ctypes.c_double))
    _check(rc, "dense_attn")
    return out, lse


def grouped_out_proj(o, w1, w2):
    """Grouped output projection. o [R, H*dv] (bf16 bits or float; heads
    consecutive); w1 [g, dg, (H/g)*dv]; w2 [d, g*dg]. Returns (y [R, d]
    float64, u [R, g*dg] float32: the intermediate rounded to bf16)."""
    w1, w2, of = _f32(w1), _f32(w2), _f32(o)
    g, dg, K1 = w1.shape
    d = w2.shape[0]
    assert of.ndim == 2 and of.shape[1] == g * K1 and w2.shape[1] == g * dg
    R = of.shape[0]
    y = np.empty((R, d), np.float64)
    u = np.empty((R, g * dg), np.float32)
    # H*dv = g*K1 is all the layout needs: g "heads" of K1 values each
    _check(lib().csk_ref_grouped_out_proj(_p(of, ctypes.c_float), _p(w1, ctypes.c_float), _p(w2, ctypes.c_float),
                                          R, g, K1, g, dg, d, _p(u, ctypes.c_float), _p(y, ctypes.c_double)),
           "grouped_out_proj")
    return y, u


RMS_EPS = 1e-6


def rmsnorm(x, gamma, eps=RMS_EPS):
    """RMSNorm over the last dim: x * gamma / sqrt(mean(x^2) + eps), float64."""
    xf = _f32(x)
    D = xf.shape[-1]
    y = np.empty(xf.shape, np.float64)
    _check(lib().csk_ref_rmsnorm(_p(xf, ctypes.c_float), _p(_f32(gamma), ctypes.c_float), xf.size // D, D,
                                 float(eps), _p(y, ctypes.c_double)), "rmsnorm")
    return y


def project_compress(x, w, bias_a, bias_b, m, gamma=None, eps=RMS_EPS, d_rope=0, rope_base=10000.0,
                     entry_pos=None):
    """Projection then compression. x [B,S,hidden]; w [4,D,hidden] (CSA:
    W_ca, W_za, W_cb, W_zb) or [2,D,hidden] (HCA: W_c, W_z; bias_b None).
    Returns [B,S//m,D] float64."""
    xf, wf = _f32(x), _f32(w)
    B, S, hidden = xf.shape
    ns, D, _ = wf.shape
    csa = 1 if ns == 4 else 0
    out = np.empty((B, S // m, D), np.float64)
    ba = _f32(bias_a)
    bb = _f32(bias_b) if bias_b is not None else ba
    ep = _i32(entry_pos) if entry_pos is not None else None
    _check(lib().csk_ref_project_compress(_p(xf, ctypes.c_float), _p(wf, ctypes.c_float), _p(ba, ctypes.c_float),
                                          _p(bb, ctypes.c_float),
                                          _p(_f32(gamma), ctypes.c_float) if gamma is not None else None,
                                          float(eps), csa, B, S, hidden, D, m, d_rope, float(rope_base),
                                          _p(ep, ctypes.c_int32), _p(out, ctypes.c_double)), "project_compress")
    return out
