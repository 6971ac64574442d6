"""Python binding of libcsk (hybrid compressed attention on MI355X / gfx950).

Argument marshalling only: every function forwards torch tensors' device
pointers, sizes and torch's current HIP stream to the C ABI declared in
include/csk.h and raises on a non-zero return code. Outputs and workspaces
are allocated here with torch when the caller does not pass them; all
computation happens in the library's kernels. There is no fallback: if the
library is missing or fails to load, every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsk.so")

CSK_F32, CSK_BF16, CSK_MXFP4, CSK_FP8KV = 0, 1, 2, 3
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float
_sz = ctypes.c_size_t


class CskError(RuntimeError):
    pass


def lib():
    """Load libcsk.so (built by compressed_sparse_kv_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CskError(f"{LIB_PATH} is not built; run compressed_sparse_kv_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.csk_last_error.restype = ctypes.c_char_p
        L.csk_abi_version.restype = _i
        L.csk_fp8kv_entry_bytes.argtypes = [_i, _i]
        L.csk_fp8kv_entry_bytes.restype = _i
        L.csa_compress.argtypes = [_vp] * 6 + [_i] * 5 + [_i64, _i, _f, _vp, _i, _i, _vp, _vp, _i64, _vp]
        L.hca_compress.argtypes = [_vp] * 3 + [_i] * 5 + [_i64, _i, _f, _vp, _i, _i, _vp, _vp, _i64, _vp]
        L.mxfp4_quantize.argtypes = [_vp, _i, _i64, _i, _vp, _vp, _vp]
        L.csk_compress_batch.argtypes = [ctypes.POINTER(CompressJob), _i, _vp]
        L.indexer_topk.argtypes = [_vp] * 7 + [_i] * 9 + [_vp, _vp, _vp, _sz, _vp]
        L.indexer_topk_workspace_size.argtypes = [_i] * 7
        L.indexer_topk_workspace_size.restype = _sz
        L.indexer_topk_noalloc.argtypes = [_vp] * 7 + [_i] * 9 + [_vp, _vp, _vp]
        L.sparse_attn.argtypes = ([_vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _i, _i, _vp] + [_i] * 6
                                  + [_f, _f, _i, _i, _vp, _vp, _i, _vp, _sz, _vp])
        L.dense_compressed_attn.argtypes = ([_vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _i, _i, _vp] + [_i] * 6
                                            + [_f, _f, _i, _i, _vp, _vp, _i, _vp, _sz, _vp])
        L.sparse_attn_workspace_size.argtypes = [_i] * 9
        L.sparse_attn_workspace_size.restype = _sz
        L.dense_compressed_attn_workspace_size.argtypes = [_i] * 10
        L.dense_compressed_attn_workspace_size.restype = _sz
        L.grouped_out_proj.argtypes = [_vp] * 3 + [_i] * 7 + [_vp, _vp, _sz, _vp]
        L.grouped_out_proj_workspace_size.argtypes = [_i] * 3
        L.grouped_out_proj_workspace_size.restype = _sz
        L.project_compress.argtypes = ([_i] + [_vp] * 5 + [_f] + [_i] * 6 + [_i64, _i, _f, _vp, _i, _vp, _vp, _i64,
                                                                       _vp, _sz, _vp])
        L.project_compress_workspace_size.argtypes = [_i] * 5
        L.project_compress_workspace_size.restype = _sz
        L.rmsnorm.argtypes = [_vp, _vp, _i64, _i, _f, _i, _i, _vp, _vp]
        L.csk_kernel_timer_arm.argtypes = [ctypes.c_char_p, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i]
        L.csk_kernel_timer_count.restype = _i
        L.csk_kernel_timer_disarm.restype = None
        _lib = L
    return _lib


def _check(rc, fn):
    if rc != 0:
        raise CskError(f"{fn} failed ({rc}): {lib().csk_last_error().decode()}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dt(t):
    if t.dtype == torch.float32:
        return CSK_F32
    if t.dtype == torch.bfloat16:
        return CSK_BF16
    raise CskError(f"unsupported dtype {t.dtype}")


def _torch_dt(code):
    return {CSK_F32: torch.float32, CSK_BF16: torch.bfloat16}[code]


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def fp8kv_entry_bytes(D, d_rope):
    """Bytes of one CSK_FP8KV entry (see csk.h)."""
    return lib().csk_fp8kv_entry_bytes(D, d_rope)


def csa_compress(ca, za, cb, zb, bias_a, bias_b, m, d_rope=0, rope_base=10000.0, entry_pos=None,
                 out_dtype=None, entry0=0, src_bstride=0, out=None, out_scale=None, dst_bstride=0,
                 B=None, S=None):
    """CSA compression of [B,S,D] series (see csa_compress in csk.h).

    Returns out ([B,S//m,D] in out_dtype) or (codes, scales) for MXFP4.
    """
    B = ca.shape[0] if B is None else B
    S = ca.shape[1] if S is None else S
    D = ca.shape[-1]
    out_dtype = _dt(ca) if out_dtype is None else out_dtype
    out, out_scale = _alloc_compress_out(out, out_scale, B, S // m, D, out_dtype, ca.device, d_rope)
    rc = lib().csa_compress(_ptr(ca), _ptr(za), _ptr(cb), _ptr(zb), _ptr(bias_a), _ptr(bias_b), B, S, D, m,
                            entry0, src_bstride, d_rope, rope_base, _ptr(entry_pos), _dt(ca), out_dtype,
                            _ptr(out), _ptr(out_scale), dst_bstride, _stream())
    _check(rc, "csa_compress")
    return (out, out_scale) if out_dtype == CSK_MXFP4 else out


def hca_compress(c, z, bias, m, d_rope=0, rope_base=10000.0, entry_pos=None, out_dtype=None, entry0=0,
                 src_bstride=0, out=None, out_scale=None, dst_bstride=0, B=None, S=None):
    B = c.shape[0] if B is None else B
    S = c.shape[1] if S is None else S
    D = c.shape[-1]
    out_dtype = _dt(c) if out_dtype is None else out_dtype
    out, out_scale = _alloc_compress_out(out, out_scale, B, S // m, D, out_dtype, c.device, d_rope)
    rc = lib().hca_compress(_ptr(c), _ptr(z), _ptr(bias), B, S, D, m, entry0, src_bstride, d_rope, rope_base,
                            _ptr(entry_pos), _dt(c), out_dtype, _ptr(out), _ptr(out_scale), dst_bstride,
                            _stream())
    _check(rc, "hca_compress")
    return (out, out_scale) if out_dtype == CSK_MXFP4 else out


def _alloc_compress_out(out, out_scale, B, N, D, out_dtype, device, d_rope=0):
    if out is None:
        if out_dtype == CSK_MXFP4:
            out = torch.empty((B, N, D // 2), dtype=torch.uint8, device=device)
        elif out_dtype == CSK_FP8KV:
            out = torch.empty((B, N, fp8kv_entry_bytes(D, d_rope)), dtype=torch.uint8, device=device)
        else:
            out = torch.empty((B, N, D), dtype=_torch_dt(out_dtype), device=device)
    if out_dtype == CSK_MXFP4 and out_scale is None:
        out_scale = torch.empty((B, N, D // 32), dtype=torch.uint8, device=device)
    return out, out_scale


def mxfp4_quantize(x, codes=None, scales=None):
    """x [..., cols] (fp32/bf16) -> (codes [..., cols/2], scales [..., cols/32])."""
    cols = x.shape[-1]
    rows = x.numel() // cols
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=x.device)
    rc = lib().mxfp4_quantize(_ptr(x), _dt(x), rows, cols, _ptr(codes), _ptr(scales), _stream())
    _check(rc, "mxfp4_quantize")
    return codes, scales


CSK_JOB_CSA, CSK_JOB_MXFP4 = 1, 2
CSK_MAX_JOBS = 4


class CompressJob(ctypes.Structure):
    """csk_compress_job of csk.h (same fields, same order)."""
    _fields_ = [("kind", _i), ("ca", _vp), ("za", _vp), ("cb", _vp), ("zb", _vp), ("bias_a", _vp),
                ("bias_b", _vp), ("B", _i), ("S", _i), ("D", _i), ("m", _i), ("entry0", _i),
                ("src_bstride", _i64), ("d_rope", _i), ("rope_base", _f), ("entry_pos", _vp),
                ("in_dtype", _i), ("out_dtype", _i), ("out", _vp), ("out_scale", _vp),
                ("dst_bstride", _i64), ("x", _vp), ("rows", _i64), ("cols", _i)]


class BatchJob:
    """One job of compress_batch: its C record, the tensors it names (kept
    alive until the launch) and its outputs."""

    def __init__(self, rec, tensors, result):
        self.rec, self.tensors, self.result = rec, tensors, result


def csa_job(ca, za, cb, zb, bias_a, bias_b, m, d_rope=0, rope_base=10000.0, entry_pos=None,
            out_dtype=None, entry0=0, src_bstride=0, out=None, out_scale=None, dst_bstride=0,
            B=None, S=None):
    """A csa_compress call (same arguments) for compress_batch."""
    B = ca.shape[0] if B is None else B
    S = ca.shape[1] if S is None else S
    D = ca.shape[-1]
    out_dtype = _dt(ca) if out_dtype is None else out_dtype
    out, out_scale = _alloc_compress_out(out, out_scale, B, S // m, D, out_dtype, ca.device, d_rope)
    rec = CompressJob(kind=CSK_JOB_CSA, ca=_ptr(ca), za=_ptr(za), cb=_ptr(cb), zb=_ptr(zb),
                      bias_a=_ptr(bias_a), bias_b=_ptr(bias_b), B=B, S=S, D=D, m=m, entry0=entry0,
                      src_bstride=src_bstride, d_rope=d_rope, rope_base=rope_base,
                      entry_pos=_ptr(entry_pos), in_dtype=_dt(ca), out_dtype=out_dtype, out=_ptr(out),
                      out_scale=_ptr(out_scale), dst_bstride=dst_bstride)
    result = (out, out_scale) if out_dtype == CSK_MXFP4 else out
    return BatchJob(rec, (ca, za, cb, zb, bias_a, bias_b, entry_pos, out, out_scale), result)


def mxfp4_job(x, codes=None, scales=None):
    """An mxfp4_quantize call (same arguments) for compress_batch."""
    cols = x.shape[-1]
    rows = x.numel() // cols
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=x.device)
    rec = CompressJob(kind=CSK_JOB_MXFP4, x=_ptr(x), in_dtype=_dt(x), rows=rows, cols=cols, out=_ptr(codes),
                      out_scale=_ptr(scales))
    return BatchJob(rec, (x, codes, scales), (codes, scales))


def compress_batch(jobs):
    """Runs csa_job / mxfp4_job records in one launch (csk_compress_batch);
    returns each job's result as its own call would."""
    arr = (CompressJob * len(jobs))(*[j.rec for j in jobs])
    _check(lib().csk_compress_batch(arr, len(jobs), _stream()), "csk_compress_batch")
    return [j.result for j in jobs]


def indexer_topk_workspace_size(B, T, HI, dI, Nmax, k, dtype):
    return lib().indexer_topk_workspace_size(B, T, HI, dI, Nmax, k, dtype)


def indexer_topk(q, w, kk, q_pos, n_entries, m, k, q_scale=None, k_scale=None, idx=None, score=None,
                 workspace=None, with_score=True, score_dtype=CSK_F32):
    """Top-k compressed entries per query row (see indexer_topk in csk.h).

    MXFP4: q [B,T,HI,dI/2] uint8 + q_scale, kk [B,Nmax,dI/2] uint8 + k_scale.
    fp32:  q [B,T,HI,dI] float32, kk [B,Nmax,dI] float32.
    score_dtype: CSK_F32, or CSK_BF16 (scores rounded to bf16 before the top-k).
    Returns (idx [B,T,k] int32, score [B,T,k] float32 or None).
    """
    B, T, HI = w.shape
    mx = q_scale is not None
    dI = q.shape[-1] * 2 if mx else q.shape[-1]
    Nmax = kk.shape[1]
    dtype = CSK_MXFP4 if mx else CSK_F32
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=w.device)
    if score is None and with_score:
        score = torch.empty((B, T, k), dtype=torch.float32, device=w.device)
    nbytes = indexer_topk_workspace_size(B, T, HI, dI, Nmax, k, dtype)
    if workspace is None:
        workspace = _ws(nbytes, w.device)
    rc = lib().indexer_topk(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(kk), _ptr(k_scale), _ptr(q_pos),
                            _ptr(n_entries), B, T, HI, dI, Nmax, m, k, dtype, score_dtype, _ptr(idx),
                            _ptr(score), _ptr(workspace), workspace.numel(), _stream())
    _check(rc, "indexer_topk")
    return idx, score


def indexer_topk_noalloc(q, w, kk, q_pos, n_entries, m, k, q_scale=None, k_scale=None, idx=None, score=None,
                         with_score=True, score_dtype=CSK_F32):
    """indexer_topk without a workspace: the library's static device
    scratch serves instead (see indexer_topk_noalloc in csk.h; calls that
    overlap on one device race). Returns (idx, score or None)."""
    B, T, HI = w.shape
    mx = q_scale is not None
    dI = q.shape[-1] * 2 if mx else q.shape[-1]
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=w.device)
    if score is None and with_score:
        score = torch.empty((B, T, k), dtype=torch.float32, device=w.device)
    rc = lib().indexer_topk_noalloc(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(kk), _ptr(k_scale), _ptr(q_pos),
                                    _ptr(n_entries), B, T, HI, dI, kk.shape[1], m, k,
                                    CSK_MXFP4 if mx else CSK_F32, score_dtype, _ptr(idx), _ptr(score), _stream())
    _check(rc, "indexer_topk_noalloc")
    return idx, score


def sparse_attn_workspace_size(B, T, H, D, dv, k, W, dtype, max_workgroups=0):
    return lib().sparse_attn_workspace_size(B, T, H, D, dv, k, W, dtype, max_workgroups)


def dense_compressed_attn_workspace_size(B, T, H, D, dv, Nmax, m, W, dtype, max_workgroups=0):
    return lib().dense_compressed_attn_workspace_size(B, T, H, D, dv, Nmax, m, W, dtype, max_workgroups)


def _kv_dt(q, kv_c):
    """The KV dtype code: uint8 entries are CSK_FP8KV, else the query's."""
    return CSK_FP8KV if kv_c.dtype == torch.uint8 else _dt(q)


def _attn_io(q, kv_w, dv, out, lse, want_lse):
    B, T, H, D = q.shape
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    S_w = 0 if kv_w is None else kv_w.shape[1]
    return B, T, H, D, S_w, out, lse


def sparse_attn(q, q_pos, kv_c, idx, kv_w, w_pos0, W, sink, dv, d_rope, scale, rope_base=10000.0,
                out=None, lse=None, workspace=None, want_lse=True, max_workgroups=0):
    """CSA attention (see sparse_attn in csk.h). Returns (out, lse)."""
    B, T, H, D, S_w, out, lse = _attn_io(q, kv_w, dv, out, lse, want_lse)
    k = idx.shape[-1]
    nbytes = sparse_attn_workspace_size(B, T, H, D, dv, k, W if S_w else 0, _dt(q), max_workgroups)
    if workspace is None:
        workspace = _ws(nbytes, q.device)
    rc = lib().sparse_attn(_ptr(q), _ptr(q_pos), _ptr(kv_c), kv_c.shape[1], _ptr(idx), k, _ptr(kv_w),
                           _ptr(w_pos0), S_w, W, _ptr(sink), B, T, H, D, dv, d_rope, rope_base, scale, _dt(q),
                           _kv_dt(q, kv_c), _ptr(out), _ptr(lse), max_workgroups, _ptr(workspace),
                           workspace.numel(), _stream())
    _check(rc, "sparse_attn")
    return out, lse


def dense_compressed_attn(q, q_pos, kv_c, n_entries, m, kv_w, w_pos0, W, sink, dv, d_rope, scale,
                          rope_base=10000.0, out=None, lse=None, workspace=None, want_lse=True,
                          max_workgroups=0):
    """HCA attention (see dense_compressed_attn in csk.h). Returns (out, lse)."""
    B, T, H, D, S_w, out, lse = _attn_io(q, kv_w, dv, out, lse, want_lse)
    Nmax = kv_c.shape[1]
    nbytes = dense_compressed_attn_workspace_size(B, T, H, D, dv, Nmax, m, W if S_w else 0, _dt(q),
                                                  max_workgroups)
    if workspace is None:
        workspace = _ws(nbytes, q.device)
    rc = lib().dense_compressed_attn(_ptr(q), _ptr(q_pos), _ptr(kv_c), Nmax, _ptr(n_entries), m, _ptr(kv_w),
                                     _ptr(w_pos0), S_w, W, _ptr(sink), B, T, H, D, dv, d_rope, rope_base, scale,
                                     _dt(q), _kv_dt(q, kv_c), _ptr(out), _ptr(lse), max_workgroups,
                                     _ptr(workspace), workspace.numel(), _stream())
    _check(rc, "dense_compressed_attn")
    return out, lse


def grouped_out_proj_workspace_size(R, g, dg):
    return lib().grouped_out_proj_workspace_size(R, g, dg)


def grouped_out_proj(o, w1, w2, y_dtype=None, out=None, workspace=None):
    """Grouped output projection (see grouped_out_proj in csk.h). o
    [..., H, dv] or [..., H*dv] bf16 (R = the leading dims' product); w1
    [g, dg, (H/g)*dv] bf16; w2 [d, g*dg] bf16. Returns (y [..., d] in
    y_dtype, default bf16; u [R, g*dg] bf16, the intermediate, a view of
    the workspace)."""
    g, dg, K1 = w1.shape
    d = w2.shape[0]
    HD = g * K1
    lead = o.shape[:-2] if o.shape[-1] != HD else o.shape[:-1]
    R = 1
    for x in lead:
        R *= int(x)
    H = g if o.shape[-1] == HD else o.shape[-2]
    dv = HD // H
    y_dtype = CSK_BF16 if y_dtype is None else y_dtype
    if out is None:
        out = torch.empty(tuple(lead) + (d,), dtype=_torch_dt(y_dtype), device=o.device)
    nbytes = grouped_out_proj_workspace_size(R, g, dg)
    if workspace is None:
        workspace = _ws(nbytes, o.device)
    rc = lib().grouped_out_proj(_ptr(o), _ptr(w1), _ptr(w2), R, H, dv, g, dg, d, y_dtype, _ptr(out),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    _check(rc, "grouped_out_proj")
    u = workspace[:nbytes].view(torch.bfloat16).view(R, g * dg) if R > 0 else None
    return out, u


RMS_EPS = 1e-6


def project_compress_workspace_size(csa, B, S, D, m):
    return lib().project_compress_workspace_size(csa, B, S, D, m)


def project_compress(x, w, bias_a, bias_b, m, gamma=None, eps=RMS_EPS, d_rope=0, rope_base=10000.0,
                     entry_pos=None, out_dtype=None, entry0=0, src_bstride=0, out=None, out_scale=None,
                     dst_bstride=0, B=None, S=None, workspace=None):
    """Projection then compression (see project_compress in csk.h). x
    [B,S,hidden] bf16; w [4,D,hidden] (CSA) or [2,D,hidden] (HCA) bf16.
    Returns out ([B,S//m,D] in out_dtype, default bf16) or (codes, scales)
    for MXFP4."""
    csa = 1 if w.shape[0] == 4 else 0
    B = x.shape[0] if B is None else B
    S = x.shape[1] if S is None else S
    hidden, D = x.shape[-1], w.shape[1]
    out_dtype = CSK_BF16 if out_dtype is None else out_dtype
    out, out_scale = _alloc_compress_out(out, out_scale, B, S // m, D, out_dtype, x.device, d_rope)
    nbytes = project_compress_workspace_size(csa, B, S, D, m)
    if workspace is None:
        workspace = _ws(nbytes, x.device)
    rc = lib().project_compress(csa, _ptr(x), _ptr(w), _ptr(bias_a), _ptr(bias_b), _ptr(gamma), eps, B, S, hidden,
                                D, m, entry0, src_bstride, d_rope, rope_base, _ptr(entry_pos), out_dtype, _ptr(out),
                                _ptr(out_scale), dst_bstride, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream())
    _check(rc, "project_compress")
    return (out, out_scale) if out_dtype == CSK_MXFP4 else out


def rmsnorm(x, gamma, eps=RMS_EPS, out_dtype=None, out=None):
    """RMSNorm over the last dim (see rmsnorm in csk.h)."""
    D = x.shape[-1]
    out_dtype = _dt(x) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(x.shape, dtype=_torch_dt(out_dtype), device=x.device)
    rc = lib().rmsnorm(_ptr(x), _ptr(gamma), x.numel() // D, D, eps, _dt(x), out_dtype, _ptr(out), _stream())
    _check(rc, "rmsnorm")
    return out


class KernelTimer:
    """Brackets the next n launches of one library kernel with HIP events
    recorded on the launch stream (see csk_kernel_timer_arm)."""

    def __init__(self, kernel, n):
        self.kernel = kernel
        self.start = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.stop = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.start + self.stop:
            e.record()  # materialise the underlying hipEvent_t
        torch.cuda.synchronize()
        arr = _vp * n
        self._s = arr(*[e.cuda_event for e in self.start])
        self._e = arr(*[e.cuda_event for e in self.stop])
        _check(lib().csk_kernel_timer_arm(kernel.encode(), self._s, self._e, n), "csk_kernel_timer_arm")

    def count(self):
        return lib().csk_kernel_timer_count()

    def disarm(self):
        lib().csk_kernel_timer_disarm()

    def durations_ms(self):
        n = self.count()
        return [self.start[i].elapsed_time(self.stop[i]) for i in range(n)]
