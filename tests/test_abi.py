"""Host-side checks of the C ABI library (no GPU needed): it loads, exports
every function include/csk.h declares, sizes workspaces and rejects bad
arguments before touching a device."""
import ctypes
import os

import pytest

from util import ROOT, header_functions

LIB = os.path.join(ROOT, "compressed_sparse_kv_amd", "libcsk.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libcsk.so is not built (run compressed_sparse_kv_amd/build.py)")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_function(lib):
    names = header_functions()
    expected = {"csa_compress", "hca_compress", "indexer_topk", "sparse_attn", "dense_compressed_attn",
                "mxfp4_quantize", "csk_last_error"}
    assert expected <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libcsk.so does not export {n}"


def test_workspace_sizes(lib):
    lib.indexer_topk_workspace_size.restype = ctypes.c_size_t
    lib.sparse_attn_workspace_size.restype = ctypes.c_size_t
    lib.dense_compressed_attn_workspace_size.restype = ctypes.c_size_t
    # decode over 262144 entries: scores plus the filtered-selection buffers
    ws = lib.indexer_topk_workspace_size(4, 1, 64, 128, 262144, 2048, 2)
    assert ws >= 4 * 262144 * 4 * 5
    # short rows need only the score buffer
    assert lib.indexer_topk_workspace_size(1, 256, 2, 32, 64, 8, 0) >= 256 * 64 * 4
    assert lib.indexer_topk_workspace_size(0, 1, 1, 32, 1, 1, 0) == 0
    # prefill rows fit one chunk: no split-K partials
    assert lib.sparse_attn_workspace_size(1, 65536, 64, 576, 512, 2048, 128, 1, 0) == 0
    # decode splits the candidates: partial (m, l, o) per chunk
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, 0) > 0


def _split_bytes(R, nch, H=64, dv=512):
    # bf16 partial O per run, then fp32 (m, l) per run, each 256-byte aligned
    al = lambda x: (x + 255) & ~255
    return al(R * nch * H * dv * 2) + al(R * nch * H * 2 * 4)


def test_attn_split_runs(lib):
    """A decode row's 64-row tiles go to the fewest runs that keep the longest
    one, within about one workgroup per CU or the call's cap (the workspace
    holds one set of partials per run)."""
    lib.sparse_attn_workspace_size.restype = ctypes.c_size_t
    lib.dense_compressed_attn_workspace_size.restype = ctypes.c_size_t
    # 32 rows x (2048 + 128) candidates = 34 tiles: at most 8 runs a row -> 7 runs of <= 5 tiles
    assert lib.sparse_attn_workspace_size(32, 1, 64, 576, 512, 2048, 128, 1, 0) == _split_bytes(32, 7)
    # 4 rows: at most 64 runs a row -> one tile each, 34 runs
    assert lib.sparse_attn_workspace_size(4, 1, 64, 576, 512, 2048, 128, 1, 0) == _split_bytes(4, 34)
    # 4 rows x (8192 + 128) = 130 tiles capped at 64 workgroups: at most 16 a row -> 15 runs of <= 9
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, 64) == _split_bytes(4, 15)
    # uncapped: at most 64 a row -> 44 runs of <= 3 tiles
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, 0) == _split_bytes(4, 44)


def test_argument_errors_without_device(lib):
    lib.csk_last_error.restype = ctypes.c_char_p
    nul = ctypes.c_void_p(0)
    rc = lib.mxfp4_quantize(nul, 0, ctypes.c_int64(4), 32, nul, nul, nul)
    assert rc == -1 and b"null" in lib.csk_last_error()
    fake = ctypes.c_void_p(16)
    rc = lib.mxfp4_quantize(fake, 0, ctypes.c_int64(4), 30, fake, fake, nul)
    assert rc == -1 and b"cols" in lib.csk_last_error()
    rc = lib.mxfp4_quantize(fake, 7, ctypes.c_int64(4), 32, fake, fake, nul)
    assert rc == -2
    lib.csk_abi_version.restype = ctypes.c_int
    assert lib.csk_abi_version() == 2


def test_attn_workgroup_cap(lib):
    # host-side plan only: the per-call cap shrinks the split (and its
    # workspace); a negative cap is rejected by the workspace query (0) and
    # by the call itself before anything else is checked against a device
    lib.csk_last_error.restype = ctypes.c_char_p
    lib.dense_compressed_attn_workspace_size.restype = ctypes.c_size_t
    lib.sparse_attn_workspace_size.restype = ctypes.c_size_t
    full = lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, 0)
    capped = lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, 64)
    assert 0 < capped < full
    # the same query twice gives the same answer: no state carried between calls
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, 0) == full
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1, -1) == 0
    # four workgroups over four rows: every row whole, no partials
    assert lib.sparse_attn_workspace_size(4, 1, 64, 576, 512, 2048, 128, 1, 4) == 0
    assert lib.sparse_attn_workspace_size(4, 1, 64, 576, 512, 2048, 128, 1, 0) > 0
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.sparse_attn.argtypes = ([vp, vp, vp, i, vp, i, vp, vp, i, i, vp] + [i] * 6
                                + [f, f, i, i, vp, vp, i, vp, ctypes.c_size_t, vp])
    fake = 4096
    rc = lib.sparse_attn(fake, fake, fake, 100, fake, 8, None, None, 0, 0, None, 1, 1, 64, 576, 512, 64,
                         10000.0, 0.05, 1, 1, fake, None, -5, None, 0, None)
    assert rc == -1 and b"max_workgroups" in lib.csk_last_error()
    # FP8 KV entries are built for the 64-head 512 + 64 shape only
    rc = lib.sparse_attn(fake, fake, fake, 100, fake, 8, None, None, 0, 0, None, 1, 1, 16, 576, 512, 64,
                         10000.0, 0.05, 1, 3, fake, None, 0, None, 0, None)
    assert rc == -2 and b"FP8" in lib.csk_last_error()
    rc = lib.sparse_attn(fake, fake, fake, 100, fake, 8, None, None, 0, 0, None, 1, 1, 64, 576, 512, 64,
                         10000.0, 0.05, 0, 3, fake, None, 0, None, 0, None)
    assert rc == -2
    # q, the caches and the output move in 16-byte pieces: a 4-byte-aligned
    # output is refused before anything runs
    rc = lib.sparse_attn(fake, fake, fake, 100, fake, 8, None, None, 0, 0, None, 1, 1, 64, 576, 512, 64,
                         10000.0, 0.05, 1, 1, fake + 4, None, 0, None, 0, None)
    assert rc == -1 and b"16-byte" in lib.csk_last_error()


def test_fp8kv_entry_bytes(lib):
    assert lib.csk_fp8kv_entry_bytes(576, 64) == 656
    assert lib.csk_fp8kv_entry_bytes(64, 32) == 112
    assert lib.csk_fp8kv_entry_bytes(576, 63) == 0 and lib.csk_fp8kv_entry_bytes(100, 20) == 0


def test_no_device_is_unsupported(lib):
    # valid arguments on a host without a HIP device: the call stops at the
    # device check with CSK_EUNSUPPORTED (never launches). Skipped where a
    # GPU is visible: there the call would run on the fake pointers.
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    lib.csk_last_error.restype = ctypes.c_char_p
    fake = ctypes.c_void_p(4096)
    rc = lib.mxfp4_quantize(fake, 0, ctypes.c_int64(4), 32, fake, fake, None)
    assert rc == -2 and b"gfx950" in lib.csk_last_error()


def test_compress_job_layout(tmp_path):
    # the binding's record must have the C struct's size and field offsets
    import subprocess
    from compressed_sparse_kv_amd import CompressJob
    fields = [f for f, _ in CompressJob._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "csk.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(csk_compress_job));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(csk_compress_job, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(CompressJob)
    assert got[1:] == [getattr(CompressJob, f).offset for f in fields]


def test_compress_batch_errors_without_device(lib):
    from compressed_sparse_kv_amd import CompressJob, CSK_JOB_CSA, CSK_JOB_MXFP4
    lib.csk_last_error.restype = ctypes.c_char_p
    lib.csk_compress_batch.argtypes = [ctypes.POINTER(CompressJob), ctypes.c_int, ctypes.c_void_p]
    fake = 16

    def run(*jobs, n=None):
        arr = (CompressJob * max(len(jobs), 1))(*jobs)
        return lib.csk_compress_batch(arr, len(jobs) if n is None else n, None)

    quant = CompressJob(kind=CSK_JOB_MXFP4, x=fake, in_dtype=0, rows=4, cols=64, out=fake, out_scale=fake)
    assert run(quant, n=0) == -1 and b"n_jobs" in lib.csk_last_error()
    assert run(quant, n=5) == -1
    assert run(CompressJob(kind=7)) == -1 and b"kind" in lib.csk_last_error()
    # a bad second job is reported by index and nothing runs
    bad_cols = CompressJob(kind=CSK_JOB_MXFP4, x=fake, in_dtype=0, rows=4, cols=48, out=fake, out_scale=fake)
    assert run(quant, bad_cols) == -1 and b"job 1" in lib.csk_last_error()
    csa = dict(kind=CSK_JOB_CSA, ca=fake, za=fake, cb=fake, zb=fake, bias_a=fake, bias_b=fake, B=1, S=64,
               D=64, m=4, in_dtype=0, out_dtype=1, out=fake)
    assert run(CompressJob(**dict(csa, m=16))) == -2 and b"m <= 8" in lib.csk_last_error()
    assert run(CompressJob(**dict(csa, S=4 * 70000))) == -2 and b"65535" in lib.csk_last_error()
    assert run(CompressJob(**dict(csa, zb=0))) == -1 and b"null" in lib.csk_last_error()
    # jobs that produce nothing launch nothing (no device needed)
    assert run(CompressJob(**dict(csa, S=3)), CompressJob(kind=CSK_JOB_MXFP4, x=fake, rows=0, cols=32,
                                                          out=fake, out_scale=fake)) == 0


def test_indexer_rejects_misaligned_key_scales(lib):
    # the MXFP4 key scales are read as whole dwords: a misaligned array is an
    # argument error, caught before any launch
    lib.csk_last_error.restype = ctypes.c_char_p
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.indexer_topk.argtypes = [vp] * 7 + [i] * 9 + [vp, vp, vp, ctypes.c_size_t, vp]
    fake, odd = 4096, 4097
    rc = lib.indexer_topk(fake, fake, fake, fake, odd, fake, fake, 1, 1, 64, 128, 4096, 4, 8, 2, 0,
                          fake, fake, fake, ctypes.c_size_t(1 << 30), None)
    assert rc == -1 and b"aligned" in lib.csk_last_error()


def test_indexer_rejects_unknown_score_dtype(lib):
    lib.csk_last_error.restype = ctypes.c_char_p
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.indexer_topk.argtypes = [vp] * 7 + [i] * 9 + [vp, vp, vp, ctypes.c_size_t, vp]
    fake = 4096
    rc = lib.indexer_topk(fake, fake, fake, fake, fake, fake, fake, 1, 1, 64, 128, 4096, 4, 8, 2, 7,
                          fake, fake, fake, ctypes.c_size_t(1 << 30), None)
    assert rc == -2 and b"score_dtype" in lib.csk_last_error()


def test_grouped_out_proj_arguments(lib):
    lib.csk_last_error.restype = ctypes.c_char_p
    lib.grouped_out_proj_workspace_size.restype = ctypes.c_size_t
    assert lib.grouped_out_proj_workspace_size(4, 8, 1024) == 4 * 8 * 1024 * 2
    assert lib.grouped_out_proj_workspace_size(0, 8, 1024) == 0
    fake = ctypes.c_void_p(4096)
    sz = ctypes.c_size_t

    def call(R=4, H=64, dv=512, g=8, dg=1024, d=4096, y_dtype=1, ws=sz(1 << 20), o=fake):
        return lib.grouped_out_proj(o, fake, fake, R, H, dv, g, dg, d, y_dtype, fake, fake, ws, None)

    assert call(g=3) == -1                       # g does not divide H
    assert call(dv=40) == -2                     # (H/g)*dv = 320 is not a multiple of 64
    assert call(dg=36) == -2                     # g*dg = 288 likewise
    assert call(d=100) == -2                     # d not a multiple of 8
    assert call(y_dtype=2) == -2
    assert call(ws=sz(100)) == -3 and b"workspace" in lib.csk_last_error()
    assert call(o=ctypes.c_void_p(4098)) == -1 and b"aligned" in lib.csk_last_error()
    assert call(R=0, o=None) == 0                # nothing to do


def test_project_compress_and_rmsnorm_arguments(lib):
    # the binding's argument lists, checked against the library without a
    # device: every call below fails on its arguments before any launch
    import compressed_sparse_kv_amd as csk
    L = csk.lib()
    assert L.project_compress_workspace_size(1, 1, 65536, 576, 4) == 16384 * 576 * 4 + 16384 * 9 * 4
    assert L.project_compress_workspace_size(0, 2, 1024, 576, 128) == 16 * 576 * 4 + 16 * 9 * 4
    fake = ctypes.c_void_p(4096)

    def call(csa=1, m=4, hidden=4096, D=576, S=256, ws=1 << 30, x=fake, out_dtype=1, entry0=0):
        return L.project_compress(csa, x, fake, fake, fake, None, 1e-6, 1, S, hidden, D, m, entry0, 0, 64, 1e4,
                                  None, out_dtype, fake, None, 0, fake, ws, None)

    assert call(m=8) == -2 and b"m = 4" in L.csk_last_error()
    assert call(csa=0, m=4) == -2
    assert call(hidden=96) == -2
    assert call(D=48) == -2
    assert call(out_dtype=7) == -2
    assert call(out_dtype=2) == -1                   # MXFP4 without out_scale
    assert call(ws=16) == -3
    assert call(x=ctypes.c_void_p(4100)) == -1       # misaligned
    assert call(S=3) == 0                            # no whole block: nothing to do
    assert L.rmsnorm(fake, fake, 4, 576, ctypes.c_float(1e-6), 1, 5, fake, None) == -2
    assert L.rmsnorm(None, fake, 4, 576, ctypes.c_float(1e-6), 1, 1, fake, None) == -1
    assert L.rmsnorm(fake, fake, 0, 576, ctypes.c_float(1e-6), 1, 1, fake, None) == 0
