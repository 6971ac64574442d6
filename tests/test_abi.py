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
    assert lib.sparse_attn_workspace_size(1, 65536, 64, 576, 512, 2048, 128, 1) == 0
    # decode splits the candidates: partial (m, l, o) per chunk
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1) > 0


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
    assert lib.csk_abi_version() == 1


def test_attn_workgroup_cap(lib):
    # host-side plan only: the cap shrinks the split (and its workspace) and
    # is restored; a negative cap is rejected
    lib.csk_set_attn_workgroups.restype = ctypes.c_int
    lib.csk_last_error.restype = ctypes.c_char_p
    lib.dense_compressed_attn_workspace_size.restype = ctypes.c_size_t
    full = lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1)
    assert lib.csk_set_attn_workgroups(64) == 0
    capped = lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1)
    assert 0 < capped < full
    assert lib.csk_set_attn_workgroups(-3) == -1 and b"negative" in lib.csk_last_error()
    assert lib.csk_set_attn_workgroups(0) == 64
    assert lib.dense_compressed_attn_workspace_size(4, 1, 64, 576, 512, 8192, 128, 128, 1) == full


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
    lib.indexer_topk.argtypes = [vp] * 7 + [i] * 8 + [vp, vp, vp, ctypes.c_size_t, vp]
    fake, odd = 4096, 4097
    rc = lib.indexer_topk(fake, fake, fake, fake, odd, fake, fake, 1, 1, 64, 128, 4096, 4, 8, 2,
                          fake, fake, fake, ctypes.c_size_t(1 << 30), None)
    assert rc == -1 and b"aligned" in lib.csk_last_error()
