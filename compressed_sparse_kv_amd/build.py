"""Build libcsk.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 code
generation disabled, and linked into compressed_sparse_kv_amd/libcsk.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "csk")
LIB = os.path.join(HERE, "libcsk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["abi.hip", "compress.hip", "indexer.hip", "attention.hip", "gemm.hip", "project.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# Per-source code generation choices: MFMA results in VGPRs. indexer.hip:
# with the compiler's default the score tiles land in AGPRs, and each of
# them is copied out before the lane swaps and the head chain.
# attention.hip: with the default the output accumulators sit in AGPRs and
# are copied to VGPRs and back around every tile step.
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build():
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
