"""Build the gfx950 HIP library in-tree with hipcc.

``build()`` compiles every source under ``csrc/`` for gfx950 and links
``libgqa_decode.so`` next to this file.  Packed-fp32 instructions are
disabled for device code; the host pass warns that it does not know that
target feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgqa_decode.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.cpp", "prologue.hip", "attn_decode_mfma.hip", "merge.hip", "attn_prefill_mfma.hip",
           "qkv_gemv.hip", "probe.hip", "step_noalloc.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _flags():
    return ["-O3", *os.environ.get("GQA_EXTRA_CFLAGS", "").split(), "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile all sources and link the shared library; return its path."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="gqa_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
            if verbose and r.stderr.strip():
                print(r.stderr)
            return obj
        with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        staged = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
