"""Host check of the memory ordering around the arrival tickets.

The fused decode step and the prefill key splits publish partial results
with write-through (device-scope) stores and then take a ticket with an
atomic add; the workgroup that draws the last ticket reads every partial
back.  That is only correct if each wave's partial stores are complete
before the barrier that precedes the ticket, and if the last arriver
invalidates what it may hold before it reads.  The GPU tests cannot show a
missing wait reliably (the window is a few hundred cycles), so this test
compiles the two kernels for gfx950 to assembly on the host and checks, in
every instance that takes a ticket:

* between the last device-scope store and the barrier ahead of the ticket
  there is a wait for the vector-memory counter to reach zero;
* the wave that draws the last ticket takes a device-scope cache
  invalidation (the acquire) right after it, before the barrier that the
  merging reads follow.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_attention_kv_amd", "csrc")
SOURCES = ("attn_decode_mfma.hip", "attn_prefill_mfma.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def assembly():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="gqa_isa_")
    try:
        def one(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang",
                   "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
                   "-I", CSRC, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr
            with open(out) as f:
                return src, f.read()
        with cf.ThreadPoolExecutor(max_workers=2) as ex:
            yield dict(ex.map(one, SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _ticket_functions(text):
    """(name, lines) of every kernel whose body takes a ticket."""
    for body in re.split(r"\n(?=_Z\w+:)", text):
        m = re.match(r"(_Z\w+):", body)
        if not m:
            continue
        lines = body.split("\n")
        if any("atomic_add" in ln for ln in lines):
            yield m.group(1), lines


def _check(lines):
    ia = next(i for i, ln in enumerate(lines) if "atomic_add" in ln)
    ib = max(j for j in range(ia) if "s_barrier" in lines[j])
    stores = [j for j in range(ib) if "store" in lines[j] and "sc1" in lines[j]]
    assert stores, "no device-scope partial store ahead of the ticket"
    waits = [j for j in range(stores[-1] + 1, ib) if "vmcnt(0)" in lines[j]]
    acquire = any("buffer_inv sc1" in ln for ln in lines[ia:ia + 40])
    return bool(waits), acquire


@pytest.mark.parametrize("src,pattern,expected", [
    # Step: 2 D x 2 q types x ((1 + 4 x 2) column/token instances + 5 pair instances)
    ("attn_decode_mfma.hip", "attn_decode_mfma_kernel", 56),
    ("attn_prefill_mfma.hip", "attn_prefill_kernel", 16),      # key splits: 2 D x 4 q modes x 2 P forms
], ids=["decode_step", "prefill_split"])
def test_ticket_release_and_acquire(assembly, src, pattern, expected):
    found = 0
    for name, lines in _ticket_functions(assembly[src]):
        assert pattern in name, name
        waited, acquired = _check(lines)
        assert waited, f"{name}: partial stores not waited for before the ticket"
        assert acquired, f"{name}: no device-scope acquire before the merge"
        found += 1
    assert found == expected, found
