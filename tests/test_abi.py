"""The C-ABI library: loads without a GPU, exports exactly what the header
declares, and rejects bad arguments on the host (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")


@pytest.fixture(scope="module")
def G():
    import importlib.util
    path = os.path.join(ROOT, "gqa_attention_kv_amd", "_build.py")
    spec = importlib.util.spec_from_file_location("_gqa_build_t", path)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    if not os.path.exists(b.LIB_PATH):
        b.build()
    import gqa_attention_kv_amd
    return gqa_attention_kv_amd


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", text)))


def test_header_symbols_exported(G):
    decl = _declared()
    assert decl == sorted(G.SYMBOLS), (decl, sorted(G.SYMBOLS))
    for name in decl:
        assert hasattr(G.lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", G.lib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT (gqa_\w+)", out)))
    assert exported == decl, exported


A16 = 0x100000       # stand-in device addresses: never dereferenced, the
A_ODD = 0x100002     # calls below all fail validation on the host


def _attn(G, **kw):
    a = dict(q=A16, qd=0, k=A16, v=A16, lens=A16, window=0, scale=0.0, out=A16, od=0,
             lse=None, B=1, Hq=8, Hkv=2, D=128, T=16)
    a.update(kw)
    return G.lib.gqa_attn_decode(a["q"], a["qd"], a["k"], a["v"], a["lens"], a["window"],
                                 a["scale"], a["out"], a["od"], a["lse"], a["B"], a["Hq"],
                                 a["Hkv"], a["D"], a["T"], None)


def test_attn_validation(G):
    assert _attn(G, q=None) == -1
    assert _attn(G, lens=None) == -1
    assert _attn(G, B=0) == -2
    assert _attn(G, T=0) == -2
    assert _attn(G, Hq=6, Hkv=4) == -2
    assert _attn(G, D=96) == -3
    assert _attn(G, Hq=6, Hkv=2) == -3          # G = 3
    assert _attn(G, Hq=64, Hkv=2) == -3         # G = 32
    assert _attn(G, qd=7) == -3
    assert _attn(G, od=2) == -3
    assert _attn(G, k=A_ODD) == -6
    assert _attn(G, out=A16 + 8) == -6
    assert _attn(G, scale=float("nan")) == -7
    assert _attn(G, B=1 << 21) == -2           # B * Hq workgroups past the grid limit


def _split(G, **kw):
    a = dict(q=A16, k=A16, v=A16, lens=A16, window=0, scale=0.0, P=64, ws=A16, wsb=1 << 30,
             B=1, Hq=8, Hkv=2, D=128, T=1000)
    a.update(kw)
    return G.lib.gqa_attn_decode_splitk(a["q"], 0, a["k"], a["v"], a["lens"], a["window"],
                                        a["scale"], a["P"], a["ws"], a["wsb"], a["B"],
                                        a["Hq"], a["Hkv"], a["D"], a["T"], None)


def test_splitk_and_merge_validation(G):
    assert _split(G, ws=None) == -1
    assert _split(G, P=0) == -7
    assert _split(G, ws=A16 + 16) == -6
    need = G.splitk_workspace_bytes(1, 8, 128, 1000, 0, 64)
    assert _split(G, wsb=need - 1) == -4
    m = G.lib.gqa_attn_decode_merge
    assert m(None, need, 0, 64, A16, 0, None, 1, 8, 128, 1000, None) == -1
    assert m(A16, need - 1, 0, 64, A16, 0, None, 1, 8, 128, 1000, None) == -4
    assert m(A16, need, 0, 0, A16, 0, None, 1, 8, 128, 1000, None) == -7
    assert m(A16, need, 0, 64, A16, 0, None, 1, 8, 96, 1000, None) == -3
    assert m(A16 + 4, need, 0, 64, A16, 0, None, 1, 8, 128, 1000, None) == -6


def test_prologue_validation(G):
    f = G.lib.gqa_qkv_prologue

    def call(**kw):
        a = dict(q=A16, kn=A16, vn=A16, dt=1, qs=8 * 128, kvs=2 * 128, wq=None, wk=None,
                 eps=1e-6, theta=1e4, pos=A16, qo=A16, kc=A16, vc=A16, B=1, Hq=8, Hkv=2,
                 D=128, T=16)
        a.update(kw)
        return f(a["q"], a["kn"], a["vn"], a["dt"], a["qs"], a["kvs"], a["wq"], a["wk"],
                 a["eps"], a["theta"], a["pos"], a["qo"], a["kc"], a["vc"], a["B"], a["Hq"],
                 a["Hkv"], a["D"], a["T"], None)
    assert call(pos=None) == -1
    assert call(wq=A16) == -1                   # one norm weight without the other
    assert call(qs=100) == -2
    assert call(kvs=10) == -2
    assert call(eps=-1.0) == -7
    assert call(theta=float("inf")) == -7
    assert call(dt=5) == -3
    assert call(D=80) == -3
    assert call(q=A_ODD + 1, dt=0) == -6


def test_decode_step_validation(G):
    f = G.lib.gqa_decode_step
    need = G.decode_step_workspace_bytes(1, 8, 2, 128, 1000, 0, 64)

    def call(**kw):
        a = dict(q=A16, kn=A16, vn=A16, dt=1, qs=8 * 128, kvs=2 * 128, wq=None, wk=None,
                 eps=1e-6, theta=1e4, pos=A16, kc=A16, vc=A16, lens=A16, window=0,
                 scale=0.0, P=64, ws=A16, wsb=need, out=A16, od=0, lse=None, qo=None,
                 B=1, Hq=8, Hkv=2, D=128, T=1000)
        a.update(kw)
        return f(a["q"], a["kn"], a["vn"], a["dt"], a["qs"], a["kvs"], a["wq"], a["wk"],
                 a["eps"], a["theta"], a["pos"], a["kc"], a["vc"], a["lens"], a["window"],
                 a["scale"], a["P"], a["ws"], a["wsb"], a["out"], a["od"], a["lse"], a["qo"],
                 a["B"], a["Hq"], a["Hkv"], a["D"], a["T"], None)
    assert call(ws=None) == -1
    assert call(lens=None) == -1
    assert call(kn=None) == -1                  # pos without k_new
    assert call(pos=None, kn=None) == -1        # v_new without pos
    assert call(pos=None, kn=None, vn=None, qo=A16) == -1     # q_out needs the prologue
    assert call(pos=None, kn=None, vn=None, wq=A16, wk=A16) == -1
    assert call(wk=A16) == -1
    assert call(Hq=7) == -2                     # Hq not a multiple of Hkv
    assert call(qs=100) == -2
    assert call(P=0) == -7
    assert call(eps=float("nan")) == -7
    assert call(theta=float("nan")) == -7
    assert call(D=96) == -3
    assert call(dt=3) == -3
    assert call(qs=8 * 128 + 1) == -6           # q rows lose 16-byte alignment
    assert call(ws=A16 + 16) == -6
    assert call(wsb=need - 1) == -4
    # split-K workspace rounded to 256 B, then one ticket per (seq, KV head)
    base = G.splitk_workspace_bytes(1, 8, 128, 1000, 0, 64)
    assert need == base + (-base) % 256 + 2 * 4


def test_partition_counts_and_workspace(G):
    assert G.num_partitions(131072, 0, 2048) == 64
    assert G.num_partitions(32768, 4096, 512) == 8
    assert G.num_partitions(100, 1000, 7) == 15
    assert G.num_partitions(100, 0, 0) == 0
    # config 4: lse 1*32*64*4 = 8192 B (256-aligned) + o 32*64*128*4 B
    assert G.splitk_workspace_bytes(1, 32, 128, 131072, 0, 2048) == 8192 + 1048576
    assert G.splitk_workspace_bytes(1, 3, 64, 10, 0, 4) == 256 + 3 * 3 * 64 * 4


def test_status_strings(G):
    for s in range(-7, 1):
        assert G.lib.gqa_status_string(s)
    assert G.lib.gqa_status_string(-99) == b"unknown status"


def test_probe_validation(G):
    f = G.lib.gqa_probe_stream_read

    def call(**kw):
        a = dict(buf=A16, n=1 << 20, wg=256, th=256, u=8, sink=A16)
        a.update(kw)
        return f(a["buf"], a["n"], a["wg"], a["th"], a["u"], a["sink"], None)
    assert call(buf=None) == -1
    assert call(sink=None) == -1
    assert call(n=8) == -2
    assert call(n=(1 << 31) + 16) == -2
    assert call(wg=0) == -2
    assert call(n=(1 << 20) + 8) == -6
    assert call(buf=A16 + 8) == -6
    assert call(th=96) == -7
    assert call(th=2048) == -7
    assert call(u=5) == -3
