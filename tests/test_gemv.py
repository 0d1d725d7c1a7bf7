"""Packed QKV projection (gqa_qkv_gemv): y = x W^T for the decode batch,
the step ahead of the prologue.  CPU: host-side validation of the C ABI.
GPU: against the fp64 oracle -- a bf16 output within one bf16 ulp of the
exact value, an fp32 output within 1e-3 --
over ragged row blocks, every M up to 16, row-strided x and y, K from one
128-column step up, the full-size 70B-shaped batch and the PyGPUkit table
shapes; bit-identical reruns; and the chain projection -> prologue (reading
q | k_new | v_new straight from the packed rows) -> attention."""
import numpy as np
import pytest

import workloads as W
from oracle import reference as O

A16 = 0x100000        # stand-in device addresses: every call below fails on the host


@pytest.fixture(scope="module")
def G():
    import gqa_attention_kv_amd
    return gqa_attention_kv_amd


def test_gemv_validation(G):
    def call(x=A16, w=A16, y=A16, M=8, N=1024, K=1024, xs=1024, ws=1024, ys=1024, yd=1):
        return G.lib.gqa_qkv_gemv(x, xs, w, ws, y, yd, ys, M, N, K, None)
    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(M=0) == -2
    assert call(M=17) == -3
    assert call(K=1000, xs=1000, ws=1000) == -3     # K not a multiple of 128
    assert call(yd=7) == -3
    assert call(xs=512) == -2                        # stride below K
    assert call(ys=100) == -2
    assert call(xs=1028) == -6                       # stride not a multiple of 8
    assert call(w=A16 + 8) == -6
    assert call(y=A16 + 2, yd=0) == -6               # fp32 output needs 4-byte alignment
    assert call(ws=1 << 28) == -2                    # a share of rows exceeds 32-bit byte offsets
    assert call(ws=1 << 26) == -2                    # 64 rows of 2^26 elements do too


def check_gemv(got, ref64, out_dtype, what=""):
    """bf16: within one bf16 ulp (at the exact value) of the exact value --
    round to nearest gives half an ulp, float32 accumulation may cross one
    rounding boundary -- with a 1e-6 floor for values near zero; fp32:
    within 1e-3."""
    if out_dtype == "bf16":
        have = O.bf16_to_f64(got)
        ulp = np.ldexp(1.0, np.frexp(ref64)[1] - 8)
        excess = np.abs(have - ref64) - (ulp + 1e-6)
        assert float(excess.max()) <= 0.0, f"{what}: beyond one bf16 ulp by {excess.max()}"
    else:
        err = float(np.max(np.abs(got.astype(np.float64) - ref64)))
        assert err <= 1e-3, f"{what}: max|y - oracle| = {err}"


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _run(torch, G, g, out_dtype=None, x_pad=0, y_pad=0):
    dev = torch.device("cuda")
    od = out_dtype or g.out_dtype
    xt = torch.from_numpy(np.pad(g.x, ((0, 0), (0, x_pad))).view(np.int16)).to(dev)
    xt = xt.view(torch.bfloat16)[:, :g.K]
    wt = torch.from_numpy(g.w.view(np.int16)).to(dev).view(torch.bfloat16)
    tdt = torch.bfloat16 if od == "bf16" else torch.float32
    y = torch.full((g.M, g.N + y_pad), -7.0, dtype=tdt, device=dev)
    G.qkv_gemv(xt, wt, out=y[:, :g.N])
    torch.cuda.synchronize()
    full = y.cpu()
    if y_pad:
        assert torch.all(full[:, g.N:] == -7.0), "wrote past N"
    out = full[:, :g.N]
    return out.view(torch.int16).numpy().view(np.uint16) if od == "bf16" else out.numpy()


CASES = [  # (overrides, output dtype, x pad, y pad)
    (dict(M=1, K=128, Hq=0, Hkv=0, N=64), "bf16", 0, 0),
    (dict(M=3, K=384, N=100), "f32", 8, 4),          # ragged row block, strided x and y
    (dict(M=8, K=1024, N=1536), "bf16", 0, 0),
    (dict(M=16, K=512, N=272), "f32", 0, 0),
    (dict(M=5, K=640, N=33), "bf16", 16, 8),         # five 128-column steps over 4 waves
    (dict(M=2, K=2048, N=2000), "f32", 0, 0),
    (dict(M=7, K=256, N=5000), "f32", 0, 4),         # 20-row shares: a 4-row last tile
    (dict(M=4, K=384, N=20000), "bf16", 8, 0),       # 64-row shares, more than one per CU
    (dict(M=16, K=1152, N=700), "f32", 0, 0),        # 3-row shares: 13 padding rows a tile
]


@pytest.mark.gpu
@pytest.mark.parametrize("over,od,xpad,ypad", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_gpu_gemv(G, over, od, xpad, ypad):
    torch = _gpu()
    g = W.make_gemv("8", **over)
    print(f"\n[case] gemv {over} {od}", flush=True)
    got = _run(torch, G, g, od, xpad, ypad)
    check_gemv(got, O.linear(g.x, g.w), od, f"gemv {over}")


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["8", "8a", "8b"])
def test_gpu_gemv_full_size(G, name):
    torch = _gpu()
    g = W.make_gemv(name)
    print(f"\n[case] gemv full size {name}", flush=True)
    got = _run(torch, G, g)
    check_gemv(got, O.linear(g.x, g.w), g.out_dtype, f"gemv {name}")
    got32 = _run(torch, G, g, "f32")
    check_gemv(got32, O.linear(g.x, g.w), "f32", f"gemv {name} f32")


@pytest.mark.gpu
def test_gpu_gemv_bit_identical_reruns(G):
    torch = _gpu()
    g = W.make_gemv("8", K=2048)
    a = _run(torch, G, g, "f32")
    b = _run(torch, G, g, "f32")
    assert np.array_equal(a, b)


@pytest.mark.gpu
def test_gpu_projection_prologue_attention_chain(G):
    """The projection's bf16 rows feed the prologue as packed q | k | v (batch
    stride N) and the attention follows; the oracle runs the same chain from
    the projection the GPU produced (checked here against the oracle first)."""
    torch = _gpu()
    dev = torch.device("cuda")
    B, Hq, Hkv, D, K, T = 3, 8, 2, 128, 512, 300
    g = W.make_gemv("8", M=B, K=K, Hq=Hq, Hkv=Hkv, D=D)
    print("\n[case] projection -> prologue -> attention", flush=True)
    xt = torch.from_numpy(g.x.view(np.int16)).to(dev).view(torch.bfloat16)
    wt = torch.from_numpy(g.w.view(np.int16)).to(dev).view(torch.bfloat16)
    y = G.qkv_gemv(xt, wt)
    ybits = y.cpu().view(torch.int16).numpy().view(np.uint16)
    check_gemv(ybits, O.linear(g.x, g.w), "bf16", "chain projection")

    w = W.make("2a", B=B, Hq=Hq, Hkv=Hkv, L=T - 64)
    lens = np.array([T - 64 + 1, 10, T - 1], np.int32)
    pos = (lens - 1).astype(np.int32)
    kc = torch.from_numpy(w.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    vc = torch.from_numpy(w.v_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    wq = torch.from_numpy(w.w_q).to(dev)
    wk = torch.from_numpy(w.w_k).to(dev)
    q = y[:, :Hq * D].view(B, Hq, D)
    kn = y[:, Hq * D:(Hq + Hkv) * D].view(B, Hkv, D)
    vn = y[:, (Hq + Hkv) * D:].view(B, Hkv, D)
    pos_t = torch.from_numpy(pos).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    q_hat = G.qkv_prologue(q, kn, vn, pos_t, kc, vc, q_norm_w=wq, k_norm_w=wk, eps=1e-6,
                           rope_theta=w.theta)
    out = G.attn_decode(q_hat, kc, vc, lens_t)
    torch.cuda.synchronize()

    qb, kb, vb = O.split_qkv(ybits, Hq, Hkv, D)
    rq, rkc, rvc = O.qkv_prologue(O.bf16_to_f64(qb), O.bf16_to_f64(kb), O.bf16_to_f64(vb),
                                  w.w_q, w.w_k, 1e-6, w.theta, pos, w.k_cache, w.v_cache)
    ro, _ = O.attend(rq, rkc, rvc, lens)
    assert float(np.max(np.abs(q_hat.cpu().numpy() - rq))) <= 1e-4
    assert float(np.max(np.abs(out.cpu().numpy() - ro))) <= 1e-3
