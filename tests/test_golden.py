"""Closed-form fixtures of tests/golden/ (written by tests/golden/make_golden.py
with Python's math module only) against the fp64 oracle on the CPU, and the
attention fixtures against the HIP path (all three attention paths, through
the C ABI) on the GPU.  Each fixture names the page and section it follows.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import reference as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(x):
    """bf16 bit patterns of values that are exact in bf16 (checked)."""
    x = np.asarray(x, dtype=np.float64)
    b = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(b), x), "fixture input not exact in bf16"
    return b


def test_golden_rmsnorm_constant():
    g = _load("rmsnorm_constant.json")
    y = O.rmsnorm(np.array(g["x"]), np.array(g["w"]), g["eps"])
    np.testing.assert_allclose(y, g["y"], rtol=0, atol=1e-14)


def test_golden_rope_neox_d4():
    g = _load("rope_neox_d4.json")
    y = O.rope_neox(np.array(g["x"]), g["pos"], g["theta"])
    np.testing.assert_allclose(y, g["y"], rtol=0, atol=1e-14)


def _cache(rows):
    return _bits(rows)[None, None]          # [B=1, Hkv=1, T, D]


def test_golden_attention_two_keys():
    g = _load("attention_two_keys.json")
    q = np.array(g["q"])[None, None]
    out, lse = O.attend(q, _cache(g["K"]), _cache(g["V"]), np.array([2], np.int32), 0,
                        g["scale"])
    np.testing.assert_allclose(out[0, 0], g["out"], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - g["lse"]) <= 1e-14


def test_golden_attention_identical_keys():
    g = _load("attention_identical_keys.json")
    q = np.array(g["q"])[None, None]
    K = [g["k"]] * g["n"]
    out, lse = O.attend(q, _cache(K), _cache(g["V"]), np.array([g["n"]], np.int32))
    np.testing.assert_allclose(out[0, 0], g["out"], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - g["lse"]) <= 1e-13


def test_golden_split_merge_two_parts():
    g = _load("split_merge_two_parts.json")
    out, lse = O.lse_merge(np.array(g["o"])[None], np.array(g["lse_parts"])[None])
    np.testing.assert_allclose(out[0], g["out"], rtol=0, atol=1e-14)
    assert abs(lse[0] - g["lse"]) <= 1e-14


# ---------------------------------------------------------------------------
# GPU: the HIP attention paths on the same fixtures (fp32 q and output)
# ---------------------------------------------------------------------------
def _gpu_attention_cases():
    two = _load("attention_two_keys.json")
    ident = _load("attention_identical_keys.json")
    return [("two_keys", two["q"], two["K"], two["V"], two["scale"], two["out"], two["lse"]),
            ("identical_keys", ident["q"], [ident["k"]] * ident["n"], ident["V"], 0.0,
             ident["out"], ident["lse"])]


@pytest.mark.gpu
@pytest.mark.parametrize("case", _gpu_attention_cases(), ids=lambda c: c[0])
@pytest.mark.parametrize("path", ["unsplit", "split", "fused"])
def test_golden_attention_gpu(case, path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd as G
    name, q, K, V, scale, want_out, want_lse = case
    print(f"\n[case] golden {name} path={path}", flush=True)
    dev = torch.device("cuda:0")
    n, D = len(K), len(q)
    T = n + 3                                      # rows past lens are never read
    kc = np.zeros((1, 1, T, D), np.uint16)
    vc = np.zeros((1, 1, T, D), np.uint16)
    kc[0, 0, :n] = _bits(K)
    vc[0, 0, :n] = _bits(V)
    kc[0, 0, n:] = 0x7FC0                          # NaN guard rows
    vc[0, 0, n:] = 0x7FC0
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    k_t, v_t = to_dev(kc), to_dev(vc)
    q_t = torch.tensor(q, dtype=torch.float32, device=dev).reshape(1, 1, D)
    lens = torch.tensor([n], dtype=torch.int32, device=dev)
    out = torch.empty((1, 1, D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, 1), dtype=torch.float32, device=dev)
    if path == "unsplit":
        G.attn_decode(q_t, k_t, v_t, lens, scale=scale, out=out, lse_out=lse)
    elif path == "split":
        ws = G.attn_decode_splitk(q_t, k_t, v_t, lens, 1, scale=scale)   # one row per partition
        G.attn_decode_merge(ws, 1, 1, D, T, 1, out=out, lse_out=lse)
    else:
        nb = G.decode_step_workspace_bytes(1, 1, 1, D, T, 0, 1)
        ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
        G.decode_step(q_t, None, None, None, k_t, v_t, lens, 1, workspace=ws, scale=scale,
                      out=out, lse_out=lse)
    torch.cuda.synchronize()
    assert float(np.max(np.abs(out.cpu().numpy()[0, 0] - np.array(want_out)))) <= 1e-3
    assert abs(float(lse.cpu()[0, 0]) - want_lse) <= 1e-3
