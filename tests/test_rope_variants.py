"""RoPE pair layouts and context-extension tables (fusedtok 1.0.1 README,
Operators row RoPE: interleaved and NeoX layouts; PyGPUkit 0.2.18 page,
Positional Encoding Operations: NTK-aware, YaRN and linear-interpolation
tables).

CPU: the C library's host table builder against the oracle's own
implementation, and host-side rejection of bad rotary arguments.  GPU: the
prologue and the fused step with each layout and table against the oracle.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import reference as O

TABLES = [("default", {}), ("linear", dict(factor=4.0)), ("ntk", dict(factor=8.0)),
          ("yarn", dict(factor=4.0, orig_ctx=4096, beta_fast=32.0, beta_slow=1.0)),
          ("yarn", dict(factor=16.0, orig_ctx=512, beta_fast=16.0, beta_slow=0.5))]


@pytest.fixture(scope="module")
def G():
    import gqa_attention_kv_amd
    return gqa_attention_kv_amd


@pytest.mark.parametrize("D", [64, 128, 8])
@pytest.mark.parametrize("theta", [1e4, 5e5])
@pytest.mark.parametrize("kind,kw", TABLES, ids=lambda x: x if isinstance(x, str) else "")
def test_table_matches_oracle(G, D, theta, kind, kw):
    f, m = G.rope_table(kind, D, theta, **kw)
    g, mo = O.rope_inv_freq_scaled(D, theta, kind, **kw)
    assert np.max(np.abs(f - g) / g) <= 1e-14
    assert abs(m - mo) <= 1e-15


def test_table_validation(G):
    buf = np.zeros(64)
    call = lambda kind=0, D=128, theta=1e4, factor=2.0, ctx=4096, bf=32.0, bs=1.0, out=True: \
        G.lib.gqa_rope_table(kind, D, theta, factor, ctx, bf, bs,
                             buf.ctypes.data if out else None, None)
    assert call() == 0
    assert call(out=False) == -1
    assert call(D=7) == -2 and call(D=0) == -2
    assert call(kind=2, D=2) == -2                   # NTK needs D >= 4
    assert call(theta=0.0) == -7 and call(theta=float("nan")) == -7
    assert call(kind=4) == -7 and call(kind=-1) == -7
    assert call(kind=1, factor=0.5) == -7 and call(kind=1, factor=float("inf")) == -7
    assert call(kind=3, ctx=0) == -7 and call(kind=3, bf=1.0, bs=1.0) == -7
    assert call(kind=3, bs=-1.0) == -7
    assert call(kind=0, factor=0.5) == 0             # the plain table ignores the factor


A16 = 0x100000       # stand-in device addresses: every call below fails on the host


def test_prologue_ex_validation(G):
    good = np.full(64, 0.01)
    def call(f=good, m=1.0, lay=0, D=128, pos=A16, S=1):
        return G.lib.gqa_qkv_prologue_ex(
            A16, A16, A16, 1, S * 8 * D, S * 2 * D, None, None, 1e-6,
            None if f is None else f.ctypes.data, m, lay, pos, S, A16, A16, A16,
            1, 8, 2, D, 16, None)
    bad = good.copy(); bad[5] = float("nan")
    neg = good.copy(); neg[0] = -1.0
    assert call(f=bad) == -7 and call(f=neg) == -7
    assert call(m=0.0) == -7 and call(m=float("inf")) == -7
    assert call(lay=2) == -7
    assert call(D=96) == -3
    assert call(f=bad, pos=None) == -1                # null checks come first
    assert call(f=bad, S=0) == -2                     # S >= 1


def test_decode_step_ex_validation(G):
    good = np.full(64, 0.01)
    ws = G.decode_step_workspace_bytes(1, 8, 2, 128, 16, 0, 8)
    def call(f=good, m=1.0, lay=0, pos=A16, kn=A16, vn=A16):
        return G.lib.gqa_decode_step_ex(
            A16, kn, vn, 1, 8 * 128, 2 * 128, None, None, 1e-6,
            None if f is None else f.ctypes.data, m, lay, pos, A16, A16, A16, 0, 0.0, 8,
            A16, ws, A16, 0, None, None, 1, 8, 2, 128, 16, None)
    bad = good.copy(); bad[3] = float("inf")
    assert call(f=bad) == -7
    assert call(m=-1.0) == -7
    assert call(lay=7) == -7
    assert call(pos=None, kn=None, vn=None) == -1     # a table without a prologue


# ---------------------------------------------------------------------------
# GPU parity
# ---------------------------------------------------------------------------
VARIANTS = [("interleaved", None), ("neox", dict(kind="linear", factor=4.0)),
            ("interleaved", dict(kind="ntk", factor=8.0)),
            ("neox", dict(kind="yarn", factor=4.0, orig_ctx=4096)),
            ("interleaved", dict(kind="yarn", factor=16.0, orig_ctx=512, beta_fast=16.0,
                                 beta_slow=0.5))]


@pytest.mark.gpu
@pytest.mark.parametrize("layout,scaling", VARIANTS,
                         ids=["il", "neox_linear", "il_ntk", "neox_yarn", "il_yarn"])
@pytest.mark.parametrize("name,over", [("5", dict(B=2, L=3000, window=1000)),
                                       ("1", {}), ("3", dict(B=4, L=2000))],
                         ids=["cfg5", "cfg1_d64", "cfg3"])
def test_gpu_rope_variants(layout, scaling, name, over):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_attention_kv_amd import runner
    from test_gpu_parity import check_attention, check_prologue
    w = W.make(name, rope_layout=layout, rope_scaling=scaling, **over)
    ref = O.decode_step(w)
    for mode in ("split", "fused"):
        print(f"\n[case] rope {layout} {scaling} cfg={name} mode={mode}", flush=True)
        step = runner.DeviceStep(w, mode=mode, part_tokens=256)
        assert step.rope_ex
        step.run()
        got = step.results()
        check_attention(got, ref, w.out_dtype, f"rope {layout} {mode}")
        check_prologue(w, got, ref, f"rope {layout} {mode}")


@pytest.mark.gpu
def test_gpu_rope_variant_full_size():
    """Workload 5 at full size with interleaved pairs and a YaRN table."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_attention_kv_amd import runner
    from test_gpu_parity import check_attention, check_prologue
    w = W.make("5", rope_layout="interleaved",
               rope_scaling=dict(kind="yarn", factor=4.0, orig_ctx=8192))
    print("\n[case] rope interleaved yarn cfg=5 full size fused", flush=True)
    ref = O.decode_step(w)
    step = runner.DeviceStep(w, mode="fused")
    step.run()
    got = step.results()
    check_attention(got, ref, w.out_dtype, "rope full size")
    check_prologue(w, got, ref, "rope full size")
