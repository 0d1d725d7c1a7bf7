"""Several query tokens per sequence (draft-token verification; the fusedtok
README's attention_prefill attends S query rows causally): token s of
sequence b attends lens[b] - (S-1-s) rows, all G*S (token, head) rows of a KV
head sharing each cache row read.  CPU: host-side validation of the C ABI.
GPU: the prologue with S tokens and the unsplit and split attention paths
against the fp64 oracle, including S that is not a power of two (padding
columns), windows, and the full-size config 6."""
import numpy as np
import pytest

import workloads as W
from oracle import reference as O

A16 = 0x100000        # stand-in device addresses: every call below fails on the host


@pytest.fixture(scope="module")
def G():
    import gqa_attention_kv_amd
    return gqa_attention_kv_amd


def test_multi_validation(G):
    def attn(S=4, Hq=32, Hkv=8, q=A16):
        return G.lib.gqa_attn_decode_multi(q, 1, A16, A16, A16, S, 0, 0.0, A16, 0, None,
                                           1, Hq, Hkv, 128, 16, None)
    assert attn(q=None) == -1
    assert attn(S=0) == -2
    assert attn(S=5) == -3            # 4 heads x 5 tokens = 20 > 16 columns
    assert attn(S=17, Hq=8, Hkv=8) == -3
    ws = G.splitk_multi_workspace_bytes(1, 4, 32, 128, 16, 0, 8)
    def split(S=4, wsb=ws, P=8):
        return G.lib.gqa_attn_decode_splitk_multi(A16, 1, A16, A16, A16, S, 0, 0.0, P, A16,
                                                  wsb, 1, 32, 8, 128, 16, None)
    assert split(wsb=ws - 1) == -4
    assert split(P=0) == -7
    assert split(S=8) == -3
    def merge(S=4, wsb=ws):
        return G.lib.gqa_attn_decode_merge_multi(A16, wsb, S, 0, 8, A16, 0, None, 1, 32, 128,
                                                 16, None)
    assert merge(wsb=ws - 1) == -4
    assert merge(S=0) == -2


def test_multi_workspace_and_partitions(G):
    # window 100 with S = 4 tokens: the union spans 103 rows -> 13 partitions of 8
    np_ = (100 + 4 - 1 + 7) // 8
    rows = 2 * 4 * 8
    want = rows * np_ * 4
    want += (-want) % 256 + rows * np_ * 64 * 4
    assert G.splitk_multi_workspace_bytes(2, 4, 8, 64, 1000, 100, 8) == want
    # S = 1 is the single-token layout
    assert G.splitk_multi_workspace_bytes(3, 1, 8, 64, 500, 0, 16) == \
        G.splitk_workspace_bytes(3, 8, 64, 500, 0, 16)


def check_prologue_multi(w, got, ref, what=""):
    qerr = float(np.max(np.abs(got["q"] - ref["q_hat"])))
    assert qerr <= 1e-4, f"{what}: max|q_out - oracle| = {qerr}"
    assert np.array_equal(got["v_cache"], ref["v_cache"]), f"{what}: V cache differs"
    rk, gk = ref["k_cache"], got["k_cache"]
    for b, g, t, _ in np.argwhere(gk != rk):
        assert int(w.pos[b]) <= t < int(w.pos[b]) + w.S, f"{what}: row {t} changed"
    diff = gk != rk
    if diff.any():
        a, c = gk[diff].astype(np.int32), rk[diff].astype(np.int32)
        assert np.all(np.abs(a - c) <= 1) and np.all((a >> 15) == (c >> 15))


CASES = [("6", dict(B=2, L=2000)),                               # S=4, G=4: 16 columns
         ("6", dict(B=3, L=1500, S=3)),                          # 12 columns (4 padding)
         ("6", dict(B=2, L=900, S=2, Hq=16, Hkv=2)),             # G=8, S=2
         ("6", dict(B=2, L=700, S=16, Hq=8, Hkv=8)),             # G=1, S=16
         ("5", dict(B=2, L=3000, window=1000, S=2)),             # window per token, QK-norm
         ("1", dict(S=2)),                                       # D=64, 8 columns
         ("3", dict(B=4, L=2000, S=4, lmin=1)),                  # ragged lengths
         ("6", dict(B=2, L=600, S=4, layout="noprologue"))]      # q given in bf16


@pytest.mark.gpu
@pytest.mark.parametrize("name,over", CASES, ids=[f"cfg{c[0]}_{i}" for i, c in enumerate(CASES)])
@pytest.mark.parametrize("mode", ["unsplit", "split"])
def test_gpu_multi_token(name, over, mode):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_attention_kv_amd import runner
    from test_gpu_parity import check_attention
    w = W.make(name, **over)
    print(f"\n[case] multi-token cfg={name} {over} mode={mode}", flush=True)
    ref = O.decode_step(w)
    step = runner.DeviceStep(w, mode=mode, part_tokens=256)
    step.run()
    got = step.results()
    check_attention(got, ref, w.out_dtype, f"multi {name} {mode}")
    if w.pos is not None:
        check_prologue_multi(w, got, ref, f"multi {name} {mode}")


@pytest.mark.gpu
def test_gpu_multi_token_full_size():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_attention_kv_amd import runner
    from test_gpu_parity import check_attention
    w = W.make("6")
    print("\n[case] multi-token cfg=6 full size split", flush=True)
    ref = O.decode_step(w)
    step = runner.DeviceStep(w, mode="split")
    step.run()
    got = step.results()
    check_attention(got, ref, w.out_dtype, "multi full size")
    check_prologue_multi(w, got, ref, "multi full size")


@pytest.mark.gpu
def test_gpu_multi_token_s1_equals_single():
    """S = 1 through the multi-token entry points is the single-token path,
    bit for bit."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd as Gm
    from gqa_attention_kv_amd import runner
    w = W.make("3", B=4, L=2000)
    print("\n[case] multi-token S=1 vs single", flush=True)
    step = runner.DeviceStep(w, mode="unsplit", out_dtype="f32")
    step.run()
    q4 = step.q.unsqueeze(1).contiguous()
    out = Gm.attn_decode_multi(q4, step.k_cache, step.v_cache, step.lens, window=w.window)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0], step.out)
