"""Several query tokens per sequence (draft-token verification; the fusedtok
README's attention_prefill attends S query rows causally): token s of
sequence b attends lens[b] - (S-1-s) rows, all G*S (token, head) rows of a KV
head sharing each cache row read.  CPU: host-side validation of the C ABI.
GPU: the prologue with S tokens and the unsplit, split and one-launch
(gqa_decode_step_multi) paths against the fp64 oracle, including S that is
not a power of two (padding columns), windows, new rows straddling
partitions and tiles, rows past the cache end, NaN outside the attended rows,
and the full-size config 6."""
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


def _step_multi(G, S=4, Hq=32, Hkv=8, q=A16, pos=A16, qbs=None, wsb=None, P=64, T=4096,
                window=0, kn=A16):
    ws = G.decode_step_multi_workspace_bytes(1, S, Hq, Hkv, 128, T, window, P) if wsb is None \
        else wsb
    qbs = S * Hq * 128 if qbs is None else qbs
    return G.lib.gqa_decode_step_multi(q, kn, A16 if kn else None, 1, qbs, S * Hkv * 128, None,
                                       None, 1e-6, None, 1.0, 0, pos, S, A16, A16, A16, window,
                                       0.0, P, A16, ws, A16, 0, None, None, 1, Hq, Hkv, 128, T,
                                       None)


def test_step_multi_validation(G):
    assert _step_multi(G, q=None) == -1
    assert _step_multi(G, pos=None) == -1          # k_new without pos
    assert _step_multi(G, S=0, wsb=1 << 20) == -2
    assert _step_multi(G, S=5, wsb=1 << 20) == -3  # 4 heads x 5 tokens > 16 columns
    assert _step_multi(G, qbs=31 * 128 * 4) == -2  # batch stride below S * Hq * D
    ws = G.decode_step_multi_workspace_bytes(1, 4, 32, 8, 128, 4096, 0, 64)
    assert _step_multi(G, wsb=ws - 1) == -4
    assert _step_multi(G, P=0, wsb=1 << 20) == -7
    assert _step_multi(G, q=A16 + 8) == -6
    # one (sequence, KV head)'s partials ((S-1) Hq + G rows) must stay below 2 GiB
    assert _step_multi(G, S=2, Hq=64, Hkv=8, P=1, T=80000, wsb=1 << 40) == -2


def test_step_multi_workspace(G):
    # S = 1 is the single-token step's layout; S > 1: the multi-token split-K
    # layout, then B * Hkv tickets at the next 256-byte boundary
    assert G.decode_step_multi_workspace_bytes(3, 1, 32, 8, 128, 5000, 0, 256) == \
        G.decode_step_workspace_bytes(3, 32, 8, 128, 5000, 0, 256)
    base = G.splitk_multi_workspace_bytes(2, 4, 32, 128, 5000, 700, 256)
    assert G.decode_step_multi_workspace_bytes(2, 4, 32, 8, 128, 5000, 700, 256) == \
        base + (-base) % 256 + 2 * 8 * 4


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
@pytest.mark.parametrize("mode", ["unsplit", "split", "fused"])
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


def _fused(w, part_tokens, **kw):
    from gqa_attention_kv_amd import runner
    step = runner.DeviceStep(w, mode="fused", part_tokens=part_tokens, **kw)
    step.run()
    return step, step.results()


# (config, overrides, partition size, what the case covers); one launch
FUSED_EDGES = [
    ("6", dict(B=2, L=700, S=16, Hq=8, Hkv=8), 8,
     "G=1, S=16: the 16 new rows span three partitions and two tiles"),
    ("6", dict(B=2, L=500, S=4, Hq=16, Hkv=4), 3,
     "partitions of 3 rows: every new row in another partition"),
    ("5", dict(B=2, L=3000, window=700, S=2, rope_layout="interleaved"), 256,
     "window per token, QK-norm, interleaved pairs"),
    ("6", dict(B=2, L=900, S=2, Hq=16, Hkv=2,
               rope_scaling=dict(kind="yarn", factor=4.0, orig_ctx=512)), 128,
     "G=8, S=2 (folded lo columns), YaRN table and magnitude factor"),
    ("1", dict(S=3, L=100), 16, "D=64, S=3: padding columns"),
    ("3", dict(B=5, L=1200, S=4, lmin=1), 300, "ragged lengths, one partition for some"),
    ("6", dict(B=2, L=600, S=4, layout="noprologue"), 128, "no prologue: q given in bf16"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,over,P,what", FUSED_EDGES,
                         ids=[f"e{i}" for i in range(len(FUSED_EDGES))])
def test_gpu_step_multi_edges(name, over, P, what):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_gpu_parity import check_attention
    w = W.make(name, **over)
    print(f"\n[case] one-launch multi-token cfg={name} {over} P={P} ({what})", flush=True)
    ref = O.decode_step(w)
    step, got = _fused(w, P)
    check_attention(got, ref, w.out_dtype, f"step multi {name} {over}")
    if w.pos is not None:
        check_prologue_multi(w, got, ref, f"step multi {name} {over}")
    assert int(step.ws_counters().abs().sum()) == 0, "tickets not reset"


@pytest.mark.gpu
def test_gpu_step_multi_rows_past_end_and_empty():
    """Sequence 0's last two new rows fall past the cache end (not written,
    not attended); sequence 1 is empty (no row written, every token sees no
    row: out = 0, lse = -inf); NaN in every row no token attends."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_gpu_parity import check_attention
    w = W.make("6", B=3, L=800, S=4, Hq=16, Hkv=4)
    T = w.T
    w.pos = w.pos.copy()
    w.lens = w.lens.copy()
    w.pos[0], w.lens[0] = T - 2, T
    w.pos[1], w.lens[1] = -4, 0
    print(f"\n[case] one-launch multi-token past end / empty pos={w.pos.tolist()}", flush=True)
    ref = O.decode_step(w)
    _, got = _fused(w, 64)
    check_attention(got, ref, w.out_dtype, "step multi edges")
    check_prologue_multi(w, got, ref, "step multi edges")
    assert np.all(got["out"][1] == 0) and np.all(got["lse"][1] == -np.inf)
    _, bad = _fused(w, 64, poison=True)      # the caches now hold NaN rows: attention only
    check_attention(bad, ref, w.out_dtype, "step multi edges, poisoned")


@pytest.mark.gpu
def test_gpu_step_multi_reruns_and_s1():
    """Reruns are bit-identical; S = 1 through gqa_decode_step_multi is
    gqa_decode_step, bit for bit."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd as Gm
    from gqa_attention_kv_amd import runner
    w = W.make("6", B=3, L=1500, S=3)
    print("\n[case] one-launch multi-token reruns", flush=True)
    step = runner.DeviceStep(w, mode="fused", part_tokens=256)
    step.run()
    r1 = step.results()
    step.run()
    r2 = step.results()
    for k in ("out", "lse", "q", "k_cache", "v_cache"):
        assert np.array_equal(r1[k], r2[k]), k
    w1 = W.make("2a", B=2)
    one = runner.DeviceStep(w1, mode="fused", part_tokens=128)
    one.run()
    a = one.results()
    out = torch.empty((w1.B, 1, w1.Hq, w1.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w1.B, 1, w1.Hq), dtype=torch.float32, device="cuda")
    fresh = runner.DeviceStep(w1, mode="fused", part_tokens=128)
    Gm.decode_step_multi(fresh.q_in.unsqueeze(1), fresh.k_new.unsqueeze(1),
                         fresh.v_new.unsqueeze(1), fresh.pos, fresh.k_cache, fresh.v_cache,
                         fresh.lens, 128, inv_freq=Gm.rope_table("default", w1.D, w1.theta)[0],
                         q_norm_w=fresh.w_q, k_norm_w=fresh.w_k, eps=w1.eps, out=out,
                         lse_out=lse)
    torch.cuda.synchronize()
    assert np.array_equal(out[:, 0].cpu().numpy(), a["out"].astype(np.float32))
    assert np.array_equal(lse[:, 0].cpu().numpy(), a["lse"].astype(np.float32))


@pytest.mark.gpu
def test_gpu_step_multi_full_size():
    """Config 6 at full size in one launch (the launch the benchmark times)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_gpu_parity import check_attention
    w = W.make("6")
    print("\n[case] one-launch multi-token cfg=6 full size", flush=True)
    ref = O.decode_step(w)
    step, got = _fused(w, w.part_tokens)
    check_attention(got, ref, w.out_dtype, "step multi full size")
    check_prologue_multi(w, got, ref, "step multi full size")
