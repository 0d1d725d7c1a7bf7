"""gqa_decode_step_noalloc (the fused step on the library's static scratch)
through the C ABI, against gqa_decode_step_multi (the same step on a
caller-allocated workspace) and the fp64 oracle.

Two calls in a row, the second with a smaller input, so the second call
runs on scratch the first one left behind: its tickets must be back at zero
and its stale partials must not leak into the result.  The results must be
bit-identical to the workspace entry point's (same kernel, same order of
operations) and within the parity bar of the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import reference as O
from test_gpu_parity import check_attention, check_prologue
from test_multi_token import check_prologue_multi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd
    return gqa_attention_kv_amd


def _run(G, w, P, noalloc):
    import torch
    from gqa_attention_kv_amd import runner
    step = runner.DeviceStep(w, mode="fused", part_tokens=P)
    tok = lambda t: t if t is None or t.dim() == 4 else t.unsqueeze(1)  # noqa: E731
    pro = w.pos is not None
    q = tok(step.q_in if pro else step.q)
    args = dict(inv_freq=step.inv_freq if pro else None, rope_mscale=step.rope_mscale,
                rope_layout=step.rope_layout, q_norm_w=step.w_q if pro else None,
                k_norm_w=step.w_k if pro else None, eps=w.eps, window=w.window,
                out=tok(step.out), lse_out=step.lse.reshape(w.B, w.S, w.Hq),
                q_out=tok(step.q) if pro else None)
    if pro and step.inv_freq is None and w.theta > 0:
        args["inv_freq"], args["rope_mscale"] = G.rope_table("default", w.D, w.theta)
    ins = (q, tok(step.k_new) if pro else None, tok(step.v_new) if pro else None,
           step.pos if pro else None, step.k_cache, step.v_cache, step.lens, P)
    if noalloc:
        G.decode_step_noalloc(*ins, **args)
    else:
        G.decode_step_multi(*ins, workspace=step.ws, **args)
    torch.cuda.synchronize()
    return step.results()


# (workload, overrides, partition rows): the second case of each pair is
# smaller than the first (fewer sequences, heads, partitions).
PAIRS = [
    (("5", dict(B=4, L=6000, window=3000), 512), ("5", dict(B=2, L=2500, window=1000), 256)),
    (("4", dict(L=40000), 2048), ("1", {}, 48)),
    (("6", dict(B=4, L=3000), 512), ("2a", {}, 128)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["window", "long_then_tiny", "multi_then_qwen"])
def test_noalloc_matches_workspace_entry_point(G, pair):
    for (name, over, P) in pair:
        print(f"\n[case] noalloc cfg={name} {over} P={P}", flush=True)
        w = W.make(name, **over)
        got = _run(G, w, P, noalloc=True)
        want = _run(G, w, P, noalloc=False)
        assert np.array_equal(got["out"], want["out"]), f"{name}: out differs"
        assert np.array_equal(got["lse"], want["lse"]), f"{name}: lse differs"
        assert np.array_equal(got["k_cache"], want["k_cache"]), f"{name}: k_cache differs"
        assert np.array_equal(got["v_cache"], want["v_cache"]), f"{name}: v_cache differs"
        ref = O.decode_step(w)
        check_attention(got, ref, w.out_dtype, f"noalloc {name}")
        if w.pos is not None:
            check = check_prologue_multi if w.S > 1 else check_prologue
            check(w, got, ref, f"noalloc {name}")


def test_noalloc_rejects_oversized_shapes(G):
    import torch
    w = W.make("4", L=4096)
    from gqa_attention_kv_amd import runner
    step = runner.DeviceStep(w, mode="fused", part_tokens=16)
    # 256 partitions x 32 heads x 128 x 4 B = 4 MiB fits; 8 rows per
    # partition (512 partitions, 8 MiB of partials) does not
    with pytest.raises(G.GQAError) as e:
        G.decode_step_noalloc(step.q.unsqueeze(1), None, None, None, step.k_cache, step.v_cache,
                              step.lens, 8, out=step.out.unsqueeze(1))
    assert e.value.status == -8
    torch.cuda.synchronize()
