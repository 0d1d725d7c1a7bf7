"""The decode step inside a HIP graph (captured through torch.cuda.CUDAGraph
on torch's current stream), checked against the fp64 oracle on every replay.

Graph replay is what a serving loop does each step; the library allocates
nothing, reads nothing from the host and clears no memory with memset, so
capture needs no special entry point.  Between replays the test does eager
work on the same buffers -- poisons the output and lse and erases the
appended K/V rows -- and synchronises, so each replay must redo the append
and the attention itself.  Every replay is compared with ``decode_step`` of
the oracle at the parity bar (out, lse, rotated q, cache append), and with
the eager result bit for bit."""
import numpy as np
import pytest

import workloads as W
from oracle import reference as O
from test_gpu_parity import check_attention, check_prologue

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd  # noqa: F401  fails loudly if the library is missing
    return torch


CASES = [("1", {}, 48), ("2a", {}, 128), ("5", dict(B=2, L=3000, window=1000), 256),
         ("3", dict(B=4, L=2000), 256), ("4", dict(L=20000), 2048)]


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("name,over,P", CASES, ids=[c[0] for c in CASES])
def test_step_graph_replay(torch_gpu, mode, name, over, P):
    torch = torch_gpu
    from gqa_attention_kv_amd import runner
    print(f"\n[case] graph replay cfg={name} {over} mode={mode} P={P}", flush=True)
    w = W.make(name, **over)
    ref = O.decode_step(w, split=False)
    step = runner.DeviceStep(w, mode=mode, part_tokens=P)
    step.run()
    torch.cuda.synchronize()
    want_out, want_lse = step.out.clone(), step.lse.clone()
    # warm up on a side stream, as graph capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()
    for i in range(4):
        # eager work between replays: poison what the replay must rewrite
        step.out.fill_(float("nan"))
        step.lse.zero_()
        if w.pos is not None:
            step.q.fill_(float("nan"))
            for b in range(w.B):
                p = int(w.pos[b])
                if 0 <= p < w.T:
                    step.k_cache[b, :, p].zero_()
                    step.v_cache[b, :, p].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = step.results()
        check_attention(got, ref, w.out_dtype, f"replay {i}")
        if w.pos is not None:
            check_prologue(w, got, ref, f"replay {i}")
        assert torch.equal(step.out, want_out), f"replay {i}: out differs from eager"
        assert torch.equal(step.lse, want_lse), f"replay {i}: lse differs from eager"
        if mode == "fused":
            assert int(step.ws_counters().abs().sum().item()) == 0
    del graph
