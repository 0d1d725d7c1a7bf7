"""The decode step inside a HIP graph (captured through torch.cuda.CUDAGraph
on torch's current stream).  Graph replay is what a serving loop does each
step; the library allocates nothing, reads nothing from the host and clears
no memory with memset, so capture needs no special entry point.  Every
replay is checked against the eager result, with eager work and
synchronisations between the replays."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd  # noqa: F401  fails loudly if the library is missing
    return torch


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("name,over", [("5", dict(B=2, L=3000, window=1000)),
                                       ("3", dict(B=4, L=2000)), ("4", dict(L=20000))],
                         ids=["cfg5", "cfg3", "cfg4"])
def test_step_graph_replay(torch_gpu, mode, name, over):
    torch = torch_gpu
    from gqa_attention_kv_amd import runner
    print(f"\n[case] graph replay cfg={name} mode={mode}", flush=True)
    w = W.make(name, **over)
    step = runner.DeviceStep(w, mode=mode, part_tokens=256, out_dtype="f32")
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
        step.out.fill_(float("nan"))          # eager work between replays
        step.lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, want_out), f"replay {i}: out differs"
        assert torch.equal(step.lse, want_lse), f"replay {i}: lse differs"
        if mode == "fused":
            assert int(step.ws_counters().abs().sum().item()) == 0
    del graph
