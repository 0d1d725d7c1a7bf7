"""Seeded random sweep over the whole surface: the decode step (split,
unsplit and fused), several tokens per sequence (split, unsplit and in one
launch), the prefill (causal and bidirectional, with and without key
splits, with the q prologue in the kernel) and the packed QKV projection.  Each case draws its sizes
from a fixed-seed generator -- group size, head dim, batch, cache length,
lengths (ragged, some zero), window, partition size, token count, output
dtype -- and is checked against the fp64 oracle at the same bars as the
fixed cases (outputs, LSE, the rotated q and the appended K/V rows).  The
case list is the same on every run; the ids name the drawn sizes."""
import numpy as np
import pytest

import workloads as W
from oracle import reference as O

GS = [1, 2, 4, 8, 16]


def _decode_cases(n=60, seed=1234):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice(GS))
        Hkv = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 5))
        T = int(rng.integers(2, 700))
        window = 0 if rng.random() < 0.5 else int(rng.integers(1, T + 1))
        mode = str(rng.choice(["split", "unsplit", "fused"]))
        prologue = bool(rng.random() < 0.7)
        out.append(dict(G=G, Hkv=Hkv, D=D, B=B, T=T, window=window, mode=mode,
                        prologue=prologue, norm=bool(rng.random() < 0.5),
                        out=str(rng.choice(["f32", "bf16"])), P=int(rng.integers(16, 600)),
                        zero=bool(rng.random() < 0.3), seed=int(rng.integers(1 << 30))))
    return out


def _tokens_cases(n=60, seed=4321, prefill=False, fused=False, splits=False, step=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice(GS))
        Hkv = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        if prefill:
            S = int(rng.integers(1, 300))
        else:
            S = int(rng.integers(1, 16 // G + 1))
        T = int(rng.integers(S + 1, S + 700))
        window = 0 if rng.random() < 0.5 else int(rng.integers(1, T + 1))
        mode = "prefill" if prefill else str(rng.choice(["split", "unsplit"]))
        if fused:
            mode = "fused"
        out.append(dict(G=G, Hkv=Hkv, D=D, B=B, S=S, T=T, window=window, mode=mode,
                        prologue=bool(rng.random() < 0.6), norm=bool(rng.random() < 0.5),
                        causal=bool(rng.random() < 0.7) if prefill else True,
                        out=str(rng.choice(["f32", "bf16"])), P=int(rng.integers(16, 600)),
                        zero=bool(rng.random() < 0.3), seed=int(rng.integers(1 << 30))))
        if splits:
            out[-1]["splits"] = int(rng.integers(2, 7))
        if step:                       # the prefill with its prologue in the kernel
            out[-1]["mode"] = "prefill_step"
            out[-1]["prologue"] = True
    return out


def _gemv_cases(n=30, seed=99):
    rng = np.random.default_rng(seed)
    return [dict(M=int(rng.integers(1, 17)), K=128 * int(rng.integers(1, 25)),
                 N=int(rng.integers(1, 700)), out=str(rng.choice(["f32", "bf16"])),
                 xpad=8 * int(rng.integers(0, 3)), ypad=int(rng.integers(0, 5)),
                 seed=int(rng.integers(1 << 30))) for _ in range(n)]


def _cid(c):
    keys = ("mode", "G", "Hkv", "D", "B", "S", "T", "window", "out", "splits")
    return "-".join(f"{k}{c[k]}" for k in keys if k in c)


def _workload(c):
    """A ragged workload (the prologue appends token s at row lens - S + s)
    or one without a prologue (q given in bf16), per the drawn sizes."""
    S = c.get("S", 1)
    over = dict(B=c["B"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"], L=c["T"], S=S,
                window=c["window"], out_dtype=c["out"], part_tokens=c["P"], norm=c["norm"],
                causal=c.get("causal", True))
    if c["prologue"]:
        w = W.make("3", seed=c["seed"], lmin=1, theta=5e5, **over)
    else:
        over.pop("norm")
        w = W.make("4", seed=c["seed"], peaky=0.0, **over)
    if c["zero"]:                      # some sequences have no row (or fewer than S)
        w.lens = w.lens.copy()
        w.lens[0] = 0 if S == 1 else min(int(w.lens[0]), S // 2)
        if w.pos is not None:
            w.pos = (w.lens - S).astype(np.int32)
    return w


def _run(c):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_attention_kv_amd import runner
    from test_gpu_parity import check_attention, check_prologue
    from test_multi_token import check_prologue_multi
    w = _workload(c)
    print(f"\n[case] sweep {c}", flush=True)
    ref = O.decode_step(w)
    step = runner.DeviceStep(w, mode=c["mode"], part_tokens=c["P"], splits=c.get("splits", 1))
    step.run()
    got = step.results()
    check_attention(got, ref, w.out_dtype, _cid(c))
    if w.pos is not None:
        if w.S > 1:
            check_prologue_multi(w, got, ref, _cid(c))
        else:
            check_prologue(w, got, ref, _cid(c))


@pytest.mark.gpu
@pytest.mark.parametrize("c", _decode_cases(), ids=_cid)
def test_gpu_sweep_decode(c):
    _run(c)


@pytest.mark.gpu
@pytest.mark.parametrize("c", _tokens_cases(), ids=_cid)
def test_gpu_sweep_tokens(c):
    _run(c)


@pytest.mark.gpu
@pytest.mark.parametrize("c", _tokens_cases(n=40, seed=5678, fused=True), ids=_cid)
def test_gpu_sweep_tokens_one_launch(c):
    _run(c)


@pytest.mark.gpu
@pytest.mark.parametrize("c", _tokens_cases(n=60, seed=777, prefill=True), ids=_cid)
def test_gpu_sweep_prefill(c):
    _run(c)


@pytest.mark.gpu
@pytest.mark.parametrize("c", _tokens_cases(n=30, seed=2468, prefill=True, splits=True),
                         ids=_cid)
def test_gpu_sweep_prefill_split(c):
    _run(c)


@pytest.mark.gpu
@pytest.mark.parametrize("c", _tokens_cases(n=30, seed=1357, prefill=True, splits=True,
                                            step=True), ids=_cid)
def test_gpu_sweep_prefill_step(c):
    _run(c)


@pytest.mark.gpu
@pytest.mark.parametrize("c", _gemv_cases(), ids=lambda c: f"M{c['M']}-K{c['K']}-N{c['N']}-{c['out']}")
def test_gpu_sweep_gemv(c):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd as G
    from test_gemv import _run as run_gemv, check_gemv
    g = W.make_gemv("8", seed=c["seed"], M=c["M"], K=c["K"], N=c["N"])
    print(f"\n[case] sweep gemv {c}", flush=True)
    got = run_gemv(torch, G, g, c["out"], c["xpad"], c["ypad"])
    check_gemv(got, O.linear(g.x, g.w), c["out"], f"sweep gemv {c}")
