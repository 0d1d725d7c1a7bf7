"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (from the required precision of the decode output): max abs error
1e-3 for float32 output, 1.5e-2 for bf16 output; lse 1e-3; q_out 1e-4 abs.
Cache append: the set of changed rows is exactly {(b, g, pos_b)}, V rows are
bit-exact, K rows within one bf16 ulp of the oracle's single rounding, every
other row bit-identical.

Each test prints the case it runs before touching the GPU.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import reference as O

pytestmark = pytest.mark.gpu

OUT_TOL = {"f32": 1e-3, "bf16": 1.5e-2}
LSE_TOL = 1e-3
Q_TOL = 1e-4


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_kv_amd  # noqa: F401  fails loudly if the library is missing
    from gqa_attention_kv_amd import runner
    return runner


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def check_attention(got, ref, out_dtype, what=""):
    tol = OUT_TOL[out_dtype]
    assert np.all(np.isfinite(got["out"])), f"{what}: non-finite output"
    err = float(np.max(np.abs(got["out"] - ref["out"]))) if ref["out"].size else 0.0
    assert err <= tol, f"{what}: max|out - oracle| = {err} > {tol}"
    rl, gl = ref["lse"], got["lse"]
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: lse finiteness differs"
    assert np.all(gl[~fin] == -math.inf)
    if fin.any():
        lerr = float(np.max(np.abs(gl[fin] - rl[fin])))
        assert lerr <= LSE_TOL, f"{what}: max|lse - oracle| = {lerr}"
    return err


def check_prologue(w, got, ref, what=""):
    qerr = float(np.max(np.abs(got["q"] - ref["q_hat"])))
    assert qerr <= Q_TOL, f"{what}: max|q_out - oracle| = {qerr}"
    rk, gk = ref["k_cache"], got["k_cache"]
    assert np.array_equal(got["v_cache"], ref["v_cache"]), f"{what}: V cache differs"
    diff = np.argwhere(gk != rk)
    for b, g, t, _ in diff:
        assert t == w.pos[b], f"{what}: K row ({b},{g},{t}) changed but pos is {w.pos[b]}"
    if len(diff):
        a = gk[gk != rk].astype(np.int32)
        c = rk[gk != rk].astype(np.int32)
        assert np.all(np.abs(a - c) <= 1), f"{what}: K append differs by more than 1 ulp"
        assert np.all((a >> 15) == (c >> 15)), f"{what}: K append sign differs"
    # the rows at pos really were written (unless out of range)
    for b in range(w.B):
        p = int(w.pos[b])
        if 0 <= p < w.T:
            np.testing.assert_array_equal(ref["v_cache"][b, :, p], w.v_new[b])


def modes_for(w):
    """Paths every workload runs through."""
    return ["unsplit", "split", "fused"]


def run_and_check(gpu, w, split=True, part_tokens=None, out_dtype=None, q_dtype="bf16",
                  poison=False, scale=0.0, what="", mode=None):
    od = out_dtype or w.out_dtype
    pt = part_tokens or w.part_tokens
    mode = mode or ("split" if split else "unsplit")
    _say(f"{what} cfg={w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} T={w.T} "
         f"window={w.window} mode={mode} P={pt} out={od} q={q_dtype} poison={poison}")
    step = gpu.DeviceStep(w, part_tokens=pt, out_dtype=od, q_dtype=q_dtype,
                          poison=poison, scale=scale, mode=mode)
    step.run()
    got = step.results()
    # q in float32 holds the exact widening of the bf16 draws, and the oracle
    # reads only attended rows, so the unpoisoned bf16 workload serves as
    # the reference in every variant.
    ref = O.decode_step(w, split=False, scale=scale)
    err = check_attention(got, ref, od, what)
    if w.pos is not None and not poison:
        check_prologue(w, got, ref, what)
    return step, got, ref, err


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["1", "2a", "2b", "3", "4", "5"])
def test_full_size_split(gpu, name):
    w = W.make(name)
    run_and_check(gpu, w, split=True, what="full split")


@pytest.mark.parametrize("name", ["1", "2a", "2b", "3", "5"])
def test_full_size_unsplit(gpu, name):
    w = W.make(name)
    run_and_check(gpu, w, split=False, what="full unsplit")


@pytest.mark.parametrize("name", ["1", "2a", "2b", "3", "4", "5"])
def test_full_size_fused(gpu, name):
    w = W.make(name)
    run_and_check(gpu, w, mode="fused", what="full fused")


# ---------------------------------------------------------------------------
# Reduced sizes spanning several tiles and a ragged tail
# ---------------------------------------------------------------------------
REDUCED = [
    ("1", {}, [1, 7, 64, 100, 128]),
    ("2a", dict(L=700), [1, 33, 128, 256, 1000]),
    ("3", dict(B=6, L=1500, lmin=1), [17, 128, 512, 2048]),
    ("4", dict(L=6000), [64, 100, 2048, 5999, 8192]),
    ("5", dict(B=3, L=3000, window=700), [64, 129, 512, 700, 701]),
]


@pytest.mark.parametrize("name,over,parts", REDUCED, ids=[r[0] for r in REDUCED])
def test_reduced_split_sweep(gpu, name, over, parts):
    w = W.make(name, **over)
    ref = O.decode_step(w)
    for mode in [m for m in modes_for(w) if m != "unsplit"]:
        for pt in parts:
            _say(f"reduced cfg={name} {over} mode={mode} P={pt}")
            step = gpu.DeviceStep(w, part_tokens=pt, mode=mode)
            step.run()
            got = step.results()
            check_attention(got, ref, w.out_dtype, f"cfg {name} {mode} P={pt}")
            if w.pos is not None:
                check_prologue(w, got, ref, f"cfg {name} {mode} P={pt}")


@pytest.mark.parametrize("name,over,parts", REDUCED, ids=[r[0] for r in REDUCED])
def test_reduced_unsplit(gpu, name, over, parts):
    w = W.make(name, **over)
    run_and_check(gpu, w, split=False, what="reduced unsplit")


def test_split_partials_match_oracle(gpu):
    """The workspace holds the oracle's per-partition (o_k, lse_k)."""
    import gqa_attention_kv_amd as G
    w = W.make("5", B=2, L=1200, window=500)
    pt = 128
    _say("split partials cfg 5 reduced")
    step = gpu.DeviceStep(w, split=True, part_tokens=pt)
    step.prologue()
    step.attention()
    import torch
    torch.cuda.synchronize()
    lse, o = G.workspace_views(step.ws, w.B, w.Hq, w.D, w.T, w.window, pt)
    lse = lse.cpu().numpy().astype(np.float64)
    o = o.cpu().numpy().astype(np.float64)
    ref = O.decode_step(w, split=False)
    ro, rl = O.attend_partials(ref["q_hat"], ref["k_cache"], ref["v_cache"], w.lens,
                               w.window, 0.0, pt)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - rl[fin])) <= LSE_TOL
    assert np.max(np.abs(o[fin] - ro[fin])) <= 1e-3


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def _edge_workload(G=4, D=128, T=200, B=3, Hkv=2, name="3", lens=None, window=0,
                   out_dtype="f32", seed=11):
    over = dict(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, L=T, lmin=1, window=window,
                out_dtype=out_dtype)
    w = W.make(name, seed=seed, **over)
    if lens is not None:
        w.lens = np.asarray(lens, np.int32)
        if w.pos is not None:
            w.pos = np.clip(w.lens - 1, 0, None).astype(np.int32)
    return w


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_group_sizes_and_head_dims(gpu, G, D):
    w = _edge_workload(G=G, D=D, T=300, B=2, Hkv=2, lens=[300, 77])
    for mode in modes_for(w):
        run_and_check(gpu, w, mode=mode, part_tokens=64, what=f"G={G} D={D}")


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 129, 256])
def test_lengths_around_tiles(gpu, n):
    P = 128
    w = _edge_workload(G=4, D=128, T=256, B=2, lens=[n, max(1, 256 - n)])
    for mode in modes_for(w):
        run_and_check(gpu, w, mode=mode, part_tokens=P, what=f"n={n}")


@pytest.mark.parametrize("window", [1, 2, 99, 100, 101, 500])
def test_windows(gpu, window):
    w = _edge_workload(G=8, D=128, T=256, B=3, lens=[100, 256, 1], window=window)
    for mode, pt in (("split", 32), ("split", 1), ("unsplit", None), ("fused", 32),
                     ("fused", 1), ("fused", 4096)):
        run_and_check(gpu, w, mode=mode, part_tokens=pt, what=f"window={window}")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("q_dtype", ["f32", "bf16"])
def test_dtypes(gpu, out_dtype, q_dtype):
    w = W.make("4", L=3000, out_dtype=out_dtype)
    for mode in modes_for(w):
        run_and_check(gpu, w, mode=mode, part_tokens=512, out_dtype=out_dtype,
                      q_dtype=q_dtype, what=f"dtypes q={q_dtype} out={out_dtype}")


def test_explicit_scale(gpu):
    w = W.make("4", L=1000)
    for mode in modes_for(w):
        run_and_check(gpu, w, mode=mode, part_tokens=128, scale=0.3, what="scale=0.3")


def test_out_of_contract_lens(gpu):
    """lens = 0 / negative -> out 0, lse -inf; lens > T clamped to T."""
    w = _edge_workload(name="4", G=4, D=128, T=256, B=4, lens=[0, -5, 10_000, 256])
    for mode in modes_for(w):
        step, got, ref, _ = run_and_check(gpu, w, mode=mode, part_tokens=64,
                                          what="lens out of contract")
        assert np.all(got["out"][:2] == 0) and np.all(got["lse"][:2] == -math.inf)


def test_pos_out_of_range_writes_nothing(gpu):
    w = W.make("5", B=3, L=300, window=100)
    w.pos = np.array([-1, 300, 5000], np.int32)
    _say("prologue pos out of range")
    step = gpu.DeviceStep(w, split=True, part_tokens=64)
    step.prologue()
    got = step.results()
    assert np.array_equal(got["k_cache"], w.k_cache)
    assert np.array_equal(got["v_cache"], w.v_cache)
    ref_q, _, _ = O.qkv_prologue(O.bf16_to_f64(w.q), O.bf16_to_f64(w.k_new),
                                 O.bf16_to_f64(w.v_new), w.w_q, w.w_k, w.eps, w.theta,
                                 w.pos, w.k_cache[:, :, :1], w.v_cache[:, :, :1])
    assert np.max(np.abs(got["q"] - ref_q)) <= Q_TOL


def test_nan_poison_outside_window(gpu):
    """bf16 NaN in every row outside [lo, n): any stray read turns out into NaN."""
    for name, over in (("5", dict(B=3, L=2000, window=300)),
                       ("3", dict(B=5, L=1000, lmin=1)),
                       ("4", dict(L=3000))):
        w = W.make(name, **over)
        if name == "4":
            w.lens = np.array([1777], np.int32)
        for mode in modes_for(w):
            for pt in ((64, 100) if mode != "unsplit" else (None,)):
                run_and_check(gpu, w, mode=mode, part_tokens=pt, poison=True,
                              what=f"poison cfg {name}")


def test_prologue_fp32_inputs_and_packed_qkv(gpu):
    """fp32 inputs, and q/k/v as views of one packed [B, Hq+2Hkv, D] buffer."""
    import torch
    import gqa_attention_kv_amd as G
    from gqa_attention_kv_amd.runner import bf16_tensor, bf16_bits
    w = W.make("2a", B=3, L=100)
    B, Hq, Hkv, D, T = w.B, w.Hq, w.Hkv, w.D, w.T
    ref = O.decode_step(w)
    for dt in (torch.bfloat16, torch.float32):
        _say(f"prologue packed qkv dtype={dt}")
        packed = torch.empty((B, Hq + 2 * Hkv, D), dtype=dt, device="cuda")
        packed[:, :Hq] = bf16_tensor(w.q, "cuda").to(dt)
        packed[:, Hq:Hq + Hkv] = bf16_tensor(w.k_new, "cuda").to(dt)
        packed[:, Hq + Hkv:] = bf16_tensor(w.v_new, "cuda").to(dt)
        kc = bf16_tensor(w.k_cache, "cuda")
        vc = bf16_tensor(w.v_cache, "cuda")
        qo = G.qkv_prologue(packed[:, :Hq], packed[:, Hq:Hq + Hkv], packed[:, Hq + Hkv:],
                            torch.from_numpy(w.pos).cuda(), kc, vc,
                            q_norm_w=torch.from_numpy(w.w_q).cuda(),
                            k_norm_w=torch.from_numpy(w.w_k).cuda(),
                            eps=w.eps, rope_theta=w.theta)
        torch.cuda.synchronize()
        got = dict(q=qo.cpu().numpy().astype(np.float64), k_cache=bf16_bits(kc),
                   v_cache=bf16_bits(vc))
        check_prologue(w, got, ref, f"packed {dt}")


def test_bit_identical_reruns(gpu):
    # Every order is fixed (partitions, the merge, no float atomics): reruns
    # are bit-identical in all three modes.
    import torch
    for name, over, mode in (("5", dict(B=2, L=3000, window=1000), "split"),
                             ("3", dict(B=4, L=2000), "split"),
                             ("3", dict(B=4, L=2000), "unsplit"),
                             ("5", dict(B=2, L=3000, window=1000), "fused"),
                             ("3", dict(B=4, L=2000), "fused")):
        w = W.make(name, **over)
        _say(f"determinism cfg {name} mode={mode}")
        step = gpu.DeviceStep(w, mode=mode, part_tokens=256)
        step.run()
        a = (step.out.clone(), step.lse.clone())
        for _ in range(3):
            step.run()
            assert torch.equal(step.out, a[0]) and torch.equal(step.lse, a[1])


def test_fused_leaves_tickets_zero(gpu):
    # Every fused call leaves the arrival tickets at zero for the next one
    # (a stale ticket would make the wrong workgroup merge, or none).
    import torch
    for name, over in (("5", dict(B=2, L=3000, window=1000)), ("3", dict(B=4, L=2000)),
                       ("4", dict(L=20000))):
        w = W.make(name, **over)
        _say(f"fused tickets cfg {name}")
        step = gpu.DeviceStep(w, mode="fused", part_tokens=256, out_dtype="f32")
        for _ in range(3):
            step.run()
            torch.cuda.synchronize()
            assert int(step.ws_counters().abs().sum().item()) == 0


def test_split_matches_unsplit(gpu):
    w = W.make("3", B=4, L=2500, lmin=1)
    _say("split vs unsplit")
    outs = []
    for split, pt in ((False, None), (True, 64), (True, 1000), (True, 4096)):
        s = gpu.DeviceStep(w, split=split, part_tokens=pt, out_dtype="f32")
        s.run()
        outs.append(s.results()["out"])
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2e-5


# ---------------------------------------------------------------------------
# The fused whole-step launch
# ---------------------------------------------------------------------------
def test_fused_pos_not_attended_still_appends(gpu):
    """pos outside the attended window / past lens: the row is still written
    (by partition 0) and attention ignores it."""
    w = W.make("5", B=3, L=600, window=100)
    w.pos = np.array([599, 10, 300], np.int32)       # attended, before lo, before lo
    w.lens = np.array([600, 600, 200], np.int32)      # b=2: pos 300 >= n = 200
    run_and_check(gpu, w, mode="fused", part_tokens=32, what="fused pos not attended")


def test_fused_pos_out_of_range_and_empty(gpu):
    w = W.make("5", B=4, L=300, window=100)
    w.pos = np.array([-1, 300, 5000, 299], np.int32)
    w.lens = np.array([300, 0, 300, -7], np.int32)
    _say("fused pos out of range / empty lens")
    step = gpu.DeviceStep(w, mode="fused", part_tokens=32)
    step.run()
    got = step.results()
    ref = O.decode_step(w)
    check_attention(got, ref, "f32", "fused oob")
    assert np.all(got["out"][1] == 0) and np.all(got["out"][3] == 0)
    # rows of b=0..2 untouched; b=3 writes row 299
    kc = got["k_cache"]
    assert np.array_equal(kc[:3], w.k_cache[:3])
    check_prologue(w, got, ref, "fused oob")


def test_fused_single_partition_and_q_out(gpu):
    """One partition per (sequence, KV head): the workgroup writes the final
    output itself; q_out equals the oracle's rotated query."""
    w = W.make("2a", B=2, L=200)
    run_and_check(gpu, w, mode="fused", part_tokens=100000, what="fused one partition")


def test_fused_fp32_inputs_and_packed_qkv(gpu):
    import torch
    import gqa_attention_kv_amd as G
    from gqa_attention_kv_amd.runner import bf16_tensor, bf16_bits
    w = W.make("5", B=3, L=700, window=300)
    B, Hq, Hkv, D, T = w.B, w.Hq, w.Hkv, w.D, w.T
    ref = O.decode_step(w)
    for dt in (torch.bfloat16, torch.float32):
        _say(f"fused packed qkv dtype={dt}")
        packed = torch.empty((B, Hq + 2 * Hkv, D), dtype=dt, device="cuda")
        packed[:, :Hq] = bf16_tensor(w.q, "cuda").to(dt)
        packed[:, Hq:Hq + Hkv] = bf16_tensor(w.k_new, "cuda").to(dt)
        packed[:, Hq + Hkv:] = bf16_tensor(w.v_new, "cuda").to(dt)
        kc = bf16_tensor(w.k_cache, "cuda")
        vc = bf16_tensor(w.v_cache, "cuda")
        q_out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        out, _ = G.decode_step(packed[:, :Hq], packed[:, Hq:Hq + Hkv], packed[:, Hq + Hkv:],
                               torch.from_numpy(w.pos).cuda(), kc, vc,
                               torch.from_numpy(w.lens).cuda(), 64,
                               q_norm_w=torch.from_numpy(w.w_q).cuda(),
                               k_norm_w=torch.from_numpy(w.w_k).cuda(), eps=w.eps,
                               rope_theta=w.theta, window=w.window, lse_out=lse, q_out=q_out)
        torch.cuda.synchronize()
        got = dict(out=out.cpu().numpy().astype(np.float64),
                   lse=lse.cpu().numpy().astype(np.float64),
                   q=q_out.cpu().numpy().astype(np.float64),
                   k_cache=bf16_bits(kc), v_cache=bf16_bits(vc))
        check_attention(got, ref, "f32", f"fused packed {dt}")
        check_prologue(w, got, ref, f"fused packed {dt}")


def test_fused_matches_three_launch_path(gpu):
    w = W.make("3", B=6, L=3000, lmin=1)
    res = {}
    for mode in ("split", "fused"):
        _say(f"fused vs split {mode}")
        s = gpu.DeviceStep(w, mode=mode, part_tokens=256, out_dtype="f32")
        s.run()
        res[mode] = s.results()
    assert np.max(np.abs(res["split"]["out"] - res["fused"]["out"])) <= 2e-5
    assert np.max(np.abs(res["split"]["q"] - res["fused"]["q"])) <= 1e-5
