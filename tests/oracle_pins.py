"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each pin takes a namespace ``O`` exposing the oracle's functions and raises
AssertionError when the oracle disagrees with a closed form, an invariant,
brute force, or an independent library routine.  ``test_oracle_pins``
runs every pin on the real oracle; ``test_oracle_mutants`` runs them on
copies of the oracle with planted mistakes and requires at least one pin to
fail for each mistake.

Sources: fusedtok 1.0.1 README ("Operators", "Usage", "Benchmarks");
cutileGPT README ("Why tiles" RMSNorm figure; feature list).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import bruteforce as BF

RNG_SEED = 1234


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _bits(rng, shape):
    """Random finite bf16 bit patterns of N(0,1) draws (no dependence on oracle)."""
    x = rng.standard_normal(shape).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _torch_bf16_to_f64(bits):
    t = torch.from_numpy(np.asarray(bits, np.uint16).astype(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def _close(a, b, tol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


# ---------------------------------------------------------------------------
# bf16 conversion
# ---------------------------------------------------------------------------
def pin_bf16_decode_matches_torch(O):
    """Every non-NaN bf16 pattern widens exactly as torch's bfloat16 does."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _torch_bf16_to_f64(allb)
    ok = ~np.isnan(ref)
    got = O.bf16_to_f64(allb)
    assert np.array_equal(got[ok], ref[ok])
    assert np.all(np.isnan(got[~ok]))


def pin_bf16_roundtrip_all_patterns(O):
    """Rounding an exact bf16 value returns its own bit pattern (all 65536)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = _torch_bf16_to_f64(allb)
    ok = ~np.isnan(x)
    got = O.f64_to_bf16(x[ok])
    assert np.array_equal(got, allb[ok])


def pin_bf16_rne_matches_torch_on_fp32(O):
    """For float32-representable inputs one RNE rounding equals torch's
    float32 -> bfloat16 conversion (round to nearest even)."""
    rng = _rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * 3
    # add exact ties: bf16 value + half an ulp
    base = x[:5000].view(np.uint32) & np.uint32(0xFFFF0000)
    x[:5000] = (base | np.uint32(0x8000)).view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = O.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def pin_bf16_single_rounding_cases(O):
    """Hand-worked cases: ties go to even; a value just above a tie rounds up
    (which a float32 intermediate would lose); specials."""
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (1 + 2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),    # above tie -> up
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),    # below tie -> down
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
        (0.0, 0x0000), (-0.0, 0x8000),
        (math.inf, 0x7F80), (-math.inf, 0xFF80),
        (3.3895313892515355e38, 0x7F7F),          # largest finite bf16
        (3.4e38, 0x7F80),                          # rounds past the max -> inf
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # tie -> even (0)
        (3 * 2.0 ** -135, 0x0001),                 # 0.75 ulp -> 1 ulp
        (2.0 ** -126, 0x0080),                     # smallest normal
    ]
    xs = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases], np.uint16)
    got = O.f64_to_bf16(xs)
    assert np.array_equal(got, want), (got, want)
    assert O.f64_to_bf16(np.array([math.nan]))[0] & 0x7FFF > 0x7F80


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def pin_rmsnorm_matches_torch(O):
    rng = _rng(2)
    x = rng.standard_normal((7, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,),
                                       torch.from_numpy(w), eps=1e-6).numpy()
    _close(O.rmsnorm(x, w, 1e-6), ref, 1e-12, "rmsnorm vs torch")


def pin_rmsnorm_closed_forms(O):
    # x = c * 1: y = c / sqrt(c^2 + eps) * w
    w = np.array([0.5, 2.0, -1.0, 3.0])
    for c, eps in [(2.0, 0.0), (0.5, 1e-2), (-3.0, 1.0)]:
        _close(O.rmsnorm(np.full(4, c), w, eps), c / math.sqrt(c * c + eps) * w,
               1e-14, "rmsnorm const")
    # hand example: x=[3,4], w=[1,2], eps=0 -> mean square 12.5
    _close(O.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0),
           [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], 1e-15, "rmsnorm hand")
    # scale invariance with eps = 0
    rng = _rng(3)
    x = rng.standard_normal(64)
    w = rng.standard_normal(64)
    _close(O.rmsnorm(7.5 * x, w, 0.0), O.rmsnorm(x, w, 0.0), 1e-13, "rmsnorm scale")


# ---------------------------------------------------------------------------
# RoPE (NeoX)
# ---------------------------------------------------------------------------
def pin_rope_identity_and_norm(O):
    rng = _rng(4)
    x = rng.standard_normal((3, 128))
    assert np.array_equal(O.rope_neox(x, 0, 1e4), x)
    for pos in (1, 17, 4095, 32767, 131071):
        y = O.rope_neox(x, pos, 5e5)
        _close(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), 1e-12, "rope norm")


def pin_rope_relative_and_composition(O):
    rng = _rng(5)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    for p, r in [(3, 10), (100, 37), (4096, 5000)]:
        a = np.dot(O.rope_neox(q, p, 1e4), O.rope_neox(k, r, 1e4))
        b = np.dot(q, O.rope_neox(k, r - p, 1e4))
        assert abs(a - b) <= 1e-10 * (1 + abs(a)), (p, r, a, b)
        _close(O.rope_neox(O.rope_neox(q, p, 1e4), r, 1e4),
               O.rope_neox(q, p + r, 1e4), 1e-11, "rope composition")


def pin_rope_small_closed_forms(O):
    # D = 2: f_0 = 1, rotation by pos radians.
    x = np.array([0.3, -1.7])
    for p in (1, 2, 5):
        c, s = math.cos(p), math.sin(p)
        _close(O.rope_neox(x, p, 1e4), [x[0] * c - x[1] * s, x[1] * c + x[0] * s],
               1e-15, "rope D=2")
    # D = 4, theta = 4: f = [1, 4**-0.5 = 0.5]; pairs (0,2) and (1,3).
    x = np.array([1.0, 2.0, 3.0, 4.0])
    p = 3
    a0, a1 = p * 1.0, p * 0.5
    want = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
            3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    _close(O.rope_neox(x, p, 4.0), want, 1e-15, "rope D=4")


def pin_rope_complex_form(O):
    """NeoX rotation = multiplying z_i = x_i + j x_{i+D/2} by exp(j pos f_i)."""
    rng = _rng(6)
    x = rng.standard_normal(128)
    pos, theta = 777, 1e6
    f = theta ** (-np.arange(64) * 2.0 / 128)
    z = (x[:64] + 1j * x[64:]) * np.exp(1j * pos * f)
    _close(O.rope_neox(x, pos, theta), np.concatenate([z.real, z.imag]), 1e-12, "rope complex")


def pin_rope_interleaved_complex_form(O):
    """Interleaved rotation = multiplying z_i = x_{2i} + j x_{2i+1} by
    exp(j pos f_i); also the identity at pos 0, norm preservation and the
    relative-position property for that layout."""
    rng = _rng(7)
    x = rng.standard_normal(64)
    f = O.rope_inv_freq(64, 1e4)
    for pos in (0, 5, 1234):
        z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * pos * f)
        want = np.empty(64)
        want[0::2], want[1::2] = z.real, z.imag
        _close(O.rope(x, pos, f, "interleaved"), want, 1e-12, "interleaved complex")
    assert np.array_equal(O.rope(x, 0, f, "interleaved"), x)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    lhs = O.rope(q, 40, f, "interleaved") @ O.rope(k, 73, f, "interleaved")
    rhs = q @ O.rope(k, 33, f, "interleaved")
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(rhs))
    assert abs(np.linalg.norm(O.rope(q, 9, f, "interleaved")) - np.linalg.norm(q)) <= 1e-12


def pin_rope_layouts_related_by_permutation(O):
    """Gathering the even elements, then the odd ones, turns interleaved pairs
    (2i, 2i+1) into NeoX pairs (i, i + D/2): rope_il(x) = P^-1 rope_neox(P x)."""
    rng = _rng(8)
    for D in (8, 64, 128):
        x = rng.standard_normal(D)
        f = rng.uniform(0.01, 1.0, D // 2)
        perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
        y = O.rope(x[perm], 17, f, "neox")
        back = np.empty(D)
        back[perm] = y
        _close(O.rope(x, 17, f, "interleaved"), back, 1e-14, "layout permutation")
        _close(O.rope(x, 17, f, "neox"), BF.rope_pairs(list(x), 17, list(f), "neox"),
               1e-14, "neox vs scalar loops")


def pin_rope_mscale(O):
    """The magnitude factor scales the rotated vector and nothing else."""
    rng = _rng(9)
    x = rng.standard_normal(16)
    f = O.rope_inv_freq(16, 1e4)
    for layout in ("neox", "interleaved"):
        _close(O.rope(x, 11, f, layout, 1.25), 1.25 * O.rope(x, 11, f, layout), 1e-15,
               "mscale")
        assert abs(np.linalg.norm(O.rope(x, 11, f, layout, 1.25))
                   - 1.25 * np.linalg.norm(x)) <= 1e-12


def pin_rope_scaled_tables(O):
    """Limits and closed forms of the context-extension tables."""
    D, theta = 128, 5e5
    f = O.rope_inv_freq(D, theta)
    for kind in ("default", "linear", "ntk", "yarn"):       # factor 1: the plain table
        g, m = O.rope_inv_freq_scaled(D, theta, kind, 1.0, 4096)
        _close(g, f, 1e-15, f"{kind} factor 1")
        assert m == 1.0
    s = 4.0
    g, m = O.rope_inv_freq_scaled(D, theta, "linear", s)
    _close(g / f, np.full(D // 2, 1 / s), 1e-15, "linear ratio")
    assert m == 1.0
    g, m = O.rope_inv_freq_scaled(D, theta, "ntk", s)
    assert g[0] == 1.0 and m == 1.0                    # highest frequency unchanged
    assert abs(g[-1] / f[-1] - 1 / s) <= 1e-12        # lowest divided by exactly s
    # middle index by hand: (theta s^(D/(D-2)))^(-2i/D) = f_i s^(-2i/(D-2))
    i = 20
    assert abs(g[i] - f[i] * s ** (-2.0 * i / (D - 2))) <= 1e-15 * f[i]
    # YaRN: r_i = L f_i / 2 pi; r >= beta_fast keeps f, r <= beta_slow takes f/s
    L, bf_, bs_ = 4096, 32.0, 1.0
    g, m = O.rope_inv_freq_scaled(D, theta, "yarn", s, L, bf_, bs_)
    r = L * f / (2 * math.pi)
    hi, lo = r >= bf_, r <= bs_
    assert hi.any() and lo.any() and (~hi & ~lo).any()
    assert np.array_equal(g[hi], f[hi])
    _close(g[lo], f[lo] / s, 1e-15, "yarn interpolated dims")
    assert abs(m - (1 + 0.1 * math.log(s))) <= 1e-15
    ratio = g / f                                      # 1/s ... 1, monotone in r
    order = np.argsort(r)
    assert np.all(np.diff(ratio[order]) >= -1e-15)
    # a dimension exactly at the middle of the ramp takes the mean of f and f/s
    D2, th2 = 4, 16.0                                  # f = [1, 1/4]
    L2 = 2 * math.pi * 16.5 / 1.0                      # r_0 = 16.5 = (1 + 32) / 2
    g2, _ = O.rope_inv_freq_scaled(D2, th2, "yarn", 2.0, L2, 32.0, 1.0)
    assert abs(g2[0] - 0.5 * (1.0 + 0.5)) <= 1e-15


def pin_prologue_table_and_layout(O):
    """The prologue with a frequency table, either layout and a magnitude
    factor matches scalar loops (brute force) on tiny shapes."""
    for k, layout in enumerate(("interleaved", "neox")):
        q, kn, vn, wq, wk, pos, kc, vc = _prologue_case(20 + k)
        D = q.shape[-1]
        f, m = O.rope_inv_freq_scaled(D, 1e4, "yarn", 3.0, 64)
        qh, kc2, _ = O.qkv_prologue(q, kn, vn, wq, wk, 1e-6, 0.0, pos, kc, vc,
                                    inv_freq=f, layout=layout, mscale=m)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                x = BF.rope_pairs(BF.rmsnorm(list(q[b, h]), list(wq), 1e-6), int(pos[b]),
                                  list(f), layout, m)
                _close(qh[b, h], x, 1e-12, f"q_hat {layout}")
            for g in range(kn.shape[1]):
                x = np.array(BF.rope_pairs(BF.rmsnorm(list(kn[b, g]), list(wk), 1e-6),
                                           int(pos[b]), list(f), layout, m))
                row = _torch_bf16_to_f64(kc2[b, g, pos[b]])
                half_ulp = np.ldexp(1.0, np.frexp(x)[1] - 9)
                assert np.all(np.abs(row - x) <= half_ulp + 1e-300)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _rand_case(k, B=2, Hq=8, Hkv=2, D=16, T=40, lens=None):
    rng = _rng(100 + k)
    q = rng.standard_normal((B, Hq, D))
    kc = _bits(rng, (B, Hkv, T, D))
    vc = _bits(rng, (B, Hkv, T, D))
    if lens is None:
        lens = rng.integers(1, T + 1, size=B).astype(np.int32)
    return q, kc, vc, np.asarray(lens, np.int32)


def _sdpa(q, kc, vc, lens, window, scale):
    """torch CPU fp64 SDPA over repeat_interleave-expanded KV heads, plus lse."""
    B, Hq, D = q.shape
    Hkv, T = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    K = torch.from_numpy(_torch_bf16_to_f64(kc)).repeat_interleave(G, dim=1)
    V = torch.from_numpy(_torch_bf16_to_f64(vc)).repeat_interleave(G, dim=1)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        n = min(max(int(lens[b]), 0), T)
        lo = max(0, n - window) if window > 0 else 0
        if n - lo == 0:
            continue
        mask = torch.zeros(1, T, dtype=torch.bool)
        mask[0, lo:n] = True
        qb = torch.from_numpy(q[b]).unsqueeze(1)           # [Hq,1,D]
        o = torch.nn.functional.scaled_dot_product_attention(
            qb, K[b], V[b], attn_mask=mask, scale=scale)
        out[b] = o[:, 0].numpy()
        s = (qb @ K[b].transpose(-1, -2))[:, 0, lo:n] * scale
        lse[b] = torch.logsumexp(s, dim=-1).numpy()
    return out, lse


def pin_attend_matches_sdpa(O):
    for k, (Hq, Hkv, D, window) in enumerate([(8, 2, 16, 0), (8, 8, 8, 0), (6, 3, 32, 0),
                                              (8, 2, 16, 5), (4, 1, 8, 13)]):
        q, kc, vc, lens = _rand_case(k, Hq=Hq, Hkv=Hkv, D=D)
        scale = 1 / math.sqrt(D)
        out, lse = O.attend(q, kc, vc, lens, window, 0.0)
        ro, rl = _sdpa(q, kc, vc, lens, window, scale)
        _close(out, ro, 1e-12, "attend vs sdpa")
        _close(lse, rl, 1e-12, "lse vs logsumexp")


def pin_attend_matches_bruteforce(O):
    for k, (B, Hq, Hkv, D, T, window) in enumerate(
            [(2, 4, 2, 8, 9, 0), (1, 4, 1, 4, 7, 3), (2, 2, 2, 6, 5, 0), (2, 4, 2, 8, 9, 1)]):
        q, kc, vc, lens = _rand_case(10 + k, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T)
        K = _torch_bf16_to_f64(kc).tolist()
        V = _torch_bf16_to_f64(vc).tolist()
        bo, bl = BF.attend(q.tolist(), K, V, lens.tolist(), window, 0.0)
        out, lse = O.attend(q, kc, vc, lens, window, 0.0)
        _close(out, bo, 1e-12, "attend vs brute force")
        _close(lse, bl, 1e-12, "lse vs brute force")


def pin_attend_special_cases(O):
    rng = _rng(20)
    B, Hq, Hkv, D, T = 1, 4, 2, 16, 12
    q = rng.standard_normal((B, Hq, D))
    kc = _bits(rng, (B, Hkv, T, D))
    vc = _bits(rng, (B, Hkv, T, D))
    Kf, Vf = _torch_bf16_to_f64(kc), _torch_bf16_to_f64(vc)
    scale = 1 / math.sqrt(D)
    # n = 1 -> V[0] exactly, lse = s_0
    out, lse = O.attend(q, kc, vc, np.array([1], np.int32), 0, 0.0)
    for h in range(Hq):
        g = h // 2
        assert np.array_equal(out[0, h], Vf[0, g, 0])
        assert abs(lse[0, h] - scale * np.dot(q[0, h], Kf[0, g, 0])) <= 1e-14
    # V = all ones -> weights sum to one
    ones = np.full_like(vc, 0x3F80)
    out, _ = O.attend(q, kc, ones, np.array([T], np.int32), 0, 0.0)
    _close(out, np.ones_like(out), 1e-14, "weights sum")
    # identical keys -> mean(V), lse = s + ln n
    kc_same = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    out, lse = O.attend(q, kc_same, vc, np.array([T], np.int32), 0, 0.0)
    for h in range(Hq):
        g = h // 2
        _close(out[0, h], Vf[0, g].mean(0), 1e-14, "mean V")
        s = scale * np.dot(q[0, h], Kf[0, g, 0])
        assert abs(lse[0, h] - (s + math.log(T))) <= 1e-13
    # window = 1 -> V[n-1]
    out, _ = O.attend(q, kc, vc, np.array([9], np.int32), 1, 0.0)
    for h in range(Hq):
        assert np.array_equal(out[0, h], Vf[0, h // 2, 8])
    # window >= n -> full attention
    full, fl = O.attend(q, kc, vc, np.array([9], np.int32), 0, 0.0)
    for W in (9, 10, 1000):
        o2, l2 = O.attend(q, kc, vc, np.array([9], np.int32), W, 0.0)
        _close(o2, full, 0.0, "window>=n")
        _close(l2, fl, 0.0, "window>=n lse")
    # lens clamped to [0, T]; lens = 0 -> out 0, lse -inf
    for W in (0, 5):
        o_big, _ = O.attend(q, kc, vc, np.array([T + 50], np.int32), W, 0.0)
        o_T, _ = O.attend(q, kc, vc, np.array([T], np.int32), W, 0.0)
        _close(o_big, o_T, 0.0, "lens clamp")
    for n0 in (0, -3):
        o0, l0 = O.attend(q, kc, vc, np.array([n0], np.int32), 0, 0.0)
        assert np.all(o0 == 0) and np.all(l0 == -math.inf)


def pin_attend_two_key_closed_form(O):
    """q = e_0, scale = 1, keys (a,0..), (b,0..): weights e^a, e^b."""
    D = 4
    a_, b_ = 1.5, -0.25                       # exact in bf16
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    K = np.zeros((2, D)); K[0, 0] = a_; K[1, 0] = b_
    V = np.array([[1.0, 2.0, -1.0, 0.5], [3.0, -2.0, 0.25, 4.0]])
    kc = O.f64_to_bf16(K)[None, None]
    vc = O.f64_to_bf16(V)[None, None]
    out, lse = O.attend(q, kc, vc, np.array([2], np.int32), 0, 1.0)
    ea, eb = math.exp(a_), math.exp(b_)
    _close(out[0, 0], (ea * V[0] + eb * V[1]) / (ea + eb), 1e-15, "two keys")
    assert abs(lse[0, 0] - math.log(ea + eb)) <= 1e-15


def pin_attend_affine_and_shift(O):
    """V -> aV + c maps out -> a out + c; a constant added to every score
    (through an extra key component) leaves out unchanged even at scores of
    several hundred, where exp without max-subtraction overflows."""
    rng = _rng(30)
    B, Hq, Hkv, D, T = 1, 4, 2, 8, 20
    q = rng.standard_normal((B, Hq, D))
    kc = _bits(rng, (B, Hkv, T, D))
    lens = np.array([T], np.int32)
    # V on a grid k/8 so that 2V + 0.5 is exact in bf16 as well
    grid = rng.integers(-16, 17, size=(B, Hkv, T, D)) / 8.0
    to_bits = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    vc = to_bits(grid)
    vc2 = to_bits(2.0 * grid + 0.5)
    out, lse = O.attend(q, kc, vc, lens, 0, 0.0)
    o2, l2 = O.attend(q, kc, vc2, lens, 0, 0.0)
    _close(o2, 2.0 * out + 0.5, 1e-13, "affine V")
    _close(l2, lse, 0.0, "affine V lse")
    # shift: append a key component equal to 1 and a query component c.
    K1 = np.concatenate([_torch_bf16_to_f64(kc), np.ones((B, Hkv, T, 1))], axis=-1)
    kc1 = to_bits(K1)
    for c in (0.0, 400.0, 2000.0):
        q1 = np.concatenate([q, np.full((B, Hq, 1), c)], axis=-1)
        o1, l1 = O.attend(q1, kc1, vc, lens, 0, 1 / math.sqrt(D))
        _close(o1, out, 1e-12, f"shift {c}")
        _close(l1 - c / math.sqrt(D), lse, 1e-9, f"shift lse {c}")


# ---------------------------------------------------------------------------
# Split-K partitions and the log-sum-exp merge
# ---------------------------------------------------------------------------
def pin_split_equals_unsplit(O):
    for k, (T, window) in enumerate([(40, 0), (40, 11), (33, 0), (64, 64)]):
        q, kc, vc, lens = _rand_case(40 + k, B=3, Hq=4, Hkv=2, D=8, T=T,
                                     lens=[T, 1, max(2, T // 2 + 1)])
        full, fl = O.attend(q, kc, vc, lens, window, 0.0)
        for P in (1, 3, 8, T, T + 5):
            o, l = O.attend_partials(q, kc, vc, lens, window, 0.0, P)
            assert o.shape[2] == O.num_partitions(T, window, P)
            mo, ml = O.lse_merge(o, l)
            _close(mo, full, 1e-12, f"split P={P}")
            _close(ml, fl, 1e-12, f"split lse P={P}")


def pin_merge_random_cuts(O):
    """Uneven cuts, including empty pieces, merge back to the whole."""
    rng = _rng(50)
    D, n = 8, 37
    q = rng.standard_normal(D)
    K = _torch_bf16_to_f64(_bits(rng, (n, D)))
    V = _torch_bf16_to_f64(_bits(rng, (n, D)))
    whole, wl = O.attend_rows(q, K, V, 0.3)
    for trial in range(5):
        cuts = np.sort(rng.integers(0, n + 1, size=6))
        edges = [0] + list(cuts) + [n]
        os_, ls_ = [], []
        for a, e in zip(edges[:-1], edges[1:]):
            o, l = O.attend_rows(q, K[a:e], V[a:e], 0.3)
            os_.append(o)
            ls_.append(l)
        mo, ml = O.lse_merge(np.array(os_)[None], np.array(ls_)[None])
        _close(mo[0], whole, 1e-12, "random cuts")
        assert abs(ml[0] - wl) <= 1e-12
    # all-empty -> zeros and -inf
    mo, ml = O.lse_merge(np.zeros((1, 3, D)), np.full((1, 3), -math.inf))
    assert np.all(mo == 0) and ml[0] == -math.inf


def pin_merge_peaky_partials(O):
    """Partials whose lse differ by hundreds: max-subtraction keeps it finite
    and the dominant partition wins."""
    D = 4
    o = np.array([[[1.0, 2, 3, 4], [5.0, 6, 7, 8], [9.0, 1, 1, 1]]])
    lse = np.array([[800.0, 0.0, -math.inf]])
    mo, ml = O.lse_merge(o, lse)
    w1 = math.exp(-800.0)
    _close(mo[0], (o[0, 0] + w1 * o[0, 1]) / (1 + w1), 1e-15, "peaky merge")
    assert abs(ml[0] - (800.0 + math.log1p(w1))) <= 1e-12
    # equal lse -> plain mean
    mo, ml = O.lse_merge(o[:, :2], np.array([[2.0, 2.0]]))
    _close(mo[0], (o[0, 0] + o[0, 1]) / 2, 1e-15, "equal merge")
    assert abs(ml[0] - (2.0 + math.log(2))) <= 1e-15


def pin_num_partitions(O):
    assert O.num_partitions(131072, 0, 2048) == 64
    assert O.num_partitions(32768, 4096, 512) == 8
    assert O.num_partitions(100, 0, 7) == 15
    assert O.num_partitions(100, 30, 7) == 5
    assert O.num_partitions(10, 30, 7) == 2


# ---------------------------------------------------------------------------
# Fused prologue
# ---------------------------------------------------------------------------
def _prologue_case(k, norm=True, theta=1e4, B=2, Hq=4, Hkv=2, D=8, T=6, pos=(2, 5)):
    rng = _rng(60 + k)
    q = _torch_bf16_to_f64(_bits(rng, (B, Hq, D)))
    kn = _torch_bf16_to_f64(_bits(rng, (B, Hkv, D)))
    vn = _torch_bf16_to_f64(_bits(rng, (B, Hkv, D)))
    kc = _bits(rng, (B, Hkv, T, D))
    vc = _bits(rng, (B, Hkv, T, D))
    wq = 1 + 0.1 * rng.standard_normal(D) if norm else None
    wk = 1 + 0.1 * rng.standard_normal(D) if norm else None
    return q, kn, vn, wq, wk, np.array(pos, np.int32), kc, vc


def pin_prologue_matches_bruteforce(O):
    for k, (norm, theta) in enumerate([(True, 1e4), (False, 5e5), (True, 0.0), (False, 0.0)]):
        q, kn, vn, wq, wk, pos, kc, vc = _prologue_case(k, norm, theta)
        eps = 1e-6
        qh, kc2, vc2 = O.qkv_prologue(q, kn, vn, wq, wk, eps, theta, pos, kc, vc)
        B, Hq, D = q.shape
        for b in range(B):
            for h in range(Hq):
                x = list(q[b, h])
                if norm:
                    x = BF.rmsnorm(x, list(wq), eps)
                if theta > 0:
                    x = BF.rope_neox(x, int(pos[b]), theta)
                _close(qh[b, h], x, 1e-12, "q_hat")
            for g in range(kn.shape[1]):
                x = list(kn[b, g])
                if norm:
                    x = BF.rmsnorm(x, list(wk), eps)
                if theta > 0:
                    x = BF.rope_neox(x, int(pos[b]), theta)
                row = _torch_bf16_to_f64(kc2[b, g, pos[b]])
                x = np.array(x)
                # within half a bf16 ulp (2^-9 relative) of the exact value
                half_ulp = np.ldexp(1.0, np.frexp(x)[1] - 9)
                assert np.all(np.abs(row - x) <= half_ulp + 1e-300), (row, x)
                if not norm and theta <= 0:
                    assert np.array_equal(row, kn[b, g])


def pin_prologue_writes_only_pos_rows(O):
    q, kn, vn, wq, wk, pos, kc, vc = _prologue_case(9)
    _, kc2, vc2 = O.qkv_prologue(q, kn, vn, wq, wk, 1e-6, 1e4, pos, kc, vc)
    B, Hkv, T, D = kc.shape
    for b in range(B):
        for g in range(Hkv):
            for t in range(T):
                same_k = np.array_equal(kc2[b, g, t], kc[b, g, t])
                same_v = np.array_equal(vc2[b, g, t], vc[b, g, t])
                if t == pos[b]:
                    # V row is the new value, bit for bit (bf16 in, bf16 out)
                    assert np.array_equal(_torch_bf16_to_f64(vc2[b, g, t]), vn[b, g])
                else:
                    assert same_k and same_v, (b, g, t)
    # out-of-range positions write nothing but still rotate q
    for bad in ((-1, 6), (6, 100)):
        qh, kc3, vc3 = O.qkv_prologue(q, kn, vn, wq, wk, 1e-6, 1e4,
                                      np.array(bad, np.int32), kc, vc)
        assert np.array_equal(kc3, kc) and np.array_equal(vc3, vc)
        x = BF.rope_neox(BF.rmsnorm(list(q[1, 0]), list(wq), 1e-6), bad[1], 1e4)
        _close(qh[1, 0], x, 1e-12, "q_hat out of range pos")


# ---------------------------------------------------------------------------
# Several query tokens per sequence
# ---------------------------------------------------------------------------
def pin_attend_multi_matches_bruteforce(O):
    """Token s of S attends lens - (S-1-s) rows (causal among the new
    tokens), with the window counted back from each token's own end."""
    rng = _rng(70)
    B, S, Hq, Hkv, D, T = 2, 3, 4, 2, 6, 9
    q = rng.standard_normal((B, S, Hq, D))
    kc, vc = _bits(rng, (B, Hkv, T, D)), _bits(rng, (B, Hkv, T, D))
    K, V = _torch_bf16_to_f64(kc), _torch_bf16_to_f64(vc)
    for lens, window in (((9, 5), 0), ((7, 3), 4), ((2, 9), 2), ((1, 0), 0)):
        out, lse = O.attend_multi(q, kc, vc, np.array(lens, np.int32), window, 0.0)
        for s in range(S):
            lens_s = [l - (S - 1 - s) for l in lens]
            bo, bl = BF.attend(q[:, s].tolist(), K.tolist(), V.tolist(), lens_s, window, 0.0)
            _close(out[:, s], np.array(bo), 1e-12, "multi out")
            assert np.allclose(lse[:, s], np.array(bl), atol=1e-12, rtol=0) or \
                np.array_equal(np.isinf(lse[:, s]), np.isinf(np.array(bl)))


def pin_attend_multi_causal(O):
    """A token's output does not depend on rows after its own end."""
    rng = _rng(71)
    B, S, Hq, Hkv, D, T = 1, 4, 2, 1, 8, 12
    q = rng.standard_normal((B, S, Hq, D))
    kc, vc = _bits(rng, (B, Hkv, T, D)), _bits(rng, (B, Hkv, T, D))
    lens = np.array([10], np.int32)
    out, _ = O.attend_multi(q, kc, vc, lens)
    for s in range(S):
        end = 10 - (S - 1 - s)
        kc2, vc2 = kc.copy(), vc.copy()
        kc2[:, :, end:] = _bits(rng, (B, Hkv, T - end, D))
        vc2[:, :, end:] = _bits(rng, (B, Hkv, T - end, D))
        out2, _ = O.attend_multi(q, kc2, vc2, lens)
        assert np.array_equal(out2[:, s], out[:, s]), s
        if end < T and s < S - 1:
            assert not np.array_equal(out2[:, S - 1], out[:, S - 1])


def pin_attend_multi_bidirectional_matches_bruteforce(O):
    """Bidirectional (attention_prefill row, "causal / bidirectional"):
    every token attends the same lens[b] rows, window counted from there."""
    rng = _rng(73)
    B, S, Hq, Hkv, D, T = 2, 3, 4, 2, 6, 9
    q = rng.standard_normal((B, S, Hq, D))
    kc, vc = _bits(rng, (B, Hkv, T, D)), _bits(rng, (B, Hkv, T, D))
    K, V = _torch_bf16_to_f64(kc), _torch_bf16_to_f64(vc)
    for lens, window in (((9, 5), 0), ((7, 3), 4), ((0, 2), 0)):
        out, lse = O.attend_multi(q, kc, vc, np.array(lens, np.int32), window, 0.0,
                                  causal=False)
        for s in range(S):
            bo, bl = BF.attend(q[:, s].tolist(), K.tolist(), V.tolist(), list(lens), window, 0.0)
            _close(out[:, s], np.array(bo), 1e-12, "bidirectional out")
            assert np.allclose(lse[:, s], np.array(bl), atol=1e-12, rtol=0) or \
                np.array_equal(np.isinf(lse[:, s]), np.isinf(np.array(bl)))


def pin_prefill_equal_keys_closed_form(O):
    """Fresh sequence of S tokens whose K rows are all equal: every score of a
    row is the same, so causal token s averages V rows 0..s and its LSE is
    scale * q.k + ln(s + 1); bidirectional tokens all average the S rows."""
    rng = _rng(74)
    B, S, Hq, Hkv, D = 1, 5, 2, 1, 8
    T = S + 3
    q = rng.standard_normal((B, S, Hq, D))
    krow = _bits(rng, (D,))
    kc = np.broadcast_to(krow, (B, Hkv, T, D)).copy()
    vc = _bits(rng, (B, Hkv, T, D))
    V = _torch_bf16_to_f64(vc)[0, 0]
    k = _torch_bf16_to_f64(krow)
    lens = np.array([S], np.int32)
    out, lse = O.attend_multi(q, kc, vc, lens)
    outb, lseb = O.attend_multi(q, kc, vc, lens, causal=False)
    for s in range(S):
        for h in range(Hq):
            sc = float(q[0, s, h] @ k) / math.sqrt(D)
            _close(out[0, s, h], V[:s + 1].mean(axis=0), 1e-12, "causal mean")
            assert abs(lse[0, s, h] - (sc + math.log(s + 1))) < 1e-12
            _close(outb[0, s, h], V[:S].mean(axis=0), 1e-12, "bidirectional mean")
            assert abs(lseb[0, s, h] - (sc + math.log(S))) < 1e-12


def pin_linear_matches_bruteforce(O):
    """The projection against scalar loops, on values whose sums are exact in
    float64 (so any dropped or misplaced term shows)."""
    rng = _rng(80)
    M, N, K = 3, 5, 8
    xb, wb = _bits(rng, (M, K)), _bits(rng, (N, K))
    y = O.linear(xb, wb)
    ref = BF.linear(_torch_bf16_to_f64(xb).tolist(), _torch_bf16_to_f64(wb).tolist())
    _close(y, np.array(ref), 1e-12, "linear")
    assert y.shape == (M, N)


def pin_linear_identity_and_onehot(O):
    """Identity weights return x; a cyclic-shift permutation returns
    y[m][n] = x[m][(n+1) mod K] (its transpose would shift the other way); a
    one-hot weight row picks one column of x; powers of two add exactly."""
    rng = _rng(81)
    K = 6
    xb = _bits(rng, (2, K))
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80          # bf16 1.0
    assert np.array_equal(O.linear(xb, eye), _torch_bf16_to_f64(xb))
    shift = np.zeros((K, K), np.uint16)
    shift[np.arange(K), (np.arange(K) + 1) % K] = 0x3F80
    assert np.array_equal(O.linear(xb, shift), np.roll(_torch_bf16_to_f64(xb), -1, axis=1))
    w = np.zeros((1, K), np.uint16)
    w[0, 4] = 0x4000                                  # 2.0
    assert np.array_equal(O.linear(xb, w)[:, 0], 2.0 * _torch_bf16_to_f64(xb)[:, 4])
    xs = np.array([[0x3F80, 0x3F00, 0x3E80, 0x3E00, 0, 0]], np.uint16)   # 1, 1/2, 1/4, 1/8
    ws = np.array([[0x3F80, 0x3F80, 0, 0x3F80, 0x3F80, 0x3F80]], np.uint16)
    assert O.linear(xs, ws)[0, 0] == 1.0 + 0.5 + 0.125


def pin_split_qkv_layout(O):
    """q | k | v along the packed row, each head's D values contiguous."""
    Hq, Hkv, D = 4, 2, 3
    y = np.arange(2 * (Hq + 2 * Hkv) * D, dtype=np.float64).reshape(2, -1)
    q, k, v = O.split_qkv(y, Hq, Hkv, D)
    assert q.shape == (2, Hq, D) and k.shape == (2, Hkv, D) and v.shape == (2, Hkv, D)
    assert q[1, 3, 2] == y[1, 3 * D + 2]
    assert k[0, 1, 0] == y[0, Hq * D + D]
    assert v[1, 0, 1] == y[1, (Hq + Hkv) * D + 1]


def pin_prologue_multi_matches_bruteforce(O):
    """S new tokens: token s normalised and rotated at pos + s, its K/V row
    appended at row pos + s, every other row untouched."""
    rng = _rng(72)
    B, S, Hq, Hkv, D, T = 2, 3, 4, 2, 8, 10
    q = _torch_bf16_to_f64(_bits(rng, (B, S, Hq, D)))
    kn = _torch_bf16_to_f64(_bits(rng, (B, S, Hkv, D)))
    vn = _torch_bf16_to_f64(_bits(rng, (B, S, Hkv, D)))
    kc, vc = _bits(rng, (B, Hkv, T, D)), _bits(rng, (B, Hkv, T, D))
    wq, wk = 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D)
    pos = np.array([2, 7], np.int32)                 # 7, 8, 9: the last row is T-1
    qh, kc2, vc2 = O.qkv_prologue_multi(q, kn, vn, wq, wk, 1e-6, 1e4, pos, kc, vc)
    for b in range(B):
        for s in range(S):
            p = int(pos[b]) + s
            for h in range(Hq):
                x = BF.rope_neox(BF.rmsnorm(list(q[b, s, h]), list(wq), 1e-6), p, 1e4)
                _close(qh[b, s, h], x, 1e-12, "multi q_hat")
            for g in range(Hkv):
                x = np.array(BF.rope_neox(BF.rmsnorm(list(kn[b, s, g]), list(wk), 1e-6), p, 1e4))
                row = _torch_bf16_to_f64(kc2[b, g, p])
                half_ulp = np.ldexp(1.0, np.frexp(x)[1] - 9)
                assert np.all(np.abs(row - x) <= half_ulp + 1e-300)
                assert np.array_equal(_torch_bf16_to_f64(vc2[b, g, p]), vn[b, s, g])
        written = {int(pos[b]) + s for s in range(S)}
        for t in range(T):
            if t not in written:
                assert np.array_equal(kc2[b, :, t], kc[b, :, t])
                assert np.array_equal(vc2[b, :, t], vc[b, :, t])


# ---------------------------------------------------------------------------
# The whole decode step: prologue, then attention over the appended cache
# ---------------------------------------------------------------------------
def _bf16_rne_scalar(x: float) -> int:
    """One round-to-nearest-even of a Python float to bf16 bits, by hand:
    8 significant bits from frexp, Python's round() (ties to even)."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    m, e = math.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    r = round(m * 256.0)                       # exact product; ties to even
    y = math.ldexp(r, e - 8)
    u = int.from_bytes(np.float32(y).tobytes(), "little")
    return u >> 16


def _bf16_value(bits: int) -> float:
    return float(np.frombuffer((bits << 16).to_bytes(4, "little"), np.float32)[0])


def _step_bruteforce(O, w, scale):
    """The decode step composed by hand from the scalar brute force: each
    token's q and k normalised (if the workload has weights), rotated at its
    own position with the workload's pair layout, table and magnitude
    factor, the k row rounded once to bf16 and written with the raw v row at
    that position, then attention of the rotated q over the appended cache
    (token s attends lens - (S-1-s) rows when causal, lens rows otherwise)."""
    S = w.S
    B, Hq, Hkv, D, T = w.B, w.Hq, w.Hkv, w.D, w.T
    q = O.bf16_to_f64(w.q).reshape(B, S, Hq, D)
    kc = w.k_cache.copy()
    vc = w.v_cache.copy()
    if w.theta > 0:
        if w.rope_scaling is not None:
            inv, msc = O.rope_inv_freq_scaled(D, w.theta, **w.rope_scaling)
            inv = [float(f) for f in inv]
        else:
            inv, msc = [w.theta ** (-2.0 * i / D) for i in range(D // 2)], 1.0
    qh = np.array(q)
    if w.pos is not None:
        kn = O.bf16_to_f64(w.k_new).reshape(B, S, Hkv, D)
        vbits = np.asarray(w.v_new).reshape(B, S, Hkv, D)

        def pro(x, wt, p):
            x = list(x)
            if wt is not None:
                x = BF.rmsnorm(x, [float(v) for v in wt], w.eps)
            if w.theta > 0:
                x = BF.rope_pairs(x, p, inv, w.rope_layout, msc)
            return x
        for b in range(B):
            for s in range(S):
                p = int(w.pos[b]) + s
                for h in range(Hq):
                    qh[b, s, h] = pro(q[b, s, h], w.w_q, p)
                if not 0 <= p < T:
                    continue
                for g in range(Hkv):
                    kx = pro(kn[b, s, g], w.w_k, p)
                    kc[b, g, p] = [_bf16_rne_scalar(v) for v in kx]
                    vc[b, g, p] = vbits[b, s, g]
    Kf = O.bf16_to_f64(kc).tolist()
    Vf = O.bf16_to_f64(vc).tolist()
    out = np.zeros((B, S, Hq, D))
    lse = np.zeros((B, S, Hq))
    for s in range(S):
        back = (S - 1 - s) if w.causal else 0
        lens_s = [int(n) - back for n in w.lens]
        o_s, l_s = BF.attend(qh[:, s].tolist(), Kf, Vf, lens_s, w.window, scale)
        out[:, s], lse[:, s] = np.array(o_s), np.array(l_s)
    if S == 1:
        qh, out, lse = qh[:, 0], out[:, 0], lse[:, 0]
    return qh, kc, vc, out, lse


def pin_decode_step_composition(O):
    """oracle.decode_step (the reference of every GPU parity test) against the
    step composed by hand from the brute force: rotated q, appended caches
    (bit for bit), output and lse; with split=True also every partition's
    (o_k, lse_k) against the brute force over that partition's rows alone."""
    import workloads as WL
    cases = [
        # QK-norm + NeoX RoPE + window, split over partitions of 5 rows
        ("5", dict(B=2, Hq=8, Hkv=2, D=8, L=23, window=11, part_tokens=5), 0.0),
        # QK-norm + interleaved pairs + YaRN table (magnitude factor), explicit scale
        ("2a", dict(B=2, Hq=4, Hkv=2, D=8, L=13, part_tokens=4, rope_layout="interleaved",
                    rope_scaling=dict(kind="yarn", factor=4.0, orig_ctx=8)), 0.37),
        # RoPE only, ragged lengths
        ("3", dict(B=3, Hq=4, Hkv=1, D=8, L=17, lmin=2, part_tokens=6), 0.0),
        # no prologue: q as given
        ("4", dict(B=1, Hq=4, Hkv=2, D=8, L=19, peaky=0.2, part_tokens=7), 0.0),
        # several causal tokens with QK-norm, NTK table, interleaved pairs, window
        ("6", dict(B=2, Hq=4, Hkv=2, D=8, L=9, S=3, norm=True, window=6,
                   rope_layout="interleaved", rope_scaling=dict(kind="ntk", factor=2.0)), 0.0),
        # several bidirectional tokens of a fresh sequence, YaRN magnitude factor
        ("7f", dict(B=1, Hq=4, Hkv=1, D=8, L=6, S=5, causal=False, norm=True,
                    rope_scaling=dict(kind="yarn", factor=2.0, orig_ctx=4)), 0.0),
    ]
    for name, over, scale in cases:
        w = WL.make(name, **over)
        qh, kc, vc, out, lse = _step_bruteforce(O, w, scale)
        for split in ((False, True) if w.S == 1 else (False,)):
            res = O.decode_step(w, split=split, scale=scale)
            what = f"decode_step {name} split={split}"
            _close(res["q_hat"], qh, 1e-12, what + " q_hat")
            assert np.array_equal(res["k_cache"], kc), what + " k_cache"
            assert np.array_equal(res["v_cache"], vc), what + " v_cache"
            _close(res["out"], out, 1e-12, what + " out")
            fin = np.isfinite(lse)
            assert np.array_equal(np.isfinite(res["lse"]), fin), what + " lse finiteness"
            _close(res["lse"][fin], lse[fin], 1e-12, what + " lse")
            if not split:
                continue
            # each partition alone: rows [lo + kP, lo + (k+1)P) of the window
            Kf = O.bf16_to_f64(kc).tolist()
            Vf = O.bf16_to_f64(vc).tolist()
            P = w.part_tokens
            for b in range(w.B):
                n = min(max(int(w.lens[b]), 0), w.T)
                lo = max(0, n - w.window) if w.window > 0 else 0
                for k in range(res["lse_parts"].shape[-1]):
                    a, e = min(lo + k * P, n), min(lo + (k + 1) * P, n)
                    if a == e:
                        assert np.all(res["lse_parts"][b, :, k] == -math.inf), what
                        continue
                    o_k, l_k = BF.attend([qh[b].tolist()], [Kf[b]], [Vf[b]], [e], e - a, scale)
                    _close(res["o_parts"][b, :, k], o_k[0], 1e-12, what + " o_k")
                    _close(res["lse_parts"][b, :, k], l_k[0], 1e-12, what + " lse_k")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
