"""Mutation tests for the oracle's pins (CPU only).

Each case plants one plausible mistake in the oracle -- a dropped term, a
wrong sign or index, a transposed operand, a wrong rounding -- by replacing
one of its module-level functions, then runs every pin.  The pins are good
enough only if at least one of them fails for every planted mistake.
"""
import math

import numpy as np
import pytest

import oracle_pins
from oracle import reference as R

_orig = {k: getattr(R, k) for k in dir(R) if not k.startswith("__")}


# --- bf16 --------------------------------------------------------------------
def _bf16_truncate(x):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_double_round(x):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_ties_away(x):
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    r = np.sign(m) * np.floor(np.abs(np.ldexp(m, 8)) + 0.5)
    r = np.ldexp(r, e - 8)
    with np.errstate(over="ignore"):
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_decode_abs(bits):
    return np.abs(_orig["bf16_to_f64"](bits))


# --- rmsnorm -----------------------------------------------------------------
def _rms_no_eps(x, w, eps):
    return _orig["rmsnorm"](x, w, 0.0)


def _rms_one_plus_w(x, w, eps):
    return _orig["rmsnorm"](x, 1.0 + np.asarray(w, np.float64), eps)


def _rms_sum_not_mean(x, w, eps):
    n = np.asarray(x).shape[-1]
    return _orig["rmsnorm"](x, np.asarray(w, np.float64) / math.sqrt(n), eps / n)


def _rms_no_sqrt(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / (np.mean(x * x, axis=-1, keepdims=True) + eps) * w


# --- rope --------------------------------------------------------------------
def _rope_neg(x, pos, theta):
    return _orig["rope_neox"](x, -np.asarray(pos), theta)


def _rope_interleaved(x, pos, theta):
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    y = _orig["rope_neox"](x[..., perm], pos, theta)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def _rope_pos_plus_one(x, pos, theta):
    return _orig["rope_neox"](x, np.asarray(pos) + 1, theta)


def _inv_freq_half_exponent(D, theta):
    return np.power(float(theta), -1.0 * np.arange(D // 2) / D)


def _rope_cos_sin_swapped(x, pos, theta):
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    h = D // 2
    a = np.asarray(pos, np.float64)[..., None] * _orig["rope_inv_freq"](D, theta)
    c, s = np.sin(a), np.cos(a)
    return np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], -1)


def _rope_general_pairs_swapped(x, pos, inv_freq, layout="neox", mscale=1.0):
    if layout != "interleaved":
        return _orig["rope"](x, pos, inv_freq, layout, mscale)
    x = np.asarray(x, np.float64)
    sw = x.copy()
    sw[..., 0::2], sw[..., 1::2] = x[..., 1::2], x[..., 0::2]
    y = _orig["rope"](sw, pos, inv_freq, layout, mscale)
    out = y.copy()
    out[..., 0::2], out[..., 1::2] = y[..., 1::2], y[..., 0::2]
    return out


def _rope_general_mscale_squared(x, pos, inv_freq, layout="neox", mscale=1.0):
    return _orig["rope"](x, pos, inv_freq, layout, mscale * mscale)


def _rope_general_ignores_layout(x, pos, inv_freq, layout="neox", mscale=1.0):
    return _orig["rope"](x, pos, inv_freq, "neox", mscale)


def _table_variant(kind):
    def f(D, theta, k="default", factor=1.0, orig_ctx=0, beta_fast=32.0, beta_slow=1.0):
        g, m = _orig["rope_inv_freq_scaled"](D, theta, k, factor, orig_ctx, beta_fast,
                                              beta_slow)
        base = _orig["rope_inv_freq"](D, theta)
        if kind == "yarn_ramp_inverted" and k == "yarn":
            r = orig_ctx * base / (2 * math.pi)
            gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0, 1)
            return gamma * base / factor + (1 - gamma) * base, m
        if kind == "ntk_base_linear" and k == "ntk":
            i = np.arange(D // 2)
            return np.power(theta * factor, -2.0 * i / D), m
        if kind == "linear_multiplies" and k == "linear":
            return base * factor, m
        if kind == "yarn_no_mscale" and k == "yarn":
            return g, 1.0
        return g, m
    return f


def _multi_off_by_one(q, k_cache, v_cache, lens, window=0, scale=0.0, causal=True):
    q = np.asarray(q, np.float64)
    B, S = q.shape[:2]
    out = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -math.inf)
    for s in range(S):
        out[:, s], lse[:, s] = R.attend(q[:, s], k_cache, v_cache,
                                        np.asarray(lens, np.int64) - (S - s if causal else 1),
                                        window, scale)
    return out, lse


def _multi_window_from_last(q, k_cache, v_cache, lens, window=0, scale=0.0, causal=True):
    q = np.asarray(q, np.float64)
    B, S = q.shape[:2]
    out = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -math.inf)
    T = k_cache.shape[2]
    for s in range(S):
        for b in range(B):
            n = min(max(int(lens[b]) - (S - 1 - s), 0), T)
            lo = max(0, int(lens[b]) - window) if window > 0 else 0
            for h in range(q.shape[2]):
                g = h // (q.shape[2] // k_cache.shape[1])
                K = R.bf16_to_f64(k_cache[b, g, lo:n])
                V = R.bf16_to_f64(v_cache[b, g, lo:n])
                sc = scale if scale > 0 else 1.0 / math.sqrt(q.shape[3])
                out[b, s, h], lse[b, s, h] = R.attend_rows(q[b, s, h], K, V, sc)
    return out, lse


def _prologue_multi_same_pos(q, k_new, v_new, w_q, w_k, eps, theta, pos, k_cache, v_cache,
                             inv_freq=None, layout="neox", mscale=1.0):
    q = np.asarray(q, np.float64)
    qh = np.empty_like(q)
    kc, vc = k_cache, v_cache
    for s in range(q.shape[1]):
        qh[:, s], kc, vc = R.qkv_prologue(q[:, s], np.asarray(k_new)[:, s],
                                          np.asarray(v_new)[:, s], w_q, w_k, eps, theta,
                                          np.asarray(pos) + (s if s < q.shape[1] - 1 else 0),
                                          kc, vc)
    return qh, kc, vc


# --- attention -----------------------------------------------------------------
def _rows_no_max(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1]), -math.inf
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(scale * (K @ q))
        l = np.sum(p)
        return (p @ V) / l, math.log(l) if np.isfinite(l) and l > 0 else math.inf


def _rows_lse_no_m(q, K, V, scale):
    o, l = _orig["attend_rows"](q, K, V, scale)
    if K.shape[0] == 0:
        return o, l
    return o, l - np.max(scale * (K @ q))


def _rows_swapped(q, K, V, scale):
    return _orig["attend_rows"](q, V, K, scale)


def _rows_unnormalised(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1]), -math.inf
    s = scale * (K @ q)
    m = np.max(s)
    p = np.exp(s - m)
    return p @ V, m + math.log(np.sum(p))


def _rows_scale_ignored(q, K, V, scale):
    return _orig["attend_rows"](q, K, V, 1.0)


def _window_off_by_one(n_raw, T, window):
    n = min(max(int(n_raw), 0), T)
    lo = max(0, n - window + 1) if window > 0 else 0
    return lo, n


def _window_no_clamp(n_raw, T, window):
    n = max(int(n_raw), 0)
    lo = max(0, n - window) if window > 0 else 0
    return min(lo, T), n


def _attend_head_mod(q, k_cache, v_cache, lens, window=0, scale=0.0):
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, v_cache.shape[3]))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        lo, n = R._window(lens[b], T, window)
        for h in range(Hq):
            g = h % Hkv
            K = R.bf16_to_f64(k_cache[b, g, lo:n])
            V = R.bf16_to_f64(v_cache[b, g, lo:n])
            out[b, h], lse[b, h] = R.attend_rows(q[b, h], K, V, scale)
    return out, lse


# --- split / merge ---------------------------------------------------------------
def _ranges_from_zero(lo, n, P, count):
    return _orig["partition_ranges"](0, n, P, count)


def _num_parts_floor(T, window, P):
    span = min(T, window) if window > 0 else T
    return max(1, span // P)


def _merge_no_max(o_parts, lse_parts):
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(lse_parts)
        W = np.sum(w, -1)
        return np.einsum("...k,...kd->...d", w, o_parts) / W[..., None], np.log(W)


def _merge_unweighted(o_parts, lse_parts):
    o, l = _orig["lse_merge"](o_parts, lse_parts)
    o_parts = np.asarray(o_parts, np.float64)
    fin = np.isfinite(np.asarray(lse_parts))
    cnt = np.maximum(fin.sum(-1), 1)
    return (o_parts * fin[..., None]).sum(-2) / cnt[..., None], l


def _merge_log2(o_parts, lse_parts):
    o, l = _orig["lse_merge"](o_parts, lse_parts)
    return o, l / math.log(2)


def _merge_no_empty_guard(o_parts, lse_parts):
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    with np.errstate(invalid="ignore"):
        M = np.max(lse_parts, -1, keepdims=True)
        w = np.exp(lse_parts - M)
        W = np.sum(w, -1)
        return np.einsum("...k,...kd->...d", w, o_parts) / W[..., None], M[..., 0] + np.log(W)


# --- prologue ----------------------------------------------------------------------
def _prologue_variant(kind):
    def f(q, k_new, v_new, w_q, w_k, eps, theta, pos, k_cache, v_cache, inv_freq=None,
          layout="neox", mscale=1.0):
        if inv_freq is not None:     # these mistakes concern the plain-theta path
            return _orig["qkv_prologue"](q, k_new, v_new, w_q, w_k, eps, theta, pos,
                                         k_cache, v_cache, inv_freq, layout, mscale)
        q = np.array(q, np.float64)
        k = np.array(k_new, np.float64)
        v = np.array(v_new, np.float64)
        B, Hq, D = q.shape
        Hkv, T = k.shape[1], k_cache.shape[2]
        kc, vc = k_cache.copy(), v_cache.copy()
        qh = np.empty_like(q)

        def proc(x, w, p):
            if kind == "rope_first":
                if theta > 0:
                    x = R.rope_neox(x, p, theta)
                if w is not None:
                    x = R.rmsnorm(x, w, eps)
                return x
            if w is not None:
                x = R.rmsnorm(x, w, eps)
            if theta > 0:
                x = R.rope_neox(x, p, theta)
            return x
        for b in range(B):
            p = int(pos[b])
            for h in range(Hq):
                qh[b, h] = proc(q[b, h], w_k if kind == "wk_for_q" else w_q, p)
            for g in range(Hkv):
                x = proc(k[b, g], w_k, p)
                vv = v[b, g]
                if kind == "rotate_v" and theta > 0:
                    vv = R.rope_neox(vv, p, theta)
                row = p + 1 if kind == "pos_plus_one" else p
                if 0 <= row < T:
                    kc[b, g, row] = R.f64_to_bf16(x)
                    vc[b, g, row] = R.f64_to_bf16(vv)
        return qh, kc, vc
    return f


def _multi_causal_flag_ignored(q, k_cache, v_cache, lens, window=0, scale=0.0, causal=True):
    return _orig["attend_multi"](q, k_cache, v_cache, lens, window, scale)


def _multi_bidirectional_first_token_rows(q, k_cache, v_cache, lens, window=0, scale=0.0,
                                          causal=True):
    if causal:
        return _orig["attend_multi"](q, k_cache, v_cache, lens, window, scale)
    S = np.asarray(q).shape[1]
    return _orig["attend_multi"](q, k_cache, v_cache, np.asarray(lens, np.int64) - (S - 1),
                                 window, scale, causal=False)


def _linear_transposed_w(x_bits, w_bits):
    x, w = R.bf16_to_f64(x_bits), R.bf16_to_f64(w_bits)
    if w.shape[0] == w.shape[1]:
        return x @ w
    return x @ w.T


def _linear_drops_last_column(x_bits, w_bits):
    x, w = R.bf16_to_f64(x_bits), R.bf16_to_f64(w_bits)
    return x[:, :-1] @ w[:, :-1].T


def _split_qkv_k_v_swapped(y, Hq, Hkv, D):
    q, k, v = _orig["split_qkv"](y, Hq, Hkv, D)
    return q, v, k


# --- the whole step (decode_step composes the pieces above) ------------------------
def _decode_step_variant(kind):
    """decode_step with one composition slip; everything else as written."""
    def f(w, split=False, scale=0.0):
        q = R.bf16_to_f64(w.q)
        S = getattr(w, "S", 1)
        inv_freq, mscale = None, 1.0
        if w.rope_scaling is not None and w.theta > 0:
            inv_freq, mscale = R.rope_inv_freq_scaled(w.D, w.theta, **w.rope_scaling)
        if kind == "drops_mscale":
            mscale = 1.0
        layout = "neox" if kind == "drops_layout" else w.rope_layout
        if kind == "ignores_scale":
            scale = 0.0
        pro = R.qkv_prologue_multi if S > 1 else R.qkv_prologue
        if w.pos is not None and not (kind == "multi_skips_prologue" and S > 1):
            q_hat, kc, vc = pro(q, R.bf16_to_f64(w.k_new), R.bf16_to_f64(w.v_new), w.w_q,
                                w.w_k, w.eps, w.theta, w.pos, w.k_cache, w.v_cache,
                                inv_freq=inv_freq, layout=layout, mscale=mscale)
        else:
            q_hat, kc, vc = q, w.k_cache, w.v_cache
        res = dict(q_hat=q_hat, k_cache=kc, v_cache=vc)
        qa = q if kind == "attends_raw_q" else q_hat
        ka, va = (w.k_cache, w.v_cache) if kind == "attends_pre_append_cache" else (kc, vc)
        if S > 1:
            causal = True if kind == "drops_causal" else w.causal
            res["out"], res["lse"] = R.attend_multi(qa, ka, va, w.lens, w.window, scale,
                                                    causal=causal)
            return res
        if split:
            o, l = R.attend_partials(qa, ka, va, w.lens, w.window, scale, w.part_tokens)
            res["o_parts"], res["lse_parts"] = o, l
            res["out"], res["lse"] = R.lse_merge(o, l)
        else:
            res["out"], res["lse"] = R.attend(qa, ka, va, w.lens, w.window, scale)
        return res
    return f


MUTANTS = {
    "bf16_truncate": {"f64_to_bf16": _bf16_truncate},
    "bf16_double_round": {"f64_to_bf16": _bf16_double_round},
    "bf16_ties_away": {"f64_to_bf16": _bf16_ties_away},
    "bf16_decode_abs": {"bf16_to_f64": _bf16_decode_abs},
    "rms_no_eps": {"rmsnorm": _rms_no_eps},
    "rms_one_plus_w": {"rmsnorm": _rms_one_plus_w},
    "rms_sum_not_mean": {"rmsnorm": _rms_sum_not_mean},
    "rms_no_sqrt": {"rmsnorm": _rms_no_sqrt},
    "rope_negative_angle": {"rope_neox": _rope_neg},
    "rope_interleaved_pairs": {"rope_neox": _rope_interleaved},
    "rope_pos_plus_one": {"rope_neox": _rope_pos_plus_one},
    "rope_half_exponent": {"rope_inv_freq": _inv_freq_half_exponent},
    "rope_cos_sin_swapped": {"rope_neox": _rope_cos_sin_swapped},
    "attn_no_max_subtraction": {"attend_rows": _rows_no_max},
    "attn_lse_without_max": {"attend_rows": _rows_lse_no_m},
    "attn_k_v_swapped": {"attend_rows": _rows_swapped},
    "attn_unnormalised": {"attend_rows": _rows_unnormalised},
    "attn_scale_ignored": {"attend_rows": _rows_scale_ignored},
    "attn_window_off_by_one": {"_window": _window_off_by_one},
    "attn_lens_not_clamped": {"_window": _window_no_clamp},
    "attn_head_map_modulo": {"attend": _attend_head_mod},
    "split_ignores_window_start": {"partition_ranges": _ranges_from_zero},
    "split_count_floor": {"num_partitions": _num_parts_floor},
    "merge_no_max_subtraction": {"lse_merge": _merge_no_max},
    "merge_unweighted": {"lse_merge": _merge_unweighted},
    "merge_lse_base2": {"lse_merge": _merge_log2},
    "merge_no_empty_guard": {"lse_merge": _merge_no_empty_guard},
    "prologue_rope_before_norm": {"qkv_prologue": _prologue_variant("rope_first")},
    "prologue_wk_for_q": {"qkv_prologue": _prologue_variant("wk_for_q")},
    "prologue_rotates_v": {"qkv_prologue": _prologue_variant("rotate_v")},
    "prologue_writes_pos_plus_one": {"qkv_prologue": _prologue_variant("pos_plus_one")},
    "rope_interleaved_pairs_swapped": {"rope": _rope_general_pairs_swapped},
    "rope_mscale_squared": {"rope": _rope_general_mscale_squared},
    "rope_layout_ignored": {"rope": _rope_general_ignores_layout},
    "yarn_ramp_inverted": {"rope_inv_freq_scaled": _table_variant("yarn_ramp_inverted")},
    "ntk_base_times_factor": {"rope_inv_freq_scaled": _table_variant("ntk_base_linear")},
    "linear_multiplies_frequencies": {"rope_inv_freq_scaled": _table_variant("linear_multiplies")},
    "yarn_without_mscale": {"rope_inv_freq_scaled": _table_variant("yarn_no_mscale")},
    "multi_token_off_by_one": {"attend_multi": _multi_off_by_one},
    "multi_window_from_last_token": {"attend_multi": _multi_window_from_last},
    "multi_prologue_last_token_position": {"qkv_prologue_multi": _prologue_multi_same_pos},
    "prefill_causal_flag_ignored": {"attend_multi": _multi_causal_flag_ignored},
    "linear_transposed_weights": {"linear": _linear_transposed_w},
    "linear_drops_a_column": {"linear": _linear_drops_last_column},
    "split_qkv_k_v_swapped": {"split_qkv": _split_qkv_k_v_swapped},
    "prefill_bidirectional_first_token_rows": {"attend_multi": _multi_bidirectional_first_token_rows},
    "step_attends_raw_q": {"decode_step": _decode_step_variant("attends_raw_q")},
    "step_attends_pre_append_cache": {"decode_step": _decode_step_variant("attends_pre_append_cache")},
    "step_drops_mscale": {"decode_step": _decode_step_variant("drops_mscale")},
    "step_drops_layout": {"decode_step": _decode_step_variant("drops_layout")},
    "step_drops_causal": {"decode_step": _decode_step_variant("drops_causal")},
    "step_ignores_scale": {"decode_step": _decode_step_variant("ignores_scale")},
    "step_multi_skips_prologue": {"decode_step": _decode_step_variant("multi_skips_prologue")},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name].items():
        monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(R)
        except Exception as e:  # noqa: BLE001 - any failure counts as a catch
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects the planted mistake {name}"
