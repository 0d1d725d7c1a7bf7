"""Plain fp64 CPU oracle for single-token GQA decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path (no kernels, headers, helpers or tables) and imports nothing
from it; the only thing both sides share is the seeded input generator in
``workloads``.

Every function computes the plain definition, slowly and in float64, one
(batch, head) at a time.  bf16 inputs are widened exactly to float64; the
only rounding the oracle performs on purpose is the bf16 store of the
appended K row (and of a bf16 output, when a caller asks for it).

Sources (titles of the pages this follows):
  * fusedtok 1.0.1 README, "Operators" table (rows RMSNorm, RoPE, Softmax,
    attention_decode) and "Usage" (the attention_decode call with a GQA cache
    [B,Hkv,T,D] and per-sequence int32 lens; RoPE with pos_offset, NeoX
    layout; the dtype rule "compute in float32, convert at load/store").
  * fusedtok 1.0.1 README, "Benchmarks" (attention references use heads
    pre-expanded with repeat_interleave, i.e. query head h reads KV head
    h // (Hq/Hkv)).
  * cutileGPT README, "Why tiles" (the RMSNorm kernel figure:
    rstd = 1/sqrt(sum(x*x)/N + eps), y = x*rstd*w) and its feature list
    (RoPE, MHA/GQA, sliding-window attention, fused QK-Norm + RoPE +
    KV-cache writes).
Readings where the pages are silent are listed per function.

Every function here is pinned by tests against closed forms, invariants,
brute force and independent library routines, except where a docstring says
"parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16", "linear", "split_qkv", "rmsnorm", "rope_inv_freq", "rope_inv_freq_scaled",
    "rope", "rope_neox", "qkv_prologue", "attend_rows", "attend", "num_partitions",
    "partition_ranges", "attend_partials", "lse_merge", "decode_step",
    "qkv_prologue_multi", "attend_multi",
]


# ---------------------------------------------------------------------------
# bf16 <-> float64
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the upper half of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Packed QKV projection (cutileGPT README runtime list: packed QKV
# projections; PyGPUkit 0.2.18, optimized BF16 GEMV with weights B[N,K])
# ---------------------------------------------------------------------------
def linear(x_bits, w_bits) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] w[n, k] in float64, from bf16 bit patterns:
    x [M,K], w [N,K] (each output's weights are one row).  The product is
    the library matrix product of the exactly widened values."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    if x.shape[-1] != w.shape[-1]:
        raise ValueError("x and w must share K")
    return x @ w.T


def split_qkv(y: np.ndarray, Hq: int, Hkv: int, D: int):
    """Views of a packed projection row: q [.., Hq, D], k [.., Hkv, D],
    v [.., Hkv, D], in that order along the last axis."""
    lead = y.shape[:-1]
    if y.shape[-1] != (Hq + 2 * Hkv) * D:
        raise ValueError("last axis must be (Hq + 2 Hkv) D")
    q = y[..., :Hq * D].reshape(lead + (Hq, D))
    k = y[..., Hq * D:(Hq + Hkv) * D].reshape(lead + (Hkv, D))
    v = y[..., (Hq + Hkv) * D:].reshape(lead + (Hkv, D))
    return q, k, v


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even), one rounding.

    The dtype rule of the fusedtok README ("Usage": float32 compute, convert at
    the store) leaves the rounding mode open; nearest-even is the reading.
    bf16 keeps 8 significant bits and float32's exponent range, so a finite
    x = m * 2**e (0.5 <= |m| < 1) rounds to rint(m * 2**8) * 2**(e-8) for
    normal results and to a multiple of 2**-133 for subnormal ones.  Values
    whose rounded magnitude reaches 2**128 become infinity; NaN becomes the
    quiet NaN 0x7FC0.  Returns uint16 bit patterns.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_x)
    m, e = np.frexp(flat_x)                     # x = m * 2**e
    normal = e - 1 >= -126                      # |x| >= 2**-126
    r = np.where(normal, np.ldexp(np.rint(np.ldexp(m, 8)), e - 8),
                 np.ldexp(np.rint(np.ldexp(flat_x, 133)), -133))
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)              # exact: r has <= 8 sig. bits
    # r32 is now exactly a bf16 value (or +-inf); keep its upper 16 bits.
    flat_o[:] = (r32.view(np.uint32) >> 16).astype(np.uint16)
    flat_o[nan] = 0x7FC0
    return out


# ---------------------------------------------------------------------------
# RMSNorm (cutileGPT "Why tiles" figure; fusedtok Operators row RMSNorm)
# ---------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x * rstd * w with rstd = 1 / sqrt(mean(x*x) + eps), over the last axis.

    The weight multiplies directly (not 1 + w), and eps is added to the mean
    of squares inside the square root, as the cutileGPT RMSNorm figure shows.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n = x.shape[-1]
    rstd = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) / n + eps)
    return x * rstd * w


# ---------------------------------------------------------------------------
# RoPE, NeoX layout (fusedtok Operators row RoPE; Usage: neox=True, pos_offset)
# ---------------------------------------------------------------------------
def rope_inv_freq(D: int, theta: float) -> np.ndarray:
    """f_i = theta ** (-2i/D) for i < D/2 (the standard rotary schedule).

    Parity unpinned by the pages: they name the NeoX layout and a position
    offset but print no frequency formula.  theta comes with each workload.
    """
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / D)


def rope_inv_freq_scaled(D: int, theta: float, kind: str = "default", factor: float = 1.0,
                         orig_ctx: int = 0, beta_fast: float = 32.0,
                         beta_slow: float = 1.0):
    """(inv_freq [D/2], mscale) of a RoPE context-extension scheme.

    The PyGPUkit 0.2.18 page ("Positional Encoding Operations") names three
    table builders -- NTK-aware RoPE, YaRN dimension-wise interpolation and
    linear position interpolation -- without formulas; each is written here
    from its published definition (parity unpinned by the pages beyond the
    limits and closed forms the tests check):
      linear  positions divided by ``factor`` s: f_i / s.
      ntk     the base grows to theta * s^(D/(D-2)), so the highest
              frequency (i = 0) is unchanged and the lowest (i = D/2-1) is
              divided by exactly s.
      yarn    (YaRN paper) with wavelength lambda_i = 2 pi / f_i and
              r_i = orig_ctx / lambda_i rotations over the original context,
              gamma_i = clip((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1)
              and f'_i = (1 - gamma_i) f_i / s + gamma_i f_i: dimensions that
              turn many times keep their frequency, those that turn less
              than once are interpolated.  The rotated vectors are scaled by
              mscale = 1 + 0.1 ln s (the paper's attention temperature,
              applied to both q and k).
      default the plain table, mscale 1.
    """
    f = rope_inv_freq(D, theta)
    s = float(factor)
    if kind == "default":
        return f, 1.0
    if kind == "linear":
        return f / s, 1.0
    if kind == "ntk":
        i = np.arange(D // 2, dtype=np.float64)
        return np.power(float(theta) * s ** (D / (D - 2.0)), -2.0 * i / D), 1.0
    if kind == "yarn":
        r = float(orig_ctx) * f / (2.0 * math.pi)
        gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
        return (1.0 - gamma) * f / s + gamma * f, 1.0 + 0.1 * math.log(s)
    raise ValueError(kind)


def rope(x: np.ndarray, pos, inv_freq: np.ndarray, layout: str = "neox",
         mscale: float = 1.0) -> np.ndarray:
    """Rotate pair i of the last axis by angle pos * inv_freq[i], times mscale.

    Pairs (the fusedtok README's RoPE row names both layouts):
      neox         (i, i + D/2), "rotate half" (its NeoX / LLaMA-HF layout)
      interleaved  (2i, 2i + 1)
    For a pair (u, v): u' = m (u cos a - v sin a), v' = m (v cos a + u sin a).
    The whole head dimension is rotated (cutileGPT lists partial RoPE as
    unsupported).  ``pos`` broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    a = np.asarray(pos, dtype=np.float64)[..., None] * np.asarray(inv_freq, np.float64)
    c, s = mscale * np.cos(a), mscale * np.sin(a)
    y = np.empty_like(x)
    if layout == "neox":
        u, v = x[..., :h], x[..., h:]
        y[..., :h], y[..., h:] = u * c - v * s, v * c + u * s
    elif layout == "interleaved":
        u, v = x[..., 0::2], x[..., 1::2]
        y[..., 0::2], y[..., 1::2] = u * c - v * s, v * c + u * s
    else:
        raise ValueError(layout)
    return y


def rope_neox(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """NeoX RoPE with the plain table: pairs (i, i + D/2) rotate by
    pos * theta^(-2i/D).

    y_i       = x_i cos a - x_{i+D/2} sin a
    y_{i+D/2} = x_{i+D/2} cos a + x_i sin a
    NeoX ("rotate half") pairing is the reading of the README's NeoX
    (LLaMA-HF) layout.
    """
    x = np.asarray(x, dtype=np.float64)
    return rope(x, pos, rope_inv_freq(x.shape[-1], theta), "neox")


# ---------------------------------------------------------------------------
# Fused prologue (cutileGPT feature list: fused QK-Norm + RoPE + KV-cache writes)
# ---------------------------------------------------------------------------
def qkv_prologue(q, k_new, v_new, w_q, w_k, eps, theta, pos, k_cache, v_cache,
                 inv_freq=None, layout: str = "neox", mscale: float = 1.0):
    """QK-RMSNorm, then RoPE at pos[b], then append K and V at row pos[b].

    q: [B,Hq,D] float64; k_new, v_new: [B,Hkv,D] float64 (exact widenings of
    the bf16 inputs); w_q, w_k: [D] or None (None = no QK-norm; one weight
    vector per projection shared by all heads); pos: int [B]; caches: uint16
    [B,Hkv,T,D].  RoPE: the table ``inv_freq`` [D/2] with ``layout`` and
    ``mscale`` (see ``rope``) when given, else the plain NeoX table of
    ``theta``; no RoPE when neither is given (theta <= 0).

    Returns (q_hat float64 [B,Hq,D], k_cache', v_cache') with new arrays for
    the caches.  Order norm -> RoPE -> write follows the feature's name.  V is
    written unrotated and un-normalised.  A pos outside [0, T) rotates q but
    writes nothing (the safe-behaviour reading for out-of-contract values).
    The appended K row is rounded to bf16 once; q_hat stays float64.
    """
    q = np.array(q, dtype=np.float64)
    k = np.array(k_new, dtype=np.float64)
    v = np.array(v_new, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    T = k_cache.shape[2]
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    q_hat = np.empty_like(q)
    if inv_freq is None and theta > 0:
        inv_freq = rope_inv_freq(D, theta)
    for b in range(B):
        p = int(pos[b])
        for h in range(Hq):
            x = q[b, h]
            if w_q is not None:
                x = rmsnorm(x, w_q, eps)
            if inv_freq is not None:
                x = rope(x, p, inv_freq, layout, mscale)
            q_hat[b, h] = x
        for g in range(Hkv):
            x = k[b, g]
            if w_k is not None:
                x = rmsnorm(x, w_k, eps)
            if inv_freq is not None:
                x = rope(x, p, inv_freq, layout, mscale)
            if 0 <= p < T:
                kc[b, g, p] = f64_to_bf16(x)
                vc[b, g, p] = f64_to_bf16(v[b, g])
    return q_hat, kc, vc


# ---------------------------------------------------------------------------
# Attention (fusedtok Operators row attention_decode; Usage; Benchmarks)
# ---------------------------------------------------------------------------
def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one query vector over rows of K, V (float64).

    s_j = scale * <q, K_j>;  m = max_j s_j;  p_j = exp(s_j - m);
    out = sum_j p_j V_j / sum_j p_j;  lse = m + ln(sum_j p_j).
    No rows: out = 0 and lse = -inf (the empty-set convention used for empty
    split-K partitions and lens = 0).
    """
    D = V.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(D), -math.inf
    s = scale * (K @ q)
    m = np.max(s)
    p = np.exp(s - m)
    l = np.sum(p)
    return (p @ V) / l, m + math.log(l)


def _window(n_raw: int, T: int, window: int):
    n = min(max(int(n_raw), 0), T)
    lo = max(0, n - window) if window > 0 else 0
    return lo, n


def attend(q, k_cache, v_cache, lens, window: int = 0, scale: float = 0.0):
    """Single-token GQA decode attention over a [B,Hkv,T,D] bf16 cache.

    q: [B,Hq,D] float64.  Query head h reads KV head h // (Hq/Hkv) (the
    repeat_interleave expansion of the fusedtok benchmarks).  Sequence b
    attends cache rows [lo, n) with n = lens[b] clamped to [0, T] and
    lo = max(0, n - window) for window > 0 (the last ``window`` rows,
    including the newest), else 0.  scale <= 0 means 1/sqrt(D) (the
    default of the SDPA the README compares against).
    Returns (out float64 [B,Hq,D], lse float64 [B,Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, v_cache.shape[3]))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        lo, n = _window(lens[b], T, window)
        for g in range(Hkv):
            K = bf16_to_f64(k_cache[b, g, lo:n])
            V = bf16_to_f64(v_cache[b, g, lo:n])
            for h in range(g * G, (g + 1) * G):
                out[b, h], lse[b, h] = attend_rows(q[b, h], K, V, scale)
    return out, lse


# ---------------------------------------------------------------------------
# Several query tokens per sequence (fusedtok Operators row attention_prefill:
# S query rows, causal; here they sit at the end of the cache)
# ---------------------------------------------------------------------------
def qkv_prologue_multi(q, k_new, v_new, w_q, w_k, eps, theta, pos, k_cache, v_cache,
                       inv_freq=None, layout: str = "neox", mscale: float = 1.0):
    """The single-token prologue applied to token s = 0, 1, ..., S-1 in turn,
    token s at position pos[b] + s (and cache row pos[b] + s).

    q: [B,S,Hq,D]; k_new, v_new: [B,S,Hkv,D].  Returns (q_hat [B,S,Hq,D],
    k_cache', v_cache').
    """
    q = np.asarray(q, dtype=np.float64)
    S = q.shape[1]
    q_hat = np.empty_like(q)
    kc, vc = k_cache, v_cache
    for s in range(S):
        q_hat[:, s], kc, vc = qkv_prologue(
            q[:, s], np.asarray(k_new)[:, s], np.asarray(v_new)[:, s], w_q, w_k, eps, theta,
            np.asarray(pos, np.int64) + s, kc, vc, inv_freq=inv_freq, layout=layout,
            mscale=mscale)
    return q_hat, kc, vc


def attend_multi(q, k_cache, v_cache, lens, window: int = 0, scale: float = 0.0,
                 causal: bool = True):
    """Attention of S query tokens per sequence over the cache.

    q: [B,S,Hq,D].  Causal (the default): token s of sequence b is
    single-token attention with lens[b] - (S-1-s) rows (the last token sees
    lens[b] rows; each earlier token one row fewer), with the window applied
    per token.  Bidirectional (fusedtok README, attention_prefill row,
    "causal / bidirectional"): every token sees the same lens[b] rows.
    Returns (out [B,S,Hq,D], lse [B,S,Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, S, Hq, D = q.shape
    out = np.zeros((B, S, Hq, v_cache.shape[3]))
    lse = np.full((B, S, Hq), -math.inf)
    for s in range(S):
        lens_s = np.asarray(lens, np.int64) - ((S - 1 - s) if causal else 0)
        out[:, s], lse[:, s] = attend(q[:, s], k_cache, v_cache, lens_s, window, scale)
    return out, lse


# ---------------------------------------------------------------------------
# Flash-decoding split (fusedtok attention_decode row: "flash-decoding split
# over long caches") and the log-sum-exp merge
# ---------------------------------------------------------------------------
def num_partitions(T: int, window: int, part_tokens: int) -> int:
    """Partitions per (sequence, KV head): ceil(min(T, window or T) / P).

    Depends on host-known sizes only, so it bounds every sequence's count.
    """
    span = min(T, window) if window > 0 else T
    return -(-span // part_tokens)


def partition_ranges(lo: int, n: int, part_tokens: int, count: int):
    """J_k = [lo + k P, min(lo + (k+1) P, n)) for k < count; may be empty.

    Partitions start at the window's first row (reading: the split is
    window-relative; any cut gives the same merged result).
    """
    out = []
    for k in range(count):
        a = lo + k * part_tokens
        out.append((min(a, n), min(a + part_tokens, n)))
    return out


def attend_partials(q, k_cache, v_cache, lens, window, scale, part_tokens):
    """Attention restricted to each partition: (o_k, lse_k) per (b, h, k).

    o_k is the normalised partition output and lse_k its log-sum-exp; an
    empty partition gives o_k = 0, lse_k = -inf.
    Returns (o float64 [B,Hq,P,D], lse float64 [B,Hq,P]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    P = num_partitions(T, window, part_tokens)
    o = np.zeros((B, Hq, P, v_cache.shape[3]))
    lse = np.full((B, Hq, P), -math.inf)
    for b in range(B):
        lo, n = _window(lens[b], T, window)
        for k, (a, e) in enumerate(partition_ranges(lo, n, part_tokens, P)):
            for g in range(Hkv):
                K = bf16_to_f64(k_cache[b, g, a:e])
                V = bf16_to_f64(v_cache[b, g, a:e])
                for h in range(g * G, (g + 1) * G):
                    o[b, h, k], lse[b, h, k] = attend_rows(q[b, h], K, V, scale)
    return o, lse


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine partition results: M = max_k lse_k, w_k = exp(lse_k - M),
    out = sum_k w_k o_k / sum_k w_k, lse = M + ln sum_k w_k.

    Partitions with lse_k = -inf weigh nothing; if all are -inf the result is
    out = 0, lse = -inf.  Works over the second-to-last axis of o_parts.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    lead = lse_parts.shape[:-1]
    D = o_parts.shape[-1]
    out = np.zeros(lead + (D,))
    lse = np.full(lead, -math.inf)
    for idx in np.ndindex(*lead):
        L = lse_parts[idx]
        M = np.max(L) if L.size else -math.inf
        if M == -math.inf:
            continue
        w = np.exp(L - M)
        W = np.sum(w)
        out[idx] = (w @ o_parts[idx]) / W
        lse[idx] = M + math.log(W)
    return out, lse


# ---------------------------------------------------------------------------
# One whole decode step on a workload
# ---------------------------------------------------------------------------
def decode_step(w, split: bool = False, scale: float = 0.0):
    """Prologue (if the workload has one) followed by attention.

    ``w`` carries the workload's arrays (see workloads.Workload).  Returns a
    dict with q_hat, k_cache, v_cache (after the append), out, lse and, when
    ``split`` is true, the partitions o_parts / lse_parts and the merged
    result in out / lse.
    """
    q = bf16_to_f64(w.q)
    S = getattr(w, "S", 1)
    inv_freq, mscale = None, 1.0
    scaling = getattr(w, "rope_scaling", None)
    if scaling is not None and w.theta > 0:
        inv_freq, mscale = rope_inv_freq_scaled(w.D, w.theta, **scaling)
    if S > 1:                 # several tokens per sequence: q is [B,S,Hq,D]
        if w.pos is not None:
            q_hat, kc, vc = qkv_prologue_multi(
                q, bf16_to_f64(w.k_new), bf16_to_f64(w.v_new), w.w_q, w.w_k, w.eps,
                w.theta, w.pos, w.k_cache, w.v_cache, inv_freq=inv_freq,
                layout=getattr(w, "rope_layout", "neox"), mscale=mscale)
        else:
            q_hat, kc, vc = q, w.k_cache, w.v_cache
        res = dict(q_hat=q_hat, k_cache=kc, v_cache=vc)
        res["out"], res["lse"] = attend_multi(q_hat, kc, vc, w.lens, w.window, scale,
                                              causal=getattr(w, "causal", True))
        return res
    if w.pos is not None:
        q_hat, kc, vc = qkv_prologue(
            q, bf16_to_f64(w.k_new), bf16_to_f64(w.v_new), w.w_q, w.w_k,
            w.eps, w.theta, w.pos, w.k_cache, w.v_cache, inv_freq=inv_freq,
            layout=getattr(w, "rope_layout", "neox"), mscale=mscale)
    else:
        q_hat, kc, vc = q, w.k_cache, w.v_cache
    res = dict(q_hat=q_hat, k_cache=kc, v_cache=vc)
    if split:
        o, l = attend_partials(q_hat, kc, vc, w.lens, w.window, scale,
                               w.part_tokens)
        res["o_parts"], res["lse_parts"] = o, l
        res["out"], res["lse"] = lse_merge(o, l)
    else:
        res["out"], res["lse"] = attend(q_hat, kc, vc, w.lens, w.window, scale)
    return res
