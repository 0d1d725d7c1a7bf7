"""Seeded synthetic inputs for single-token GQA decode attention.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It only draws random numbers and lays them out; it performs
none of the attention method's arithmetic (no normalisation, rotation,
softmax, or rounding of computed values).  The one numeric conversion here
is fp32 -> bf16 of freshly drawn N(0,1) samples, which is how bf16 inputs
are produced in the first place.

Workload shapes follow the five decode configurations the build targets:
a tiny step, a Qwen3-0.6B-shaped layer, a Llama-3-8B-shaped batch with
ragged lengths, a 128K-token long-context split-K case with a peaky
softmax, and a 70B-shaped sliding-window case.  Every array is produced
from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed draw order:

    lens (ragged configs only), q, k_new, v_new,
    w_q, w_k (QK-norm configs only), peaky row indices (peaky configs only)

Normal draws are float32 ``standard_normal`` rounded to bf16 with
round-to-nearest-even.  The two caches are the exception to the single
stream: each fixed chunk of 2**24 elements of a cache is drawn from its own
PCG64 stream seeded with (seed, cache tag, chunk index), so chunks can be
filled by parallel threads with results independent of the thread count,
and the host never holds a float32 copy of a whole cache.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "make", "CONFIGS", "kv_bytes", "fp32_to_bf16_bits"]

# Chunk (in elements) for drawing cache contents: 16M float32 = 64 MiB.
_CHUNK = 1 << 24


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); return uint16 bits.

    Used only to turn freshly drawn finite float32 samples into bf16 inputs
    (finite inputs never overflow the 32-bit sum below).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    return r.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) bf16 draws from the workload's main stream."""
    return fp32_to_bf16_bits(rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
                             ).reshape(shape)


_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1)))


def _cache_bf16(seed: int, tag: int, shape) -> np.ndarray:
    """N(0,1) bf16 cache contents; chunk j comes from PCG64(SeedSequence((seed, tag, j)))."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(j):
        s = j * _CHUNK
        e = min(n, s + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, tag, j))))
        out[s:e] = fp32_to_bf16_bits(g.standard_normal(e - s, dtype=np.float32))

    chunks = range(-(-n // _CHUNK))
    if _THREADS > 1 and len(chunks) > 1:
        with cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    else:
        for j in chunks:
            fill(j)
    return out.reshape(shape)


@dataclasses.dataclass
class Workload:
    """One decode step's inputs (host arrays) plus its launch configuration.

    Shapes: q [B,Hq,D], k_new/v_new [B,Hkv,D], k_cache/v_cache [B,Hkv,T,D],
    all bf16 stored as uint16 bit patterns.  ``pos`` is the RoPE position of
    the new token, which is also the cache row it is written to; ``lens`` is
    the number of cache rows [0, lens[b]) attended after the append.
    ``prologue`` False means q is given directly to attention (no norm, RoPE
    or append).  ``theta`` <= 0 disables RoPE; ``w_q``/``w_k`` None disables
    QK-RMSNorm.  ``window`` <= 0 is full attention.
    """

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int
    lens: np.ndarray                 # int32 [B]
    pos: Optional[np.ndarray]        # int32 [B] (None without a prologue)
    window: int
    theta: float
    eps: float
    out_dtype: str                   # "f32" | "bf16"
    part_tokens: int                 # split-K partition size used by the bench
    q: np.ndarray                    # uint16 [B,Hq,D]
    k_new: Optional[np.ndarray]      # uint16 [B,Hkv,D]
    v_new: Optional[np.ndarray]
    k_cache: np.ndarray              # uint16 [B,Hkv,T,D]
    v_cache: np.ndarray
    w_q: Optional[np.ndarray]        # float32 [D]
    w_k: Optional[np.ndarray]
    peaky_rows: Optional[np.ndarray] = None  # int64 [B,Hkv,m] rows of K scaled by 4
    rope_layout: str = "neox"        # RoPE pairs: "neox" (i, i+D/2) | "interleaved" (2i, 2i+1)
    # RoPE context-extension scheme (None: the plain theta table), e.g.
    # dict(kind="yarn", factor=4.0, orig_ctx=4096, beta_fast=32.0, beta_slow=1.0)
    rope_scaling: Optional[dict] = None
    # query tokens per sequence (causal among themselves); with S > 1, q is
    # [B,S,Hq,D], k_new/v_new [B,S,Hkv,D], token s at position pos[b] + s
    S: int = 1
    # False: every token attends all lens[b] rows (bidirectional prefill)
    causal: bool = True

    @property
    def prologue(self) -> bool:
        return self.pos is not None

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def attended(self) -> np.ndarray:
        """Rows read per sequence: the union of the tokens' ranges, n_b - lo_b
        with n_b = lens_b (clamped to [0,T]) and lo_b the first token's window
        start (the window counts back from each token's own end)."""
        n = np.clip(self.lens.astype(np.int64), 0, self.T)
        if self.window > 0:
            back = (self.S - 1) if self.causal else 0
            n0 = np.clip(self.lens.astype(np.int64) - back, 0, self.T)
            return n - np.maximum(0, n0 - self.window)
        return n

    def token_rows(self) -> np.ndarray:
        """Rows each (sequence, token) attends, int64 [B,S]: n_s - lo_s."""
        back = np.arange(self.S - 1, -1, -1) if self.causal else np.zeros(self.S, np.int64)
        n = np.clip(self.lens.astype(np.int64)[:, None] - back[None, :], 0, self.T)
        lo = np.maximum(0, n - self.window) if self.window > 0 else np.zeros_like(n)
        return n - lo


def kv_bytes(w: Workload) -> int:
    """Algorithmic KV-cache bytes one decode step reads: K and V rows of the
    attended window, bf16, every KV head of every sequence."""
    return int(w.attended().sum()) * w.Hkv * w.D * 2 * 2


def attention_flops(w: Workload) -> int:
    """Algorithmic FLOPs of the attention contractions: 2 D for q.k plus 2 D
    for p v per (query head, attended row) pair."""
    return int(w.token_rows().sum()) * w.Hq * 4 * w.D


# name -> (base parameters).  Sizes may be overridden for reduced test cases.
CONFIGS: Dict[str, dict] = {
    # tiny step: B1 Hq8 Hkv2 D64 L128, RoPE 1e4 at pos L-1, no QK-norm; one
    # 128-row partition per KV head (the step then needs no merge)
    "1": dict(seed=1, B=1, Hq=8, Hkv=2, D=64, L=128, layout="last",
              window=0, theta=1e4, norm=False, out_dtype="f32", part_tokens=128),
    # Qwen3-0.6B-shaped layer, L in {512, 2048}; new token at pos=L
    "2a": dict(seed=2, B=1, Hq=16, Hkv=8, D=128, L=512, layout="append",
               window=0, theta=1e6, norm=True, out_dtype="f32", part_tokens=128),
    "2b": dict(seed=2, B=1, Hq=16, Hkv=8, D=128, L=2048, layout="append",
               window=0, theta=1e6, norm=True, out_dtype="f32", part_tokens=256),
    # Llama-3-8B-shaped batch, ragged lens ~ U{128..4096}, bf16 output
    "3": dict(seed=3, B=32, Hq=32, Hkv=8, D=128, L=4096, layout="ragged",
              lmin=128, window=0, theta=5e5, norm=False, out_dtype="bf16",
              part_tokens=1024),
    # long context, no prologue, q given in bf16, 1% of K rows x4, P=2048
    "4": dict(seed=4, B=1, Hq=32, Hkv=8, D=128, L=131072, layout="noprologue",
              window=0, theta=0.0, norm=False, out_dtype="f32", part_tokens=2048,
              peaky=0.01),
    # 70B-shaped sliding window: B8 Hq64 Hkv8 L32768, W=4096
    "5": dict(seed=5, B=8, Hq=64, Hkv=8, D=128, L=32768, layout="last",
              window=4096, theta=5e5, norm=True, out_dtype="f32", part_tokens=1024),
    # several query tokens per sequence (draft-token verification): the
    # Llama-3-8B shape with S=4 new tokens appended at L=8192, so the 4 x 4
    # (token, head) rows of each KV head share every cache row read
    "6": dict(seed=6, B=8, Hq=32, Hkv=8, D=128, L=8192, layout="append", S=4,
              window=0, theta=5e5, norm=False, out_dtype="bf16", part_tokens=1024),
    # chunked prefill: the Llama-3-8B shape with the last S=1024 tokens of an
    # 8192-row cache as causal queries, q given in bf16 (the matrix-core path)
    "7": dict(seed=7, B=4, Hq=32, Hkv=8, D=128, L=8192, layout="noprologue", S=1024,
              window=0, theta=0.0, norm=False, out_dtype="bf16", part_tokens=1024),
    # fresh-sequence causal prefill of S=1024 tokens at D=128 (the shape of the
    # fusedtok attention_prefill benchmark row), Llama-3-8B heads, prologue
    # on every token
    "7f": dict(seed=8, B=1, Hq=32, Hkv=8, D=128, L=1024, layout="fresh", S=1024,
               window=0, theta=5e5, norm=False, out_dtype="bf16", part_tokens=1024),
}


def make(name: str, seed: Optional[int] = None, **over) -> Workload:
    """Build workload ``name`` (a key of CONFIGS) with optional overrides.

    Overrides accept any base key (B, Hq, Hkv, D, L, window, theta, norm,
    out_dtype, part_tokens, peaky, lmin) plus ``T`` for ragged layouts and
    ``rope_layout`` / ``rope_scaling`` (the RoPE variant; no effect on the
    random draws).
    Layouts:
      last       T = L, new tokens at pos = L-S .. L-1, lens = L
      append     T = L + 64, new tokens at pos = L .. L+S-1, lens = L + S
      ragged     T = L, lens ~ U{lmin..L}, pos = lens - S
      noprologue T = L, lens = L, q given directly
      fresh      T = L (>= S), the S tokens of a new sequence at pos = 0 .. S-1,
                 lens = S
    (S = 1 unless overridden: the query tokens per sequence.)
    """
    p = dict(CONFIGS[name])
    p.update(over)
    seed = p["seed"] if seed is None else seed
    B, Hq, Hkv, D, L = p["B"], p["Hq"], p["Hkv"], p["D"], p["L"]
    S = int(p.get("S", 1))
    layout = p["layout"]
    rng = np.random.default_rng(seed)

    if layout == "last":
        T = L
        lens = np.full(B, L, np.int32)
        pos = np.full(B, L - S, np.int32)
    elif layout == "append":
        T = p.get("T", L + 64)
        lens = np.full(B, L + S, np.int32)
        pos = np.full(B, L, np.int32)
    elif layout == "ragged":
        T = p.get("T", L)
        lens = rng.integers(max(p["lmin"], S), L, size=B, endpoint=True).astype(np.int32)
        pos = (lens - S).astype(np.int32)
    elif layout == "noprologue":
        T = L
        lens = np.full(B, L, np.int32)
        pos = None
    elif layout == "fresh":
        T = p.get("T", L)
        if T < S:
            raise ValueError("a fresh sequence needs T >= S")
        lens = np.full(B, S, np.int32)
        pos = np.zeros(B, np.int32)
    else:
        raise ValueError(layout)

    tok = (S,) if S > 1 else ()
    q = _normal_bf16(rng, (B,) + tok + (Hq, D))
    if pos is not None:
        k_new = _normal_bf16(rng, (B,) + tok + (Hkv, D))
        v_new = _normal_bf16(rng, (B,) + tok + (Hkv, D))
    else:
        k_new = v_new = None
    k_cache = _cache_bf16(seed, 1, (B, Hkv, T, D))
    v_cache = _cache_bf16(seed, 2, (B, Hkv, T, D))
    if p["norm"]:
        w_q = (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
        w_k = (1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)).astype(np.float32)
    else:
        w_q = w_k = None

    peaky_rows = None
    frac = p.get("peaky", 0.0)
    if frac:
        # Scale round(frac * n) distinct rows of K by 4 in every (b, kv head).
        # Multiplying a bf16 value by 4 adds 2 to its exponent: exact.
        n = int(lens[0])
        m = int(round(frac * n))
        peaky_rows = np.empty((B, Hkv, m), np.int64)
        for b in range(B):
            for g in range(Hkv):
                rows = rng.choice(n, size=m, replace=False)
                peaky_rows[b, g] = rows
                blk = k_cache[b, g, rows].astype(np.uint32) << 16
                blk = (blk.view(np.float32) * np.float32(4.0)).view(np.uint32)
                k_cache[b, g, rows] = (blk >> 16).astype(np.uint16)

    return Workload(
        name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, lens=lens, pos=pos,
        window=int(p["window"]), theta=float(p["theta"]), eps=1e-6,
        out_dtype=p["out_dtype"], part_tokens=int(p["part_tokens"]),
        q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
        w_q=w_q, w_k=w_k, peaky_rows=peaky_rows,
        rope_layout=p.get("rope_layout", "neox"), rope_scaling=p.get("rope_scaling"), S=S,
        causal=bool(p.get("causal", True)))


# ---------------------------------------------------------------------------
# Packed QKV projection (the step ahead of the prologue)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class GemvWorkload:
    """y = x W^T for the decode batch: x [M,K] and W [N,K] bf16 bit patterns,
    N = (Hq + 2 Hkv) D, so row m of y is q | k_new | v_new of sequence m."""

    name: str
    seed: int
    M: int
    N: int
    K: int
    Hq: int
    Hkv: int
    D: int
    x: np.ndarray                    # uint16 [M,K]
    w: np.ndarray                    # uint16 [N,K]
    out_dtype: str                   # "f32" | "bf16"


def gemv_bytes(g: GemvWorkload) -> int:
    """HBM bytes one projection moves: the weights, x and y."""
    ob = 2 if g.out_dtype == "bf16" else 4
    return g.N * g.K * 2 + g.M * g.K * 2 + g.M * g.N * ob


GEMV_CONFIGS: Dict[str, dict] = {
    # the 70B-shaped decode batch of config 5: hidden 8192, Hq 64, Hkv 8, D 128
    "8": dict(seed=9, M=8, K=8192, Hq=64, Hkv=8, D=128, out_dtype="bf16"),
    # the shapes of the PyGPUkit BF16 GEMV table (one row of x): K=2048,
    # N=8192 and K=4096, N=14336 (written as Hq D with Hkv = 0)
    "8a": dict(seed=10, M=1, K=2048, Hq=64, Hkv=0, D=128, out_dtype="bf16"),
    "8b": dict(seed=11, M=1, K=4096, Hq=112, Hkv=0, D=128, out_dtype="bf16"),
}


def make_gemv(name: str, seed: Optional[int] = None, **over) -> GemvWorkload:
    """x ~ N(0,1) and W ~ N(0,1) 2^-e (e = ceil(log2 sqrt K), an exact bf16
    scaling, so outputs are O(1)), both rounded to bf16 (nearest even)."""
    p = dict(GEMV_CONFIGS[name])
    p.update(over)
    seed = p["seed"] if seed is None else seed
    M, K, Hq, Hkv, D = p["M"], p["K"], p["Hq"], p["Hkv"], p["D"]
    N = p.get("N", (Hq + 2 * Hkv) * D)
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, (M, K))
    w = _cache_bf16(seed, 3, (N, K))
    e = int(np.ceil(np.log2(np.sqrt(K))))
    wf = (w.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** -e)
    w = (wf.view(np.uint32) >> 16).astype(np.uint16)
    return GemvWorkload(name=name, seed=seed, M=M, N=N, K=K, Hq=Hq, Hkv=Hkv, D=D, x=x, w=w,
                        out_dtype=p["out_dtype"])
