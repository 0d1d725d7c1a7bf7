"""Python binding of the gfx950 GQA decode-attention library.

Argument marshalling only: each function checks torch tensors (dtype,
device, layout), passes their device pointers and torch's current HIP
stream to the C ABI in ``include/gqa_decode.h``, and raises on a non-zero
status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  Importing fails loudly when the library is missing.

Functions follow the C entry points' names without the ``gqa_`` prefix:
``qkv_prologue``, ``qkv_prologue_ex``, ``attn_decode``,
``attn_decode_splitk``, ``attn_decode_merge``, ``attn_decode_multi``,
``attn_decode_splitk_multi``, ``attn_decode_merge_multi``, ``decode_step``,
``decode_step_ex``, ``decode_step_multi``, ``attn_prefill`` (with key
``splits``: ``prefill_workspace_bytes``, ``prefill_default_splits``),
``prefill_step``, ``qkv_gemv``,
``rope_table``, ``splitk_workspace_bytes``, ``splitk_multi_workspace_bytes``,
``decode_step_workspace_bytes``, ``decode_step_multi_workspace_bytes``,
``num_partitions``, ``decode_step_noalloc`` (no workspace: the library's
static scratch); and the measurement helper ``probe_stream_read``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from ._build import LIB_PATH

__all__ = [
    "GQAError", "lib", "qkv_prologue", "qkv_prologue_ex", "attn_decode",
    "attn_decode_splitk", "attn_decode_merge", "splitk_workspace_bytes", "num_partitions",
    "decode_step", "decode_step_ex", "decode_step_workspace_bytes", "rope_table",
    "attn_decode_multi", "attn_decode_splitk_multi", "attn_decode_merge_multi",
    "splitk_multi_workspace_bytes", "decode_step_multi", "decode_step_multi_workspace_bytes",
    "attn_prefill", "qkv_gemv", "prefill_workspace_bytes", "prefill_default_splits",
    "prefill_step", "probe_stream_read", "decode_step_noalloc",
    "F32", "BF16", "SYMBOLS", "ROPE_NEOX", "ROPE_INTERLEAVED", "ROPE_KINDS",
]

F32, BF16 = 0, 1
ROPE_NEOX, ROPE_INTERLEAVED = 0, 1
ROPE_KINDS = {"default": 0, "linear": 1, "ntk": 2, "yarn": 3}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float
_d = ctypes.c_double
_sz = ctypes.c_size_t

# name -> (restype, argtypes); every symbol the header declares.
SYMBOLS = {
    "gqa_qkv_prologue": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _d, _p, _p, _p, _p,
                              _i, _i, _i, _i, _i, _p]),
    "gqa_attn_decode": (_i, [_p, _i, _p, _p, _p, _i, _f, _p, _i, _p, _i, _i, _i, _i, _i, _p]),
    "gqa_num_partitions": (_i, [_i, _i, _i]),
    "gqa_splitk_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode_splitk": (_i, [_p, _i, _p, _p, _p, _i, _f, _i, _p, _sz,
                                    _i, _i, _i, _i, _i, _p]),
    "gqa_attn_decode_merge": (_i, [_p, _sz, _i, _i, _p, _i, _p, _i, _i, _i, _i, _p]),
    "gqa_decode_step_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "gqa_decode_step": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _d, _p, _p, _p, _p,
                             _i, _f, _i, _p, _sz, _p, _i, _p, _p, _i, _i, _i, _i, _i, _p]),
    "gqa_status_string": (ctypes.c_char_p, [_i]),
    "gqa_rope_table": (_i, [_i, _i, _d, _d, _i, _d, _d, _p, _p]),
    "gqa_qkv_prologue_ex": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _p, _d, _i, _p, _i,
                                 _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "gqa_attn_decode_multi": (_i, [_p, _i, _p, _p, _p, _i, _i, _f, _p, _i, _p, _i, _i, _i, _i,
                                   _i, _p]),
    "gqa_splitk_multi_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "gqa_attn_decode_splitk_multi": (_i, [_p, _i, _p, _p, _p, _i, _i, _f, _i, _p, _sz,
                                          _i, _i, _i, _i, _i, _p]),
    "gqa_attn_decode_merge_multi": (_i, [_p, _sz, _i, _i, _i, _p, _i, _p, _i, _i, _i, _i, _p]),
    "gqa_decode_step_ex": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _p, _d, _i, _p, _p,
                                _p, _p, _i, _f, _i, _p, _sz, _p, _i, _p, _p, _i, _i, _i, _i,
                                _i, _p]),
    "gqa_decode_step_multi_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "gqa_decode_step_multi": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _p, _d, _i, _p, _i,
                                   _p, _p, _p, _i, _f, _i, _p, _sz, _p, _i, _p, _p, _i, _i,
                                   _i, _i, _i, _p]),
    "gqa_attn_prefill": (_i, [_p, _i, _p, _p, _p, _i, _i, _i, _f, _p, _i, _p, _i, _i, _i, _i,
                              _i, _p]),
    "gqa_qkv_gemv": (_i, [_p, _i64, _p, _i64, _p, _i, _i64, _i, _i, _i, _p]),
    "gqa_attn_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "gqa_prefill_step": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _p, _d, _i, _p, _i,
                              _p, _p, _p, _i, _i, _f, _i, _p, _sz, _p, _i, _p, _p,
                              _i, _i, _i, _i, _i, _p]),
    "gqa_attn_prefill_default_splits": (_i, [_i, _i, _i, _i]),
    "gqa_attn_prefill_split": (_i, [_p, _i, _p, _p, _p, _i, _i, _i, _f, _i, _p, _sz, _p, _i,
                                    _p, _i, _i, _i, _i, _i, _p]),
    "gqa_probe_stream_read": (_i, [_p, _sz, _i, _i, _i, _p, _p]),
    "gqa_decode_step_noalloc": (_i, [_p, _p, _p, _i, _i64, _i64, _p, _p, _f, _p, _d, _i, _p,
                                     _i, _p, _p, _p, _i, _f, _i, _p, _i, _p, _p, _i, _i, _i,
                                     _i, _i, _p]),
}
for _name, (_res, _args) in SYMBOLS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class GQAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"gqa status {status}: {lib.gqa_status_string(status).decode()}")


def _check(rc: int):
    if rc != 0:
        raise GQAError(rc)


_DT = {torch.float32: F32, torch.bfloat16: BF16}


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{what}: dtype {t.dtype} not supported (float32 or bfloat16)")
    return _DT[t.dtype]


def _dev(t: torch.Tensor, what: str, device=None):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")


def _contig(t: torch.Tensor, what: str):
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def num_partitions(T: int, window: int, part_tokens: int) -> int:
    return int(lib.gqa_num_partitions(T, window, part_tokens))


def splitk_workspace_bytes(B: int, Hq: int, D: int, T: int, window: int,
                           part_tokens: int) -> int:
    return int(lib.gqa_splitk_workspace_bytes(B, Hq, D, T, window, part_tokens))


def rope_table(kind: str, D: int, theta: float, factor: float = 1.0, orig_ctx: int = 0,
               beta_fast: float = 32.0, beta_slow: float = 1.0):
    """Host table of rotary frequencies for a scheme ("default", "linear",
    "ntk", "yarn"): returns (float64 numpy array [D/2], mscale)."""
    import numpy as np
    f = np.zeros(D // 2, dtype=np.float64)
    m = ctypes.c_double(0.0)
    _check(lib.gqa_rope_table(ROPE_KINDS[kind], int(D), float(theta), float(factor),
                              int(orig_ctx), float(beta_fast), float(beta_slow),
                              f.ctypes.data, ctypes.addressof(m)))
    return f, m.value


def _host_table(inv_freq, D):
    """A host float64 [D/2] array for the C ABI (kept alive by the caller)."""
    import numpy as np
    if inv_freq is None:
        return None
    f = np.ascontiguousarray(np.asarray(inv_freq, dtype=np.float64))
    if f.shape != (D // 2,):
        raise ValueError(f"inv_freq must have D/2 = {D // 2} entries")
    return f


def _layout_code(layout) -> int:
    if layout in (ROPE_NEOX, "neox"):
        return ROPE_NEOX
    if layout in (ROPE_INTERLEAVED, "interleaved"):
        return ROPE_INTERLEAVED
    raise ValueError(f"unknown RoPE layout {layout!r}")


def qkv_prologue(q, k_new, v_new, pos, k_cache, v_cache, q_norm_w=None, k_norm_w=None,
                 eps: float = 1e-6, rope_theta: float = 0.0, q_out=None):
    """QK-RMSNorm + NeoX RoPE at pos[b] + append of k/v at row pos[b].

    q [B,Hq,D], k_new/v_new [B,Hkv,D] (float32 or bfloat16, heads contiguous,
    any batch stride, k_new and v_new with the same batch stride);
    pos int32 [B]; caches bfloat16 [B,Hkv,T,D] (written in place);
    norm weights float32 [D] or None.  Returns q_out float32 [B,Hq,D].
    """
    dev, B, Hq, Hkv, D, T, code, q_out = _prologue_checks(
        q, k_new, v_new, pos, k_cache, v_cache, q_norm_w, k_norm_w, q_out)
    _check(lib.gqa_qkv_prologue(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0), k_new.stride(0),
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), float(rope_theta), _ptr(pos),
        _ptr(q_out), _ptr(k_cache), _ptr(v_cache), B, Hq, Hkv, D, T, _stream(dev)))
    return q_out


def qkv_prologue_ex(q, k_new, v_new, pos, k_cache, v_cache, inv_freq=None,
                    rope_mscale: float = 1.0, rope_layout="neox", q_norm_w=None,
                    k_norm_w=None, eps: float = 1e-6, q_out=None):
    """``qkv_prologue`` with an explicit rotary table (host float64 [D/2] or
    None for no RoPE), magnitude factor and pair layout ("neox" or
    "interleaved").  q [B,S,Hq,D] and k_new/v_new [B,S,Hkv,D] carry S tokens
    per sequence (token s at position pos[b] + s); 3-D inputs mean S = 1.
    Returns q_out float32 of q's shape."""
    S = 1
    if q.dim() == 4:
        S = q.shape[1]
        if k_new.dim() != 4 or v_new.dim() != 4 or k_new.shape[1] != S or v_new.shape[1] != S:
            raise ValueError("q, k_new and v_new must have the same token count")
        for t, w in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
            if t.stride(3) != 1 or t.stride(2) != t.shape[3] or t.stride(1) != t.shape[2] * t.shape[3]:
                raise ValueError(f"{w}: tokens and heads must be dense inside a batch row")
        qv = q.select(1, 0)
        kv_, vv = k_new.select(1, 0), v_new.select(1, 0)
        dev, B, Hq, Hkv, D, T, code, _ = _prologue_checks(
            qv, kv_, vv, pos, k_cache, v_cache, q_norm_w, k_norm_w,
            torch.empty(0, device=k_cache.device))
        if q_out is None:
            q_out = torch.empty((B, S, Hq, D), dtype=torch.float32, device=dev)
        _dev(q_out, "q_out", dev)
        _contig(q_out, "q_out")
        if q_out.dtype != torch.float32 or tuple(q_out.shape) != (B, S, Hq, D):
            raise ValueError("q_out must be float32 [B,S,Hq,D]")
    else:
        dev, B, Hq, Hkv, D, T, code, q_out = _prologue_checks(
            q, k_new, v_new, pos, k_cache, v_cache, q_norm_w, k_norm_w, q_out)
    f = _host_table(inv_freq, D)
    _check(lib.gqa_qkv_prologue_ex(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0), k_new.stride(0),
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), None if f is None else f.ctypes.data,
        float(rope_mscale), _layout_code(rope_layout), _ptr(pos), int(S), _ptr(q_out),
        _ptr(k_cache), _ptr(v_cache), B, Hq, Hkv, D, T, _stream(dev)))
    return q_out


def _prologue_checks(q, k_new, v_new, pos, k_cache, v_cache, q_norm_w, k_norm_w, q_out):
    """Checks of the single-token layout; q_out may be an empty placeholder
    (numel 0) that the caller checks itself."""
    dev = k_cache.device
    for t, w in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (pos, "pos"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, w, dev)
    B, Hq, D = q.shape
    _, Hkv, T, _ = k_cache.shape
    if q.dtype != k_new.dtype or q.dtype != v_new.dtype:
        raise TypeError("q, k_new and v_new must share a dtype")
    code = _dtype_code(q, "q")
    for t, w, h in ((q, "q", Hq), (k_new, "k_new", Hkv), (v_new, "v_new", Hkv)):
        if tuple(t.shape) != (B, h, D) or t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{w}: expected [B,{h},D] with contiguous heads")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must share a batch stride")
    for t, w in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, Hkv, T, D):
            raise ValueError(f"{w}: expected bfloat16 [B,Hkv,T,D]")
        _contig(t, w)
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,):
        raise ValueError("pos must be int32 [B]")
    _contig(pos, "pos")
    for w, nm in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _dev(w, nm, dev)
            if w.dtype != torch.float32 or tuple(w.shape) != (D,):
                raise ValueError(f"{nm} must be float32 [D]")
            _contig(w, nm)
    if q_out is None:
        q_out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if q_out.numel():
        _dev(q_out, "q_out", dev)
        _contig(q_out, "q_out")
        if q_out.dtype != torch.float32 or tuple(q_out.shape) != (B, Hq, D):
            raise ValueError("q_out must be float32 [B,Hq,D]")
    return dev, B, Hq, Hkv, D, T, code, q_out


def _attn_common(q, k_cache, v_cache, lens):
    dev = k_cache.device
    for t, w in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (lens, "lens")):
        _dev(t, w, dev)
        _contig(t, w)
    B, Hq, D = q.shape
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must be [B,Hkv,T,D] of equal shape")
    _, Hkv, T, Dk = k_cache.shape
    if k_cache.shape[0] != B or Dk != D:
        raise ValueError("cache shape does not match q")
    if k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("caches must be bfloat16")
    if lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
        raise ValueError("lens must be int32 [B]")
    return dev, B, Hq, Hkv, D, T


def _lse_check(lse_out, B, Hq, dev):
    if lse_out is not None:
        _dev(lse_out, "lse_out", dev)
        _contig(lse_out, "lse_out")
        if lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (B, Hq):
            raise ValueError("lse_out must be float32 [B,Hq]")


def attn_decode(q, k_cache, v_cache, lens, window: int = 0, scale: float = 0.0,
                out=None, out_dtype=torch.float32, lse_out=None):
    """Unsplit decode attention: one workgroup per (sequence, KV head).

    Returns ``out`` [B,Hq,D]; writes the natural-log LSE into ``lse_out``
    (float32 [B,Hq]) when given."""
    dev, B, Hq, Hkv, D, T = _attn_common(q, k_cache, v_cache, lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    _lse_check(lse_out, B, Hq, dev)
    _check(lib.gqa_attn_decode(
        _ptr(q), _dtype_code(q, "q"), _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(window),
        float(scale), _ptr(out), _dtype_code(out, "out"), _ptr(lse_out), B, Hq, Hkv, D, T,
        _stream(dev)))
    return out


def attn_decode_splitk(q, k_cache, v_cache, lens, part_tokens: int, window: int = 0,
                       scale: float = 0.0, workspace=None):
    """Partition pass of the split-K decode; returns the workspace tensor."""
    dev, B, Hq, Hkv, D, T = _attn_common(q, k_cache, v_cache, lens)
    need = splitk_workspace_bytes(B, Hq, D, T, window, part_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", dev)
    _contig(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.gqa_attn_decode_splitk(
        _ptr(q), _dtype_code(q, "q"), _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(window),
        float(scale), int(part_tokens), _ptr(workspace), nbytes, B, Hq, Hkv, D, T,
        _stream(dev)))
    return workspace


def attn_decode_merge(workspace, B: int, Hq: int, D: int, T: int, part_tokens: int,
                      window: int = 0, out=None, out_dtype=torch.float32, lse_out=None):
    """Log-sum-exp merge of the partitions in ``workspace``; returns ``out``."""
    dev = workspace.device
    _dev(workspace, "workspace")
    _contig(workspace, "workspace")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    _lse_check(lse_out, B, Hq, dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.gqa_attn_decode_merge(
        _ptr(workspace), nbytes, int(window), int(part_tokens), _ptr(out),
        _dtype_code(out, "out"), _ptr(lse_out), B, Hq, D, T, _stream(dev)))
    return out


def workspace_views(workspace, B: int, Hq: int, D: int, T: int, window: int,
                    part_tokens: int):
    """(lse [B,Hq,NP], o [B,Hq,NP,D]) float32 views of a split-K workspace,
    following the layout documented in the header."""
    npart = num_partitions(T, window, part_tokens)
    n_lse = B * Hq * npart
    off = (n_lse * 4 + 255) // 256 * 256
    flat = workspace.view(torch.uint8)
    lse = flat[: n_lse * 4].view(torch.float32).view(B, Hq, npart)
    o = flat[off: off + n_lse * D * 4].view(torch.float32).view(B, Hq, npart, D)
    return lse, o


def _multi_common(q, k_cache, v_cache, lens):
    if q.dim() != 4:
        raise ValueError("q must be [B,S,Hq,D]")
    B, S, Hq, D = q.shape
    dev, _, _, Hkv, _, T = _attn_common(q.reshape(B, S * Hq, D), k_cache, v_cache, lens)
    return dev, B, S, Hq, Hkv, D, T


def attn_decode_multi(q, k_cache, v_cache, lens, window: int = 0, scale: float = 0.0,
                      out=None, out_dtype=torch.float32, lse_out=None):
    """S causal query tokens per sequence (q [B,S,Hq,D]) in one pass per
    (sequence, KV head); token s attends lens[b] - (S-1-s) rows.  Returns out
    [B,S,Hq,D]; writes the LSE into ``lse_out`` (float32 [B,S,Hq]) when given."""
    dev, B, S, Hq, Hkv, D, T = _multi_common(q, k_cache, v_cache, lens)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B,S,Hq,D]")
    if lse_out is not None:
        _lse_check(lse_out.reshape(B, S * Hq), B, S * Hq, dev)
    _check(lib.gqa_attn_decode_multi(
        _ptr(q), _dtype_code(q, "q"), _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(S),
        int(window), float(scale), _ptr(out), _dtype_code(out, "out"), _ptr(lse_out),
        B, Hq, Hkv, D, T, _stream(dev)))
    return out


def attn_prefill(q, k_cache, v_cache, lens, causal: bool = True, window: int = 0,
                 scale: float = 0.0, out=None, out_dtype=torch.float32, lse_out=None,
                 splits: int = 1, workspace=None):
    """S query tokens per sequence (q [B,S,Hq,D]) over the cache on the matrix
    cores, any S.  causal: token s attends lens[b] - (S-1-s) rows (as
    attn_decode_multi); otherwise every token attends lens[b] rows.  Returns
    out [B,S,Hq,D]; writes the LSE into ``lse_out`` (float32 [B,S,Hq]).
    ``splits`` > 1 shares each row block's keys among that many workgroups
    (gqa_attn_prefill_split); ``workspace`` (uint8, its tickets zero) is
    allocated zeroed when None -- reuse it across calls."""
    dev, B, S, Hq, Hkv, D, T = _multi_common(q, k_cache, v_cache, lens)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B,S,Hq,D]")
    if lse_out is not None:
        _lse_check(lse_out.reshape(B, S * Hq), B, S * Hq, dev)
    nbytes = 0
    if splits > 1:
        need = prefill_workspace_bytes(B, S, Hq, Hkv, D, splits)
        if workspace is None:
            workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        _dev(workspace, "workspace", dev)
        _contig(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
    _check(lib.gqa_attn_prefill_split(
        _ptr(q), _dtype_code(q, "q"), _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(S),
        1 if causal else 0, int(window), float(scale), int(splits),
        _ptr(workspace) if splits > 1 else None, nbytes, _ptr(out), _dtype_code(out, "out"),
        _ptr(lse_out), B, Hq, Hkv, D, T, _stream(dev)))
    return out


def prefill_step(q, k_new, v_new, pos, k_cache, v_cache, lens, causal: bool = True,
                 window: int = 0, scale: float = 0.0, inv_freq=None, rope_mscale: float = 1.0,
                 rope_layout="neox", q_norm_w=None, k_norm_w=None, eps: float = 1e-6,
                 splits: int = 1, workspace=None, out=None, out_dtype=torch.float32,
                 lse_out=None, q_out=None):
    """The prefill with its prologue (gqa_prefill_step): q [B,S,Hq,D], k_new
    and v_new [B,S,Hkv,D] (tokens and heads dense, a batch stride of their
    own) in float32 or bfloat16; token s is appended at row pos[b] + s and
    the attention kernel normalises and rotates q itself.  ``inv_freq``:
    host float64 [D/2] rotary table or None.  Returns out [B,S,Hq,D]."""
    dev, B, S, Hq, Hkv, D, T = _multi_common(q, k_cache, v_cache, lens)
    code = _dtype_code(q, "q")
    for t, w, h in ((q, "q", Hq), (k_new, "k_new", Hkv), (v_new, "v_new", Hkv)):
        _dev(t, w, dev)
        if t.dtype != q.dtype:
            raise TypeError("q, k_new and v_new must share a dtype")
        if (tuple(t.shape) != (B, S, h, D) or t.stride(3) != 1 or t.stride(2) != D
                or t.stride(1) != h * D):
            raise ValueError(f"{w}: expected [B,S,{h},D] with contiguous tokens and heads")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must share a batch stride")
    for t, w in ((pos, "pos"),):
        _dev(t, w, dev)
        if t.dtype != torch.int32 or tuple(t.shape) != (B,):
            raise ValueError("pos must be int32 [B]")
        _contig(t, w)
    for w, nm in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _dev(w, nm, dev)
            if w.dtype != torch.float32 or tuple(w.shape) != (D,):
                raise ValueError(f"{nm} must be float32 [D]")
            _contig(w, nm)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B,S,Hq,D]")
    if lse_out is not None:
        _lse_check(lse_out.reshape(B, S * Hq), B, S * Hq, dev)
    if q_out is not None:
        _dev(q_out, "q_out", dev)
        _contig(q_out, "q_out")
        if q_out.dtype != torch.float32 or tuple(q_out.shape) != (B, S, Hq, D):
            raise ValueError("q_out must be float32 [B,S,Hq,D]")
    nbytes = 0
    if splits > 1:
        need = prefill_workspace_bytes(B, S, Hq, Hkv, D, splits)
        if workspace is None:
            workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        _dev(workspace, "workspace", dev)
        _contig(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
    f = _host_table(inv_freq, D)
    _check(lib.gqa_prefill_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0), k_new.stride(0),
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), None if f is None else f.ctypes.data,
        float(rope_mscale), _layout_code(rope_layout), _ptr(pos), int(S),
        _ptr(k_cache), _ptr(v_cache), _ptr(lens), 1 if causal else 0, int(window),
        float(scale), int(splits), _ptr(workspace) if splits > 1 else None, nbytes,
        _ptr(out), _dtype_code(out, "out"), _ptr(lse_out), _ptr(q_out), B, Hq, Hkv, D, T,
        _stream(dev)))
    return out


def prefill_workspace_bytes(B: int, S: int, Hq: int, Hkv: int, D: int, splits: int) -> int:
    return int(lib.gqa_attn_prefill_workspace_bytes(B, S, Hq, Hkv, D, splits))


def prefill_default_splits(B: int, S: int, Hq: int, Hkv: int) -> int:
    return int(lib.gqa_attn_prefill_default_splits(B, S, Hq, Hkv))


def qkv_gemv(x, w, out=None, out_dtype=torch.bfloat16):
    """Packed QKV projection y = x W^T for the decode batch: x [M,K] bf16
    (M <= 16), w [N,K] bf16 (rows of the projection, K a multiple of 128).
    Returns y [M,N] (or writes ``out``, which may be a row-strided view)."""
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [M,K] and w [N,K]")
    dev = x.device
    _dev(w, "w", dev)
    for t, nm in ((x, "x"), (w, "w")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{nm} must be bfloat16")
        if t.stride(1) != 1:
            raise ValueError(f"{nm} rows must be contiguous")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N,K] with the K of x")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    if tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be [M,N] with contiguous rows")
    _check(lib.gqa_qkv_gemv(_ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(out),
                            _dtype_code(out, "out"), out.stride(0), M, N, K, _stream(dev)))
    return out


def probe_stream_read(buf, workgroups: int = 256, threads: int = 256, unroll: int = 8,
                      sink=None, nbytes: Optional[int] = None):
    """Measurement helper (not part of the attention path): read the first
    ``nbytes`` bytes (default: all) of the contiguous device tensor ``buf``
    once, one contiguous share per workgroup, ``unroll`` 16-byte loads in
    flight per thread.  ``sink`` is a device uint32/int32 tensor of at least
    workgroups * threads elements (allocated when None)."""
    _dev(buf, "buf")
    _contig(buf, "buf")
    dev = buf.device
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if n > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if sink is None:
        sink = torch.empty(workgroups * threads, dtype=torch.int32, device=dev)
    _dev(sink, "sink", dev)
    if sink.numel() * sink.element_size() < 4 * workgroups * threads:
        raise ValueError("sink must hold workgroups * threads uint32")
    _check(lib.gqa_probe_stream_read(_ptr(buf), n, workgroups, threads, unroll, _ptr(sink),
                                     _stream(dev)))
    return sink


def splitk_multi_workspace_bytes(B: int, S: int, Hq: int, D: int, T: int, window: int,
                                 part_tokens: int) -> int:
    return int(lib.gqa_splitk_multi_workspace_bytes(B, S, Hq, D, T, window, part_tokens))


def attn_decode_splitk_multi(q, k_cache, v_cache, lens, part_tokens: int, window: int = 0,
                             scale: float = 0.0, workspace=None):
    """Partition pass of the split-K multi-token decode; returns the workspace."""
    dev, B, S, Hq, Hkv, D, T = _multi_common(q, k_cache, v_cache, lens)
    need = splitk_multi_workspace_bytes(B, S, Hq, D, T, window, part_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", dev)
    _contig(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.gqa_attn_decode_splitk_multi(
        _ptr(q), _dtype_code(q, "q"), _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(S),
        int(window), float(scale), int(part_tokens), _ptr(workspace), nbytes,
        B, Hq, Hkv, D, T, _stream(dev)))
    return workspace


def attn_decode_merge_multi(workspace, B: int, S: int, Hq: int, D: int, T: int,
                            part_tokens: int, window: int = 0, out=None,
                            out_dtype=torch.float32, lse_out=None):
    """Merge of the multi-token partitions; returns out [B,S,Hq,D]."""
    dev = workspace.device
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    if tuple(out.shape) != (B, S, Hq, D):
        raise ValueError("out must be [B,S,Hq,D]")
    if lse_out is not None:
        _lse_check(lse_out.reshape(B, S * Hq), B, S * Hq, dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.gqa_attn_decode_merge_multi(
        _ptr(workspace), nbytes, int(S), int(window), int(part_tokens), _ptr(out),
        _dtype_code(out, "out"), _ptr(lse_out), B, Hq, D, T, _stream(dev)))
    return out


def decode_step_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, T: int, window: int,
                                part_tokens: int) -> int:
    return int(lib.gqa_decode_step_workspace_bytes(B, Hq, Hkv, D, T, window, part_tokens))


def decode_step(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens: int,
                workspace=None, q_norm_w=None, k_norm_w=None, eps: float = 1e-6,
                rope_theta: float = 0.0, window: int = 0, scale: float = 0.0, out=None,
                out_dtype=torch.float32, lse_out=None, q_out=None):
    """Whole decode step in one launch: prologue + split-K attention + merge.

    Inputs as for ``qkv_prologue`` plus ``lens``; ``workspace`` is a uint8
    device tensor whose arrival tickets start at zero (allocated zeroed when
    None; reuse it across calls).  Returns ``(out, workspace)``.
    """
    a = _step_checks(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens, workspace,
                     q_norm_w, k_norm_w, window, out, out_dtype, lse_out, q_out)
    dev, B, Hq, Hkv, D, T, code, workspace, out, nbytes, pro = a
    _check(lib.gqa_decode_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0),
        k_new.stride(0) if pro else Hkv * D,
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), float(rope_theta), _ptr(pos),
        _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(window), float(scale), int(part_tokens),
        _ptr(workspace), nbytes, _ptr(out), _dtype_code(out, "out"), _ptr(lse_out),
        _ptr(q_out), B, Hq, Hkv, D, T, _stream(dev)))
    return out, workspace


def decode_step_ex(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens: int,
                   workspace=None, inv_freq=None, rope_mscale: float = 1.0,
                   rope_layout="neox", q_norm_w=None, k_norm_w=None, eps: float = 1e-6,
                   window: int = 0, scale: float = 0.0, out=None, out_dtype=torch.float32,
                   lse_out=None, q_out=None):
    """``decode_step`` with an explicit rotary table (host float64 [D/2] or
    None), magnitude factor and pair layout."""
    a = _step_checks(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens, workspace,
                     q_norm_w, k_norm_w, window, out, out_dtype, lse_out, q_out)
    dev, B, Hq, Hkv, D, T, code, workspace, out, nbytes, pro = a
    f = _host_table(inv_freq, D)
    _check(lib.gqa_decode_step_ex(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0),
        k_new.stride(0) if pro else Hkv * D,
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), None if f is None else f.ctypes.data,
        float(rope_mscale), _layout_code(rope_layout), _ptr(pos),
        _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(window), float(scale), int(part_tokens),
        _ptr(workspace), nbytes, _ptr(out), _dtype_code(out, "out"), _ptr(lse_out),
        _ptr(q_out), B, Hq, Hkv, D, T, _stream(dev)))
    return out, workspace


def decode_step_multi_workspace_bytes(B: int, S: int, Hq: int, Hkv: int, D: int, T: int,
                                      window: int, part_tokens: int) -> int:
    return int(lib.gqa_decode_step_multi_workspace_bytes(B, S, Hq, Hkv, D, T, window,
                                                         part_tokens))


def decode_step_multi(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens: int,
                      workspace=None, inv_freq=None, rope_mscale: float = 1.0,
                      rope_layout="neox", q_norm_w=None, k_norm_w=None, eps: float = 1e-6,
                      window: int = 0, scale: float = 0.0, out=None, out_dtype=torch.float32,
                      lse_out=None, q_out=None):
    """The whole multi-token step in one launch: q [B,S,Hq,D], k_new and
    v_new [B,S,Hkv,D] (tokens and heads dense; a batch stride of their own),
    token s rotated at pos[b] + s and appended at row pos[b] + s, then the
    attention of ``attn_decode_multi``.  ``inv_freq``: host float64 [D/2]
    rotary table or None.  Returns ``(out [B,S,Hq,D], workspace)``; the
    workspace's tickets start at zero (allocated zeroed when None)."""
    a = _step_checks(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens, workspace,
                     q_norm_w, k_norm_w, window, out, out_dtype, lse_out, q_out, multi=True)
    dev, B, S, Hq, Hkv, D, T, code, workspace, out, nbytes, pro = a
    f = _host_table(inv_freq, D)
    _check(lib.gqa_decode_step_multi(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0),
        k_new.stride(0) if pro else S * Hkv * D,
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), None if f is None else f.ctypes.data,
        float(rope_mscale), _layout_code(rope_layout), _ptr(pos), S,
        _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(window), float(scale), int(part_tokens),
        _ptr(workspace), nbytes, _ptr(out), _dtype_code(out, "out"), _ptr(lse_out),
        _ptr(q_out), B, Hq, Hkv, D, T, _stream(dev)))
    return out, workspace


def decode_step_noalloc(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens: int,
                        inv_freq=None, rope_mscale: float = 1.0, rope_layout="neox",
                        q_norm_w=None, k_norm_w=None, eps: float = 1e-6, window: int = 0,
                        scale: float = 0.0, out=None, out_dtype=torch.float32, lse_out=None,
                        q_out=None):
    """``decode_step_multi`` without a workspace: the library's static
    per-device scratch holds the tickets and partials (for callers that
    cannot allocate; ``out`` must then be given, since allocating it here
    would defeat the purpose).  Calls that overlap in time on one GPU race.
    Returns ``out``."""
    if out is None:
        raise ValueError("decode_step_noalloc needs a preallocated out")
    a = _step_checks(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens, None,
                     q_norm_w, k_norm_w, window, out, out_dtype, lse_out, q_out, multi=True,
                     no_workspace=True)
    dev, B, S, Hq, Hkv, D, T, code, _, out, _, pro = a
    f = _host_table(inv_freq, D)
    _check(lib.gqa_decode_step_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), code, q.stride(0),
        k_new.stride(0) if pro else S * Hkv * D,
        _ptr(q_norm_w), _ptr(k_norm_w), float(eps), None if f is None else f.ctypes.data,
        float(rope_mscale), _layout_code(rope_layout), _ptr(pos), S,
        _ptr(k_cache), _ptr(v_cache), _ptr(lens), int(window), float(scale), int(part_tokens),
        _ptr(out), _dtype_code(out, "out"), _ptr(lse_out), _ptr(q_out), B, Hq, Hkv, D, T,
        _stream(dev)))
    return out


def _step_checks(q, k_new, v_new, pos, k_cache, v_cache, lens, part_tokens, workspace,
                 q_norm_w, k_norm_w, window, out, out_dtype, lse_out, q_out, multi=False,
                 no_workspace=False):
    """Checks of the one-launch step.  ``multi``: q, k_new, v_new, out and
    q_out carry a token axis ([B,S,H,D], tokens and heads dense).
    ``no_workspace``: the call takes no workspace (none is allocated)."""
    dev = k_cache.device
    pro = pos is not None
    if (k_new is None) == pro or (v_new is None) == pro:
        raise ValueError("pos, k_new and v_new come together (or all None: no prologue)")
    for t, w in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (lens, "lens")):
        _dev(t, w, dev)
    if multi:
        if q.dim() != 4:
            raise ValueError("q: expected [B,S,Hq,D]")
        B, S, Hq, D = q.shape
    else:
        B, Hq, D = q.shape
        S = 1
    _, Hkv, T, _ = k_cache.shape
    code = _dtype_code(q, "q")
    news = ((k_new, "k_new", Hkv), (v_new, "v_new", Hkv)) if pro else ()
    for t, w, h in ((q, "q", Hq),) + news:
        _dev(t, w, dev)
        if t.dtype != q.dtype:
            raise TypeError("q, k_new and v_new must share a dtype")
        if multi:
            if (tuple(t.shape) != (B, S, h, D) or t.stride(3) != 1 or t.stride(2) != D
                    or t.stride(1) != h * D):
                raise ValueError(f"{w}: expected [B,S,{h},D] with contiguous tokens and heads")
        elif tuple(t.shape) != (B, h, D) or t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{w}: expected [B,{h},D] with contiguous heads")
    if pro and k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must share a batch stride")
    for t, w in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, Hkv, T, D):
            raise ValueError(f"{w}: expected bfloat16 [B,Hkv,T,D]")
        _contig(t, w)
    for t, w in ((pos, "pos"), (lens, "lens")):
        if t is None:
            continue
        _dev(t, w, dev)
        if t.dtype != torch.int32 or tuple(t.shape) != (B,):
            raise ValueError(f"{w} must be int32 [B]")
        _contig(t, w)
    for w, nm in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _dev(w, nm, dev)
            if w.dtype != torch.float32 or tuple(w.shape) != (D,):
                raise ValueError(f"{nm} must be float32 [D]")
            _contig(w, nm)
    if not no_workspace:
        need = (decode_step_multi_workspace_bytes(B, S, Hq, Hkv, D, T, window, part_tokens)
                if multi else decode_step_workspace_bytes(B, Hq, Hkv, D, T, window, part_tokens))
        if workspace is None:
            workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        _dev(workspace, "workspace", dev)
        _contig(workspace, "workspace")
    rows = (B, S, Hq) if multi else (B, Hq)
    if out is None:
        out = torch.empty(rows + (D,), dtype=out_dtype, device=dev)
    _dev(out, "out", dev)
    _contig(out, "out")
    if multi:
        if tuple(out.shape) != rows + (D,):
            raise ValueError("out: expected [B,S,Hq,D]")
        if lse_out is not None:
            _dev(lse_out, "lse_out", dev)
            _contig(lse_out, "lse_out")
            if lse_out.dtype != torch.float32 or tuple(lse_out.shape) != rows:
                raise ValueError("lse_out must be float32 [B,S,Hq]")
    else:
        _lse_check(lse_out, B, Hq, dev)
    if q_out is not None:
        _dev(q_out, "q_out", dev)
        _contig(q_out, "q_out")
        if q_out.dtype != torch.float32 or tuple(q_out.shape) != rows + (D,):
            raise ValueError(f"q_out must be float32 {list(rows + (D,))}")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if multi:
        return dev, B, S, Hq, Hkv, D, T, code, workspace, out, nbytes, pro
    return dev, B, Hq, Hkv, D, T, code, workspace, out, nbytes, pro
