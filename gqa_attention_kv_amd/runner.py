"""Device-resident decode step: upload a workload once, then enqueue
prologue -> attention (unsplit, or split-K partitions + merge) on torch's
current stream as often as needed.

Only plumbing lives here (uploads, buffer allocation, the order of the C-ABI
calls); every arithmetic step runs in the HIP kernels.  The prologue's append
is idempotent (same row, same bytes), so ``run()`` can be repeated.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import attn_decode, attn_decode_merge, attn_decode_splitk, decode_step, qkv_prologue
from . import decode_step_ex, qkv_prologue_ex, rope_table
from . import attn_decode_merge_multi, attn_decode_multi, attn_decode_splitk_multi, attn_prefill
from . import splitk_multi_workspace_bytes
from . import decode_step_multi, decode_step_multi_workspace_bytes, prefill_workspace_bytes
from . import prefill_step, qkv_gemv

BF16_NAN = 0x7FC0


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> torch.bfloat16 tensor on ``device``."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceStep:
    """One decode step of workload ``w`` with all inputs resident in HBM.

    ``mode``: "fused" runs the whole step as one launch (gqa_decode_step, or
    gqa_decode_step_multi with several tokens); "split" runs the prologue,
    the split-K partition pass over ``part_tokens``-row partitions (default:
    the workload's own size) and the merge as three launches; "unsplit" runs
    the prologue and the unsplit kernel; "prefill" runs the prologue and the
    matrix-core prefill kernel (any number of tokens, causal or
    bidirectional as the workload says; ``splits`` > 1 shares each row
    block's keys among that many workgroups); "prefill_step" runs the K/V
    append and the prefill kernel, which rotates q itself
    (gqa_prefill_step).  ``split`` (bool) is the older spelling of
    split/unsplit.  ``q_dtype`` selects the dtype attention reads q in when
    the workload has no prologue.  ``poison`` writes bf16 NaN into every
    cache row outside each sequence's attended range [lo, n) (rows the step
    must never read); rows written by the prologue are left alone.
    """

    def __init__(self, w, device="cuda", split: bool = True,
                 part_tokens: Optional[int] = None, out_dtype: Optional[str] = None,
                 q_dtype: str = "bf16", poison: bool = False, scale: float = 0.0,
                 mode: Optional[str] = None, splits: int = 1):
        self.w = w
        self.dev = torch.device(device)
        self.S = int(getattr(w, "S", 1))     # query tokens per sequence
        self.mode = mode or ("split" if split else "unsplit")
        self.causal = bool(getattr(w, "causal", True))
        if self.mode == "prefill_step" and w.pos is None:
            raise ValueError("prefill_step needs a workload with a prologue")
        if not self.causal and self.mode not in ("prefill", "prefill_step"):
            raise NotImplementedError("bidirectional attention runs on the prefill kernel")
        self.split = self.mode == "split"
        self.splits = int(splits)           # prefill: key splits per row block
        self.part_tokens = int(part_tokens or w.part_tokens)
        self.scale = float(scale)
        od = out_dtype or w.out_dtype
        self.out_dtype = torch.bfloat16 if od == "bf16" else torch.float32
        kc, vc = w.k_cache, w.v_cache
        if poison:
            kc, vc = kc.copy(), vc.copy()
            n = np.clip(w.lens.astype(np.int64), 0, w.T)
            back = (self.S - 1) if self.causal else 0
            for b in range(w.B):
                n0 = max(0, min(int(w.lens[b]) - back, w.T))   # first token's end
                lo = max(0, n0 - w.window) if w.window > 0 else 0
                keep = np.zeros(w.T, bool)
                keep[lo:int(n[b])] = True
                if w.pos is not None:
                    for st in range(self.S):
                        if 0 <= int(w.pos[b]) + st < w.T:
                            keep[int(w.pos[b]) + st] = True
                kc[b][:, ~keep] = BF16_NAN
                vc[b][:, ~keep] = BF16_NAN
        d = self.dev
        self.k_cache = bf16_tensor(kc, d)
        self.v_cache = bf16_tensor(vc, d)
        self.lens = torch.from_numpy(w.lens.astype(np.int32)).to(d)
        self.rope_ex, self.inv_freq, self.rope_mscale, self.rope_layout = False, None, 1.0, "neox"
        if w.pos is not None:
            self.q_in = bf16_tensor(w.q, d)
            self.k_new = bf16_tensor(w.k_new, d)
            self.v_new = bf16_tensor(w.v_new, d)
            self.pos = torch.from_numpy(w.pos.astype(np.int32)).to(d)
            self.w_q = None if w.w_q is None else torch.from_numpy(w.w_q).to(d)
            self.w_k = None if w.w_k is None else torch.from_numpy(w.w_k).to(d)
            self.q = torch.empty(tuple(w.q.shape), dtype=torch.float32, device=d)
            # A RoPE variant (interleaved pairs or a context-extension table)
            # or several tokens go through the *_ex entry points with the
            # library's own table.
            sc = getattr(w, "rope_scaling", None)
            self.rope_layout = getattr(w, "rope_layout", "neox")
            self.rope_ex = (sc is not None or self.rope_layout != "neox" or self.S > 1)
            self.inv_freq, self.rope_mscale = None, 1.0
            if self.rope_ex and w.theta > 0:
                sc = dict(sc or {"kind": "default"})
                self.inv_freq, self.rope_mscale = rope_table(sc.pop("kind"), w.D, w.theta, **sc)
        else:
            qb = bf16_tensor(w.q, d)
            self.q = qb if q_dtype == "bf16" else qb.float()
        tok = (self.S,) if self.S > 1 else ()
        self.out = torch.empty((w.B,) + tok + (w.Hq, w.D), dtype=self.out_dtype, device=d)
        self.lse = torch.empty((w.B,) + tok + (w.Hq,), dtype=torch.float32, device=d)
        self.ws = None
        self.pws = None
        if self.mode == "prefill_step" and self.inv_freq is None and w.theta > 0:
            self.inv_freq, self.rope_mscale = rope_table("default", w.D, w.theta)
        if self.mode in ("prefill", "prefill_step") and self.splits > 1:
            nb = prefill_workspace_bytes(w.B, self.S, w.Hq, w.Hkv, w.D, self.splits)
            self.pws = torch.zeros(nb, dtype=torch.uint8, device=d)   # tickets start at 0
        if self.mode == "split":
            nb = splitk_multi_workspace_bytes(w.B, self.S, w.Hq, w.D, w.T, w.window,
                                              self.part_tokens)
            self.ws = torch.empty(nb, dtype=torch.uint8, device=d)
        elif self.mode == "fused":
            nb = decode_step_multi_workspace_bytes(w.B, self.S, w.Hq, w.Hkv, w.D, w.T, w.window,
                                                   self.part_tokens)
            self.ws = torch.zeros(nb, dtype=torch.uint8, device=d)   # tickets start at 0

    # -- the three stages, each one C-ABI call ------------------------------
    def prologue(self):
        w = self.w
        if w.pos is None:
            return
        if self.rope_ex:
            qkv_prologue_ex(self.q_in, self.k_new, self.v_new, self.pos, self.k_cache,
                            self.v_cache, inv_freq=self.inv_freq, rope_mscale=self.rope_mscale,
                            rope_layout=self.rope_layout, q_norm_w=self.w_q, k_norm_w=self.w_k,
                            eps=w.eps, q_out=self.q)
            return
        qkv_prologue(self.q_in, self.k_new, self.v_new, self.pos, self.k_cache, self.v_cache,
                     q_norm_w=self.w_q, k_norm_w=self.w_k, eps=w.eps,
                     rope_theta=w.theta, q_out=self.q)

    def attention(self):
        w = self.w
        if self.mode == "prefill":
            q = self.q if self.q.dim() == 4 else self.q.unsqueeze(1)
            out = self.out if self.out.dim() == 4 else self.out.unsqueeze(1)
            attn_prefill(q, self.k_cache, self.v_cache, self.lens, causal=self.causal,
                         window=w.window, scale=self.scale, out=out,
                         lse_out=self.lse.reshape(w.B, self.S, w.Hq), splits=self.splits,
                         workspace=self.pws)
            return
        if self.S > 1:
            if self.split:
                attn_decode_splitk_multi(self.q, self.k_cache, self.v_cache, self.lens,
                                         self.part_tokens, window=w.window, scale=self.scale,
                                         workspace=self.ws)
            else:
                attn_decode_multi(self.q, self.k_cache, self.v_cache, self.lens,
                                  window=w.window, scale=self.scale, out=self.out,
                                  lse_out=self.lse)
            return
        if self.split:
            attn_decode_splitk(self.q, self.k_cache, self.v_cache, self.lens, self.part_tokens,
                               window=w.window, scale=self.scale, workspace=self.ws)
        else:
            attn_decode(self.q, self.k_cache, self.v_cache, self.lens, window=w.window,
                        scale=self.scale, out=self.out, lse_out=self.lse)

    def merge(self):
        if not self.split:
            return
        w = self.w
        if self.S > 1:
            attn_decode_merge_multi(self.ws, w.B, self.S, w.Hq, w.D, w.T, self.part_tokens,
                                    window=w.window, out=self.out, lse_out=self.lse)
            return
        attn_decode_merge(self.ws, w.B, w.Hq, w.D, w.T, self.part_tokens, window=w.window,
                          out=self.out, lse_out=self.lse)

    def fused(self):
        w = self.w
        if self.S > 1:
            pro = w.pos is not None
            decode_step_multi(self.q_in if pro else self.q, self.k_new if pro else None,
                              self.v_new if pro else None, self.pos if pro else None,
                              self.k_cache, self.v_cache, self.lens, self.part_tokens,
                              workspace=self.ws, inv_freq=self.inv_freq if pro else None,
                              rope_mscale=self.rope_mscale, rope_layout=self.rope_layout,
                              q_norm_w=self.w_q if pro else None,
                              k_norm_w=self.w_k if pro else None, eps=w.eps,
                              window=w.window, scale=self.scale, out=self.out,
                              lse_out=self.lse, q_out=self.q if pro else None)
            return
        if w.pos is None:        # no prologue: attention and merge in one launch
            decode_step(self.q, None, None, None, self.k_cache, self.v_cache, self.lens,
                        self.part_tokens, workspace=self.ws, window=w.window,
                        scale=self.scale, out=self.out, lse_out=self.lse)
            return
        if self.rope_ex:
            decode_step_ex(self.q_in, self.k_new, self.v_new, self.pos, self.k_cache,
                           self.v_cache, self.lens, self.part_tokens, workspace=self.ws,
                           inv_freq=self.inv_freq, rope_mscale=self.rope_mscale,
                           rope_layout=self.rope_layout, q_norm_w=self.w_q, k_norm_w=self.w_k,
                           eps=w.eps, window=w.window, scale=self.scale, out=self.out,
                           lse_out=self.lse, q_out=self.q)
            return
        decode_step(self.q_in, self.k_new, self.v_new, self.pos, self.k_cache, self.v_cache,
                    self.lens, self.part_tokens, workspace=self.ws, q_norm_w=self.w_q,
                    k_norm_w=self.w_k, eps=w.eps, rope_theta=w.theta, window=w.window,
                    scale=self.scale, out=self.out, lse_out=self.lse, q_out=self.q)

    def ws_counters(self) -> torch.Tensor:
        """The fused step's arrival tickets (int32 view of the workspace
        tail, [B*Hkv]); they are zero between calls."""
        w = self.w
        base = splitk_multi_workspace_bytes(w.B, self.S, w.Hq, w.D, w.T, w.window,
                                            self.part_tokens)
        off = base + (-base) % 256
        return self.ws[off:off + 4 * w.B * w.Hkv].view(torch.int32)

    def prefill_step(self):
        w = self.w
        q = self.q_in if self.q_in.dim() == 4 else self.q_in.unsqueeze(1)
        kn = self.k_new if self.k_new.dim() == 4 else self.k_new.unsqueeze(1)
        vn = self.v_new if self.v_new.dim() == 4 else self.v_new.unsqueeze(1)
        out = self.out if self.out.dim() == 4 else self.out.unsqueeze(1)
        qo = self.q if self.q.dim() == 4 else self.q.unsqueeze(1)
        prefill_step(q, kn, vn, self.pos, self.k_cache, self.v_cache, self.lens,
                     causal=self.causal, window=w.window, scale=self.scale,
                     inv_freq=self.inv_freq, rope_mscale=self.rope_mscale,
                     rope_layout=self.rope_layout, q_norm_w=self.w_q, k_norm_w=self.w_k,
                     eps=w.eps, splits=self.splits, workspace=self.pws, out=out,
                     lse_out=self.lse.reshape(w.B, self.S, w.Hq), q_out=qo)

    def run(self):
        if self.mode == "fused":
            self.fused()
            return
        if self.mode == "prefill_step":
            self.prefill_step()
            return
        self.prologue()
        self.attention()
        self.merge()

    def results(self) -> dict:
        torch.cuda.synchronize(self.dev)
        out = self.out.float().cpu().numpy().astype(np.float64)
        return dict(out=out, lse=self.lse.cpu().numpy().astype(np.float64),
                    q=self.q.float().cpu().numpy().astype(np.float64),
                    k_cache=bf16_bits(self.k_cache), v_cache=bf16_bits(self.v_cache))


class DeviceGemv:
    """The packed QKV projection of a projection workload with x and W
    resident in HBM; ``run()`` enqueues y = x W^T on torch's current
    stream."""

    def __init__(self, g, device="cuda", out_dtype: Optional[str] = None):
        self.g = g
        d = torch.device(device)
        self.x = bf16_tensor(g.x, d)
        self.w = bf16_tensor(g.w, d)
        od = out_dtype or g.out_dtype
        self.y = torch.empty((g.M, g.N), dtype=torch.bfloat16 if od == "bf16" else torch.float32,
                             device=d)

    def run(self):
        qkv_gemv(self.x, self.w, out=self.y)
