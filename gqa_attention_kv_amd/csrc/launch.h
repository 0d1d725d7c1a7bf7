// Launchers behind the C ABI.  Arguments are validated by the caller (the
// extern "C" entry points); these only pick a kernel instance and enqueue it.
// Each returns 0 on success or a negative gqa status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gqa_decode.h"

namespace gqa {

constexpr int kMaxHalfDim = 64;   // D/2 for the largest supported head dim

// Arguments of the standalone prologue kernel, passed by value.
struct PrologueArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  int in_bf16;
  int64_t q_bstride, kv_bstride;
  const float* q_norm_w;
  const float* k_norm_w;
  float eps;
  int rope;                    // 0: no RoPE
  int rope_interleaved;        // pairs (2i, 2i+1) instead of (i, i+D/2)
  float rope_mscale;           // magnitude factor of the rotated vectors
  const int32_t* pos;          // token s of sequence b sits at pos[b] + s
  int S;                       // tokens per sequence
  float* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int B, Hq, Hkv, D, T;
  int kv_only;                 // only the K/V append (q is rotated elsewhere; q_out unused)
  double inv_freq_rev[kMaxHalfDim];   // rotary frequency of pair i / (2 pi), float64
};

// Arguments of the attention kernel in all three modes, passed by value.
struct KernelArgs {
  // query [B,S,Hq,D]: sequences q_bstride elements apart, tokens q_sstride
  // apart, heads dense
  const void* q;
  int64_t q_bstride;
  int64_t q_sstride;
  int S;                       // query tokens per sequence (causal among themselves)
  int in_bf16;                 // q (and, in Step, k_new / v_new) are bf16
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* lens;
  int window;
  float qscale;                // softmax scale * log2(e)
  int part_tokens;             // Split / Step
  int num_parts;
  float* ws_lse;               // [B,S,Hq,num_parts]
  float* ws_o;                 // [B,S,Hq,num_parts,D]
  uint32_t* ws_cnt;            // Step: [B,Hkv] arrival tickets, zero between launches
  void* out;                   // Final / Step
  int out_bf16;
  float* lse_out;              // may be null
  int B, Hq, Hkv, D, T;
  // Step only: the fused prologue
  const void* k_new;           // [B,S,Hkv,D]: sequences kv_bstride apart, tokens Hkv*D
  const void* v_new;
  int64_t kv_bstride;
  const float* wq;             // null: no QK-norm
  const float* wk;
  float eps;
  int rope;                    // 0: no RoPE
  int rope_interleaved;        // pairs (2i, 2i+1) instead of (i, i+D/2)
  float rope_mscale;           // magnitude factor of the rotated vectors
  const int32_t* pos;          // token s at position (and cache row) pos[b] + s
  float* q_out;                // [B,S,Hq,D] or null
  uint16_t* k_cache_w;         // same buffers as k_cache / v_cache
  uint16_t* v_cache_w;
  double inv_freq_rev[kMaxHalfDim];   // frequency of pair i / (2 pi), float64
};

struct MergeArgs {
  const float* ws_lse;
  const float* ws_o;
  int num_parts;
  void* out;
  int out_bf16;
  float* lse_out;
  int B, Hq, D;
};

// Arguments of the prefill kernel (S query tokens per sequence over the
// cache, causal or bidirectional), passed by value.
struct PrefillArgs {
  const void* q;               // [B,S,Hq,D]: sequences q_bstride apart, tokens and heads dense
  int64_t q_bstride;
  int in_bf16;
  const uint16_t* k_cache;     // [B,Hkv,T,D]
  const uint16_t* v_cache;
  const int32_t* lens;
  int S;
  int causal;
  int window;
  float qscale;                // softmax scale * log2(e)
  void* out;                   // [B,S,Hq,D]
  int out_bf16;
  float* lse_out;              // [B,S,Hq] or null
  int B, Hq, Hkv, D, T;
  int row_blocks;              // ceil(S * G / prefill_rows_per_block())
  // Key splits: each row block's tiles are shared out among `splits`
  // workgroups whose partials (normalised o, natural-log lse) go to ws_o /
  // ws_lse; the last of them to arrive (ticket ws_cnt, one per row block,
  // zero between launches) merges them.  splits = 1: no workspace.
  int splits;
  float* ws_o;                 // [teams, splits, rows per block, D]
  float* ws_lse;               // [teams, splits, rows per block]
  uint32_t* ws_cnt;            // [teams]
  // q prologue in the kernel (q raw): RMSNorm with wq (or none), then RoPE
  // of token s at pos[b] + s; q_out [B,S,Hq,D] float32 or null
  int pro;
  const float* wq;
  float eps;
  int rope;
  int rope_interleaved;
  float rope_mscale;
  const int32_t* pos;
  float* q_out;
  double inv_freq_rev[kMaxHalfDim];   // rotary frequency of pair i / (2 pi), float64
};

// Arguments of the packed QKV projection y[M,N] = x[M,K] W^T, passed by
// value.  Strides are in elements.
struct GemvArgs {
  const uint16_t* x;           // [M, x_stride] bf16
  int64_t x_stride;
  const uint16_t* w;           // [N, w_stride] bf16
  int64_t w_stride;
  void* y;                     // [M, y_stride] fp32 or bf16
  int64_t y_stride;
  int out_bf16;
  int M, N, K;
};

int launch_prologue(const PrologueArgs& a, hipStream_t s);
int launch_attn_final(const KernelArgs& a, hipStream_t s);   // one pass per (seq, KV head)
int launch_attn_split(const KernelArgs& a, hipStream_t s);   // partition pass
int launch_decode_step(const KernelArgs& a, hipStream_t s);  // fused whole step
int launch_merge(const MergeArgs& a, hipStream_t s);
int prefill_rows_per_block();                                 // (token, head) rows per workgroup
int launch_attn_prefill(const PrefillArgs& a, hipStream_t s);
int launch_qkv_gemv(const GemvArgs& a, hipStream_t s);
// Host checks of a fused decode step's arguments (all but its workspace),
// shared by gqa_decode_step_multi and gqa_decode_step_noalloc: fills `a`
// except ws_lse / ws_o / ws_cnt and returns GQA_OK, or a negative status.
int decode_step_args(const void* q, const void* k_new, const void* v_new,
                     gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                     const float* q_norm_w, const float* k_norm_w, float eps,
                     const double* inv_freq, double rope_mscale, int rope_layout,
                     const int32_t* pos, int S,
                     uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                     int window, float scale, int part_tokens,
                     void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                     int B, int Hq, int Hkv, int D, int T, KernelArgs* a);
// Bytes of the step's lse partials [B,S,Hq,num_parts] fp32, rounded up to 256.
size_t step_lse_bytes(int B, int S, int Hq, int num_parts);
int launch_stream_read(const void* buf, uint32_t bytes, int workgroups, int threads, int unroll,
                       uint32_t* sink, hipStream_t s);   // read-ceiling probe

}  // namespace gqa
