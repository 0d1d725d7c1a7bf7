// Launchers behind the C ABI.  Arguments are validated by the caller (the
// extern "C" entry points); these only pick a kernel instance and enqueue it.
// Each returns 0 on success or a negative gqa status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct PrologueArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  int in_bf16;
  int64_t q_bstride, kv_bstride;
  const float* q_norm_w;
  const float* k_norm_w;
  float eps;
  double theta;
  const int32_t* pos;
  float* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int B, Hq, Hkv, D, T;
};

struct AttnArgs {
  const void* q;
  int q_bf16;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* lens;
  int window;
  float qscale;        // softmax scale * log2(e)
  int part_tokens;     // split mode: partition length
  int num_parts;       // split mode: partitions per (sequence, KV head)
  float* ws_lse;       // split mode: [B,Hq,num_parts]
  float* ws_o;         // split mode: [B,Hq,num_parts,D]
  void* out;           // final mode
  int out_bf16;
  float* lse_out;      // final mode, may be null
  int B, Hq, Hkv, D, T;
  bool split;
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

int launch_prologue(const PrologueArgs& a, hipStream_t s);
int launch_attn_valu(const AttnArgs& a, hipStream_t s);   // VALU dot products
int launch_attn_mfma(const AttnArgs& a, hipStream_t s);   // matrix-core dot products
int launch_merge(const MergeArgs& a, hipStream_t s);

// The attention pass used by the C ABI.
inline int launch_attn(const AttnArgs& a, hipStream_t s) {
#ifdef GQA_ATTN_VALU
  return launch_attn_valu(a, s);
#else
  return launch_attn_mfma(a, s);
#endif
}

}  // namespace gqa
