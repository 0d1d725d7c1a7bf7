// extern "C" entry points declared in include/gqa_decode.h: host-side
// argument checks, then the launcher calls (one, or two for
// gqa_prefill_step).  Nothing is enqueued when a check fails, and no entry
// point allocates, frees, synchronises or reads device memory
// (gqa_attn_prefill_default_splits only reads a device attribute).
#include <math.h>
#include <stdint.h>

#include "../../include/gqa_decode.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxIndex = INT64_C(1) << 62;
// Workgroups per launch: one-dimensional grids of up to 512 threads per
// workgroup stay below 2^32 threads.
constexpr int64_t kMaxWorkgroups = INT64_C(1) << 23;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dtype_ok(gqa_dtype_t t) { return t == GQA_F32 || t == GQA_BF16; }

bool group_ok(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

// Shared shape checks for [B,Hq,D] queries against a [B,Hkv,T,D] cache.
int check_shapes(int B, int Hq, int Hkv, int D, int T) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || T < 1) return GQA_ERR_SHAPE;
  if (Hq % Hkv != 0) return GQA_ERR_SHAPE;
  if ((int64_t)B * Hkv * T > kMaxIndex / D) return GQA_ERR_SHAPE;
  // the attention kernels address one (sequence, KV head) slab of T rows
  // with 32-bit byte offsets
  if ((int64_t)T * D * 2 > (int64_t)UINT32_MAX) return GQA_ERR_SHAPE;
  if ((int64_t)B * Hq > kMaxWorkgroups) return GQA_ERR_SHAPE;
  if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
  if (!group_ok(Hq / Hkv)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Rows the S tokens of one sequence attend together span at most T, or
// window + S - 1 with a window (token s's window ends S-1-s rows earlier).
int num_parts(int T, int window, int part_tokens, int S = 1) {
  const int64_t w = window > 0 ? (int64_t)window + S - 1 : (int64_t)T;
  const int64_t span = w < T ? w : T;
  return (int)((span + part_tokens - 1) / part_tokens);
}

// Split-K checks; B * Hkv * partitions is the attention pass's grid.
int check_split(int B, int Hkv, int T, int window, int part_tokens, int S = 1) {
  if (part_tokens < 1) return GQA_ERR_VALUE;
  if ((int64_t)T + part_tokens >= INT32_MAX) return GQA_ERR_SHAPE;
  if ((int64_t)B * Hkv * num_parts(T, window, part_tokens, S) > kMaxWorkgroups)
    return GQA_ERR_SHAPE;
  return GQA_OK;
}

// S query tokens per sequence: all G * S (token, head) rows of a KV head
// share one 16-column matrix tile.
int check_tokens(int S, int B, int Hq, int Hkv) {
  if (S < 1 || S > 16) return S < 1 ? GQA_ERR_SHAPE : GQA_ERR_UNSUPPORTED;
  if ((Hq / Hkv) * S > 16) return GQA_ERR_UNSUPPORTED;
  if ((int64_t)B * S * Hq > kMaxWorkgroups) return GQA_ERR_SHAPE;
  return GQA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A rotary table (host, D/2 finite non-negative frequencies, or NULL for no
// RoPE), its magnitude factor and its pair layout.
int check_rope(const double* inv_freq, double mscale, int layout, int D) {
  if (layout != GQA_ROPE_NEOX && layout != GQA_ROPE_INTERLEAVED) return GQA_ERR_VALUE;
  if (!(mscale > 0.0) || !isfinite(mscale)) return GQA_ERR_VALUE;
  if (inv_freq)
    for (int i = 0; i < D / 2; ++i)
      if (!(inv_freq[i] >= 0.0) || !isfinite(inv_freq[i])) return GQA_ERR_VALUE;
  return GQA_OK;
}

float softmax_qscale(float scale, int D) {
  const double s = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)D);
  return (float)(s * 1.4426950408889634);
}

}  // namespace

namespace gqa {

size_t step_lse_bytes(int B, int S, int Hq, int num_parts) {
  return align256((size_t)B * S * Hq * num_parts * sizeof(float));
}

int decode_step_args(const void* q, const void* k_new, const void* v_new,
                     gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                     const float* q_norm_w, const float* k_norm_w, float eps,
                     const double* inv_freq, double rope_mscale, int rope_layout,
                     const int32_t* pos, int S,
                     uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                     int window, float scale, int part_tokens,
                     void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                     int B, int Hq, int Hkv, int D, int T, KernelArgs* args) {
  if (!q || !k_cache || !v_cache || !lens || !out) return GQA_ERR_NULL;
  // the prologue inputs come all together or not at all
  const bool pro = pos != nullptr;
  if ((k_new != nullptr) != pro || (v_new != nullptr) != pro) return GQA_ERR_NULL;
  if ((q_norm_w == nullptr) != (k_norm_w == nullptr)) return GQA_ERR_NULL;
  if (!pro && (q_norm_w != nullptr || q_out != nullptr || inv_freq != nullptr))
    return GQA_ERR_NULL;
  int rc = check_shapes(B, Hq, Hkv, D, T);
  if (rc) return rc;
  if ((rc = check_tokens(S, B, Hq, Hkv))) return rc;
  if ((rc = check_split(B, Hkv, T, window, part_tokens, S))) return rc;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (q_bstride < (int64_t)S * Hq * D || kv_bstride < (int64_t)S * Hkv * D) return GQA_ERR_SHAPE;
  if (q_bstride > kMaxIndex / B || kv_bstride > kMaxIndex / B) return GQA_ERR_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return GQA_ERR_VALUE;
  if ((rc = check_rope(inv_freq, rope_mscale, rope_layout, D))) return rc;
  if (isnan(scale) || isinf(scale)) return GQA_ERR_VALUE;
  const uintptr_t ea = in_dtype == GQA_BF16 ? 2 : 4;
  // q rows are read as 16-byte vectors: the batch stride must keep that alignment
  if (!aligned(q, 16) || (q_bstride * (int64_t)ea) % 16 != 0 || !aligned(k_new, ea) ||
      !aligned(v_new, ea) || !aligned(q_norm_w, 16) || !aligned(k_norm_w, 4) ||
      !aligned(pos, 4) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(lens, 4) ||
      !aligned(out, 16) || !aligned(lse_out, 4) || !aligned(q_out, 16))
    return GQA_ERR_ALIGN;
  const int np = num_parts(T, window, part_tokens, S);
  // the merge reads one (sequence, KV head)'s partials -- rows of S tokens,
  // Hq apart -- with 32-bit offsets
  const int64_t team_rows = (int64_t)(S - 1) * Hq + Hq / Hkv;
  if (team_rows * np * D * 4 >= (INT64_C(1) << 31)) return GQA_ERR_SHAPE;
  KernelArgs& a = *args;
  a = KernelArgs{};
  a.q = q; a.q_bstride = q_bstride; a.in_bf16 = in_dtype == GQA_BF16;
  a.S = S; a.q_sstride = (int64_t)Hq * D;
  a.k_cache = k_cache; a.v_cache = v_cache; a.k_cache_w = k_cache; a.v_cache_w = v_cache;
  a.lens = lens; a.window = window; a.qscale = softmax_qscale(scale, D);
  a.part_tokens = part_tokens; a.num_parts = np;
  a.out = out; a.out_bf16 = out_dtype == GQA_BF16; a.lse_out = lse_out;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T = T;
  a.k_new = k_new; a.v_new = v_new; a.kv_bstride = kv_bstride;
  a.wq = q_norm_w; a.wk = k_norm_w; a.eps = eps;
  a.rope = pro && inv_freq != nullptr;
  a.rope_interleaved = rope_layout == GQA_ROPE_INTERLEAVED;
  a.rope_mscale = (float)rope_mscale;
  a.pos = pos; a.q_out = q_out;
  if (a.rope)
    for (int i = 0; i < D / 2; ++i) a.inv_freq_rev[i] = inv_freq[i] / 6.283185307179586476925;
  return GQA_OK;
}

}  // namespace gqa

extern "C" {

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "a size is < 1, inconsistent, or too large";
    case GQA_ERR_UNSUPPORTED: return "head dim, group size or dtype not supported";
    case GQA_ERR_WORKSPACE: return "split-K workspace too small";
    case GQA_ERR_LAUNCH: return "HIP kernel launch failed";
    case GQA_ERR_ALIGN: return "pointer not aligned as required";
    case GQA_ERR_VALUE: return "scalar argument out of range";
    case GQA_ERR_SCRATCH: return "shape too large for the static scratch of the no-allocation step";
    default: return "unknown status";
  }
}

int gqa_rope_table(int kind, int D, double theta, double factor, int orig_ctx,
                   double beta_fast, double beta_slow, double* inv_freq, double* mscale) {
  if (!inv_freq) return GQA_ERR_NULL;
  if (D < 2 || D % 2 != 0) return GQA_ERR_SHAPE;
  if (!(theta > 0.0) || !isfinite(theta)) return GQA_ERR_VALUE;
  if (kind < GQA_ROPE_DEFAULT || kind > GQA_ROPE_YARN) return GQA_ERR_VALUE;
  if (kind != GQA_ROPE_DEFAULT && (!(factor >= 1.0) || !isfinite(factor)))
    return GQA_ERR_VALUE;
  if (kind == GQA_ROPE_NTK && D < 4) return GQA_ERR_SHAPE;
  if (kind == GQA_ROPE_YARN &&
      (orig_ctx < 1 || !(beta_slow >= 0.0) || !(beta_fast > beta_slow) || !isfinite(beta_fast)))
    return GQA_ERR_VALUE;
  const double two_pi = 6.283185307179586476925;
  for (int i = 0; i < D / 2; ++i) {
    const double e = -2.0 * i / D;
    const double f = pow(theta, e);
    double out = f;
    switch (kind) {
      case GQA_ROPE_LINEAR:   // positions divided by the factor
        out = f / factor;
        break;
      case GQA_ROPE_NTK:      // base stretched so the lowest frequency drops by the factor
        out = pow(theta * pow(factor, D / (D - 2.0)), e);
        break;
      case GQA_ROPE_YARN: {   // blend by rotations over the original context
        const double r = (double)orig_ctx * f / two_pi;
        double gm = (r - beta_slow) / (beta_fast - beta_slow);
        gm = gm < 0.0 ? 0.0 : (gm > 1.0 ? 1.0 : gm);
        out = (1.0 - gm) * f / factor + gm * f;
        break;
      }
      default:
        break;
    }
    inv_freq[i] = out;
  }
  if (mscale) *mscale = kind == GQA_ROPE_YARN ? 1.0 + 0.1 * log(factor) : 1.0;
  return GQA_OK;
}

int gqa_qkv_prologue_ex(const void* q, const void* k_new, const void* v_new,
                        gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                        const float* q_norm_w, const float* k_norm_w, float eps,
                        const double* inv_freq, double rope_mscale, int rope_layout,
                        const int32_t* pos, int S, float* q_out,
                        uint16_t* k_cache, uint16_t* v_cache,
                        int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (!q || !k_new || !v_new || !pos || !q_out || !k_cache || !v_cache) return GQA_ERR_NULL;
  if ((q_norm_w == nullptr) != (k_norm_w == nullptr)) return GQA_ERR_NULL;
  int rc = check_shapes(B, Hq, Hkv, D, T);
  if (rc) return rc;
  if (!dtype_ok(in_dtype)) return GQA_ERR_UNSUPPORTED;
  if (S < 1 || (int64_t)B * S * (Hq + Hkv) > kMaxIndex / D) return GQA_ERR_SHAPE;
  // the prologue's grid: one row of workgroups per (sequence, token)
  if ((int64_t)B * S > kMaxWorkgroups || Hq + Hkv > 65535) return GQA_ERR_SHAPE;
  if (q_bstride < (int64_t)S * Hq * D || kv_bstride < (int64_t)S * Hkv * D) return GQA_ERR_SHAPE;
  if (q_bstride > kMaxIndex / B || kv_bstride > kMaxIndex / B) return GQA_ERR_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return GQA_ERR_VALUE;
  if ((rc = check_rope(inv_freq, rope_mscale, rope_layout, D))) return rc;
  const uintptr_t ea = in_dtype == GQA_BF16 ? 2 : 4;
  if (!aligned(q, ea) || !aligned(k_new, ea) || !aligned(v_new, ea) || !aligned(q_out, 4) ||
      !aligned(k_cache, 2) || !aligned(v_cache, 2) || !aligned(pos, 4) ||
      !aligned(q_norm_w, 4) || !aligned(k_norm_w, 4))
    return GQA_ERR_ALIGN;
  gqa::PrologueArgs a{};
  a.q = q; a.k_new = k_new; a.v_new = v_new; a.in_bf16 = in_dtype == GQA_BF16;
  a.q_bstride = q_bstride; a.kv_bstride = kv_bstride;
  a.q_norm_w = q_norm_w; a.k_norm_w = k_norm_w; a.eps = eps;
  a.rope = inv_freq != nullptr;
  a.rope_interleaved = rope_layout == GQA_ROPE_INTERLEAVED;
  a.rope_mscale = (float)rope_mscale;
  if (a.rope)
    for (int i = 0; i < D / 2; ++i) a.inv_freq_rev[i] = inv_freq[i] / 6.283185307179586476925;
  a.pos = pos; a.S = S; a.q_out = q_out; a.k_cache = k_cache; a.v_cache = v_cache;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T = T;
  return gqa::launch_prologue(a, stream);
}

int gqa_qkv_prologue(const void* q, const void* k_new, const void* v_new,
                     gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                     const float* q_norm_w, const float* k_norm_w, float eps,
                     double rope_theta, const int32_t* pos, float* q_out,
                     uint16_t* k_cache, uint16_t* v_cache,
                     int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (isnan(rope_theta) || isinf(rope_theta)) return GQA_ERR_VALUE;
  double table[gqa::kMaxHalfDim];
  const double* f = nullptr;
  if (rope_theta > 0.0 && (D == 64 || D == 128)) {
    gqa_rope_table(GQA_ROPE_DEFAULT, D, rope_theta, 1.0, 0, 0.0, 0.0, table, nullptr);
    f = table;
  }
  return gqa_qkv_prologue_ex(q, k_new, v_new, in_dtype, q_bstride, kv_bstride, q_norm_w,
                             k_norm_w, eps, f, 1.0, GQA_ROPE_NEOX, pos, 1, q_out, k_cache,
                             v_cache, B, Hq, Hkv, D, T, stream);
}

int gqa_attn_decode(const void* q, gqa_dtype_t q_dtype,
                    const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* lens, int window, float scale,
                    void* out, gqa_dtype_t out_dtype, float* lse_out,
                    int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  return gqa_attn_decode_multi(q, q_dtype, k_cache, v_cache, lens, 1, window, scale, out,
                               out_dtype, lse_out, B, Hq, Hkv, D, T, stream);
}

int gqa_attn_decode_multi(const void* q, gqa_dtype_t q_dtype,
                          const uint16_t* k_cache, const uint16_t* v_cache,
                          const int32_t* lens, int S, int window, float scale,
                          void* out, gqa_dtype_t out_dtype, float* lse_out,
                          int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !lens || !out) return GQA_ERR_NULL;
  int rc = check_shapes(B, Hq, Hkv, D, T);
  if (rc) return rc;
  if ((rc = check_tokens(S, B, Hq, Hkv))) return rc;
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (isnan(scale) || isinf(scale)) return GQA_ERR_VALUE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lens, 4) || !aligned(lse_out, 4))
    return GQA_ERR_ALIGN;
  gqa::KernelArgs a{};
  a.q = q; a.q_bstride = (int64_t)S * Hq * D; a.q_sstride = (int64_t)Hq * D; a.S = S;
  a.in_bf16 = q_dtype == GQA_BF16;
  a.k_cache = k_cache; a.v_cache = v_cache; a.lens = lens; a.window = window;
  a.qscale = softmax_qscale(scale, D);
  a.out = out; a.out_bf16 = out_dtype == GQA_BF16; a.lse_out = lse_out;
  a.num_parts = 1;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T = T;
  return gqa::launch_attn_final(a, stream);
}

int gqa_attn_prefill(const void* q, gqa_dtype_t q_dtype,
                     const uint16_t* k_cache, const uint16_t* v_cache,
                     const int32_t* lens, int S, int causal, int window, float scale,
                     void* out, gqa_dtype_t out_dtype, float* lse_out,
                     int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  return gqa_attn_prefill_split(q, q_dtype, k_cache, v_cache, lens, S, causal, window, scale, 1,
                                nullptr, 0, out, out_dtype, lse_out, B, Hq, Hkv, D, T, stream);
}

// Prefill key-split workspace: partial o [teams, splits, rows, D], then
// (256-byte aligned) partial lse [teams, splits, rows], then tickets
// [teams]; teams = B * Hkv * row blocks.
static int64_t prefill_teams(int B, int S, int Hq, int Hkv) {
  const int64_t rows = (int64_t)S * (Hq / Hkv);
  const int per = gqa::prefill_rows_per_block();
  return (int64_t)B * Hkv * ((rows + per - 1) / per);
}

// Point the key-split buffers of `a` (sizes and splits set) into `workspace`.
static void prefill_workspace_layout(gqa::PrefillArgs& a, void* workspace) {
  const size_t part =
      (size_t)a.B * a.Hkv * a.row_blocks * a.splits * gqa::prefill_rows_per_block();
  char* ws = static_cast<char*>(workspace);
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_lse = reinterpret_cast<float*>(ws + align256(part * a.D * sizeof(float)));
  a.ws_cnt = reinterpret_cast<uint32_t*>(ws + align256(part * a.D * sizeof(float)) +
                                         align256(part * sizeof(float)));
}

size_t gqa_attn_prefill_workspace_bytes(int B, int S, int Hq, int Hkv, int D, int splits) {
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || D < 1 || splits < 1 || Hq % Hkv != 0) return 0;
  if (splits == 1) return 0;
  const int64_t teams = prefill_teams(B, S, Hq, Hkv);
  const size_t part = (size_t)teams * splits * gqa::prefill_rows_per_block();
  return align256(part * D * sizeof(float)) + align256(part * sizeof(float)) +
         (size_t)teams * sizeof(uint32_t);
}

int gqa_attn_prefill_default_splits(int B, int S, int Hq, int Hkv) {
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 1;
  // Fewer row blocks than CUs: two splits.  With as many row blocks as CUs
  // (the fresh S = 1024 prefill) one split measured faster than two, and
  // three or four slower still: each split writes and the last reads back
  // a 64 KB partial, as much as its share of the keys.
  const int64_t wgs = prefill_teams(B, S, Hq, Hkv);
  return wgs < (int64_t)cus ? 2 : 1;
}

int gqa_attn_prefill_split(const void* q, gqa_dtype_t q_dtype,
                           const uint16_t* k_cache, const uint16_t* v_cache,
                           const int32_t* lens, int S, int causal, int window, float scale,
                           int splits, void* workspace, size_t workspace_bytes,
                           void* out, gqa_dtype_t out_dtype, float* lse_out,
                           int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !lens || !out) return GQA_ERR_NULL;
  int rc = check_shapes(B, Hq, Hkv, D, T);
  if (rc) return rc;
  if (S < 1) return GQA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return GQA_ERR_VALUE;
  if (splits < 1 || splits > 16) return GQA_ERR_VALUE;
  if (splits > 1 && !workspace) return GQA_ERR_NULL;
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (isnan(scale) || isinf(scale)) return GQA_ERR_VALUE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lens, 4) || !aligned(lse_out, 4) || !aligned(workspace, 256))
    return GQA_ERR_ALIGN;
  const int64_t rows = (int64_t)S * (Hq / Hkv);   // (token, head) rows per KV head
  if (rows > INT32_MAX / 2 || (int64_t)B * S * Hq > kMaxIndex / D) return GQA_ERR_SHAPE;
  const int per = gqa::prefill_rows_per_block();
  const int64_t row_blocks = (rows + per - 1) / per;
  if ((int64_t)B * Hkv * row_blocks * splits > kMaxWorkgroups) return GQA_ERR_SHAPE;
  if (splits > 1 &&
      workspace_bytes < gqa_attn_prefill_workspace_bytes(B, S, Hq, Hkv, D, splits))
    return GQA_ERR_WORKSPACE;
  gqa::PrefillArgs a{};
  a.q = q; a.q_bstride = (int64_t)S * Hq * D; a.in_bf16 = q_dtype == GQA_BF16;
  a.k_cache = k_cache; a.v_cache = v_cache; a.lens = lens;
  a.S = S; a.causal = causal; a.window = window;
  a.qscale = softmax_qscale(scale, D);
  a.out = out; a.out_bf16 = out_dtype == GQA_BF16; a.lse_out = lse_out;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T = T;
  a.row_blocks = (int)row_blocks;
  a.splits = splits;
  if (splits > 1) prefill_workspace_layout(a, workspace);
  return gqa::launch_attn_prefill(a, stream);
}

int gqa_prefill_step(const void* q, const void* k_new, const void* v_new,
                     gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                     const float* q_norm_w, const float* k_norm_w, float eps,
                     const double* inv_freq, double rope_mscale, int rope_layout,
                     const int32_t* pos, int S,
                     uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                     int causal, int window, float scale, int splits,
                     void* workspace, size_t workspace_bytes,
                     void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                     int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (!q || !k_new || !v_new || !pos || !k_cache || !v_cache || !lens || !out)
    return GQA_ERR_NULL;
  if ((q_norm_w == nullptr) != (k_norm_w == nullptr)) return GQA_ERR_NULL;
  int rc = check_shapes(B, Hq, Hkv, D, T);
  if (rc) return rc;
  if (S < 1) return GQA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return GQA_ERR_VALUE;
  if (splits < 1 || splits > 16) return GQA_ERR_VALUE;
  if (splits > 1 && !workspace) return GQA_ERR_NULL;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (isnan(scale) || isinf(scale)) return GQA_ERR_VALUE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return GQA_ERR_VALUE;
  if ((rc = check_rope(inv_freq, rope_mscale, rope_layout, D))) return rc;
  if (q_bstride < (int64_t)S * Hq * D || kv_bstride < (int64_t)S * Hkv * D) return GQA_ERR_SHAPE;
  if (q_bstride > kMaxIndex / B || kv_bstride > kMaxIndex / B) return GQA_ERR_SHAPE;
  if ((int64_t)B * S > kMaxWorkgroups) return GQA_ERR_SHAPE;
  const uintptr_t ea = in_dtype == GQA_BF16 ? 2 : 4;
  // q rows are read as 16-byte vectors: the batch stride keeps that alignment
  if (!aligned(q, 16) || (q_bstride * (int64_t)ea) % 16 != 0 || !aligned(k_new, ea) ||
      !aligned(v_new, ea) || !aligned(q_norm_w, 16) || !aligned(k_norm_w, 4) ||
      !aligned(pos, 4) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(lens, 4) || !aligned(out, 16) || !aligned(lse_out, 4) || !aligned(q_out, 16) ||
      !aligned(workspace, 256))
    return GQA_ERR_ALIGN;
  const int64_t rows = (int64_t)S * (Hq / Hkv);
  if (rows > INT32_MAX / 2 || (int64_t)B * S * Hq > kMaxIndex / D) return GQA_ERR_SHAPE;
  const int per = gqa::prefill_rows_per_block();
  const int64_t row_blocks = (rows + per - 1) / per;
  if ((int64_t)B * Hkv * row_blocks * splits > kMaxWorkgroups) return GQA_ERR_SHAPE;
  if (splits > 1 &&
      workspace_bytes < gqa_attn_prefill_workspace_bytes(B, S, Hq, Hkv, D, splits))
    return GQA_ERR_WORKSPACE;
  // 1: the K/V append of the S tokens (the prologue kernel on the K/V head
  // vectors only)
  gqa::PrologueArgs pa{};
  pa.q = q; pa.k_new = k_new; pa.v_new = v_new; pa.in_bf16 = in_dtype == GQA_BF16;
  pa.q_bstride = q_bstride; pa.kv_bstride = kv_bstride;
  pa.q_norm_w = q_norm_w; pa.k_norm_w = k_norm_w; pa.eps = eps;
  pa.rope = inv_freq != nullptr;
  pa.rope_interleaved = rope_layout == GQA_ROPE_INTERLEAVED;
  pa.rope_mscale = (float)rope_mscale;
  pa.pos = pos; pa.S = S; pa.q_out = nullptr; pa.k_cache = k_cache; pa.v_cache = v_cache;
  pa.B = B; pa.Hq = Hq; pa.Hkv = Hkv; pa.D = D; pa.T = T; pa.kv_only = 1;
  if (pa.rope)
    for (int i = 0; i < D / 2; ++i) pa.inv_freq_rev[i] = inv_freq[i] / 6.283185307179586476925;
  if ((rc = gqa::launch_prologue(pa, stream))) return rc;
  // 2: the attention, which normalises and rotates q itself
  gqa::PrefillArgs a{};
  a.q = q; a.q_bstride = q_bstride; a.in_bf16 = in_dtype == GQA_BF16;
  a.k_cache = k_cache; a.v_cache = v_cache; a.lens = lens;
  a.S = S; a.causal = causal; a.window = window;
  a.qscale = softmax_qscale(scale, D);
  a.out = out; a.out_bf16 = out_dtype == GQA_BF16; a.lse_out = lse_out;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T = T;
  a.row_blocks = (int)row_blocks;
  a.splits = splits;
  if (splits > 1) prefill_workspace_layout(a, workspace);
  a.pro = 1;
  a.wq = q_norm_w; a.eps = eps;
  a.rope = pa.rope; a.rope_interleaved = pa.rope_interleaved; a.rope_mscale = pa.rope_mscale;
  a.pos = pos; a.q_out = q_out;
  for (int i = 0; i < D / 2; ++i) a.inv_freq_rev[i] = pa.inv_freq_rev[i];
  return gqa::launch_attn_prefill(a, stream);
}

int gqa_qkv_gemv(const uint16_t* x, int64_t x_stride, const uint16_t* w, int64_t w_stride,
                 void* y, gqa_dtype_t y_dtype, int64_t y_stride, int M, int N, int K,
                 hipStream_t stream) {
  if (!x || !w || !y) return GQA_ERR_NULL;
  if (M < 1 || N < 1 || K < 1) return GQA_ERR_SHAPE;
  if (M > 16 || K % 128 != 0 || !dtype_ok(y_dtype)) return GQA_ERR_UNSUPPORTED;
  if (x_stride < K || w_stride < K || y_stride < N) return GQA_ERR_SHAPE;
  if (x_stride % 8 != 0 || w_stride % 8 != 0) return GQA_ERR_ALIGN;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, y_dtype == GQA_BF16 ? 2 : 4))
    return GQA_ERR_ALIGN;
  // a workgroup addresses its share of up to 64 weight rows with 32-bit
  // byte offsets
  if ((63 * w_stride + K) * 2 > (int64_t)UINT32_MAX) return GQA_ERR_SHAPE;
  if ((int64_t)N > kMaxWorkgroups * 16 || (int64_t)M * y_stride > kMaxIndex ||
      (int64_t)N * w_stride > kMaxIndex || (int64_t)M * x_stride > kMaxIndex)
    return GQA_ERR_SHAPE;
  gqa::GemvArgs a{};
  a.x = x; a.x_stride = x_stride; a.w = w; a.w_stride = w_stride;
  a.y = y; a.y_stride = y_stride; a.out_bf16 = y_dtype == GQA_BF16;
  a.M = M; a.N = N; a.K = K;
  return gqa::launch_qkv_gemv(a, stream);
}

int gqa_probe_stream_read(const void* buf, size_t bytes, int workgroups, int threads, int unroll,
                          uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return GQA_ERR_NULL;
  if (bytes < 16 || bytes > ((size_t)1 << 31) || workgroups < 1 || workgroups > 65536)
    return GQA_ERR_SHAPE;
  if (bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4)) return GQA_ERR_ALIGN;
  if (threads < 64 || threads > 1024 || threads % 64 != 0) return GQA_ERR_VALUE;
  if (unroll != 4 && unroll != 8 && unroll != 16) return GQA_ERR_UNSUPPORTED;
  return gqa::launch_stream_read(buf, (uint32_t)bytes, workgroups, threads, unroll, sink, stream);
}

int gqa_num_partitions(int T, int window, int part_tokens) {
  if (T < 1 || part_tokens < 1) return 0;
  return num_parts(T, window, part_tokens);
}

static size_t lse_bytes(size_t rows, int np) { return rows * np * sizeof(float); }

size_t gqa_splitk_workspace_bytes(int B, int Hq, int D, int T, int window, int part_tokens) {
  return gqa_splitk_multi_workspace_bytes(B, 1, Hq, D, T, window, part_tokens);
}

size_t gqa_splitk_multi_workspace_bytes(int B, int S, int Hq, int D, int T, int window,
                                        int part_tokens) {
  if (B < 1 || S < 1 || Hq < 1 || D < 1 || T < 1 || part_tokens < 1) return 0;
  const int np = num_parts(T, window, part_tokens, S);
  const size_t rows = (size_t)B * S * Hq;
  return align256(lse_bytes(rows, np)) + (size_t)rows * np * D * sizeof(float);
}

int gqa_attn_decode_splitk(const void* q, gqa_dtype_t q_dtype,
                           const uint16_t* k_cache, const uint16_t* v_cache,
                           const int32_t* lens, int window, float scale,
                           int part_tokens, void* workspace, size_t workspace_bytes,
                           int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  return gqa_attn_decode_splitk_multi(q, q_dtype, k_cache, v_cache, lens, 1, window, scale,
                                      part_tokens, workspace, workspace_bytes, B, Hq, Hkv, D,
                                      T, stream);
}

int gqa_attn_decode_splitk_multi(const void* q, gqa_dtype_t q_dtype,
                                 const uint16_t* k_cache, const uint16_t* v_cache,
                                 const int32_t* lens, int S, int window, float scale,
                                 int part_tokens, void* workspace, size_t workspace_bytes,
                                 int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !lens || !workspace) return GQA_ERR_NULL;
  int rc = check_shapes(B, Hq, Hkv, D, T);
  if (rc) return rc;
  if ((rc = check_tokens(S, B, Hq, Hkv))) return rc;
  if ((rc = check_split(B, Hkv, T, window, part_tokens, S))) return rc;
  if (!dtype_ok(q_dtype)) return GQA_ERR_UNSUPPORTED;
  if (isnan(scale) || isinf(scale)) return GQA_ERR_VALUE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(lens, 4) || !aligned(workspace, 256))
    return GQA_ERR_ALIGN;
  if (workspace_bytes < gqa_splitk_multi_workspace_bytes(B, S, Hq, D, T, window, part_tokens))
    return GQA_ERR_WORKSPACE;
  const int np = num_parts(T, window, part_tokens, S);
  gqa::KernelArgs a{};
  a.q = q; a.q_bstride = (int64_t)S * Hq * D; a.q_sstride = (int64_t)Hq * D; a.S = S;
  a.in_bf16 = q_dtype == GQA_BF16;
  a.k_cache = k_cache; a.v_cache = v_cache; a.lens = lens; a.window = window;
  a.qscale = softmax_qscale(scale, D);
  a.part_tokens = part_tokens; a.num_parts = np;
  a.ws_lse = static_cast<float*>(workspace);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    align256(lse_bytes((size_t)B * S * Hq, np)));
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.T = T;
  return gqa::launch_attn_split(a, stream);
}

int gqa_attn_decode_merge(const void* workspace, size_t workspace_bytes,
                          int window, int part_tokens,
                          void* out, gqa_dtype_t out_dtype, float* lse_out,
                          int B, int Hq, int D, int T, hipStream_t stream) {
  return gqa_attn_decode_merge_multi(workspace, workspace_bytes, 1, window, part_tokens, out,
                                     out_dtype, lse_out, B, Hq, D, T, stream);
}

int gqa_attn_decode_merge_multi(const void* workspace, size_t workspace_bytes, int S,
                                int window, int part_tokens,
                                void* out, gqa_dtype_t out_dtype, float* lse_out,
                                int B, int Hq, int D, int T, hipStream_t stream) {
  if (!workspace || !out) return GQA_ERR_NULL;
  if (B < 1 || Hq < 1 || T < 1 || S < 1) return GQA_ERR_SHAPE;
  if ((int64_t)B * S * Hq > kMaxWorkgroups) return GQA_ERR_SHAPE;
  if (S > 16) return GQA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
  int rc = check_split(1, 1, T, window, part_tokens, S);
  if (rc) return rc;
  if (!dtype_ok(out_dtype)) return GQA_ERR_UNSUPPORTED;
  if (!aligned(workspace, 256) || !aligned(out, 16) || !aligned(lse_out, 4)) return GQA_ERR_ALIGN;
  if (workspace_bytes < gqa_splitk_multi_workspace_bytes(B, S, Hq, D, T, window, part_tokens))
    return GQA_ERR_WORKSPACE;
  const int np = num_parts(T, window, part_tokens, S);
  gqa::MergeArgs a{};
  a.ws_lse = static_cast<const float*>(workspace);
  a.ws_o = reinterpret_cast<const float*>(static_cast<const char*>(workspace) +
                                          align256(lse_bytes((size_t)B * S * Hq, np)));
  a.num_parts = np; a.out = out; a.out_bf16 = out_dtype == GQA_BF16; a.lse_out = lse_out;
  a.B = B * S; a.Hq = Hq; a.D = D;       // the merge works on rows of [B*S, Hq]
  return gqa::launch_merge(a, stream);
}

size_t gqa_decode_step_workspace_bytes(int B, int Hq, int Hkv, int D, int T, int window,
                                       int part_tokens) {
  return gqa_decode_step_multi_workspace_bytes(B, 1, Hq, Hkv, D, T, window, part_tokens);
}

size_t gqa_decode_step_multi_workspace_bytes(int B, int S, int Hq, int Hkv, int D, int T,
                                             int window, int part_tokens) {
  const size_t base = gqa_splitk_multi_workspace_bytes(B, S, Hq, D, T, window, part_tokens);
  if (base == 0 || Hkv < 1) return 0;
  return align256(base) + (size_t)B * Hkv * sizeof(uint32_t);
}

int gqa_decode_step_ex(const void* q, const void* k_new, const void* v_new,
                       gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                       const float* q_norm_w, const float* k_norm_w, float eps,
                       const double* inv_freq, double rope_mscale, int rope_layout,
                       const int32_t* pos,
                       uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                       int window, float scale, int part_tokens,
                       void* workspace, size_t workspace_bytes,
                       void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                       int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  return gqa_decode_step_multi(q, k_new, v_new, in_dtype, q_bstride, kv_bstride, q_norm_w,
                               k_norm_w, eps, inv_freq, rope_mscale, rope_layout, pos, 1,
                               k_cache, v_cache, lens, window, scale, part_tokens, workspace,
                               workspace_bytes, out, out_dtype, lse_out, q_out, B, Hq, Hkv, D,
                               T, stream);
}

int gqa_decode_step_multi(const void* q, const void* k_new, const void* v_new,
                          gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                          const float* q_norm_w, const float* k_norm_w, float eps,
                          const double* inv_freq, double rope_mscale, int rope_layout,
                          const int32_t* pos, int S,
                          uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                          int window, float scale, int part_tokens,
                          void* workspace, size_t workspace_bytes,
                          void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                          int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (!workspace) return GQA_ERR_NULL;
  gqa::KernelArgs a{};
  int rc = gqa::decode_step_args(q, k_new, v_new, in_dtype, q_bstride, kv_bstride, q_norm_w,
                                 k_norm_w, eps, inv_freq, rope_mscale, rope_layout, pos, S,
                                 k_cache, v_cache, lens, window, scale, part_tokens, out,
                                 out_dtype, lse_out, q_out, B, Hq, Hkv, D, T, &a);
  if (rc) return rc;
  if (!aligned(workspace, 256)) return GQA_ERR_ALIGN;
  if (workspace_bytes <
      gqa_decode_step_multi_workspace_bytes(B, S, Hq, Hkv, D, T, window, part_tokens))
    return GQA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(ws);
  a.ws_o = reinterpret_cast<float*>(ws + gqa::step_lse_bytes(B, S, Hq, a.num_parts));
  a.ws_cnt = reinterpret_cast<uint32_t*>(
      ws + align256(gqa_splitk_multi_workspace_bytes(B, S, Hq, D, T, window, part_tokens)));
  return gqa::launch_decode_step(a, stream);
}

int gqa_decode_step(const void* q, const void* k_new, const void* v_new, gqa_dtype_t in_dtype,
                    int64_t q_bstride, int64_t kv_bstride,
                    const float* q_norm_w, const float* k_norm_w, float eps,
                    double rope_theta, const int32_t* pos,
                    uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                    int window, float scale, int part_tokens,
                    void* workspace, size_t workspace_bytes,
                    void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                    int B, int Hq, int Hkv, int D, int T, hipStream_t stream) {
  if (isnan(rope_theta) || isinf(rope_theta)) return GQA_ERR_VALUE;
  double table[gqa::kMaxHalfDim];
  const double* f = nullptr;
  if (pos != nullptr && rope_theta > 0.0 && (D == 64 || D == 128)) {
    gqa_rope_table(GQA_ROPE_DEFAULT, D, rope_theta, 1.0, 0, 0.0, 0.0, table, nullptr);
    f = table;
  }
  return gqa_decode_step_ex(q, k_new, v_new, in_dtype, q_bstride, kv_bstride, q_norm_w,
                            k_norm_w, eps, f, 1.0, GQA_ROPE_NEOX, pos, k_cache, v_cache, lens,
                            window, scale, part_tokens, workspace, workspace_bytes, out,
                            out_dtype, lse_out, q_out, B, Hq, Hkv, D, T, stream);
}

}  // extern "C"
