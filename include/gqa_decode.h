/*
 * gqa_decode.h -- C ABI of an MI355X (gfx950) library for single-token
 * grouped-query-attention decode over a bf16 KV cache.
 *
 * The operations are the ones two pages describe:
 *   - fusedtok 1.0.1 README, "Operators" table, row attention_decode:
 *     single-token causal attention with GQA over a contiguous KV cache,
 *     online softmax, flash-decoding split over long caches, per-sequence
 *     lengths; "Usage": attention_decode(q_heads [B,Hq,D],
 *     k_cache/v_cache [B,Hkv,T,D], lens int32 [B]), rope(..., pos_offset,
 *     neox=True), rmsnorm(x, w, eps); zero-copy device buffers, stream
 *     ordered, no host synchronisation; bf16 tensors computed in float32
 *     and converted at load and store.
 *   - cutileGPT README, feature list: fused QK-Norm + RoPE + KV-cache
 *     writes; MHA/GQA and sliding-window attention; "Why tiles" figure:
 *     RMSNorm rstd = 1/sqrt(sum(x*x)/N + eps), y = x*rstd*w.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer, except where noted.  The
 *     caller allocates and frees every buffer, including the split-K
 *     workspace.  The library never allocates, frees, synchronises, or reads
 *     device memory from the host; each call only enqueues kernels on
 *     `stream` (0 = the null stream), so calls are asynchronous and may be
 *     captured in a HIP graph.
 *   - bf16 values are passed as their uint16 bit patterns.  Arithmetic is
 *     float32; bf16 stores round to nearest, ties to even.
 *   - Layouts are dense and row-major: q [B,Hq,D], caches [B,Hkv,T,D]
 *     (element (b,g,t,d) at ((b*Hkv+g)*T+t)*D+d), outputs [B,Hq,D],
 *     lse [B,Hq].  Query head h uses KV head h / (Hq/Hkv).
 *   - Outputs must not alias inputs.
 *   - Supported: D in {64, 128}; G = Hq/Hkv in {1, 2, 4, 8, 16}; one
 *     (sequence, KV head) slab of the cache below 4 GiB (T * D * 2 bytes
 *     < 2^32, i.e. T < 16,777,216 rows at D = 128), else GQA_ERR_SHAPE.
 *   - Errors: arguments are checked on the host before anything is
 *     enqueued; on error the call returns a negative status and enqueues
 *     nothing.  A launch failure reported by HIP returns GQA_ERR_LAUNCH.
 *   - Device values outside the contract are handled safely, not trapped:
 *     lens[b] is clamped to [0, T]; a sequence with no attended rows
 *     produces out = 0 and lse = -inf; a pos[b] outside [0, T) still
 *     produces q_out but writes nothing to the cache.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype_t;

enum {
  GQA_OK = 0,
  GQA_ERR_NULL = -1,        /* a required pointer is NULL                  */
  GQA_ERR_SHAPE = -2,       /* a size is < 1, inconsistent, or overflows   */
  GQA_ERR_UNSUPPORTED = -3, /* head dim, group size or dtype not built     */
  GQA_ERR_WORKSPACE = -4,   /* split-K workspace too small                 */
  GQA_ERR_LAUNCH = -5,      /* HIP reported an error for the launch        */
  GQA_ERR_ALIGN = -6,       /* a pointer lacks the required alignment      */
  GQA_ERR_VALUE = -7,       /* a scalar argument is out of its range       */
  GQA_ERR_SCRATCH = -8      /* the shape needs more than the library's
                               static scratch (gqa_decode_step_noalloc)     */
};

/*
 * Fused prologue for one decode step (cutileGPT: fused QK-Norm + RoPE +
 * KV-cache writes; fusedtok: RMSNorm, RoPE NeoX layout with a position
 * offset).  For every sequence b:
 *   each query head:  q_out[b,h,:] = RoPE_pos[b]( RMSNorm(q[b,h,:], q_norm_w) )
 *   each KV head g:   k_cache[b,g,pos[b],:] = bf16( RoPE_pos[b]( RMSNorm(k_new[b,g,:], k_norm_w) ) )
 *                     v_cache[b,g,pos[b],:] = bf16( v_new[b,g,:] )
 * RMSNorm: y = x * w / sqrt(mean(x^2) + eps).  RoPE (NeoX, rotate-half):
 * element i < D/2 pairs with i + D/2 and both rotate by pos * theta^(-2i/D);
 * angles are formed and reduced in float64.
 *
 *   q, k_new, v_new  [B,Hq,D] / [B,Hkv,D] / [B,Hkv,D] in `in_dtype`
 *                    (GQA_F32 or GQA_BF16).  Heads are contiguous inside a
 *                    batch row; consecutive batch rows are `q_bstride` /
 *                    `kv_bstride` elements apart (>= Hq*D / Hkv*D), so one
 *                    packed QKV projection output can be passed directly.
 *   q_norm_w, k_norm_w  float32 [D] each, or both NULL for no QK-norm.
 *   eps              >= 0, added to the mean of squares.
 *   rope_theta       base of the rotary schedule; <= 0 disables RoPE.
 *   pos              int32 [B]: RoPE position of the new token, which is
 *                    also the cache row it is written to.
 *   q_out            float32 [B,Hq,D] (dense), the rotated queries.
 *   k_cache, v_cache bf16 [B,Hkv,T,D]; only rows pos[b] are written.
 */
int gqa_qkv_prologue(const void* q, const void* k_new, const void* v_new,
                     gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                     const float* q_norm_w, const float* k_norm_w, float eps,
                     double rope_theta, const int32_t* pos, float* q_out,
                     uint16_t* k_cache, uint16_t* v_cache,
                     int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/* RoPE pair layouts (fusedtok 1.0.1 README, Operators row RoPE: interleaved
 * and NeoX layouts). */
enum {
  GQA_ROPE_NEOX = 0,         /* pair i = elements (i, i + D/2), "rotate half" */
  GQA_ROPE_INTERLEAVED = 1   /* pair i = elements (2i, 2i + 1)                */
};

/* Rotary frequency schemes (PyGPUkit 0.2.18 page, Positional Encoding
 * Operations: NTK-aware RoPE, YaRN dimension-wise interpolation, linear
 * position interpolation; the page names them without formulas). */
enum {
  GQA_ROPE_DEFAULT = 0,  /* f_i = theta^(-2i/D)                                */
  GQA_ROPE_LINEAR = 1,   /* f_i / factor (positions divided by the factor)     */
  GQA_ROPE_NTK = 2,      /* base theta * factor^(D/(D-2)): f_0 unchanged,      */
                         /* f_{D/2-1} divided by exactly the factor            */
  GQA_ROPE_YARN = 3      /* r_i = orig_ctx f_i / (2 pi) rotations over the     */
                         /* original context; g_i = clamp((r_i - beta_slow) /  */
                         /* (beta_fast - beta_slow), 0, 1); f_i' = (1 - g_i)   */
                         /* f_i / factor + g_i f_i; mscale = 1 + 0.1 ln factor */
};

/*
 * Host helper (no GPU work): fill inv_freq[D/2] (host memory, radians per
 * position of rotary pair i) for scheme `kind` and, when `mscale` is not
 * NULL, the magnitude factor the scheme applies to the rotated q and k (1
 * except YaRN).  theta > 0; factor >= 1 (ignored by GQA_ROPE_DEFAULT);
 * orig_ctx >= 1 and beta_fast > beta_slow >= 0 for YaRN (orig_ctx and the
 * betas are ignored otherwise); D even (>= 4 for NTK).  Returns GQA_OK or
 * GQA_ERR_NULL / GQA_ERR_SHAPE / GQA_ERR_VALUE; nothing is written on error.
 */
int gqa_rope_table(int kind, int D, double theta, double factor, int orig_ctx,
                   double beta_fast, double beta_slow, double* inv_freq, double* mscale);

/*
 * gqa_qkv_prologue with an explicit rotary table instead of rope_theta, and
 * S >= 1 new tokens per sequence:
 *   inv_freq     HOST pointer to D/2 float64 frequencies (radians per
 *                position, finite, >= 0), read during the call; NULL for no
 *                RoPE.  Pair i of the chosen layout rotates by
 *                position * inv_freq[i] (angle and sincos in float64).
 *   rope_mscale  > 0: both rotated vectors (q and k) are multiplied by it
 *                (1 for a plain rotation; YaRN's attention temperature).
 *   rope_layout  GQA_ROPE_NEOX or GQA_ROPE_INTERLEAVED.
 *   S            tokens per sequence: q is [B,S,Hq,D] and k_new, v_new are
 *                [B,S,Hkv,D] (batch rows q_bstride >= S*Hq*D and kv_bstride
 *                >= S*Hkv*D elements apart, tokens dense inside a row);
 *                token s of sequence b sits at position pos[b] + s and is
 *                written to cache row pos[b] + s; q_out is [B,S,Hq,D].
 * Every other argument, and every error, as for gqa_qkv_prologue.
 * gqa_qkv_prologue(theta) is this call with the GQA_ROPE_DEFAULT table,
 * mscale 1, the NeoX layout and S = 1.
 */
int gqa_qkv_prologue_ex(const void* q, const void* k_new, const void* v_new,
                        gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                        const float* q_norm_w, const float* k_norm_w, float eps,
                        const double* inv_freq, double rope_mscale, int rope_layout,
                        const int32_t* pos, int S, float* q_out,
                        uint16_t* k_cache, uint16_t* v_cache,
                        int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * Single-token GQA decode attention, one pass over the cache per KV head
 * (fusedtok attention_decode; cutileGPT sliding-window attention).
 * For sequence b let n = clamp(lens[b], 0, T) and lo = max(0, n - window)
 * when window > 0, else 0.  For every query head h (KV head g = h/(Hq/Hkv)):
 *   s_j = scale * <q[b,h,:], K[b,g,j,:]>   for j in [lo, n)
 *   out[b,h,:] = sum_j softmax(s)_j V[b,g,j,:];  lse[b,h] = log sum_j exp(s_j)
 *
 *   q        [B,Hq,D] in q_dtype (GQA_F32 or GQA_BF16), 16-byte aligned.
 *   k_cache, v_cache  bf16 [B,Hkv,T,D], 16-byte aligned.
 *   lens     int32 [B]: rows [0, lens[b]) are valid.
 *   window   <= 0: attend to all valid rows; > 0: only the last `window`.
 *   scale    softmax scale; <= 0 selects 1/sqrt(D).
 *   out      [B,Hq,D] in out_dtype (GQA_F32 or GQA_BF16), 16-byte aligned.
 *   lse_out  float32 [B,Hq] natural-log log-sum-exp of the scores, or NULL.
 * One workgroup per (sequence, KV head) streams the rows; for long caches
 * use the split-K pair below.
 */
int gqa_attn_decode(const void* q, gqa_dtype_t q_dtype,
                    const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* lens, int window, float scale,
                    void* out, gqa_dtype_t out_dtype, float* lse_out,
                    int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * Flash-decoding split (fusedtok attention_decode: "flash-decoding split
 * over long caches").  The attended rows [lo, n) of each (sequence, KV head)
 * are cut into partitions J_k = [lo + k*P, min(lo + (k+1)*P, n)),
 * k < num_parts, P = part_tokens.  num_parts depends on host-known sizes
 * only: ceil(min(T, window > 0 ? window : T) / P).
 */
int gqa_num_partitions(int T, int window, int part_tokens);

/*
 * Bytes of workspace gqa_attn_decode_splitk needs (0 for invalid sizes).
 * Layout, with NP = num_parts:
 *   offset 0:                 lse_k float32 [B,Hq,NP]   natural-log LSE of
 *                             partition k, -inf for an empty partition
 *   offset align256(4*B*Hq*NP): o_k float32 [B,Hq,NP,D] softmax-normalised
 *                             partition output (undefined where lse_k=-inf)
 */
size_t gqa_splitk_workspace_bytes(int B, int Hq, int D, int T, int window,
                                  int part_tokens);

/*
 * Partition pass: one workgroup per (partition, KV head, sequence) writes
 * (o_k, lse_k) for the G query heads of its KV head into `workspace`
 * (256-byte aligned, at least gqa_splitk_workspace_bytes bytes).  Every
 * partition slot is written, empty ones with lse_k = -inf.  Other
 * arguments as for gqa_attn_decode.
 */
int gqa_attn_decode_splitk(const void* q, gqa_dtype_t q_dtype,
                           const uint16_t* k_cache, const uint16_t* v_cache,
                           const int32_t* lens, int window, float scale,
                           int part_tokens, void* workspace, size_t workspace_bytes,
                           int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * Log-sum-exp merge of the partitions written by gqa_attn_decode_splitk
 * with the same (B, Hq, D, T, window, part_tokens):
 *   M = max_k lse_k;  w_k = exp(lse_k - M);
 *   out = sum_k w_k o_k / sum_k w_k;  lse = M + log sum_k w_k
 * in ascending k, so results are bit-identical run to run.  All partitions
 * empty: out = 0, lse = -inf.
 */
int gqa_attn_decode_merge(const void* workspace, size_t workspace_bytes,
                          int window, int part_tokens,
                          void* out, gqa_dtype_t out_dtype, float* lse_out,
                          int B, int Hq, int D, int T, hipStream_t stream);

/*
 * The whole decode step in one launch (cutileGPT README: fused QK-Norm +
 * RoPE + KV-cache writes; fusedtok 1.0.1 README: attention_decode with the
 * flash-decoding split): the effect of gqa_qkv_prologue followed by
 * gqa_attn_decode_splitk and gqa_attn_decode_merge, with q_out optional.
 * Each workgroup -- one partition of a (sequence, KV head), or two
 * consecutive ones for long contexts -- rotates the new query itself and
 * writes one partial (o, lse) for the rows it attends; the last workgroup of
 * each (sequence, KV head) to finish merges the partials in a fixed order,
 * so reruns are bit-identical.  The workgroup whose partition attends row
 * pos[b] computes the appended K/V row and uses it in place of reading that
 * row; partition 0 writes it to the cache.  Rotary angles are reduced in
 * float64 (a host-computed theta^(-2i/D) table) before a float32 sincos.
 *
 * Arguments are those of the three calls it replaces, plus:
 *   workspace  256-byte aligned, gqa_decode_step_workspace_bytes() bytes:
 *              the split-K layout above, then (at the next 256-byte
 *              boundary) uint32 [B,Hkv] arrival tickets.  The tickets must be
 *              zero before the first call (e.g. a zero-filled allocation);
 *              every call that completes leaves them zero again.  Calls that
 *              share a workspace must not overlap in time.
 *   q          16-byte aligned and q_bstride * element size a multiple of 16.
 *   q_out      float32 [B,Hq,D] rotated queries, or NULL.
 * One (sequence, KV head)'s partials, (Hq/Hkv) * partitions * D * 4 bytes,
 * must stay below 2 GiB (else GQA_ERR_SHAPE; only reached with very small
 * part_tokens).
 * With pos, k_new and v_new all NULL (and no norm weights, no q_out) the
 * prologue is skipped: q [B,Hq,D] in in_dtype is attended as given and the
 * cache is only read -- the split-K pass and the merge in one launch.
 */
size_t gqa_decode_step_workspace_bytes(int B, int Hq, int Hkv, int D, int T, int window,
                                       int part_tokens);
int gqa_decode_step(const void* q, const void* k_new, const void* v_new, gqa_dtype_t in_dtype,
                    int64_t q_bstride, int64_t kv_bstride,
                    const float* q_norm_w, const float* k_norm_w, float eps,
                    double rope_theta, const int32_t* pos,
                    uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                    int window, float scale, int part_tokens,
                    void* workspace, size_t workspace_bytes,
                    void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                    int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * gqa_decode_step with an explicit rotary table, magnitude factor and pair
 * layout (arguments and errors as for gqa_qkv_prologue_ex; inv_freq must be
 * NULL when the prologue is skipped).  gqa_decode_step(theta) is this call
 * with the GQA_ROPE_DEFAULT table, mscale 1 and the NeoX layout.
 */
int gqa_decode_step_ex(const void* q, const void* k_new, const void* v_new,
                       gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                       const float* q_norm_w, const float* k_norm_w, float eps,
                       const double* inv_freq, double rope_mscale, int rope_layout,
                       const int32_t* pos,
                       uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                       int window, float scale, int part_tokens,
                       void* workspace, size_t workspace_bytes,
                       void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                       int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * Multi-token decode: S >= 1 query tokens per sequence (e.g. draft tokens
 * being verified), causal among themselves, over the same cache.  The
 * fusedtok README's attention_prefill attends S query rows causally; here
 * the rows sit at the end of a cache that already holds them:
 *   token s of sequence b attends rows [lo_s, n_s) with
 *   n_s = clamp(lens[b] - (S-1-s), 0, T) and lo_s = max(0, n_s - window)
 *   (or 0 without a window), so the last token sees lens[b] rows.
 * q, out [B,S,Hq,D] dense, lse_out [B,S,Hq]; every other argument as for
 * the single-token call (which is this call with S = 1).  G = Hq/Hkv times
 * S must be at most 16 (all (token, head) rows of a KV head share each
 * cache row read), else GQA_ERR_UNSUPPORTED.
 * The split-K variant partitions the union of the tokens' rows (at most T,
 * or window + S - 1 rows) and its workspace holds [B,S,Hq] rows of
 * partials; gqa_attn_decode_merge_multi merges them.
 */
int gqa_attn_decode_multi(const void* q, gqa_dtype_t q_dtype,
                          const uint16_t* k_cache, const uint16_t* v_cache,
                          const int32_t* lens, int S, int window, float scale,
                          void* out, gqa_dtype_t out_dtype, float* lse_out,
                          int B, int Hq, int Hkv, int D, int T, hipStream_t stream);
size_t gqa_splitk_multi_workspace_bytes(int B, int S, int Hq, int D, int T, int window,
                                        int part_tokens);
int gqa_attn_decode_splitk_multi(const void* q, gqa_dtype_t q_dtype,
                                 const uint16_t* k_cache, const uint16_t* v_cache,
                                 const int32_t* lens, int S, int window, float scale,
                                 int part_tokens, void* workspace, size_t workspace_bytes,
                                 int B, int Hq, int Hkv, int D, int T, hipStream_t stream);
int gqa_attn_decode_merge_multi(const void* workspace, size_t workspace_bytes, int S,
                                int window, int part_tokens,
                                void* out, gqa_dtype_t out_dtype, float* lse_out,
                                int B, int Hq, int D, int T, hipStream_t stream);

/*
 * The whole multi-token step in one launch: the effect of
 * gqa_qkv_prologue_ex over S tokens followed by gqa_attn_decode_splitk_multi
 * and gqa_attn_decode_merge_multi, as gqa_decode_step_ex is for one token
 * (which is this call with S = 1).  Token s of sequence b is rotated at
 * position pos[b] + s and appended at cache row pos[b] + s (rows outside
 * [0, T) are not written); the attended rows are those of
 * gqa_attn_decode_multi.  Every workgroup whose partition attends one of the
 * new rows computes it and uses it in place of reading it; partition 0
 * writes them to the cache.
 *   q       [B,S,Hq,D] in in_dtype: sequences q_bstride >= S*Hq*D elements
 *           apart, tokens Hq*D apart, heads dense.
 *   k_new, v_new  [B,S,Hkv,D]: sequences kv_bstride >= S*Hkv*D apart,
 *           tokens Hkv*D apart.
 *   out     [B,S,Hq,D]; lse_out [B,S,Hq] or NULL; q_out float32 [B,S,Hq,D]
 *           or NULL.
 *   workspace  gqa_decode_step_multi_workspace_bytes() bytes, 256-byte
 *           aligned: the layout of gqa_splitk_multi_workspace_bytes, then
 *           (at the next 256-byte boundary) the uint32 [B,Hkv] tickets, zero
 *           before the first call and left zero by every call that completes.
 * G * S <= 16 (else GQA_ERR_UNSUPPORTED); the partials of one (sequence, KV
 * head), ((S-1)*Hq + G) * partitions * D * 4 bytes, below 2 GiB (else
 * GQA_ERR_SHAPE).  Other arguments and errors as for gqa_decode_step_ex.
 */
size_t gqa_decode_step_multi_workspace_bytes(int B, int S, int Hq, int Hkv, int D, int T,
                                             int window, int part_tokens);
int gqa_decode_step_multi(const void* q, const void* k_new, const void* v_new,
                          gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                          const float* q_norm_w, const float* k_norm_w, float eps,
                          const double* inv_freq, double rope_mscale, int rope_layout,
                          const int32_t* pos, int S,
                          uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                          int window, float scale, int part_tokens,
                          void* workspace, size_t workspace_bytes,
                          void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                          int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * Prefill: attention of S query tokens per sequence over the cache, causal
 * or bidirectional (fusedtok README, "Operators" row attention_prefill),
 * with the GQA head mapping, lengths and window of attention_decode.  The S
 * tokens are the last rows of each sequence's cache (a fresh sequence:
 * lens[b] = S, T >= S):
 *   causal = 1: token s attends rows [lo_s, n_s), n_s = clamp(lens[b] -
 *               (S-1-s), 0, T) -- the same rows as gqa_attn_decode_multi;
 *   causal = 0: every token attends [lo, n), n = clamp(lens[b], 0, T);
 *   lo = max(0, n - window) with window > 0, else 0.
 * q [B,S,Hq,D] fp32 or bf16, dense; out [B,S,Hq,D] fp32 or bf16;
 * lse_out [B,S,Hq] fp32 (natural log) or NULL.  Any S >= 1 and any G =
 * Hq/Hkv in {1,2,4,8,16}; D in {64,128}.  A row with no key gets out = 0 and
 * lse = -inf.  Runs on the matrix cores: K and V tiles are shared through
 * LDS by 128 (token, head) rows of one KV head; P keeps ~16 mantissa bits
 * (bf16 hi + lo) and an fp32 q is split the same way.  Errors:
 * GQA_ERR_NULL, GQA_ERR_SHAPE (S < 1, sizes), GQA_ERR_VALUE (causal not 0 or
 * 1, non-finite scale), GQA_ERR_UNSUPPORTED (D, G, dtypes), GQA_ERR_ALIGN
 * (q, caches, out 16-byte aligned; lens, lse_out 4-byte aligned).  Nothing
 * is allocated; outputs must not alias inputs.
 */
int gqa_attn_prefill(const void* q, gqa_dtype_t q_dtype,
                     const uint16_t* k_cache, const uint16_t* v_cache,
                     const int32_t* lens, int S, int causal, int window, float scale,
                     void* out, gqa_dtype_t out_dtype, float* lse_out,
                     int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * gqa_attn_prefill with the keys of every 128-row block shared out among
 * `splits` workgroups (1..16; gqa_attn_prefill is splits = 1): the
 * flash-decoding split of the fusedtok README's attention_decode applied to
 * the prefill, for launches whose row blocks are too few -- or, under the
 * causal mask, too unequal -- to keep every CU busy.  Each split writes its
 * rows' partial (normalised o, lse) to `workspace`; the last split of a row
 * block to finish merges them in split order (bit-identical reruns) and
 * writes out / lse_out.  Results equal gqa_attn_prefill's up to rounding.
 *   workspace  256-byte aligned, gqa_attn_prefill_workspace_bytes() bytes
 *              (0 for splits = 1, when it may be NULL): partial o, partial
 *              lse, then uint32 tickets, one per row block, which must be
 *              zero before the first call and are left zero by every call
 *              that completes.  Calls sharing a workspace must not overlap.
 * Errors as for gqa_attn_prefill, plus GQA_ERR_VALUE (splits outside 1..16),
 * GQA_ERR_NULL (splits > 1 without a workspace), GQA_ERR_WORKSPACE (too
 * small) and GQA_ERR_ALIGN (workspace not 256-byte aligned).
 * gqa_attn_prefill_default_splits suggests a split count for the current
 * device: 2 when the launch has fewer row blocks than CUs, else 1;
 * it reads device attributes only and returns 1 when they cannot be read.
 */
/*
 * The prefill with its prologue, in two launches: the effect of
 * gqa_qkv_prologue_ex over S tokens followed by gqa_attn_prefill_split.
 * The first launch appends the S tokens' K/V rows (rows pos[b] + s inside
 * [0, T)); the second is the attention kernel, which normalises and rotates
 * its own rows of q as it loads them, so the rotated q never goes through
 * memory (q_out, float32 [B,S,Hq,D], is written only when not NULL).  q's
 * rotary sin and cos come from the float64-reduced phase through the
 * hardware sine and cosine (which take turns), so q_out can differ from
 * gqa_qkv_prologue_ex's float64 rotation in the last bits; the appended K
 * rows are those of gqa_qkv_prologue_ex.  Arguments as for
 * gqa_qkv_prologue_ex (q [B,S,Hq,D] and k_new, v_new [B,S,Hkv,D] with batch
 * strides, tokens and heads dense; pos, k_new, v_new required) and
 * gqa_attn_prefill_split (causal, window, scale, splits, workspace, out,
 * out_dtype, lse_out); the same errors.
 */
int gqa_prefill_step(const void* q, const void* k_new, const void* v_new,
                     gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                     const float* q_norm_w, const float* k_norm_w, float eps,
                     const double* inv_freq, double rope_mscale, int rope_layout,
                     const int32_t* pos, int S,
                     uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                     int causal, int window, float scale, int splits,
                     void* workspace, size_t workspace_bytes,
                     void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                     int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

size_t gqa_attn_prefill_workspace_bytes(int B, int S, int Hq, int Hkv, int D, int splits);
int gqa_attn_prefill_default_splits(int B, int S, int Hq, int Hkv);
int gqa_attn_prefill_split(const void* q, gqa_dtype_t q_dtype,
                           const uint16_t* k_cache, const uint16_t* v_cache,
                           const int32_t* lens, int S, int causal, int window, float scale,
                           int splits, void* workspace, size_t workspace_bytes,
                           void* out, gqa_dtype_t out_dtype, float* lse_out,
                           int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/*
 * Packed QKV projection of the decode batch: y[m][n] = sum_k x[m][k] w[n][k]
 * for m < M, n < N (the projection ahead of the prologue in the cutileGPT
 * README's runtime list, "packed QKV ... projections"; the weight layout
 * B[N,K] of the PyGPUkit 0.2.18 page's optimized BF16 GEMV).  With
 * N = (Hq + 2 Hkv) D, row m of y is q | k_new | v_new of sequence m, and
 * gqa_qkv_prologue reads it directly with q = y, k_new = y + Hq D,
 * v_new = y + (Hq + Hkv) D and both batch strides = y_stride.
 * x [M, x_stride] bf16 and w [N, w_stride] bf16, row-major, 16-byte aligned
 * with strides a multiple of 8 elements; y [M, y_stride] fp32 or bf16
 * (round to nearest even).  bf16 products, float32 accumulation in a fixed
 * order (bit-identical reruns).  1 <= M <= 16 and K a multiple of 128, else
 * GQA_ERR_UNSUPPORTED; GQA_ERR_SHAPE for strides below the sizes or
 * 63 * w_stride + K >= 2^31 elements; GQA_ERR_ALIGN for misaligned
 * pointers or strides.  Nothing is allocated; y must not alias x or w.
 */
int gqa_qkv_gemv(const uint16_t* x, int64_t x_stride, const uint16_t* w, int64_t w_stride,
                 void* y, gqa_dtype_t y_dtype, int64_t y_stride, int M, int N, int K,
                 hipStream_t stream);

/*
 * gqa_decode_step_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): gqa_decode_step_multi with the same arguments except
 * the workspace, which is instead a file-scope device array of the library,
 * 8 MiB on each device it runs on, held until the process ends.  The call
 * allocates nothing and calls no allocating routine.
 *   Limits: B * Hkv <= 4096 arrival tickets, and the split-K partials,
 *   256-byte-rounded B*S*Hq*NP*4 bytes of lse plus B*S*Hq*NP*D*4 bytes of o
 *   (NP = partitions, as for gqa_splitk_multi_workspace_bytes), within
 *   8 MiB - 16 KiB; beyond them it returns GQA_ERR_SCRATCH and enqueues
 *   nothing.  (For example B=1, Hq=32, L=131072, P=2048 needs 1.01 MiB, as
 *   does B=8, Hq=64, window 4096, P=1024.)
 *   The step runs on the current device; `stream` must belong to it.  The
 *   first call on a device also enqueues, ahead of the step, one small
 *   kernel that zeroes the tickets.
 *   Every call on a device shares that device's array: calls that overlap
 *   in time on one device (on different streams, or from several host
 *   threads without ordering) race and give wrong results.  Calls ordered
 *   on one stream are safe; each completed call leaves the tickets at zero,
 *   the partials are rewritten by every call.
 * Other arguments, results and errors as for gqa_decode_step_multi.
 */
int gqa_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                            gqa_dtype_t in_dtype, int64_t q_bstride, int64_t kv_bstride,
                            const float* q_norm_w, const float* k_norm_w, float eps,
                            const double* inv_freq, double rope_mscale, int rope_layout,
                            const int32_t* pos, int S,
                            uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens,
                            int window, float scale, int part_tokens,
                            void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out,
                            int B, int Hq, int Hkv, int D, int T, hipStream_t stream);

/* Measurement helper, not part of the attention path: reads `bytes` bytes
 * of the device buffer `buf` once, as one contiguous share per workgroup
 * (`workgroups` workgroups of `threads` threads, `unroll` 16-byte
 * non-temporal loads in flight per thread), and does nothing with them.
 * Timed around the launch it gives the streaming-read rate the part reaches
 * for that many bytes: the ceiling a decode step that reads each K/V row
 * once can approach.  The fusedtok README ("Benchmarks") rates its decode
 * kernel by the cache-streaming bandwidth it reaches; this is the bare
 * stream it is measured against.
 * buf 16-byte aligned, 16 <= bytes <= 2^31 and a multiple of 16, else
 * GQA_ERR_SHAPE / GQA_ERR_ALIGN; 1 <= workgroups <= 65536; threads a
 * multiple of 64 in [64, 1024] (GQA_ERR_VALUE); unroll 4, 8 or 16
 * (GQA_ERR_UNSUPPORTED).  `sink` is caller-owned device memory of
 * workgroups * threads uint32 that the kernel may write (in practice it
 * never does).  Nothing is allocated. */
int gqa_probe_stream_read(const void* buf, size_t bytes, int workgroups, int threads, int unroll,
                          uint32_t* sink, hipStream_t stream);

/* Static text for a status code (never NULL). */
const char* gqa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
