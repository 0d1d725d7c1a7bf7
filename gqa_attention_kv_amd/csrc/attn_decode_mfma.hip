// GQA decode attention on gfx950 matrix cores, one token per sequence (or
// a few: G * S <= 16 (token, head) rows per KV head), in three modes that
// share one body:
//   Final  one workgroup per (sequence, KV head) writes the output directly;
//   Split  one workgroup per (partition, KV head, sequence) writes the
//          partition's (o_k, lse_k) for the log-sum-exp merge;
//   Step   the whole decode step in one launch: per-head QK-RMSNorm and NeoX
//          RoPE of the new queries, the K/V append, the split-K pass, and the
//          merge, done by the last workgroup of each (sequence, KV head) to
//          finish.
//
// Computes what the fusedtok 1.0.1 README ("Operators" row attention_decode)
// describes -- single-token GQA attention over a contiguous KV cache with
// online softmax, per-sequence lengths and a flash-decoding split -- plus the
// sliding window and the fused QK-Norm + RoPE + KV-cache write of the
// cutileGPT README feature list.  A workgroup covers all G query heads of one
// KV head, so each K/V row is read from HBM once.
//
// Why matrix cores.  Per cached row the G heads need 2*G*D multiply-adds;
// at G = 8 the VALU form costs more issue cycles per row than HBM needs to
// deliver it at 6.4 TB/s.  Both contractions run on bf16 MFMA instead,
// leaving the VALU the softmax and some operand packing.
//
// Tiles of 16 rows.  Lane l, with n = l % 16 and g = l / 16:
//   QK: S^T[16 rows x 16 heads] += K[16 x 32] * Q^T[32 x 16] with
//       v_mfma_f32_16x16x32_bf16, one call per 32-wide slice of D.  The A
//       operand wants lane l to hold row n, elements 32c + 8g..+8.  Loading
//       that directly makes every load instruction touch 16 rows x 64 bytes,
//       which streams at only ~4.1 TB/s on MI355X against ~5.2 TB/s for
//       instructions that read whole 256-byte rows.  So K is loaded like V,
//       whole rows, and passes through a wave-private LDS slab (rows padded
//       to D*2+16 bytes; the counters still report bank conflicts at about
//       0.6 of the LDS-active cycles, small against the HBM-bound loop).
//       An fp32 q is split into bf16 hi + lo parts so the
//       scores keep ~16 mantissa bits: with G <= 8 the lo parts fill columns
//       8..15 of the same operand and one DPP step adds column n + 8 to
//       column n; with G = 16 they take a second call.  A bf16 q needs the
//       hi part only.  Heads >= G are zero columns.  A-operand row m is fed
//       tile row pi(m) = 4(m%4) + m/4, so the result leaves lane l holding S
//       for tile rows 4r + g (r < 4) of head n.
//   PV: O[16 heads x 16 cols] += P[16 x 32] * V[32 x 16] with
//       v_mfma_f32_16x16x32_bf16, one call per D/16 column block.  The 16
//       tile rows become 32 k-indices, k = 8g + 2r + x for tile row 4r + g,
//       with x = 0 carrying the bf16 hi part of P and x = 1 its lo part
//       (P keeps ~16 mantissa bits; V is exact in bf16 and appears at both
//       k of its row).  Lane l's P operand is the four scores the QK step
//       left in it, so no cross-lane movement is needed.  Output column n of
//       block b stands for d = (D/16) n + b, which makes lane l's V operand
//       for every block one contiguous (D/8)-byte load per row: a wave-wide
//       load reads 4 consecutive rows, 1 KiB contiguous for D = 128.
// Each wave streams units of two tiles (32 rows): the loads of the next
// unit's tile are issued as soon as a tile is computed (register double
// buffer, branch-free trips), and the waves of a workgroup take
// interleaved units.  K and V are read through buffer resources (the slab
// base in scalar registers, 32-bit lane offsets).
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;   // 16 bytes, register type

enum class Mode { Final, Split, Step };

// Cache policy of the K/V stream loads: non-temporal (nt).  Every cached
// row is read exactly once per step, so nothing is gained by keeping it;
// measured on MI355X, nt on both K and V took the fused step from 33.0 to
// 30.2 us (workload 5) and 103 to 94.5 us (workload 4); the coherence bits
// sc0 / sc1 on top changed nothing, nt on K or V alone gave half the gain.
constexpr int kStreamPolicy = 2;

// Buffer resource over `bytes` bytes from `base` (raw, unswizzled); loads
// through it take 32-bit byte offsets and return zeros past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int D>
struct VRow;   // lane's slice of one V row: D/16 bf16
template <>
struct VRow<128> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0,
                                                                         kStreamPolicy));
  }
  __device__ __forceinline__ uint32_t word(int w) const {
    return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
  }
};
template <>
struct VRow<64> {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStreamPolicy));
  }
  __device__ __forceinline__ uint32_t word(int w) const { return w == 0 ? v.x : v.y; }
};

// bf16 element e of a V slice, copied into both halves of a dword.
template <int D>
__device__ __forceinline__ uint32_t dup_bf16(const VRow<D>& r, int e) {
  const uint32_t w = r.word(e >> 1);
  return __builtin_amdgcn_perm(w, w, (e & 1) ? 0x03020302u : 0x01000100u);
}

// Two floats rounded to bf16 (nearest even, one v_cvt_pk_bf16_f32), a in
// the low half of the dword.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// x as a bf16 pair (hi, lo) with hi = bf16(x) and lo = bf16(x - hi): hi + lo
// carries ~16 significant bits of x.  hi in the low half of the dword.
__device__ __forceinline__ uint32_t split_bf16(float x) {
  const __bf16 h = (__bf16)x;
  const bf16x2_t v = {h, (__bf16)(x - (float)h)};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float f[8]);
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float f[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <>
__device__ __forceinline__ void load8f<uint16_t>(const uint16_t* p, float f[8]) {
  unpack8(*reinterpret_cast<const uint4*>(p), f);
}

template <typename T>
__device__ __forceinline__ float load1f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load1f<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load1f<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Eight q elements as loaded (raw) and their float32 values (unpack), so
// that the conversion of a bf16 q can be placed after later loads are issued.
template <typename T>
struct QRaw;
template <>
struct QRaw<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void unpack(float f[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};
template <>
struct QRaw<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void unpack(float f[8]) const { unpack8(v, f); }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }

__device__ __forceinline__ uint16_t bits_bf16(const float* p, int64_t i) { return f32_to_bf16(p[i]); }
__device__ __forceinline__ uint16_t bits_bf16(const uint16_t* p, int64_t i) { return p[i]; }

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

template <int D>
struct TileBuf {
  u32x4_t k[D / 32];   // K rows, whole-row pieces: lane's 16 bytes of D/32 rows
  VRow<D> v[4];        // V rows 4i + g, i < 4
};

// Register budget: three waves per SIMD (168 VGPRs); G = 16 keeps two q
// operands (hi and lo) live and gets two waves (256 VGPRs) so that nothing
// spills to scratch inside the tile loop.
constexpr int kWavesPerEU = 3;

// Lazy-rescale threshold of the online softmax, in exp2 units.
constexpr float kRescaleLog2 = 8.0f;

// The last workgroup of a (sequence, KV head) team merges the team's
// partitions (one per member): M = max_k lse_k, w_k = e^(lse_k - M),
// out = sum_k w_k o_k / sum_k w_k, lse = M + log sum_k w_k.  Thread t owns
// float4 group(s) of the G*D outputs; when there are fewer groups than
// threads, KS subsets of threads take partitions s, s + KS, ... and are
// combined through LDS at the end.  Every order is fixed, so the result is
// bit-identical from run to run.  Partials are read with device-coherent
// loads (the sc1 policy of agent-scope atomics; 16-byte buffer loads for o),
// which do not hit stale L2 lines; a batch of up to MB partitions is one
// memory round trip.  The team's slice of o is below 2 GiB (checked on the
// host), so 32-bit buffer offsets reach all of it.
// Column h of the team is output row head0 + rel(h): rel(h) = h with one
// token (CT = G columns); with several tokens (MT) column h is token h / G,
// head h % G, so rel(h) = (h / G) Hq + h % G, and columns h >= nc are padding.
template <int D, int CT, int NW, bool MT>
__device__ __forceinline__ void merge_partials(const KernelArgs& a, int64_t head0, int G,
                                               int nc, int count) {
  constexpr int NTH = NW * 64;
  constexpr int NG = CT * D / 4;                // float4 output groups
  constexpr int GPT = NG > NTH ? NG / NTH : 1;  // groups per thread
  constexpr int TPS = NG < NTH ? NG : NTH;      // threads per partition subset
  constexpr int KS = NTH / TPS;                 // partition subsets
  constexpr int MB = 16 / GPT;                  // partitions per batch (no spills)
  constexpr int kCoherent = 0x10;               // sc1: read through to the coherence point
  const int num_parts = a.num_parts;
  const int t = threadIdx.x;
  const int s = t / TPS;
  auto rel = [&](int h) -> int64_t {
    if constexpr (MT) return (int64_t)(h / G) * a.Hq + h % G;
    return h;
  };
  const int64_t span = MT ? rel(nc - 1) + 1 : CT;   // rows from head0 to the last column's
  const __amdgpu_buffer_rsrc_t Ors =
      make_rsrc(a.ws_o + head0 * num_parts * D, (uint32_t)((size_t)span * num_parts * D * 4));
  float Mx[GPT], Wx[GPT];
  float Ax[GPT][4];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    Mx[j] = -INFINITY;
    Wx[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) Ax[j][e] = 0.0f;
  }
  for (int k0 = s; k0 < count; k0 += KS * MB) {
    float lk[GPT][MB];
    f32x4_t ov[GPT][MB];
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int gi = t % TPS + j * TPS;
      const int h = gi / (D / 4);
      const int d4 = gi % (D / 4);
      const bool col = !MT || h < nc;
      const int64_t rh = rel(col ? h : 0);
      const float* Lh = a.ws_lse + (head0 + rh) * num_parts;
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        const int kk = k0 + k * KS;
        lk[j][k] = -INFINITY;
        ov[j][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (kk < count && col) {
          lk[j][k] = __hip_atomic_load(Lh + kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t off = (uint32_t)(((rh * num_parts + kk) * D + 4 * d4) * 4);
          ov[j][k] = __builtin_amdgcn_raw_buffer_load_b128(Ors, off, 0, kCoherent);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      float cm = -INFINITY;
#pragma unroll
      for (int k = 0; k < MB; ++k) cm = fmaxf(cm, lk[j][k]);
      const float Mn = fmaxf(Mx[j], cm);
      if (Mn == -INFINITY) continue;
      const float sc = __expf(Mx[j] - Mn);          // 0 while nothing was seen
      float W = Wx[j] * sc;
      float A[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) A[e] = Ax[j][e] * sc;
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        // an empty partition (lse = -inf) has weight 0 and an undefined o_k
        const bool ok = lk[j][k] != -INFINITY;
        const float w = ok ? __expf(lk[j][k] - Mn) : 0.0f;
        const float o4[4] = {ov[j][k][0], ov[j][k][1], ov[j][k][2], ov[j][k][3]};
        W += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) A[e] = fmaf(w, ok ? o4[e] : 0.0f, A[e]);
      }
      Mx[j] = Mn;
      Wx[j] = W;
#pragma unroll
      for (int e = 0; e < 4; ++e) Ax[j][e] = A[e];
    }
  }
  if constexpr (KS > 1) {   // GPT == 1: combine the subsets in ascending order
    __shared__ float sm_mx[NTH], sm_wx[NTH];
    __shared__ float4 sm_ax[NTH];
    sm_mx[t] = Mx[0];
    sm_wx[t] = Wx[0];
    sm_ax[t] = make_float4(Ax[0][0], Ax[0][1], Ax[0][2], Ax[0][3]);
    __syncthreads();
    if (t >= TPS) return;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < KS; ++q) M = fmaxf(M, sm_mx[q * TPS + t]);
    float W = 0.0f, A[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        const float f = __expf(sm_mx[q * TPS + t] - M);
        const float4 av = sm_ax[q * TPS + t];
        W = fmaf(sm_wx[q * TPS + t], f, W);
        A[0] = fmaf(av.x, f, A[0]);
        A[1] = fmaf(av.y, f, A[1]);
        A[2] = fmaf(av.z, f, A[2]);
        A[3] = fmaf(av.w, f, A[3]);
      }
    }
    Mx[0] = M;
    Wx[0] = W;
#pragma unroll
    for (int e = 0; e < 4; ++e) Ax[0][e] = A[e];
  }
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int gi = t % TPS + j * TPS;
    const int h = gi / (D / 4);
    const int d4 = gi % (D / 4);
    if (MT && h >= nc) continue;
    const bool any = Wx[j] > 0.0f;
    float ov[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = any ? Ax[j][e] / Wx[j] : 0.0f;
    const int64_t oi = (head0 + rel(h)) * D + 4 * d4;
    if (a.out_bf16) {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oi) =
          make_uint2(pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3]));
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) =
          make_float4(ov[0], ov[1], ov[2], ov[3]);
    }
    if (d4 == 0 && a.lse_out != nullptr)
      a.lse_out[head0 + rel(h)] = any ? Mx[j] + logf(Wx[j]) : -INFINITY;
  }
}

// CT is the column capacity: the NC = G * S query rows of one KV head (G
// heads of the group times S tokens of the sequence, NC <= CT) are the
// columns of the 16-column MFMA tile; column c is token c / G, head c % G.
// MT: several tokens (S > 1), whose columns attend different row ranges;
// the single-token instances keep the plainer inner loop.
template <int D, int CT, int NW, int PPW, typename IT, Mode MODE, bool MT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(CT >= 16 ? 2 : kWavesPerEU))) void
attn_decode_mfma_kernel(const KernelArgs a) {
  static_assert(CT <= 16, "one 16-column MFMA tile holds at most 16 query rows");
  constexpr int KC = D / 32;          // QK calls per tile (per q part)
  constexpr int VB = D / 16;          // PV column blocks
  constexpr int HALF = D / 2;
  constexpr int UR = 32;              // rows per unit of work: two 16-row tiles
  // fp32 q (given, or the prologue's rotated q) needs the lo part
  constexpr bool kLo = sizeof(IT) == 4 || MODE == Mode::Step;
  // With at most 8 heads the lo part takes columns 8..15 of the same
  // operand (column n + 8 holds head n's lo part) instead of a second call.
  constexpr bool kFold = kLo && CT <= 8;
  constexpr bool kPartial = MODE != Mode::Final;

  // One-dimensional grid.  The hardware hands workgroup i to XCD i % 8.
  // With 8 or more partitions per (sequence, KV head) the partition index
  // runs fastest, so consecutive partitions of one sequence land on
  // consecutive XCDs and the workgroups in flight read one stretch of the
  // cache.  With fewer, it runs slowest: workgroup i takes partition
  // i / (B*Hkv) of (sequence, KV head) i % (B*Hkv), so every XCD gets the
  // same mix of partitions -- partition 0 of every sequence is the one that
  // is never empty under ragged lengths -- and the dispatcher starts all
  // first partitions before any later one.  (Partition-slowest order with
  // many partitions puts partitions of every sequence in flight at once,
  // streams 32 MiB or more apart, and measured slower and sensitive to where
  // the K and V caches sit relative to each other.)
  //
  // Partitions per workgroup (ppw = PPW, Split and Step with one token):
  // with ppw = 2 a workgroup takes two consecutive partitions of one
  // (sequence, KV head) and its NW waves split into two groups of NW/2, one
  // per partition.  The long-context launches use it with NW = 8, so each
  // partition keeps four waves while the two partitions that share a CU are
  // one workgroup (see the launcher).  The grid's unit is then the pair.
  constexpr int ppw = (kPartial && !MT) ? PPW : 1;
  constexpr int wpp = NW / ppw;       // waves per partition
  static_assert(PPW == 1 || PPW == 2, "one or two partitions per workgroup");
  const int nbg = a.B * a.Hkv;
  const int npg = MODE == Mode::Final ? 1 : (a.num_parts + ppw - 1) / ppw;
  int pgrp, bg;
  if (MT && npg >= 8) {
    // Several tokens: the last partition of every team, often a stub (the
    // new tokens' rows past the last whole partition), after all the
    // others, so the whole partitions take the first round of resident
    // workgroups (measured on 4 draft tokens over 8192 rows: 59.0 -> 57.0 us)
    const int head = nbg * (npg - 1);
    if ((int)blockIdx.x < head) {
      bg = (int)blockIdx.x / (npg - 1);
      pgrp = (int)blockIdx.x - bg * (npg - 1);
    } else {
      bg = (int)blockIdx.x - head;
      pgrp = npg - 1;
    }
  } else if (npg >= 8) {
    bg = (int)blockIdx.x / npg;
    pgrp = (int)blockIdx.x - bg * npg;
  } else {
    pgrp = (int)blockIdx.x / nbg;
    bg = (int)blockIdx.x - pgrp * nbg;
  }
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lw = ppw == 1 ? wave : wave % wpp;   // wave within its partition's group
  const int part = ppw == 1 ? pgrp : pgrp * ppw + wave / wpp;   // this wave's partition
  const int n = lane & 15;
  const int lg = lane >> 4;
  const int T = a.T;
  const int Hq = a.Hq;
  const int Hkv = a.Hkv;
  const int num_parts = a.num_parts;
  const int S = MT ? a.S : 1;         // tokens per sequence
  const int G = MT ? Hq / Hkv : CT;   // heads per KV head (CT itself with one token)
  const int NC = MT ? G * S : CT;     // columns in use

  // Token s of sequence b attends rows [lo_s, n_s): n_s = lens[b] - (S-1-s)
  // clamped to [0, T], lo_s = n_s - window (or 0).  The workgroup streams
  // the union [lo_0, n_{S-1}), or its partition of that range.
  auto tok_end = [&](int st) {
    return (int)min(max((int64_t)a.lens[b] - (S - 1 - st), (int64_t)0), (int64_t)T);
  };
  auto tok_lo = [&](int st) { return a.window > 0 ? max(0, tok_end(st) - a.window) : 0; };
  const int nrow = MT ? tok_end(S - 1) : min(max(a.lens[b], 0), T);
  const int lo = MT ? tok_lo(0) : (a.window > 0 ? max(0, nrow - a.window) : 0);
  // Rows this wave attends: the whole range, or its partition.
  int t0 = lo, t1 = nrow;
  if (kPartial) {
    t0 = min(lo + part * a.part_tokens, nrow);
    t1 = min(t0 + a.part_tokens, nrow);
  }
  // output row (of [B, S, Hq]) of column c
  const int64_t head0 = ((int64_t)b * S) * Hq + (int64_t)g * G;
  auto orow = [&](int c) -> int64_t {
    if constexpr (MT) return ((int64_t)b * S + c / G) * Hq + (int64_t)g * G + c % G;
    return head0 + c;
  };

  if constexpr (MODE != Mode::Step) {
    // nothing to attend in this range (uniform over the workgroup when it
    // holds one partition)
    if (ppw == 1 && t0 >= t1) {
      if (MODE == Mode::Split) {
        for (int c = threadIdx.x; c < NC; c += NW * 64)
          a.ws_lse[orow(c) * num_parts + part] = -INFINITY;
      } else {
        for (int e = threadIdx.x; e < NC * D; e += NW * 64) {
          const int64_t oi = orow(e / D) * D + e % D;
          if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = 0;
          else reinterpret_cast<float*>(a.out)[oi] = 0.0f;
        }
        if (a.lse_out != nullptr)
          for (int c = threadIdx.x; c < NC; c += NW * 64) a.lse_out[orow(c)] = -INFINITY;
      }
      return;
    }
  }

  const int64_t slab_off = ((int64_t)b * Hkv + g) * T * D;
  // K whole-row layout: a load covers RPI rows; lane l takes 16-byte piece
  // kp = l % PPR of row RPI*i + kr.
  constexpr int PPR = D / 8;            // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;         // rows per load instruction
  constexpr int ROWU4 = PPR + 1;        // padded LDS row, in 16-byte units
  const int kp = lane % PPR;
  const int kr = lane / PPR;
  // This (sequence, KV head)'s T x D slab of each cache, as a buffer
  // resource: T * D * 2 < 2^32 bytes (checked on the host).
  const __amdgpu_buffer_rsrc_t Krs = make_rsrc(a.k_cache + slab_off, (uint32_t)T * D * 2u);
  const __amdgpu_buffer_rsrc_t Vrs = make_rsrc(a.v_cache + slab_off, (uint32_t)T * D * 2u);
  const uint32_t koff = 16u * kp;          // + row * 2D bytes
  const uint32_t voff = 2u * VB * n;
  // LDS: the waves' K slabs while streaming, then (after a barrier) the
  // per-wave partial results for the cross-wave combine, in one buffer.
  struct Combine {
    float m[NW][CT];
    float l[NW][CT];
    float o[NW][CT][D];
  };
  union Lds {
    u32x4_t sk[NW][16][ROWU4];
    Combine cb;
  };
  __shared__ Lds lds;
  u32x4_t* slab = &lds.sk[wave][0][0];

  // Loads are unconditional: a row index past the range is clamped to the
  // last valid row (an attended row, so finite; row 0 when the range is
  // empty), and the softmax gives such rows p = 0.  With no branches around
  // the loads the compiler can count them exactly and wait only for the tile
  // being computed.
  const int rlast = max(t1 - 1, 0);
  auto issue = [&](TileBuf<D>& buf, int base) {
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const uint32_t rk = (uint32_t)min(base + RPI * i + kr, rlast);
      buf.k[i] = __builtin_amdgcn_raw_buffer_load_b128(Krs, rk * (2u * D) + koff, 0,
                                                       kStreamPolicy);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t rv = (uint32_t)min(base + 4 * i + lg, rlast);
      buf.v[i].load(Vrs, rv * (2u * D) + voff);
    }
  };

  // Units of UR rows: the wave with index lw in its partition's group of
  // wpp waves takes units lw, lw + wpp, lw + 2 wpp, ... of the partition's
  // range (the whole workgroup's range when it holds one partition).
  auto unit_row = [&](int64_t u) -> int {
    return (int)min((int64_t)t0 + (int64_t)UR * u, (int64_t)t1);
  };
  int64_t ustep = lw;
  int rcur = unit_row(ustep);

  TileBuf<D> bf[2];
  auto prime = [&]() {
    issue(bf[0], rcur);
    issue(bf[1], rcur + 16);
  };

  // q of column hn = n (n % 8 when folded; padding columns hn >= NC load
  // column NC-1 -- no branch around the loads -- and are zeroed): lane
  // holds elements 32c + 8lg + j of token hq / G, head hq % G.
  const int hn = kFold ? (n & 7) : n;
  const float keep = hn < NC ? 1.0f : 0.0f;
  const int hq = min(hn, NC - 1);
  const int tq = MT ? hq / G : 0;     // token and head of column hq
  const int hh = MT ? hq % G : hq;
  const int64_t qoff = (int64_t)b * a.q_bstride + (int64_t)tq * a.q_sstride +
                       (int64_t)(g * G + hh) * D;
  // Rows column hn may attend, within this workgroup's range.
  const int clo = MT ? max(t0, tok_lo(tq)) : t0;
  const int chi = MT ? min(t1, tok_end(tq)) : t1;
  float qf[KC][8];
  // Step: the appended row (bf16 K row, then V row, per wave), substituted
  // into the one tile that holds row psub.
  __shared__ u32x4_t snew[NW][2][PPR];
  int psub = -1;
  // Step with several tokens: the new rows [sub_lo, sub_hi) this workgroup
  // attends, token s's row at sub_k[s] (shared by the waves), and token s's
  // rotary angles at ang[s] (cos of pair i at i, sin at D/2 + i).
  __shared__ u32x4_t sub_k[MT ? CT : 1][2][PPR];
  __shared__ float ang[MT ? CT : 1][D];
  int sub_lo = -1, sub_hi = -1, p_new = 0;

  if constexpr (MODE == Mode::Step) {
    // ---- fused prologue: QK-RMSNorm, NeoX RoPE at pos[b], K/V append ----
    // (skipped when no prologue inputs are given: q is then used as is)
    const bool has_pro = a.pos != nullptr;
    const int p = has_pro ? a.pos[b] : -1;
    // Every global load of the prologue is issued before the first tiles:
    // loads complete in order, so waiting for these never waits for a tile.
    const IT* qs = reinterpret_cast<const IT*>(a.q) + qoff;
    QRaw<IT> qraw[KC];   // several tokens: unpacked after the tiles are issued
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if constexpr (MT) qraw[c].load(qs + 32 * c + 8 * lg);
      else load8f<IT>(qs + 32 * c + 8 * lg, qf[c]);
    }
    const bool qnorm = has_pro && a.wq != nullptr;
    const bool rope = has_pro && a.rope;
    float wq8[KC][8];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (qnorm) load8f<float>(a.wq + 32 * c + 8 * lg, wq8[c]);
    }
    // Query head g*G + hq: RMSNorm over D (the lane's D/4 elements, summed
    // over the four lane groups of head n).
    auto apply_qnorm = [&]() {
      if (!qnorm) return;
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(qf[c][j], qf[c][j], ss);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[c][j] = qf[c][j] * r * wq8[c][j];
    };
    const int fi = lane % HALF;               // rotary pair of this lane
    const bool il = a.rope_interleaved != 0;  // pairs (2i, 2i+1), else (i, i+D/2)
    const int e0 = il ? 2 * fi : fi, e1 = il ? 2 * fi + 1 : fi + HALF;
    const double inv_rev = rope ? a.inv_freq_rev[fi] : 0.0;
    // The appended K pair (e0, e1) in float64 (weights, a float64 sin/cos of
    // the reduced phase fr and the rotation on the exact inputs, the RMS
    // factor last), rounded once: an element much smaller than its inputs
    // keeps ~1e-7 relative accuracy, so it lands within one bf16 ulp of the
    // exact value.  Called by whole waves (the sum of squares crosses lanes).
    auto k_pair = [&](float xf0, float xf1, float wk0, float wk1, double fr, uint16_t& k0,
                      uint16_t& k1) {
      double x0 = xf0, x1 = xf1, r = 1.0;
      if (a.wk != nullptr) {
        const float ss = group_sum_shfl<HALF>(xf0 * xf0 + xf1 * xf1);
        r = 1.0 / sqrt((double)ss / D + (double)a.eps);
        x0 *= (double)wk0;
        x1 *= (double)wk1;
      }
      if (rope) {
        double sd, cd;
        sincos_pi_f64(fr * 6.283185307179586, &sd, &cd);
        cd *= (double)a.rope_mscale;
        sd *= (double)a.rope_mscale;
        const double y0 = x0 * cd - x1 * sd, y1 = x1 * cd + x0 * sd;
        x0 = y0;
        x1 = y1;
      }
      k0 = f32_to_bf16((float)(x0 * r));
      k1 = f32_to_bf16((float)(x1 * r));
    };
    // Rotary phase p * f / (2 pi) of this lane's pair, formed and reduced to
    // [-1/2, 1/2] in float64 from the host-computed table.
    auto phase = [&](int64_t pos_s) {
      const double rev = (double)pos_s * inv_rev;
      return rev - rint(rev);
    };
    float cs = 1.0f, sn = 0.0f;
    if constexpr (!MT) {
      // The workgroup whose partition holds row pos[b] computes it, uses it
      // in place of loading it and writes it to the cache (so no workgroup
      // waits for the write); partition 0 writes it when it lies in the
      // cache but outside the attended rows.  Positions outside [0, T) write
      // nothing.
      const bool in_range = has_pro && p >= 0 && p < T;
      const bool attended = has_pro && p >= t0 && p < t1;
      const bool outside = in_range && (p < lo || p >= nrow);
      const bool kwrite = lw == 0 && (attended || (part == 0 && outside));
      const bool need_k = attended || kwrite;
      // raw values: converted only after the tiles are issued
      IT rx0 = 0, rx1 = 0, rv0 = 0, rv1 = 0;
      float wk0 = 1.0f, wk1 = 1.0f;
      if (need_k) {
        const IT* ks = reinterpret_cast<const IT*>(a.k_new) + (int64_t)b * a.kv_bstride +
                       (int64_t)g * D;
        const IT* vs = reinterpret_cast<const IT*>(a.v_new) + (int64_t)b * a.kv_bstride +
                       (int64_t)g * D;
        rx0 = ks[e0];
        rx1 = ks[e1];
        rv0 = vs[e0];
        rv1 = vs[e1];
        if (a.wk != nullptr) {
          wk0 = a.wk[e0];
          wk1 = a.wk[e1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      prime();
      __builtin_amdgcn_sched_barrier(0);
      // (the asm keeps the weights' conversion, and so the wait for them,
      // from moving ahead of the tile loads)
      asm volatile("" : "+v"(wk0), "+v"(wk1));
      // q's sin and cos from the hardware's v_sin_f32 / v_cos_f32, which
      // take the angle in turns: the reduced phase in [-1/2, 1/2] is exactly
      // that, so no range reduction is needed.  cos and sin carry the
      // magnitude factor, so it reaches both q and k.
      double fr = 0.0;
      if (rope) {
        fr = phase(p);
        sn = __builtin_amdgcn_sinf((float)fr);
        cs = __builtin_amdgcn_cosf((float)fr);
        cs *= a.rope_mscale;
        sn *= a.rope_mscale;
      }
      if (need_k) {
        uint16_t k0, k1;
        k_pair(to_f32(rx0), to_f32(rx1), wk0, wk1, fr, k0, k1);
        const uint16_t v0 = bits_bf16(&rv0, 0), v1 = bits_bf16(&rv1, 0);
        if (kwrite && lane < HALF) {
          uint16_t* krow = a.k_cache_w + slab_off + (int64_t)p * D;
          uint16_t* vrow = a.v_cache_w + slab_off + (int64_t)p * D;
          krow[e0] = k0;
          krow[e1] = k1;
          vrow[e0] = v0;
          vrow[e1] = v1;
        }
        // the wave's copy crosses lanes through LDS in program order (the
        // asm hides the index from per-lane alias analysis)
        if (attended && lane < HALF) {
          uint16_t* kh = reinterpret_cast<uint16_t*>(&snew[wave][0][0]);
          int kidx = fi;
          asm volatile("" : "+v"(kidx));
          const int k0i = il ? 2 * kidx : kidx, k1i = il ? 2 * kidx + 1 : kidx + HALF;
          kh[k0i] = k0;
          kh[k1i] = k1;
          kh[D + k0i] = v0;
          kh[D + k1i] = v1;
        }
        if (attended) psub = p;
      }
    } else {
      // Several tokens: token s sits at position p + s and is appended at
      // cache row p + s (rows inside [0, T) only).  Every workgroup computes
      // the new rows its partition holds, substitutes them for what it loads
      // (as with one token) and writes them to the cache; partition 0 writes
      // the new rows no token attends.  So each row is written once, and by
      // a workgroup that computes it anyway.  Wave w takes tokens w, w + NW,
      // ...; the angle table and the new rows are shared by the waves
      // through LDS (one barrier).
      constexpr int RW = (CT + NW - 1) / NW;   // tokens per wave at most
      if (has_pro) {
        sub_lo = (int)max((int64_t)p, (int64_t)t0);
        sub_hi = (int)min((int64_t)p + S, (int64_t)t1);
        p_new = p;
      }
      bool need[RW];
      bool any_new = false;
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int st = wave + NW * j;
        const int64_t row = (int64_t)p + st;
        // written by the workgroup whose partition holds it (that one
        // computes it anyway), or by partition 0 when it lies in the cache
        // but outside the rows the tokens attend
        const bool outside = row >= 0 && row < T && (row < lo || row >= nrow);
        need[j] = has_pro && st < S &&
                  ((row >= sub_lo && row < sub_hi) || (part == 0 && outside));
        any_new = any_new || need[j];
      }
      __builtin_amdgcn_sched_barrier(0);
      prime();
      __builtin_amdgcn_sched_barrier(0);
      // The norm waits only for the loads issued before the tiles, and frees
      // the weights' registers; the angle table needs no load.
#pragma unroll
      for (int c = 0; c < KC; ++c) qraw[c].unpack(qf[c]);
      apply_qnorm();
      if (rope) {
        // Entry e = thread + 64 NW k is pair e % HALF = this lane's pair fi
        // (HALF divides 64), whose frequency was loaded before the tiles: a
        // load here would wait behind them.
        static_assert(64 % HALF == 0, "pair of a table entry");
        for (int e = threadIdx.x; e < S * HALF; e += NW * 64) {
          const int st = e / HALF, i = e % HALF;
          const double rev = (double)((int64_t)p + st) * inv_rev;
          double sd, cd;
          sincos_pi_f64((rev - rint(rev)) * 6.283185307179586, &sd, &cd);
          ang[st][i] = (float)cd * a.rope_mscale;
          ang[st][HALF + i] = (float)sd * a.rope_mscale;
        }
      }
      // The new rows' inputs are loaded after the tiles: a value loaded
      // under a condition and merged with a default makes the compiler wait
      // for it (and for every load before it) ahead of the tile loads.
      IT rx0[RW], rx1[RW], rv0[RW], rv1[RW];
      float wk0 = 1.0f, wk1 = 1.0f;
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        if (!need[j]) continue;                         // wave-uniform
        const int st = wave + NW * j;
        const int64_t off = (int64_t)b * a.kv_bstride + ((int64_t)st * Hkv + g) * D;
        const IT* ks = reinterpret_cast<const IT*>(a.k_new) + off;
        const IT* vs = reinterpret_cast<const IT*>(a.v_new) + off;
        rx0[j] = ks[e0];
        rx1[j] = ks[e1];
        rv0[j] = vs[e0];
        rv1[j] = vs[e1];
      }
      if (any_new && a.wk != nullptr) {
        wk0 = a.wk[e0];
        wk1 = a.wk[e1];
      }
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        if (!need[j]) continue;                         // wave-uniform
        const int st = wave + NW * j;
        const int row = p + st;
        uint16_t k0, k1;
        k_pair(to_f32(rx0[j]), to_f32(rx1[j]), wk0, wk1, rope ? phase(row) : 0.0, k0, k1);
        const uint16_t v0 = bits_bf16(&rv0[j], 0), v1 = bits_bf16(&rv1[j], 0);
        if (lane < HALF) {                              // row is inside [0, T)
          uint16_t* krow = a.k_cache_w + slab_off + (int64_t)row * D;
          uint16_t* vrow = a.v_cache_w + slab_off + (int64_t)row * D;
          krow[e0] = k0;
          krow[e1] = k1;
          vrow[e0] = v0;
          vrow[e1] = v1;
        }
        if (row >= sub_lo && row < sub_hi && lane < HALF) {
          uint16_t* kh = reinterpret_cast<uint16_t*>(&sub_k[st][0][0]);
          kh[e0] = k0;
          kh[e1] = k1;
          kh[D + e0] = v0;
          kh[D + e1] = v1;
        }
      }
      __syncthreads();   // the angle table and the new rows, for every wave
    }
    // Then RoPE.  NeoX: element e < D/2 of slice c pairs with e + D/2 in
    // slice c + KC/2 of the same lane.  Interleaved: elements 2i, 2i+1 sit
    // next to each other in one slice.
    if (!MT) apply_qnorm();
    if (rope) {
      // One token: the angles cross lanes through this wave's LDS slab (in
      // order within the wave; each asm hides an index from per-lane alias
      // analysis, so the compiler keeps program order).  Several tokens:
      // column hn reads its token's row of the shared table.
      const float* af;
      if constexpr (MT) {
        af = &ang[tq][0];
      } else {
        float* aw = reinterpret_cast<float*>(slab);
        int aidx = fi;
        asm volatile("" : "+v"(aidx));
        if (lane < HALF) {
          aw[aidx] = cs;
          aw[HALF + aidx] = sn;
        }
        af = aw;
      }
      if (il) {
        int ridx = 4 * lg;                   // pair of element 32c + 8lg + j is 16c + 4lg + j/2
        asm volatile("" : "+v"(ridx));
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const float cc = af[ridx + 16 * c + j / 2], sv = af[HALF + ridx + 16 * c + j / 2];
            const float y1 = qf[c][j], y2 = qf[c][j + 1];
            qf[c][j] = y1 * cc - y2 * sv;
            qf[c][j + 1] = y2 * cc + y1 * sv;
          }
      } else {
        int ridx = 8 * lg;
        asm volatile("" : "+v"(ridx));
#pragma unroll
        for (int c = 0; c < KC / 2; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float cc = af[ridx + 32 * c + j], sv = af[HALF + ridx + 32 * c + j];
            const float y1 = qf[c][j], y2 = qf[c + KC / 2][j];
            qf[c][j] = y1 * cc - y2 * sv;
            qf[c + KC / 2][j] = y2 * cc + y1 * sv;
          }
      }
    }
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[c][j] *= keep;
    if (has_pro && a.q_out != nullptr && part == 0 && wave == 0 && n < NC) {
      float* qo = a.q_out + orow(n) * D;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        *reinterpret_cast<float4*>(qo + 32 * c + 8 * lg) =
            make_float4(qf[c][0], qf[c][1], qf[c][2], qf[c][3]);
        *reinterpret_cast<float4*>(qo + 32 * c + 8 * lg + 4) =
            make_float4(qf[c][4], qf[c][5], qf[c][6], qf[c][7]);
      }
    }
  } else {
    // The q loads go out first and the first tiles right behind them, so
    // waiting for q never waits for a tile (loads complete in order).
    const IT* qs = reinterpret_cast<const IT*>(a.q) + qoff;
#pragma unroll
    for (int c = 0; c < KC; ++c) load8f<IT>(qs + 32 * c + 8 * lg, qf[c]);
    __builtin_amdgcn_sched_barrier(0);
    prime();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[c][j] *= keep;
  }

  // Q^T operand: bf16 hi (+ lo) parts of q[head hn][32c + 8lg .. +8]; when
  // folded, columns n >= 8 take the lo part into qhi.
  uint4 qhi[KC], qlo[KC];
  const bool lo_col = kFold && n >= 8;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float x0 = qf[c][2 * w], x1 = qf[c][2 * w + 1];
      hw[w] = pack_bf16(x0, x1);
      lw[w] = pack_bf16(x0 - __uint_as_float(hw[w] << 16),
                        x1 - __uint_as_float(hw[w] & 0xffff0000u));
      if (lo_col) hw[w] = lw[w];
    }
    qhi[c] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    qlo[c] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }

  float m = -INFINITY;   // running max of head n (same in all four lane groups)
  float l = 0.0f;        // partial sum over this lane's rows
  f32x4_t o[VB];         // O[head 4lg + r][d = VB n + blk]
#pragma unroll
  for (int blk = 0; blk < VB; ++blk) o[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float qscale = a.qscale;

  auto compute = [&](TileBuf<D>& buf, int base) {
    // K rows -> LDS -> A operand (row pi(n), elements 32c + 8lg .. +8).  The
    // slab is private to the wave and the hardware runs one wave's LDS
    // operations in order, so no barrier is needed.  But the data crosses
    // lanes, and per-lane alias analysis would let the compiler hoist a
    // lane's reads above the other lanes' writes (or the next tile's writes
    // above these reads).  Passing each index through an empty asm statement
    // hides it from that analysis and keeps program order without a fence
    // (a fence pins the prefetch registers to scratch; volatile accesses
    // wait for every outstanding global load).
    int widx = kr * ROWU4 + kp;
    asm volatile("" : "+v"(widx));
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) slab[widx + RPI * i * ROWU4] = buf.k[i];
    // The appended row (Step only) replaces whatever was loaded for it, in
    // the slab (K) and in the registers (V): a wave-uniform test, taken for
    // at most one tile of the range.
    if constexpr (MODE == Mode::Step && MT) {
      // several tokens: rows [sub_lo, sub_hi) come from the shared table
      // (taken for at most two tiles; the asm keeps the table reads inside
      // the branch instead of letting the compiler run them every tile)
      if (sub_hi > base && sub_lo < base + 16) {     // wave-uniform
        int sk = kp, sv = VB * n;
        asm volatile("" : "+v"(sk), "+v"(sv));
        const u32x4_t* tk = &sub_k[0][0][0];
#pragma unroll
        for (int i = 0; i < 16 / RPI; ++i) {
          const int row = base + RPI * i + kr;
          if (row >= sub_lo && row < sub_hi)
            slab[widx + RPI * i * ROWU4] = tk[(row - p_new) * 2 * PPR + sk];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = base + 4 * r + lg;
          if (row >= sub_lo && row < sub_hi)
            buf.v[r].load(reinterpret_cast<const uint16_t*>(&sub_k[row - p_new][1][0]) + sv);
        }
      }
    }
    const int dp = psub - base;
    if (!MT && (unsigned)dp < 16u) {
      int cidx = dp * ROWU4 + lane;
      asm volatile("" : "+v"(cidx));
      if (lane < PPR) slab[cidx] = snew[wave][0][lane];
      int vidx = VB * n;
      asm volatile("" : "+v"(vidx));
      VRow<D> vn;
      vn.load(reinterpret_cast<const uint16_t*>(&snew[wave][1][0]) + vidx);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * r + lg == dp) buf.v[r] = vn;
    }
    int ridx = (4 * (n & 3) + (n >> 2)) * ROWU4 + lg;
    asm volatile("" : "+v"(ridx));
    u32x4_t ka[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = slab[ridx + 4 * c];
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[c]),
                                                  __builtin_bit_cast(bf16x8_t, qhi[c]), s,
                                                  0, 0, 0);
      if constexpr (kLo && !kFold)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[c]),
                                                    __builtin_bit_cast(bf16x8_t, qlo[c]), s,
                                                    0, 0, 0);
    }
    // Folded: hi (column n) + lo (column n + 8) of head n % 8, in both lanes.
    // Rows of heads >= G in the PV operand below are never stored.
    if constexpr (kFold) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] += dpp<kDppRowRor8>(s[r]);
    }
    float p[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = base + 4 * r + lg;
      const bool ok = MT ? (row >= clo && row < chi) : row < t1;
      p[r] = ok ? s[r] * qscale : -INFINITY;
      tmax = fmaxf(tmax, p[r]);
    }
    // The maximum over the four lane groups (rows) of head n, in VALU
    // permutes rather than LDS round trips.
    {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                      __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax),
                                                      __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
    }
    // Lazy rescale: the reference maximum m moves only when the tile's
    // maximum exceeds it by more than 2^8 (exp2 units), so p stays below 256
    // and, in most tiles, O is not rescaled at all (no cross-lane exchange
    // of the factors).  m = -inf (no valid row yet) always moves to a finite
    // maximum.
    const bool need = tmax > m + kRescaleLog2;
    if (__any(need)) {
      const float mnew = need ? tmax : m;
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;   // 0 from -inf
      m = mnew;
      l *= alpha;
      // Rescale O rows: row 4lg + r belongs to the head held by lane 4lg + r.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float al = __shfl(alpha, 4 * lg + r, 64);
#pragma unroll
        for (int blk = 0; blk < VB; ++blk) o[blk][r] *= al;
      }
    }
    // A column that has seen no valid row yet (m = -inf, several tokens)
    // takes its exponents against 0, which keeps p at 0 instead of NaN.
    const float mref = m == -INFINITY ? 0.0f : m;
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(p[r] - mref);
      psum += p[r];
    }
    l += psum;
    // PV on one bf16 call per column block, with the 16 tile rows as 32
    // k-indices: k = 8lg + 2r + x stands for tile row 4r + lg, x = 0 taking
    // the bf16 hi part of P and x = 1 its lo part, so V (exact in bf16) is
    // the same at both k of a row.  Lane (n, lg) already holds P[head n] of
    // exactly those rows (the A operand) and loaded V of the same rows at
    // columns VB n .. VB n + VB - 1 (the B operand of every block).
    u32x4_t pa;
#pragma unroll
    for (int r = 0; r < 4; ++r) pa[r] = split_bf16(p[r]);
#pragma unroll
    for (int blk = 0; blk < VB; ++blk) {
      u32x4_t vb;
#pragma unroll
      for (int r = 0; r < 4; ++r) vb[r] = dup_bf16<D>(buf.v[r], blk);
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, pa),
                                                       __builtin_bit_cast(bf16x8_t, vb), o[blk],
                                                       0, 0, 0);
    }
  };

  // One unit per trip, no branch inside the trip: the second tile may lie
  // wholly past the range, and then every row is masked (p = 0, and alpha =
  // 1 because the running max is already finite), which leaves the state
  // unchanged.  As soon as a tile is computed its buffer is refilled with
  // the same tile of the next unit.  A branch between a prefetch and its
  // use would let the compiler sink the loads past the compute they are
  // meant to overlap; the scheduling barriers keep the machine scheduler
  // from doing the same.
  while (rcur < t1) {
    ustep += wpp;
    const int rnext = unit_row(ustep);
    __builtin_amdgcn_sched_barrier(0);
    compute(bf[0], rcur);
    __builtin_amdgcn_sched_barrier(0);
    issue(bf[0], rnext);
    __builtin_amdgcn_sched_barrier(0);
    compute(bf[1], rcur + 16);
    __builtin_amdgcn_sched_barrier(0);
    issue(bf[1], rnext + 16);
    __builtin_amdgcn_sched_barrier(0);
    rcur = rnext;
  }

  // Sum l over the four lane groups (rows), per head n.
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  __syncthreads();                  // every wave is done with its K slab
  auto& sm_m = lds.cb.m;
  auto& sm_l = lds.cb.l;
  auto& sm_o = lds.cb.o;
  if (lg == 0 && n < NC) {
    sm_m[wave][n] = m;
    sm_l[wave][n] = l;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * lg + r;
    if (h < NC) {
#pragma unroll
      for (int blk = 0; blk < VB; ++blk) sm_o[wave][h][VB * n + blk] = o[blk][r];
    }
  }
  __syncthreads();

  // Step with a single partition writes the final output like Final.  Each
  // thread combines four consecutive d of one column over the waves of one
  // partition (one 16-byte LDS read per wave, one 16-byte store); with two
  // partitions per workgroup the index runs over both.
  const bool write_final = MODE == Mode::Final || (MODE == Mode::Step && num_parts == 1);
  constexpr int Q4 = D / 4;
  // Step: this team's partials, rows head0 .. head0 + span - 1 of ws_o
  // (column c is row head0 + (orow(c) - head0)), through one buffer
  // resource; the host keeps them below 2 GiB.
  const int64_t span = orow(NC - 1) - head0 + 1;
  const __amdgpu_buffer_rsrc_t Wrs =
      MODE == Mode::Step
          ? make_rsrc(a.ws_o + head0 * num_parts * D, (uint32_t)((size_t)span * num_parts * D * 4))
          : make_rsrc(nullptr, 0u);
  // A Step workgroup with two partitions combines them here and writes one
  // partial, at index pgrp: the merge reads half as many (for the 64-
  // partition long-context step, 64 KB per KV head instead of 128 KB, the
  // read one CU makes at the end of the launch).  Split writes one partial
  // per partition, its output contract.
  constexpr bool kPairOne = MODE == Mode::Step && ppw == 2;
  constexpr int npw = kPairOne ? 1 : ppw;   // partials written per workgroup
  for (int idx = threadIdx.x; idx < npw * CT * Q4; idx += NW * 64) {
    const int pp = npw == 1 ? 0 : idx / (CT * Q4);   // partition of the pair
    const int h = (idx / Q4) % CT;    // column
    const int d = 4 * (idx % Q4);
    const int pout = kPairOne ? pgrp : pgrp * ppw + pp;
    if (h >= NC) {                    // columns only grow with idx within a partition
      if (npw == 1) break;
      continue;
    }
    if (!kPairOne && ppw > 1 && pout >= num_parts) continue;
    // the waves of this partial: its partition's, or both partitions' (a
    // pair's missing second partition ran no rows: m = -inf, l = 0)
    auto mine = [&](int w) { return kPairOne || w / wpp == pp; };
    const int64_t oh = orow(h);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (mine(w)) M = fmaxf(M, sm_m[w][h]);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f;
    float4 A = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (!mine(w)) continue;
      const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - Ms);
      const float4 ow = *reinterpret_cast<const float4*>(&sm_o[w][h][d]);
      L += sm_l[w][h] * f;
      A.x = fmaf(ow.x, f, A.x);
      A.y = fmaf(ow.y, f, A.y);
      A.z = fmaf(ow.z, f, A.z);
      A.w = fmaf(ow.w, f, A.w);
    }
    const bool any = L > 0.0f;
    const float inv = any ? 1.0f / L : 0.0f;
    const float4 ov = float4{A.x * inv, A.y * inv, A.z * inv, A.w * inv};
    const float lse = any ? (M + log2f(L)) * kLn2 : -INFINITY;
    if (write_final) {
      if (a.out_bf16)
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + oh * D + d) =
            make_uint2(pack_bf16(ov.x, ov.y), pack_bf16(ov.z, ov.w));
      else
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oh * D + d) = ov;
      if (d == 0 && a.lse_out != nullptr) a.lse_out[oh] = lse;
    } else if (MODE == Mode::Split) {
      if (any) *reinterpret_cast<float4*>(a.ws_o + (oh * num_parts + pout) * D + d) = ov;
      if (d == 0) a.ws_lse[oh * num_parts + pout] = lse;
    } else {
      // Write-through (sc1) stores reach the coherence point, so the merging
      // workgroup (possibly on another XCD) can read them without any L2
      // writeback.
      constexpr int kCoherent = 0x10;
      if (any)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, ov), Wrs,
            (uint32_t)((((oh - head0) * num_parts + pout) * D + d) * 4), 0, kCoherent);
      if (d == 0)
        __hip_atomic_store(a.ws_lse + oh * num_parts + pout, lse, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if constexpr (MODE == Mode::Step) {
    if (num_parts == 1) return;
    // Arrival ticket: every workgroup of this (sequence, KV head) publishes
    // its partial and takes a ticket; the last one reads the partials back,
    // merges them, and resets the ticket for the next launch.  No workgroup
    // waits on another.
    //  * Release: every wave waits until its own write-through partial
    //    stores are complete (wait_vmem), then the workgroup meets at the
    //    barrier, and only then does thread 0 take the ticket.  So every
    //    partial of this workgroup is visible device-wide before the ticket
    //    moves.  (An agent-scope release fence would also write back the
    //    whole L2 of the XCD, per workgroup; the partials are write-through
    //    and need only the wait.)
    //  * Acquire: the last arriver alone takes an agent-scope acquire fence
    //    before it reads, and reads the partials with device-coherent loads.
    wait_vmem();
    __syncthreads();
    __shared__ int s_last;
    uint32_t* ticket = a.ws_cnt + (int64_t)b * Hkv + g;
    if (threadIdx.x == 0) {
      // one arrival per partition this workgroup holds
      const uint32_t cnt = ppw == 1 ? 1u : (uint32_t)min(ppw, num_parts - pgrp * ppw);
      const uint32_t old = __hip_atomic_fetch_add(ticket, cnt, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old + cnt == (uint32_t)num_parts;
      // the acquire: one wave invalidates the CU's and the XCD's caches
      // before the barrier that the other waves' reads follow (an
      // invalidation per wave cost up to 3 us on an eight-wave workgroup)
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    merge_partials<D, CT, NW, MT>(a, head0, G, NC, kPairOne ? npg : num_parts);
    if (threadIdx.x == 0)
      __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Waves per partition: four, one per SIMD of the CU (eight per workgroup
// when a workgroup holds two partitions).
constexpr int kWavesPerGroup = 4;

// Long-context launches (single token, Split or Step, at least kPairParts
// partitions per (sequence, KV head) and kPairFrom partitions in all) run
// two partitions per workgroup on eight waves: one workgroup per CU with
// four waves per partition.  Measured on the 64-partition long-context
// step (537 MB): 91.8 -> 87.0 us, the slowest XCD's loop ending earlier
// than with two four-wave workgroups per CU, of which the one dispatched
// first takes most of the CU's bandwidth.  Ragged batches (few partitions
// per sequence, many of them short or empty) keep one partition per
// workgroup, whose finer grain the dispatcher balances (pairs cost 6 us on
// the ragged Llama-3-8B batch).
constexpr int kPairParts = 16;
constexpr int64_t kPairFrom = 512;

template <int D, int CT, typename IT, Mode MODE>
static int launch_mode(const KernelArgs& a, hipStream_t s) {
  bool multi = false;
  if constexpr (CT > 1) multi = a.S > 1;   // one column holds one token
  const int64_t total = (int64_t)a.num_parts * a.B * a.Hkv;
  const bool pair = MODE != Mode::Final && !multi && a.num_parts >= kPairParts &&
                    total >= kPairFrom;
  if (pair) {
    if constexpr (MODE != Mode::Final) {
      constexpr int NW = 2 * kWavesPerGroup;
      const dim3 grid((a.num_parts + 1) / 2 * a.B * a.Hkv);
      hipLaunchKernelGGL((attn_decode_mfma_kernel<D, CT, NW, 2, IT, MODE, false>), grid,
                         dim3(NW * 64), 0, s, a);
    }
  } else {
    constexpr int NW = kWavesPerGroup;
    const dim3 grid((MODE == Mode::Final ? 1 : a.num_parts) * a.B * a.Hkv);
    if (multi)
      hipLaunchKernelGGL((attn_decode_mfma_kernel<D, CT, NW, 1, IT, MODE, CT != 1>), grid,
                         dim3(NW * 64), 0, s, a);
    else
      hipLaunchKernelGGL((attn_decode_mfma_kernel<D, CT, NW, 1, IT, MODE, false>), grid,
                         dim3(NW * 64), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

// Column capacity: the smallest power of two holding G * S query rows.
template <int D, typename IT, Mode MODE>
static int dispatch_g(const KernelArgs& a, hipStream_t s) {
  const int nc = (a.Hq / a.Hkv) * a.S;
  switch (nc <= 1 ? 1 : nc <= 2 ? 2 : nc <= 4 ? 4 : nc <= 8 ? 8 : nc <= 16 ? 16 : 0) {
    case 1: return launch_mode<D, 1, IT, MODE>(a, s);
    case 2: return launch_mode<D, 2, IT, MODE>(a, s);
    case 4: return launch_mode<D, 4, IT, MODE>(a, s);
    case 8: return launch_mode<D, 8, IT, MODE>(a, s);
    case 16: return launch_mode<D, 16, IT, MODE>(a, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

template <Mode MODE>
static int dispatch(const KernelArgs& a, hipStream_t s) {
  if (a.D == 128)
    return a.in_bf16 ? dispatch_g<128, uint16_t, MODE>(a, s) : dispatch_g<128, float, MODE>(a, s);
  if (a.D == 64)
    return a.in_bf16 ? dispatch_g<64, uint16_t, MODE>(a, s) : dispatch_g<64, float, MODE>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

int launch_attn_final(const KernelArgs& a, hipStream_t s) { return dispatch<Mode::Final>(a, s); }
int launch_attn_split(const KernelArgs& a, hipStream_t s) { return dispatch<Mode::Split>(a, s); }
int launch_decode_step(const KernelArgs& a, hipStream_t s) { return dispatch<Mode::Step>(a, s); }

}  // namespace gqa
