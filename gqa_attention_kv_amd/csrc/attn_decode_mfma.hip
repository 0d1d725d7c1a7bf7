// Single-token GQA decode attention on gfx950 matrix cores, in three modes
// that share one body:
//   Final  one workgroup per (sequence, KV head) writes the output directly;
//   Split  one workgroup per (partition, KV head, sequence) writes the
//          partition's (o_k, lse_k) for the log-sum-exp merge;
//   Step   the whole decode step in one launch: per-head QK-RMSNorm and NeoX
//          RoPE of the new query, the K/V append, the split-K pass, and the
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
// deliver it at 6.4 TB/s.  Both contractions run on MFMA instead, leaving
// the VALU only the bf16->fp32 widening of V and the softmax.
//
// Tiles of 16 rows.  Lane l, with n = l % 16 and g = l / 16:
//   QK: S^T[16 rows x 16 heads] += K[16 x 32] * Q^T[32 x 16] with
//       v_mfma_f32_16x16x32_bf16, one call per 32-wide slice of D.  The A
//       operand wants lane l to hold row n, elements 32c + 8g..+8.  Loading
//       that directly makes every load instruction touch 16 rows x 64 bytes,
//       which streams at only ~4.1 TB/s on MI355X against ~5.2 TB/s for
//       instructions that read whole 256-byte rows.  So K is loaded like V,
//       whole rows, and passes through a wave-private LDS slab (rows padded
//       to D*2+16 bytes: conflict-free for both the row writes and the
//       operand reads).  q is split into bf16 hi + lo parts (two calls) so
//       scores keep ~16 mantissa bits; a bf16 q needs the hi call only.
//       Heads >= G are zero columns.  A-operand row m is fed tile row
//       pi(m) = 4(m%4) + m/4, so the result leaves lane l holding S for tile
//       rows 4r + g (r < 4) of head n.
//   PV: O[16 heads x 16 cols] += P[16 x 4] * V[4 x 16] with
//       v_mfma_f32_16x16x4_f32, four calls per tile (call i takes tile rows
//       4i..4i+3, row 4i + g in lane group g) times D/16 column blocks.
//       P's A operand (head n, row 4i+g) is exactly the register the QK step
//       left in lane l, so no cross-lane movement is needed.  Output column
//       n of block b stands for d = (D/16) n + b, which makes lane l's V
//       operand for all blocks one contiguous (D/8)-byte load of row 4i+g:
//       a wave-wide load reads 4 consecutive rows, 1 KiB contiguous for
//       D = 128.  fp32 keeps P and V exact.
// Loads for tile j+1 are issued before tile j is computed (register double
// buffer, branch-free trips of two tiles), and waves of a workgroup take
// interleaved tiles.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;   // 16 bytes, register type

enum class Mode { Final, Split, Step };

template <int D>
struct VRow;   // lane's slice of one V row: D/16 bf16
template <>
struct VRow<128> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void unpack(float f[8]) const { unpack8(v, f); }
};
template <>
struct VRow<64> {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void unpack(float f[4]) const {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  }
};

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

#ifndef GQA_WAVES_PER_EU
#define GQA_WAVES_PER_EU 3
#endif
#ifndef GQA_STAGES
#define GQA_STAGES 2
#endif

template <int D, int G, int NW, typename IT, Mode MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(GQA_WAVES_PER_EU))) void
attn_decode_mfma_kernel(const KernelArgs a) {
  static_assert(G <= 16, "one 16-column MFMA tile holds at most 16 heads");
  constexpr int KC = D / 32;          // QK calls per tile (per q part)
  constexpr int VB = D / 16;          // PV column blocks
  constexpr int HALF = D / 2;
  // fp32 q (given, or the prologue's rotated q) needs the lo part
  constexpr bool kLo = sizeof(IT) == 4 || MODE == Mode::Step;
  constexpr bool kPartial = MODE != Mode::Final;

  // One-dimensional grid.  The hardware hands workgroup i to XCD i % 8.
  // With 8 or more partitions per (sequence, KV head) the partition index
  // runs fastest, so consecutive partitions of one sequence land on
  // consecutive XCDs.  With fewer, it runs slowest: workgroup i takes
  // partition i / (B*Hkv) of (sequence, KV head) i % (B*Hkv), so every XCD
  // gets the same mix of partitions -- partition 0 of every sequence is the
  // one that is never empty under ragged lengths -- and the dispatcher
  // starts all first partitions before any later one.  (Partition-fastest
  // order with few partitions puts every partition 0 on the same two XCDs;
  // partition-major order with many partitions per sequence measured slower
  // and sensitive to where the K and V caches sit relative to each other.)
  const int nbg = a.B * a.Hkv;
  const int npg = MODE == Mode::Final ? 1 : a.num_parts;
  int part, bg;
  if (npg >= 8) {
    bg = (int)blockIdx.x / npg;
    part = (int)blockIdx.x - bg * npg;
  } else {
    part = (int)blockIdx.x / nbg;
    bg = (int)blockIdx.x - part * nbg;
  }
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int lg = lane >> 4;
  const int T = a.T;
  const int Hq = a.Hq;
  const int Hkv = a.Hkv;
  const int num_parts = a.num_parts;

  const int nrow = min(max(a.lens[b], 0), T);
  const int lo = a.window > 0 ? max(0, nrow - a.window) : 0;
  int t0 = lo, t1 = nrow;
  if (kPartial) {
    t0 = min(lo + part * a.part_tokens, nrow);
    t1 = min(t0 + a.part_tokens, nrow);
  }
  const int64_t head0 = (int64_t)b * Hq + (int64_t)g * G;

  if constexpr (MODE != Mode::Step) {
    if (t0 >= t1) {   // nothing to attend in this range (uniform over the workgroup)
      if (MODE == Mode::Split) {
        for (int h = threadIdx.x; h < G; h += NW * 64)
          a.ws_lse[(head0 + h) * num_parts + part] = -INFINITY;
      } else {
        for (int e = threadIdx.x; e < G * D; e += NW * 64) {
          if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[head0 * D + e] = 0;
          else reinterpret_cast<float*>(a.out)[head0 * D + e] = 0.0f;
        }
        if (a.lse_out != nullptr)
          for (int h = threadIdx.x; h < G; h += NW * 64) a.lse_out[head0 + h] = -INFINITY;
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
  const uint16_t* Kbase = a.k_cache + slab_off + 8 * kp;        // + row*D
  const uint16_t* Vbase = a.v_cache + slab_off + VB * n;        // + row*D
  __shared__ u32x4_t sk[NW][16][ROWU4];
  u32x4_t* slab = &sk[wave][0][0];

  // Loads are unconditional: a row index past the range is clamped to the
  // last valid row (an attended row, so finite; row 0 when the range is
  // empty), and the softmax gives such rows p = 0.  With no branches around
  // the loads the compiler can count them exactly and wait only for the tile
  // being computed.
  const int rlast = max(t1 - 1, 0);
  auto issue_from = [&](TileBuf<D>& buf, int base, const uint16_t* kb, const uint16_t* vb,
                        int rstride) {
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int rk = min(base + RPI * i + kr, rlast);
      buf.k[i] = *reinterpret_cast<const u32x4_t*>(kb + (int64_t)rk * rstride);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rv = min(base + 4 * i + lg, rlast);
      buf.v[i].load(vb + (int64_t)rv * rstride);
    }
  };
  auto issue = [&](TileBuf<D>& buf, int base) { issue_from(buf, base, Kbase, Vbase, D); };

  constexpr int STEP = NW * 16;
  constexpr int S = GQA_STAGES;        // register tile buffers
  int base = t0 + wave * 16;
  TileBuf<D> bf[S];
  auto prime = [&]() {                 // the S tiles of the first trip
#pragma unroll
    for (int s = 0; s < S; ++s) issue(bf[s], base + s * STEP);
  };

  // q for head n (padding columns n >= G load head G-1 -- no branch around
  // the loads -- and are zeroed): lane holds elements 32c + 8lg + j.
  const float keep = n < G ? 1.0f : 0.0f;
  const int hq = min(n, G - 1);
  float qf[KC][8];

  if constexpr (MODE == Mode::Step) {
    // ---- fused prologue: QK-RMSNorm, NeoX RoPE at pos[b], K/V append ----
    // (skipped when no prologue inputs are given: q is then used as is)
    const bool has_pro = a.pos != nullptr;
    const int p = has_pro ? a.pos[b] : -1;
    // The row pos[b] is written by the workgroup whose partition attends it
    // (or partition 0 when it is not attended); positions outside [0, T)
    // write nothing.  No other workgroup reads that row.
    const bool in_range = has_pro && p >= 0 && p < T;
    const bool attended = p >= lo && p < nrow;
    const bool writer = in_range && (attended ? (p >= t0 && p < t1) : part == 0);
    const bool reads_row = writer && attended;
    // Every global load of the prologue is issued before the first tiles:
    // loads complete in order, so waiting for these never waits for a tile.
    const IT* qs = reinterpret_cast<const IT*>(a.q) + (int64_t)b * a.q_bstride +
                   (int64_t)(g * G + hq) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) load8f<IT>(qs + 32 * c + 8 * lg, qf[c]);
    const bool qnorm = has_pro && a.wq != nullptr;
    const bool rope = has_pro && a.rope;
    float wq8[KC][8];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (qnorm) load8f<float>(a.wq + 32 * c + 8 * lg, wq8[c]);
    }
    const int fi = lane % HALF;               // rotary frequency index of this lane
    const double inv_rev = rope ? a.inv_freq_rev[fi] : 0.0;
    const bool kwrite = writer && wave == 0;
    // raw values: converted only after the tiles are issued
    IT rx0 = 0, rx1 = 0, rv0 = 0, rv1 = 0;
    float wk0 = 1.0f, wk1 = 1.0f;
    if (kwrite) {
      const IT* ks = reinterpret_cast<const IT*>(a.k_new) + (int64_t)b * a.kv_bstride +
                     (int64_t)g * D;
      const IT* vs = reinterpret_cast<const IT*>(a.v_new) + (int64_t)b * a.kv_bstride +
                     (int64_t)g * D;
      rx0 = ks[fi];
      rx1 = ks[fi + HALF];
      rv0 = vs[fi];
      rv1 = vs[fi + HALF];
      if (a.wk != nullptr) {
        wk0 = a.wk[fi];
        wk1 = a.wk[fi + HALF];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // A writer whose appended row falls in the first tiles issues them only
    // after the append; until then its buffers are filled from its own q row
    // (same number of loads, so the compiler still counts them exactly, and
    // every lane's pieces stay inside that row: it holds D elements of at
    // least 2 bytes).  Otherwise no primed row is the appended one: a
    // partition holding pos past its first S tiles has more rows than those
    // tiles cover, so none of their rows is clamped.
    const bool late = reads_row && (p - t0) < S * STEP;
    {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(qs);
      const uint16_t* kb = late ? qrow + 8 * kp : Kbase;
      const uint16_t* vb = late ? qrow + VB * n : Vbase;
      const int rs = late ? 0 : D;
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) issue_from(bf[s2], base + s2 * STEP, kb, vb, rs);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Rotary angle of frequency index fi: the phase p * theta^(-2fi/D) / (2 pi)
    // is formed and reduced in float64 from a host-computed table, leaving a
    // float32 sincos of an angle in [-pi, pi].
    float cs = 1.0f, sn = 0.0f;
    if (rope) {
      const double rev = (double)p * inv_rev;
      const double fr = rev - rint(rev);
      sincosf((float)(fr * 6.283185307179586), &sn, &cs);
    }
    if (kwrite) {
      float x0 = to_f32(rx0), x1 = to_f32(rx1);
      if (a.wk != nullptr) {
        const float ss = group_sum_shfl<HALF>(x0 * x0 + x1 * x1);
        const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
        x0 = x0 * r * wk0;
        x1 = x1 * r * wk1;
      }
      if (a.rope) {
        const float y0 = x0 * cs - x1 * sn, y1 = x1 * cs + x0 * sn;
        x0 = y0;
        x1 = y1;
      }
      if (lane < HALF) {
        uint16_t* krow = a.k_cache_w + slab_off + (int64_t)p * D;
        uint16_t* vrow = a.v_cache_w + slab_off + (int64_t)p * D;
        krow[fi] = f32_to_bf16(x0);
        krow[fi + HALF] = f32_to_bf16(x1);
        vrow[fi] = bits_bf16(&rv0, 0);
        vrow[fi + HALF] = bits_bf16(&rv1, 0);
      }
      if (reads_row) __threadfence_block();   // the row is visible before the barrier
    }
    // Query head g*G + hq: RMSNorm over D (the lane's D/4 elements, summed
    // over the four lane groups of head n), then RoPE: element e < D/2 of
    // slice c pairs with e + D/2 in slice c + KC/2 of the same lane.
    if (qnorm) {
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
    }
    if (rope) {
      // Hand the angles across lanes through this wave's LDS slab (in-order
      // LDS; the asm hides the indices from per-lane alias analysis).
      float* af = reinterpret_cast<float*>(slab);
      int aidx = fi;
      asm volatile("" : "+v"(aidx));
      if (lane < HALF) {
        af[aidx] = cs;
        af[HALF + aidx] = sn;
      }
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
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[c][j] *= keep;
    if (has_pro && a.q_out != nullptr && part == 0 && wave == 0 && n < G) {
      float* qo = a.q_out + (head0 + n) * D;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        *reinterpret_cast<float4*>(qo + 32 * c + 8 * lg) =
            make_float4(qf[c][0], qf[c][1], qf[c][2], qf[c][3]);
        *reinterpret_cast<float4*>(qo + 32 * c + 8 * lg + 4) =
            make_float4(qf[c][4], qf[c][5], qf[c][6], qf[c][7]);
      }
    }
    if (reads_row) {
      __syncthreads();                  // appended row written before it is loaded
      if (late) prime();
    }
  } else {
    // The q loads go out first and the first tiles right behind them, so
    // waiting for q never waits for a tile (loads complete in order).
    const IT* qs = reinterpret_cast<const IT*>(a.q) + (head0 + hq) * D;
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

  // Q^T operand: bf16 hi (+ lo) parts of q[head n][32c + 8lg .. +8].
  uint4 qhi[KC], qlo[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    uint16_t h16[8], l16[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h16[j] = f32_to_bf16(qf[c][j]);
      l16[j] = f32_to_bf16(qf[c][j] - bf16_to_f32(h16[j]));
    }
    qhi[c] = make_uint4(pack2(h16[0], h16[1]), pack2(h16[2], h16[3]),
                        pack2(h16[4], h16[5]), pack2(h16[6], h16[7]));
    qlo[c] = make_uint4(pack2(l16[0], l16[1]), pack2(l16[2], l16[3]),
                        pack2(l16[4], l16[5]), pack2(l16[6], l16[7]));
  }

  float m = -INFINITY;   // running max of head n (same in all four lane groups)
  float l = 0.0f;        // partial sum over this lane's rows
  f32x4_t o[VB];         // O[head 4lg + r][d = VB n + blk]
#pragma unroll
  for (int blk = 0; blk < VB; ++blk) o[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float qscale = a.qscale;

  auto compute = [&](const TileBuf<D>& buf, int base) {
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
      if constexpr (kLo)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[c]),
                                                    __builtin_bit_cast(bf16x8_t, qlo[c]), s,
                                                    0, 0, 0);
    }
    float p[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = base + 4 * r + lg < t1;
      p[r] = ok ? s[r] * qscale : -INFINITY;
      tmax = fmaxf(tmax, p[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // finite: the trip's first tile always holds a valid row
    const float mnew = fmaxf(m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(p[r] - mnew);
      psum += p[r];
    }
    l = l * alpha + psum;
    // Rescale O rows: row 4lg + r belongs to the head held by lane 4lg + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float al = __shfl(alpha, 4 * lg + r, 64);
#pragma unroll
      for (int blk = 0; blk < VB; ++blk) o[blk][r] *= al;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vf[VB];
      buf.v[i].unpack(vf);
#pragma unroll
      for (int blk = 0; blk < VB; ++blk)
        o[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[i], vf[blk], o[blk], 0, 0, 0);
    }
  };

  // S tiles per trip, no branch inside the trip: tiles after the first may
  // lie wholly past the range, and then every row is masked (p = 0, and
  // alpha = 1 because the running max is already finite), which leaves the
  // state unchanged.  As soon as tile s is computed its buffer is refilled
  // with the tile one trip ahead, so S - 1 tiles are in flight behind each
  // compute (and S were issued before the first).  A branch between a
  // prefetch and its use would let the compiler sink the loads past the
  // compute they are meant to overlap; the scheduling barriers keep the
  // machine scheduler from doing the same.
  if (base < t1) {
    for (; base < t1; base += S * STEP) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        compute(bf[s], base + s * STEP);
        __builtin_amdgcn_sched_barrier(0);
        issue(bf[s], base + (s + S) * STEP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Sum l over the four lane groups (rows), per head n.
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_o[NW][G][D];
  if (lg == 0 && n < G) {
    sm_m[wave][n] = m;
    sm_l[wave][n] = l;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * lg + r;
    if (h < G) {
#pragma unroll
      for (int blk = 0; blk < VB; ++blk) sm_o[wave][h][VB * n + blk] = o[blk][r];
    }
  }
  __syncthreads();

  // Step with a single partition writes the final output like Final.
  const bool write_final = MODE == Mode::Final || (MODE == Mode::Step && num_parts == 1);
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - Ms);
      L += sm_l[w][h] * f;
      A += sm_o[w][h][d] * f;
    }
    const bool any = L > 0.0f;
    const float ov = any ? A / L : 0.0f;
    const float lse = any ? (M + log2f(L)) * kLn2 : -INFINITY;
    if (write_final) {
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[(head0 + h) * D + d] = f32_to_bf16(ov);
      else reinterpret_cast<float*>(a.out)[(head0 + h) * D + d] = ov;
      if (d == 0 && a.lse_out != nullptr) a.lse_out[head0 + h] = lse;
    } else if (MODE == Mode::Split) {
      if (any) a.ws_o[((head0 + h) * num_parts + part) * D + d] = ov;
      if (d == 0) a.ws_lse[(head0 + h) * num_parts + part] = lse;
    } else {
      // Agent-scope stores write through to the coherence point, so the
      // merging workgroup (possibly on another XCD) can read them without
      // any L2 writeback.
      if (any)
        __hip_atomic_store(a.ws_o + ((head0 + h) * num_parts + part) * D + d, ov,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0)
        __hip_atomic_store(a.ws_lse + (head0 + h) * num_parts + part, lse, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if constexpr (MODE == Mode::Step) {
    if (num_parts == 1) return;
    // Arrival ticket: every workgroup of this (sequence, KV head) publishes
    // its partial, waits until those write-through stores have completed,
    // and takes a ticket; the last one reads the partials back with
    // agent-scope loads (which do not hit stale L2 lines), merges them in
    // ascending partition order, and resets the ticket for the next launch.
    // No workgroup waits on another.  Agent-scope fences would write back or
    // invalidate a whole L2 per workgroup, which costs more than the step.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // stores completed
    __syncthreads();
    __shared__ int s_last;
    uint32_t* ticket = a.ws_cnt + (int64_t)b * Hkv + g;
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (uint32_t)(num_parts - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // Merge, in ascending partition order.  Thread pair j owns output (h, d);
    // h is the same across a wave (G*D and D are multiples of 64).  The LSEs
    // of 64 partitions sit one per lane and are read back with readlane, and
    // each chunk of MC partials is loaded in one batch together with them,
    // so a merge of up to MC partitions is a single memory round trip.
    constexpr int NTH = NW * 64;
    constexpr int PAIRS = (G * D + NTH - 1) / NTH;   // (head, d) outputs per thread
    constexpr int MC = PAIRS >= 8 ? 4 : 32 / PAIRS;
    float Mx[PAIRS], Wx[PAIRS], Ax[PAIRS];
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
      Mx[j] = -INFINITY;
      Wx[j] = 0.0f;
      Ax[j] = 0.0f;
    }
    for (int kb = 0; kb < num_parts; kb += 64) {
      const int kn = min(64, num_parts - kb);
      float lsev[PAIRS];
#pragma unroll
      for (int j = 0; j < PAIRS; ++j) {
        const int h = min((int)(threadIdx.x + j * NTH) / D, G - 1);
        lsev[j] = __hip_atomic_load(a.ws_lse + (head0 + h) * num_parts + kb + min(lane, kn - 1),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      for (int kc = 0; kc < kn; kc += MC) {
        float ov[PAIRS][MC];
#pragma unroll
        for (int j = 0; j < PAIRS; ++j) {
          const int idx = min((int)threadIdx.x + j * NTH, G * D - 1);
          const float* Op = a.ws_o + ((head0 + idx / D) * num_parts + kb) * D + idx % D;
#pragma unroll
          for (int k = 0; k < MC; ++k)    // rows past kn stay inside the workspace
            ov[j][k] = __hip_atomic_load(const_cast<float*>(Op) + (int64_t)min(kc + k, kn - 1) * D,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < PAIRS; ++j) {
          float lk[MC];
          float cm = -INFINITY;
#pragma unroll
          for (int k = 0; k < MC; ++k) {
            const float v = __builtin_amdgcn_readlane(__float_as_int(lsev[j]), min(kc + k, 63));
            lk[k] = kc + k < kn ? __int_as_float(v) : -INFINITY;
            cm = fmaxf(cm, lk[k]);
          }
          const float Mn = fmaxf(Mx[j], cm);
          if (Mn == -INFINITY) continue;
          const float sc = __expf(Mx[j] - Mn);          // 0 while nothing was seen
          float W = Wx[j] * sc, A = Ax[j] * sc;
#pragma unroll
          for (int k = 0; k < MC; ++k) {
            const float w = lk[k] == -INFINITY ? 0.0f : __expf(lk[k] - Mn);
            W += w;
            A = fmaf(w, lk[k] == -INFINITY ? 0.0f : ov[j][k], A);   // undefined o_k where empty
          }
          Mx[j] = Mn;
          Wx[j] = W;
          Ax[j] = A;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
      const int idx = threadIdx.x + j * NTH;
      if (idx >= G * D) break;
      const int h = idx / D;
      const int d = idx % D;
      const bool any = Wx[j] > 0.0f;
      const float ov = any ? Ax[j] / Wx[j] : 0.0f;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[(head0 + h) * D + d] = f32_to_bf16(ov);
      else reinterpret_cast<float*>(a.out)[(head0 + h) * D + d] = ov;
      if (d == 0 && a.lse_out != nullptr)
        a.lse_out[head0 + h] = any ? Mx[j] + logf(Wx[j]) : -INFINITY;
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

#ifndef GQA_MFMA_NW
#define GQA_MFMA_NW 4
#endif

template <int D, int G, typename IT, Mode MODE>
static int launch_mode(const KernelArgs& a, hipStream_t s) {
  constexpr int NW = GQA_MFMA_NW;
  const dim3 grid((MODE == Mode::Final ? 1 : a.num_parts) * a.B * a.Hkv);
  hipLaunchKernelGGL((attn_decode_mfma_kernel<D, G, NW, IT, MODE>), grid, dim3(NW * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <int D, typename IT, Mode MODE>
static int dispatch_g(const KernelArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
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
