// Single-token GQA decode attention on gfx950 matrix cores.
//
// Computes what the fusedtok 1.0.1 README ("Operators" row attention_decode)
// describes -- single-token GQA attention over a contiguous KV cache with
// online softmax, per-sequence lengths and a flash-decoding split -- plus the
// sliding window of the cutileGPT README feature list.  Same decomposition
// as the VALU kernel: one workgroup per (partition, KV head, sequence)
// covering all G query heads of that KV head, each K/V row read once.
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

template <int D>
struct VRow;   // lane's slice of one V row: D/16 bf16
template <>
struct VRow<128> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void unpack(float f[8]) const { unpack8(v, f); }
};
template <>
struct VRow<64> {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint2(0, 0); }
  __device__ __forceinline__ void unpack(float f[4]) const {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  }
};

template <typename QT>
__device__ __forceinline__ void load_q8f(const QT* p, float f[8]);
template <>
__device__ __forceinline__ void load_q8f<float>(const float* p, float f[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <>
__device__ __forceinline__ void load_q8f<uint16_t>(const uint16_t* p, float f[8]) {
  unpack8(*reinterpret_cast<const uint4*>(p), f);
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

template <int D>
struct TileBuf {
  u32x4_t k[D / 32];   // K rows, whole-row pieces: lane's 16 bytes of D/32 rows
  VRow<D> v[4];        // V rows 4i + g, i < 4
};

template <int D, int G, int NW, typename QT, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_decode_mfma_kernel(
    const QT* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ lens, int window,
    float qscale, int part_tokens, int num_parts, int Hq, int Hkv, int T,
    float* __restrict__ ws_lse, float* __restrict__ ws_o, void* __restrict__ out,
    int out_bf16, float* __restrict__ lse_out) {
  static_assert(G <= 16, "one 16-column MFMA tile holds at most 16 heads");
  constexpr int KC = D / 32;          // QK calls per tile (per q part)
  constexpr int VB = D / 16;          // PV column blocks
  constexpr bool kLo = sizeof(QT) == 4;   // fp32 q needs the lo part

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int lg = lane >> 4;

  const int nrow = min(max(lens[b], 0), T);
  const int lo = window > 0 ? max(0, nrow - window) : 0;
  int t0 = lo, t1 = nrow;
  if (SPLIT) {
    t0 = min(lo + part * part_tokens, nrow);
    t1 = min(t0 + part_tokens, nrow);
  }
  const int64_t head0 = (int64_t)b * Hq + (int64_t)g * G;

  if (t0 >= t1) {
    if (SPLIT) {
      for (int h = threadIdx.x; h < G; h += NW * 64)
        ws_lse[(head0 + h) * num_parts + part] = -INFINITY;
    } else {
      for (int e = threadIdx.x; e < G * D; e += NW * 64) {
        if (out_bf16) reinterpret_cast<uint16_t*>(out)[head0 * D + e] = 0;
        else reinterpret_cast<float*>(out)[head0 * D + e] = 0.0f;
      }
      if (lse_out != nullptr)
        for (int h = threadIdx.x; h < G; h += NW * 64) lse_out[head0 + h] = -INFINITY;
    }
    return;
  }

  float m = -INFINITY;   // running max of head n (same in all four lane groups)
  float l = 0.0f;        // partial sum over this lane's rows
  f32x4_t o[VB];         // O[head 4lg + r][d = VB n + blk]
#pragma unroll
  for (int blk = 0; blk < VB; ++blk) o[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t slab = ((int64_t)b * Hkv + g) * T * D;
  // K whole-row layout: a load covers RPI rows; lane l takes 16-byte piece
  // kp = l % PPR of row RPI*i + kr.
  constexpr int PPR = D / 8;            // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;         // rows per load instruction
  constexpr int ROWU4 = PPR + 1;        // padded LDS row, in 16-byte units
  const int kp = lane % PPR;
  const int kr = lane / PPR;
  const uint16_t* Kbase = k_cache + slab + 8 * kp;           // + row*D
  const uint16_t* Vbase = v_cache + slab + VB * n;           // + row*D
  __shared__ u32x4_t sk[NW][16][ROWU4];

  // Loads are unconditional: a row index past the range is clamped to the
  // last valid row (an attended row, so finite), and the softmax gives such
  // rows p = 0.  With no branches around the loads the compiler can count
  // them exactly and wait only for the tile being computed.
  auto issue = [&](TileBuf<D>& buf, int base) {
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int rk = min(base + RPI * i + kr, t1 - 1);
      buf.k[i] = *reinterpret_cast<const u32x4_t*>(Kbase + (int64_t)rk * D);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rv = min(base + 4 * i + lg, t1 - 1);
      buf.v[i].load(Vbase + (int64_t)rv * D);
    }
  };

  constexpr int STEP = NW * 16;
  int base = t0 + wave * 16;
  TileBuf<D> b0, b1;
  if (base < t1) issue(b0, base);      // first tile in flight before q is read
  // Q^T operand: lane holds q[head n][32c + 8lg .. +8] as bf16 hi (+ lo).
  // All q loads are issued before any is used (one memory round trip).
  uint4 qhi[KC], qlo[KC];
  {
    // Columns n >= G are padding: they load head G-1 (no branch around the
    // loads) and are zeroed.
    const float keep = n < G ? 1.0f : 0.0f;
    const int hq = min(n, G - 1);
    float qf[KC][8];
#pragma unroll
    for (int c = 0; c < KC; ++c) load_q8f<QT>(q + (head0 + hq) * D + 32 * c + 8 * lg, qf[c]);
    __builtin_amdgcn_sched_barrier(0);   // keep the q loads in one batch
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[c][j] *= keep;
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
  }

  auto compute = [&](const TileBuf<D>& buf, int base) {
    // K rows -> LDS -> A operand (row n, elements 32c + 8lg .. +8).  The slab
    // is private to the wave and the hardware runs one wave's LDS operations
    // in order, so no barrier is needed.  But the data crosses lanes, and
    // per-lane alias analysis would let the compiler hoist a lane's reads
    // above the other lanes' writes (or the next tile's writes above these
    // reads).  Passing each index through an empty asm statement hides it
    // from that analysis and keeps program order without a fence (a fence
    // pins the prefetch registers to scratch; volatile accesses wait for
    // every outstanding global load).
    u32x4_t* slab = &sk[wave][0][0];
    int widx = (RPI * 0 + kr) * ROWU4 + kp;
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
      const float a = __shfl(alpha, 4 * lg + r, 64);
#pragma unroll
      for (int blk = 0; blk < VB; ++blk) o[blk][r] *= a;
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

  // Two tiles per trip, no branch inside the trip: the second tile may lie
  // wholly past the range, and then every row is masked (p = 0, and alpha = 1
  // because the running max is already finite), which leaves the state
  // unchanged.  A branch between a prefetch and its use would let the
  // compiler sink the loads past the compute they are meant to overlap; the
  // scheduling barriers keep the machine scheduler from doing the same.
  if (base < t1) {
    for (; base < t1; base += 2 * STEP) {
      issue(b1, base + STEP);
      __builtin_amdgcn_sched_barrier(0);
      compute(b0, base);
      issue(b0, base + 2 * STEP);
      __builtin_amdgcn_sched_barrier(0);
      compute(b1, base + STEP);
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
    if (SPLIT) {
      ws_o[((head0 + h) * num_parts + part) * D + d] = ov;
      if (d == 0) ws_lse[(head0 + h) * num_parts + part] = lse;
    } else {
      if (out_bf16) reinterpret_cast<uint16_t*>(out)[(head0 + h) * D + d] = f32_to_bf16(ov);
      else reinterpret_cast<float*>(out)[(head0 + h) * D + d] = ov;
      if (d == 0 && lse_out != nullptr) lse_out[head0 + h] = lse;
    }
  }
}

#ifndef GQA_MFMA_NW
#define GQA_MFMA_NW 4
#endif

template <int D, int G, typename QT>
static int launch_mfma_t(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = GQA_MFMA_NW;
  const dim3 block(NW * 64);
  if (a.split) {
    const dim3 grid(a.num_parts, a.Hkv, a.B);
    hipLaunchKernelGGL((attn_decode_mfma_kernel<D, G, NW, QT, true>), grid, block, 0, s,
                       (const QT*)a.q, a.k_cache, a.v_cache, a.lens, a.window, a.qscale,
                       a.part_tokens, a.num_parts, a.Hq, a.Hkv, a.T, a.ws_lse, a.ws_o,
                       nullptr, 0, nullptr);
  } else {
    const dim3 grid(1, a.Hkv, a.B);
    hipLaunchKernelGGL((attn_decode_mfma_kernel<D, G, NW, QT, false>), grid, block, 0, s,
                       (const QT*)a.q, a.k_cache, a.v_cache, a.lens, a.window, a.qscale,
                       0, 1, a.Hq, a.Hkv, a.T, nullptr, nullptr, a.out, a.out_bf16,
                       a.lse_out);
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <int D, typename QT>
static int dispatch_mfma_g(const AttnArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_mfma_t<D, 1, QT>(a, s);
    case 2: return launch_mfma_t<D, 2, QT>(a, s);
    case 4: return launch_mfma_t<D, 4, QT>(a, s);
    case 8: return launch_mfma_t<D, 8, QT>(a, s);
    case 16: return launch_mfma_t<D, 16, QT>(a, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.D == 128)
    return a.q_bf16 ? dispatch_mfma_g<128, uint16_t>(a, s) : dispatch_mfma_g<128, float>(a, s);
  if (a.D == 64)
    return a.q_bf16 ? dispatch_mfma_g<64, uint16_t>(a, s) : dispatch_mfma_g<64, float>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
