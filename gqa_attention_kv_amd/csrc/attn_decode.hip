// Single-token GQA decode attention over a bf16 KV cache, for gfx950.
//
// Follows the fusedtok 1.0.1 README, "Operators" row attention_decode
// (single-token causal attention with GQA over a contiguous KV cache,
// online softmax, flash-decoding split over long caches, per-sequence
// lengths) and "Usage" (cache [B,Hkv,T,D], int32 lens [B]); the sliding
// window follows the cutileGPT README feature list.
//
// Work decomposition.  A workgroup owns one (partition, KV head, sequence)
// and all G = Hq/Hkv query heads of that KV head.  Each K and V row is read
// from HBM once and used by all G heads from registers.
//
// Lane layout (wave64).  A row of D bf16 is D/8 lanes x 16 bytes, so one
// wave-wide 16-byte load covers 64/(D/8) consecutive rows (4 rows = 1 KiB
// for D = 128), fully coalesced.  Lane (r, c) holds elements [8c, 8c+8) of
// row r of each load.  A score needs the sum over the D/8 lanes of a row;
// that is a DPP reduction inside a 16-lane row (4 steps for D = 128).
//
// Softmax.  q is pre-scaled by scale*log2(e) so scores are in base 2 and
// exponentials are exp2.  Each row slot r of each wave keeps its own running
// max m, sum l and accumulator over the rows it saw (online softmax); row
// slots are merged with cross-lane shuffles after the loop and waves through
// LDS, once per workgroup.  An empty range leaves l = 0 and gives out = 0,
// lse = -inf.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {

template <typename QT>
__device__ __forceinline__ void load_q8(const QT* p, float f[8]);
template <>
__device__ __forceinline__ void load_q8<float>(const float* p, float f[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <>
__device__ __forceinline__ void load_q8<uint16_t>(const uint16_t* p, float f[8]) {
  unpack8(*reinterpret_cast<const uint4*>(p), f);
}

// Merge (m2, l2) into (m, l): returns the factors that rescale the two
// accumulators.  -inf maxima (no rows seen) give factor 0 for that side.
__device__ __forceinline__ void lse_combine(float& m, float& l, float m2, float l2,
                                            float& f1, float& f2) {
  const float M = fmaxf(m, m2);
  const float Ms = (M == -INFINITY) ? 0.0f : M;
  f1 = __builtin_amdgcn_exp2f(m - Ms);
  f2 = __builtin_amdgcn_exp2f(m2 - Ms);
  l = l * f1 + l2 * f2;
  m = M;
}

template <int D, int G, int NW, typename QT, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_decode_kernel(
    const QT* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ lens, int window,
    float qscale, int part_tokens, int num_parts, int Hq, int Hkv, int T,
    float* __restrict__ ws_lse, float* __restrict__ ws_o, void* __restrict__ out,
    int out_bf16, float* __restrict__ lse_out) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per wave-wide load
  constexpr int U = (G >= 8) ? 2 : 4;   // loads of K (and of V) per iteration
  constexpr int ROWS_WAVE = U * RPI;    // rows per wave per iteration
  constexpr int ROWS_WG = NW * ROWS_WAVE;

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;

  const int n = min(max(lens[b], 0), T);
  const int lo = window > 0 ? max(0, n - window) : 0;
  int t0 = lo, t1 = n;
  if (SPLIT) {
    t0 = min(lo + part * part_tokens, n);
    t1 = min(t0 + part_tokens, n);
  }
  const int64_t head0 = (int64_t)b * Hq + (int64_t)g * G;   // first query head

  if (t0 >= t1) {
    // Nothing to attend in this range (uniform over the workgroup).
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

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load_q8<QT>(q + (head0 + h) * D + 8 * c, qf[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[h][e] *= qscale;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  const int64_t slab = ((int64_t)b * Hkv + g) * T * D + 8 * c;
  const uint16_t* Kp = k_cache + slab;
  const uint16_t* Vp = v_cache + slab;

  for (int base = t0 + wave * ROWS_WAVE; base < t1; base += ROWS_WG) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * RPI + r;
      valid[u] = t < t1;
      if (valid[u]) {
        kr[u] = *reinterpret_cast<const uint4*>(Kp + (int64_t)t * D);
        vr[u] = *reinterpret_cast<const uint4*>(Vp + (int64_t)t * D);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }

    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qf[h][e], kf[e], d);
        s[u][h] = d;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float t = group_sum<LPR>(s[u][h]);
        s[u][h] = valid[u] ? t : -INFINITY;
      }

    float p[U][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][h]);
      const float ms = (mx == -INFINITY) ? 0.0f : mx;
      const float alpha = __builtin_amdgcn_exp2f(m[h] - ms);
      m[h] = mx;
      float lsum = l[h] * alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u][h] = __builtin_amdgcn_exp2f(s[u][h] - ms);
        lsum += p[u][h];
      }
      l[h] = lsum;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      unpack8(vr[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p[u][h], vf[e], acc[h][e]);
    }
  }

  // Merge the RPI row slots of the wave (lanes with equal c).
#pragma unroll
  for (int mask = LPR; mask < 64; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], mask, 64);
      const float l2 = __shfl_xor(l[h], mask, 64);
      float f1, f2;
      lse_combine(m[h], l[h], m2, l2, f1, f2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a2 = __shfl_xor(acc[h][e], mask, 64);
        acc[h][e] = acc[h][e] * f1 + a2 * f2;
      }
    }
  }

  // Merge the waves through LDS, then write G x D outputs.
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_acc[NW][G][D];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][h][8 * c + e] = acc[h][e];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
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
      A += sm_acc[w][h][d] * f;
    }
    const bool any = L > 0.0f;
    const float o = any ? A / L : 0.0f;
    const float lse = any ? (M + log2f(L)) * kLn2 : -INFINITY;
    if (SPLIT) {
      ws_o[((head0 + h) * num_parts + part) * D + d] = o;
      if (d == 0) ws_lse[(head0 + h) * num_parts + part] = lse;
    } else {
      if (out_bf16) reinterpret_cast<uint16_t*>(out)[(head0 + h) * D + d] = f32_to_bf16(o);
      else reinterpret_cast<float*>(out)[(head0 + h) * D + d] = o;
      if (d == 0 && lse_out != nullptr) lse_out[head0 + h] = lse;
    }
  }
}

template <int D, int G, typename QT>
static int launch_attn_t(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = 4;
  const dim3 block(NW * 64);
  if (a.split) {
    const dim3 grid(a.num_parts, a.Hkv, a.B);
    hipLaunchKernelGGL((attn_decode_kernel<D, G, NW, QT, true>), grid, block, 0, s,
                       (const QT*)a.q, a.k_cache, a.v_cache, a.lens, a.window, a.qscale,
                       a.part_tokens, a.num_parts, a.Hq, a.Hkv, a.T, a.ws_lse, a.ws_o,
                       nullptr, 0, nullptr);
  } else {
    const dim3 grid(1, a.Hkv, a.B);
    hipLaunchKernelGGL((attn_decode_kernel<D, G, NW, QT, false>), grid, block, 0, s,
                       (const QT*)a.q, a.k_cache, a.v_cache, a.lens, a.window, a.qscale,
                       0, 1, a.Hq, a.Hkv, a.T, nullptr, nullptr, a.out, a.out_bf16,
                       a.lse_out);
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <int D, typename QT>
static int dispatch_g(const AttnArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_attn_t<D, 1, QT>(a, s);
    case 2: return launch_attn_t<D, 2, QT>(a, s);
    case 4: return launch_attn_t<D, 4, QT>(a, s);
    case 8: return launch_attn_t<D, 8, QT>(a, s);
    case 16: return launch_attn_t<D, 16, QT>(a, s);
    default: return GQA_ERR_UNSUPPORTED;
  }
}

int launch_attn_valu(const AttnArgs& a, hipStream_t s) {
  if (a.D == 128) return a.q_bf16 ? dispatch_g<128, uint16_t>(a, s) : dispatch_g<128, float>(a, s);
  if (a.D == 64) return a.q_bf16 ? dispatch_g<64, uint16_t>(a, s) : dispatch_g<64, float>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
