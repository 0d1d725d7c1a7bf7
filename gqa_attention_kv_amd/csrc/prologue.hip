// Fused decode prologue for gfx950: per-head QK-RMSNorm, RoPE at the
// sequence's position, and the append of the new K/V row to the bf16 cache.
//
// Follows the cutileGPT README feature "fused QK-Norm + RoPE + KV-cache
// writes", the RMSNorm formula of its "Why tiles" figure (x * w / sqrt(
// mean(x^2) + eps)), and the fusedtok 1.0.1 README "Operators" row RoPE
// (interleaved and NeoX layouts, kv-cache position offset).
//
// Mapping: one head vector (a query head or a KV head of one token of one
// sequence; token s of sequence b sits at position pos[b] + s) per D/2
// consecutive lanes; lane i owns rotary pair i -- elements (i, i + D/2)
// in the NeoX layout, (2i, 2i + 1) in the interleaved one -- so the
// rotation is lane-local and only the sum of squares crosses lanes.  For
// D = 128 that is one wave64 per head vector.  The rotary angle
// pos * inv_freq[i] (the caller's table) is formed in float64 with a
// float64 sincos (at pos ~ 1e5 a float32 angle would be off by ~1e-2 rad);
// the norm weights, the rotation and the magnitude factor are applied in
// float64 too, and the result is rounded once.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {

template <typename IT>
__device__ __forceinline__ float load_elem(const IT* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

__device__ __forceinline__ uint16_t to_bf16_bits(const float* p, int64_t i) {
  return f32_to_bf16(p[i]);
}
__device__ __forceinline__ uint16_t to_bf16_bits(const uint16_t* p, int64_t i) { return p[i]; }

template <int D, typename IT>
__global__ __launch_bounds__(256) void qkv_prologue_kernel(const PrologueArgs a) {
  constexpr int HALF = D / 2;        // lanes per head vector
  constexpr int VPB = 256 / HALF;    // head vectors per workgroup
  const int Hq = a.Hq, Hkv = a.Hkv, T = a.T, S = a.S;
  const int H = Hq + Hkv;
  const int64_t vec = (int64_t)blockIdx.x * VPB + threadIdx.x / HALF;
  const int i = threadIdx.x % HALF;
  const bool live = vec < (int64_t)a.B * S * H;   // lanes past the end: vector 0, no stores
  const int64_t v = live ? vec : 0;
  const int b = (int)(v / ((int64_t)S * H));
  const int st = (int)(v / H % S);  // token
  const int hh = (int)(v % H);
  const bool is_q = hh < Hq;
  const int g = hh - Hq;
  // elements of rotary pair i
  const int e0 = a.rope_interleaved ? 2 * i : i;
  const int e1 = a.rope_interleaved ? 2 * i + 1 : i + HALF;

  const IT* src = is_q ? reinterpret_cast<const IT*>(a.q) + (int64_t)b * a.q_bstride +
                             ((int64_t)st * Hq + hh) * D
                       : reinterpret_cast<const IT*>(a.k_new) + (int64_t)b * a.kv_bstride +
                             ((int64_t)st * Hkv + g) * D;
  float x0 = load_elem<IT>(src, e0);
  float x1 = load_elem<IT>(src, e1);

  // Weights and rotation act on the exact inputs in float64 and the RMS
  // factor r multiplies the result, so a rotated element much smaller than
  // its inputs (x0 c ~ x1 s) keeps the accuracy of r (~1e-7 relative)
  // instead of the ~1e-7 absolute error an fp32 rotation leaves.
  const float* w = is_q ? a.q_norm_w : a.k_norm_w;
  double y0 = x0, y1 = x1, r = 1.0;
  if (w != nullptr) {
    float ss = x0 * x0 + x1 * x1;
    ss = group_sum_shfl<HALF>(ss);
    r = 1.0 / sqrt((double)ss / D + (double)a.eps);
    y0 *= (double)w[e0];
    y1 *= (double)w[e1];
  }

  const int64_t p = (int64_t)a.pos[b] + st;
  if (a.rope) {
    double sn, cs;
    sincos((double)p * a.inv_freq[i], &sn, &cs);
    cs *= (double)a.rope_mscale;
    sn *= (double)a.rope_mscale;
    const double t0 = y0 * cs - y1 * sn;
    const double t1 = y1 * cs + y0 * sn;
    y0 = t0;
    y1 = t1;
  }
  x0 = (float)(y0 * r);
  x1 = (float)(y1 * r);
  if (!live) return;

  if (is_q) {
    float* dst = a.q_out + (((int64_t)b * S + st) * Hq + hh) * D;
    dst[e0] = x0;
    dst[e1] = x1;
  } else if (p >= 0 && p < T) {
    const int64_t row = (((int64_t)b * Hkv + g) * T + p) * D;
    a.k_cache[row + e0] = f32_to_bf16(x0);
    a.k_cache[row + e1] = f32_to_bf16(x1);
    const IT* vs = reinterpret_cast<const IT*>(a.v_new) + (int64_t)b * a.kv_bstride +
                   ((int64_t)st * Hkv + g) * D;
    a.v_cache[row + e0] = to_bf16_bits(vs, e0);
    a.v_cache[row + e1] = to_bf16_bits(vs, e1);
  }
}

template <int D, typename IT>
static int launch_prologue_t(const PrologueArgs& a, hipStream_t s) {
  constexpr int VPB = 256 / (D / 2);
  const int64_t vecs = (int64_t)a.B * a.S * (a.Hq + a.Hkv);
  const unsigned blocks = (unsigned)((vecs + VPB - 1) / VPB);
  hipLaunchKernelGGL((qkv_prologue_kernel<D, IT>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

int launch_prologue(const PrologueArgs& a, hipStream_t s) {
  if (a.D == 128) return a.in_bf16 ? launch_prologue_t<128, uint16_t>(a, s)
                                   : launch_prologue_t<128, float>(a, s);
  if (a.D == 64) return a.in_bf16 ? launch_prologue_t<64, uint16_t>(a, s)
                                  : launch_prologue_t<64, float>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
