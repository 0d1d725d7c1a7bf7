// Fused decode prologue for gfx950: per-head QK-RMSNorm, RoPE at the
// sequence's position, and the append of the new K/V row to the bf16 cache.
//
// Follows the cutileGPT README feature "fused QK-Norm + RoPE + KV-cache
// writes", the RMSNorm formula of its "Why tiles" figure (x * w / sqrt(
// mean(x^2) + eps)), and the fusedtok 1.0.1 README "Operators" row RoPE
// (interleaved and NeoX layouts, kv-cache position offset).
//
// Mapping: a group of D/2 consecutive lanes takes head vectors (query heads
// or KV heads of one token of one sequence; token s of sequence b sits at
// position pos[b] + s) one after another; lane i owns rotary pair i --
// elements (i, i + D/2) in the NeoX layout, (2i, 2i + 1) in the
// interleaved one -- so the rotation is lane-local and only the sum of
// squares crosses lanes.  For D = 128 a lane group is one wave64.  The
// rotary angle
// pos * inv_freq[i] (the caller's table) is formed in float64 as a phase
// in turns and reduced to [-pi, pi] before a float64 sin/cos (at pos ~ 1e5 a
// float32 angle would be off by ~1e-2 rad);
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

// Head vectors per lane group, loaded together: with many vectors one
// memory round trip covers R = 8 of them, so the launch takes few, full
// waves; small launches (below kManyVecs vectors) keep R = 1, which spreads
// their few vectors over more workgroups.
constexpr int kProVecs = 8;
constexpr int64_t kManyVecs = 16384;

// Grid: x = sequence * S + token, y = a chunk of VPB * R of the token's
// Hq + Hkv head vectors (query heads first; only the Hkv K/V vectors when
// the queries are rotated by the attention kernel); lane group k of the workgroup
// takes vectors r * VPB + k of the chunk.  Index arithmetic is per
// workgroup, and every input of the R vectors is loaded before any math.
template <int D, typename IT, int R>
__global__ __launch_bounds__(256) void qkv_prologue_kernel(const PrologueArgs a) {
  constexpr int HALF = D / 2;        // lanes per head vector
  constexpr int VPB = 256 / HALF;    // lane groups per workgroup
  const int Hq = a.Hq, Hkv = a.Hkv, T = a.T, S = a.S;
  const int H = Hq + Hkv;
  const int vfirst = a.kv_only ? Hq : 0;   // first head vector of the launch
  const int b = blockIdx.x / S;
  const int st = blockIdx.x - b * S;  // token
  const int grp = threadIdx.x / HALF;
  const int i = threadIdx.x % HALF;
  // elements of rotary pair i
  const int e0 = a.rope_interleaved ? 2 * i : i;
  const int e1 = a.rope_interleaved ? 2 * i + 1 : i + HALF;
  const int64_t p = (int64_t)a.pos[b] + st;

  float x0[R], x1[R];
  IT v0[R], v1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int vh = vfirst + (blockIdx.y * R + r) * VPB + grp;
    x0[r] = x1[r] = 0.0f;
    v0[r] = v1[r] = IT(0);
    if (vh >= H) continue;
    if (vh < Hq) {
      const IT* src = reinterpret_cast<const IT*>(a.q) + (int64_t)b * a.q_bstride +
                      ((int64_t)st * Hq + vh) * D;
      x0[r] = load_elem<IT>(src, e0);
      x1[r] = load_elem<IT>(src, e1);
    } else {
      const int64_t off = (int64_t)b * a.kv_bstride + ((int64_t)st * Hkv + (vh - Hq)) * D;
      const IT* ks = reinterpret_cast<const IT*>(a.k_new) + off;
      const IT* vs = reinterpret_cast<const IT*>(a.v_new) + off;
      x0[r] = load_elem<IT>(ks, e0);
      x1[r] = load_elem<IT>(ks, e1);
      v0[r] = vs[e0];
      v1[r] = vs[e1];
    }
  }
  const bool norm = a.q_norm_w != nullptr;
  const float wq0 = norm ? a.q_norm_w[e0] : 1.0f, wq1 = norm ? a.q_norm_w[e1] : 1.0f;
  const float wk0 = norm ? a.k_norm_w[e0] : 1.0f, wk1 = norm ? a.k_norm_w[e1] : 1.0f;

  // The rotary angle of pair i, shared by every head of the token: phase
  // p f / (2 pi) reduced to [-1/2, 1/2] turns, then sin/cos of the reduced
  // angle, times the magnitude factor.
  double cs = 1.0, sn = 0.0;
  if (a.rope) {
    const double rev = (double)p * a.inv_freq_rev[i];
    sincos_pi_f64((rev - rint(rev)) * 6.283185307179586, &sn, &cs);
    cs *= (double)a.rope_mscale;
    sn *= (double)a.rope_mscale;
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int vh = vfirst + (blockIdx.y * R + r) * VPB + grp;
    if (vh >= H) continue;             // uniform within the lane group
    const bool is_q = vh < Hq;
    // Weights and rotation act on the exact inputs in float64 and the RMS
    // factor rr multiplies the result, so a rotated element much smaller
    // than its inputs (x0 c ~ x1 s) keeps the accuracy of rr (~1e-7
    // relative) instead of the ~1e-7 absolute error an fp32 rotation leaves.
    double y0 = x0[r], y1 = x1[r], rr = 1.0;
    if (norm) {
      const float ss = group_sum_shfl<HALF>(x0[r] * x0[r] + x1[r] * x1[r]);
      rr = 1.0 / sqrt((double)ss / D + (double)a.eps);
      y0 *= (double)(is_q ? wq0 : wk0);
      y1 *= (double)(is_q ? wq1 : wk1);
    }
    if (a.rope) {
      const double t0 = y0 * cs - y1 * sn;
      const double t1 = y1 * cs + y0 * sn;
      y0 = t0;
      y1 = t1;
    }
    const float z0 = (float)(y0 * rr), z1 = (float)(y1 * rr);
    if (is_q) {
      float* dst = a.q_out + (((int64_t)b * S + st) * Hq + vh) * D;
      dst[e0] = z0;
      dst[e1] = z1;
    } else if (p >= 0 && p < T) {
      const int64_t row = (((int64_t)b * Hkv + (vh - Hq)) * T + p) * D;
      a.k_cache[row + e0] = f32_to_bf16(z0);
      a.k_cache[row + e1] = f32_to_bf16(z1);
      a.v_cache[row + e0] = to_bf16_bits(&v0[r], 0);
      a.v_cache[row + e1] = to_bf16_bits(&v1[r], 0);
    }
  }
}

template <int D, typename IT, int R>
static int launch_prologue_r(const PrologueArgs& a, hipStream_t s) {
  constexpr int per = 256 / (D / 2) * R;   // head vectors per workgroup
  const int nv = a.kv_only ? a.Hkv : a.Hq + a.Hkv;   // head vectors per token
  const dim3 grid((unsigned)((int64_t)a.B * a.S), (unsigned)((nv + per - 1) / per));
  hipLaunchKernelGGL((qkv_prologue_kernel<D, IT, R>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <int D, typename IT>
static int launch_prologue_t(const PrologueArgs& a, hipStream_t s) {
  const int64_t vecs = (int64_t)a.B * a.S * (a.kv_only ? a.Hkv : a.Hq + a.Hkv);
  return vecs >= kManyVecs ? launch_prologue_r<D, IT, kProVecs>(a, s)
                           : launch_prologue_r<D, IT, 1>(a, s);
}

int launch_prologue(const PrologueArgs& a, hipStream_t s) {
  if (a.D == 128) return a.in_bf16 ? launch_prologue_t<128, uint16_t>(a, s)
                                   : launch_prologue_t<128, float>(a, s);
  if (a.D == 64) return a.in_bf16 ? launch_prologue_t<64, uint16_t>(a, s)
                                  : launch_prologue_t<64, float>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
