// Log-sum-exp merge of split-K partitions, for gfx950.
//
// The flash-decoding split of the fusedtok 1.0.1 README ("Operators" row
// attention_decode) leaves, per (sequence, query head), NP partition results
// (o_k normalised, lse_k natural log; lse_k = -inf for an empty partition).
// They combine as M = max_k lse_k, w_k = exp(lse_k - M),
// out = sum_k w_k o_k / sum_k w_k, lse = M + log sum_k w_k.
//
// One 256-thread workgroup per (sequence, query head).  Threads form
// 256/(D/4) subgroups of D/4 lanes; a subgroup reads one partition row with
// 16-byte loads, subgroup j takes partitions j, j+S, j+2S, ...  The
// subgroup sums are combined through LDS in a fixed order, so the result is
// bit-identical from run to run (no atomics).
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(
    const float* __restrict__ ws_lse, const float* __restrict__ ws_o, int num_parts,
    void* __restrict__ out, int out_bf16, float* __restrict__ lse_out) {
  constexpr int TPR = D / 4;       // threads per partition row
  constexpr int S = 256 / TPR;     // partitions read in parallel
  const int64_t bh = blockIdx.x;
  const float* L = ws_lse + bh * num_parts;
  const float* O = ws_o + bh * num_parts * D;
  const int tid = threadIdx.x;

  __shared__ float red[256];
  float mx = -INFINITY;
  for (int k = tid; k < num_parts; k += 256) mx = fmaxf(mx, L[k]);
  red[tid] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];

  const int j = tid / TPR;
  const int c4 = tid % TPR;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.0f;
  if (M != -INFINITY) {
    for (int k = j; k < num_parts; k += S) {
      const float lk = L[k];
      if (lk == -INFINITY) continue;
      const float w = __expf(lk - M);
      const float4 o = *reinterpret_cast<const float4*>(O + (int64_t)k * D + 4 * c4);
      a.x = fmaf(w, o.x, a.x);
      a.y = fmaf(w, o.y, a.y);
      a.z = fmaf(w, o.z, a.z);
      a.w = fmaf(w, o.w, a.w);
      wsum += w;
    }
  }

  __shared__ float4 sa[256];
  __shared__ float sw[S];
  sa[tid] = a;
  if (c4 == 0) sw[j] = wsum;
  __syncthreads();
  if (tid < TPR) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    float W = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float4 v = sa[s * TPR + tid];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
      W += sw[s];
    }
    const bool any = W > 0.0f;
    const float inv = any ? 1.0f / W : 0.0f;
    const float o[4] = {t.x * inv, t.y * inv, t.z * inv, t.w * inv};
    if (out_bf16) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(out) + bh * D + 4 * tid;
      const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    } else {
      float* dst = reinterpret_cast<float*>(out) + bh * D + 4 * tid;
      *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (tid == 0 && lse_out != nullptr) lse_out[bh] = any ? M + logf(W) : -INFINITY;
  }
}

int launch_merge(const MergeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.Hq));
  if (a.D == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(256), 0, s, a.ws_lse, a.ws_o,
                       a.num_parts, a.out, a.out_bf16, a.lse_out);
  else if (a.D == 64)
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(256), 0, s, a.ws_lse, a.ws_o,
                       a.num_parts, a.out, a.out_bf16, a.lse_out);
  else
    return GQA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace gqa
