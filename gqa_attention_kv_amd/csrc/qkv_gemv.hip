// Packed QKV projection for the decode batch on gfx950: y[M,N] = x[M,K] W^T
// with W stored [N,K] (each output's weights contiguous), bf16 inputs and
// float32 accumulation.  This is the projection step ahead of the prologue:
// the cutileGPT README's runtime list has packed QKV projections feeding the
// fused QK-Norm + RoPE + KV-cache write, and the PyGPUkit 0.2.18 page's
// "Optimized BF16 GEMV" row describes the B[N,K] weight layout streamed at
// memory bandwidth.  With N = (Hq + 2 Hkv) D the output row of sequence m is
// q | k_new | v_new, which the prologue reads through its batch strides.
//
// The weights are read once, so the kernel is bound by HBM.  The
// contraction still runs on the matrix cores: with M = 8 rows of x the VALU
// form costs 8 multiply-adds and a conversion per weight element, about as
// many issue cycles as HBM needs to deliver the element, while one
// v_mfma_f32_16x16x32_bf16 covers 16 weight rows x 32 columns for all
// M <= 16 rows of x.
//
// Work split: a workgroup owns 16 weight rows (16 outputs per row of x); its
// 8 waves take the 128-column steps w, w + 8, ... of those rows (in an order
// rotated per workgroup).  A step is
// 16 rows x 256 bytes, loaded as whole 256-byte row segments (16 lanes per
// row) and staged through a wave-private LDS slab (rows padded to 272 bytes:
// conflict-free writes and operand reads), from which lane l = 16 k4 + n
// reads the A operand W[row n][32c + 8k4 .. + 8] of each 32-column slice c.
// The B operand is x[m][same columns] for m = l % 16 (zero for m >= M),
// read from L2.  The eight waves' partial 16 x 16 tiles are added through
// LDS in a fixed order, so reruns are bit-identical.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kWaves = 8;
constexpr int kRowsPerBlock = 16;
constexpr int kStepCols = 128;                   // columns per step (256 bytes of a row)
constexpr int kRowU4 = kStepCols * 2 / 16 + 1;   // slab row pitch in 16-byte units (272 B)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__global__ __launch_bounds__(kWaves * 64) void qkv_gemv_kernel(const GemvArgs a) {
  __shared__ u32x4_t slab[kWaves][kRowsPerBlock * kRowU4];
  __shared__ f32x4_t part[kWaves - 1][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, k4 = lane >> 4;
  const int N = a.N, K = a.K, M = a.M;
  const int n0 = blockIdx.x * kRowsPerBlock;
  const int steps = K / kStepCols;

  // Whole-row loads: instruction i reads rows 4i + lane/16 of the block,
  // 16 bytes at column 8 (lane % 16) of the step.  Rows past N are clamped
  // (their outputs are not stored).  The block's 16 rows are addressed
  // through one buffer resource with 32-bit offsets.
  const int rows_here = N - n0 < kRowsPerBlock ? N - n0 : kRowsPerBlock;
  const __amdgpu_buffer_rsrc_t rw =
      w_rsrc(a.w + (int64_t)n0 * a.w_stride,
             (uint32_t)(((int64_t)(rows_here - 1) * a.w_stride + K) * 2));
  uint32_t roff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = 4 * i + k4;
    r = r < rows_here ? r : rows_here - 1;
    roff[i] = (uint32_t)((int64_t)r * a.w_stride * 2) + 16u * n;
  }
  // x operand: row m = n of x (zero past M), 16 bytes per slice.
  const bool xrow = n < M;
  const uint16_t* xp = a.x + (int64_t)(xrow ? n : 0) * a.x_stride + 8 * k4;

  // Two tiles in flight per wave: a ring of register buffers with fixed
  // slots (the loop body is unrolled over the ring).
  constexpr int kRing = 2;
  u32x4_t wt[kRing][4], xb[kRing][4];
  auto fetch = [&](int buf, int step) {
    const uint32_t col = (uint32_t)step * (kStepCols * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wt[buf][i] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, roff[i] + col, 0, 0));
#pragma unroll
    for (int c = 0; c < 4; ++c)
      xb[buf][c] = xrow ? *reinterpret_cast<const u32x4_t*>(xp + step * kStepCols + 32 * c)
                        : u32x4_t{0u, 0u, 0u, 0u};
  };

  u32x4_t* sl = slab[wave];
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // stage a tile's rows, then read them back in operand order (one wave:
  // LDS operations complete in order; the empty asm keeps the compiler from
  // reordering the reads above the writes of other lanes)
  auto compute = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int widx = (4 * i + k4) * kRowU4 + n;
      asm volatile("" : "+v"(widx));
      sl[widx] = wt[buf][i];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int ridx = n * kRowU4 + 4 * c + k4;
      asm volatile("" : "+v"(ridx));
      const u32x4_t wa = sl[ridx];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa),
                                                    __builtin_bit_cast(bf16x8_t, xb[buf][c]),
                                                    acc, 0, 0, 0);
    }
  };

  // This wave's steps are wave, wave + 8, ...; slot j of a trip holds step
  // s + 8 j, and the fetch of the step kRing - 1 slots ahead refills the
  // slot computed just before.  Each workgroup walks its rows' columns in a
  // rotated order (by 37 * block steps): rows are K * 2 bytes apart, and
  // workgroups reading the same columns of their rows at the same time load
  // a narrow slice of the HBM channels (measured: 39.3 -> 35.1 us for the
  // 168 MB projection, 23.1 -> 22.8 us for 117 MB).
  const int first = wave, st = kWaves, last = steps;
  const int rot = (int)((blockIdx.x * 37u) % (unsigned)steps);
  auto step_of = [&](int x) { return x + rot < steps ? x + rot : x + rot - steps; };
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j)
    if (first + st * j < last) fetch(j, step_of(first + st * j));
  for (int s = first; s < last; s += st * kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int cur = s + st * j;
      if (cur >= last) break;                        // wave-uniform
      const int ahead = cur + st * (kRing - 1);
      if (ahead < last) fetch((j + kRing - 1) % kRing, step_of(ahead));
      compute(j);
    }
  }

  // acc[i] = sum over this wave's steps of W[n0 + 4 k4 + i] . x[m], m = n.
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) acc += part[w][lane];
  if (n >= M) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = n0 + 4 * k4 + i;
    if (row >= N) continue;
    const int64_t o = (int64_t)n * a.y_stride + row;
    if (a.out_bf16)
      reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16(acc[i]);
    else
      reinterpret_cast<float*>(a.y)[o] = acc[i];
  }
}

}  // namespace

int launch_qkv_gemv(const GemvArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.N + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(qkv_gemv_kernel, dim3(blocks), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace gqa
