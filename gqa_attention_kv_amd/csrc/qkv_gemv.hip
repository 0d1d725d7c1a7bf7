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
// Work split: the N weight rows are cut into one contiguous share per
// workgroup, ceil(N / CUs) rows, so every CU streams the same number of
// bytes (with 16-row workgroups the 640 blocks of a 10240-row projection
// ran two or three to a CU, and the CUs holding three set the time).  A
// share is NT 16-row tiles (the last rows of the last tile are padding that
// loads nothing).  The 8 waves take the 128-column steps w, w + 8, ... of
// the share (in an order rotated per workgroup); for each step a wave loads
// x once and then the step's 16 rows x 256 bytes of every tile, so x is
// read from L2 once per step and share instead of once per tile.  A tile's
// rows are loaded as whole 256-byte row segments (16 lanes per row) and
// staged through a wave-private LDS slab (rows padded to 272 bytes), from
// which lane l = 16 k4 + n reads the A operand W[row n][32c + 8k4 .. + 8]
// of each 32-column slice c; the B operand is x[m][same columns] for m =
// l % 16 (zero for m >= M).  One (step, tile) item is in flight while the
// previous one is computed.  The eight waves' partial 16 x 16 tiles are
// added through LDS in a fixed order, so reruns are bit-identical.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kWaves = 8;
constexpr int kRowsPerTile = 16;
constexpr int kMaxTiles = 4;                     // tiles per workgroup share
constexpr int kAhead = 1;                        // items in flight beyond the one computed
constexpr int kStepCols = 128;                   // columns per step (256 bytes of a row)
constexpr int kRowU4 = kStepCols * 2 / 16 + 1;   // slab row pitch in 16-byte units (272 B)
// The weights are read exactly once per launch: their loads carry the
// non-temporal policy (nt), so they do not displace what the L2 and the
// Infinity Cache should keep.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int NT, int AHEAD>
__global__ __launch_bounds__(kWaves * 64) void qkv_gemv_kernel(const GemvArgs a, int share) {
  __shared__ u32x4_t slab[kWaves][kRowsPerTile * kRowU4];
  __shared__ f32x4_t part[NT][kWaves - 1][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, k4 = lane >> 4;
  const int N = a.N, K = a.K, M = a.M;
  const int n0 = blockIdx.x * share;
  const int rows_here = N - n0 < share ? N - n0 : share;
  const int steps = K / kStepCols;
  // this wave's steps: wave, wave + 8, ... < steps
  const int nsw = wave < steps ? (steps - wave + kWaves - 1) / kWaves : 0;

  // The share's rows through one buffer resource (32-bit offsets).  Load
  // instruction i of tile t reads row 16 t + 4 i + lane / 16 of the share,
  // 16 bytes at column 8 (lane % 16) of the step; a padding row past the
  // share gets an offset past the resource and loads zeros from nowhere.
  const uint32_t wbytes = (uint32_t)(((int64_t)(rows_here - 1) * a.w_stride + K) * 2);
  const __amdgpu_buffer_rsrc_t rw = w_rsrc(a.w + (int64_t)n0 * a.w_stride, wbytes);
  uint32_t roff[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = kRowsPerTile * t + 4 * i + k4;
      roff[t][i] = r < rows_here ? (uint32_t)((int64_t)r * a.w_stride * 2) + 16u * n : wbytes;
    }
  // x operand: row m = n of x (zero past M), 16 bytes per slice.
  const bool xrow = n < M;
  const uint16_t* xp = a.x + (int64_t)(xrow ? n : 0) * a.x_stride + 8 * k4;

  // Each workgroup walks its columns in a rotated order (by 37 * block
  // steps): rows are K * 2 bytes apart, and workgroups reading the same
  // columns of their rows at the same time load a narrow slice of the HBM
  // channels (measured: 39.3 -> 35.1 us for the 168 MB projection with
  // 16-row workgroups).
  const int rot = (int)((blockIdx.x * 37u) % (unsigned)steps);
  auto step_of = [&](int j) {
    const int x = wave + kWaves * j;
    return x + rot < steps ? x + rot : x + rot - steps;
  };

  // Items (step j, tile t), tile fastest, AHEAD items in flight beyond the
  // one being computed: a ring of R = AHEAD + 1 register slots for the W
  // tiles and R for x (one per step in flight); the loop runs R steps per
  // trip so every slot index is a compile-time constant.
  constexpr int R = AHEAD + 1;
  u32x4_t wt[R][4], xb[R][4];
  auto fetch_w = [&](int slot, int j, int t) {
    const uint32_t col = (uint32_t)step_of(j) * (kStepCols * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wt[slot][i] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       rw, roff[t][i] == wbytes ? wbytes : roff[t][i] + col, 0, kStreamPolicy));
  };
  auto fetch_x = [&](int slot, int j) {
    const int c0 = step_of(j) * kStepCols;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      xb[slot][c] = xrow ? *reinterpret_cast<const u32x4_t*>(xp + c0 + 32 * c)
                         : u32x4_t{0u, 0u, 0u, 0u};
  };
  // item q of a trip (q = jj NT + t, possibly past the trip's R NT items:
  // then it is item q - R NT of the next trip); slot q % R either way
  auto fetch_item = [&](int j0, int q) {
    const int jj = q / NT, t = q % NT;
    const int j = j0 + jj;
    if (j >= nsw) return;                                  // wave-uniform
    fetch_w(q % R, j, t);
    if (t == 0) fetch_x(jj % R, j);
  };

  u32x4_t* sl = slab[wave];
  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // stage an item's rows, then read them back in operand order (one wave:
  // LDS operations complete in order; the empty asm keeps the compiler from
  // reordering the reads above the writes of other lanes)
  auto compute = [&](int slot, int xs, f32x4_t& c_acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int widx = (4 * i + k4) * kRowU4 + n;
      asm volatile("" : "+v"(widx));
      sl[widx] = wt[slot][i];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int ridx = n * kRowU4 + 4 * c + k4;
      asm volatile("" : "+v"(ridx));
      const u32x4_t wa = sl[ridx];
      c_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa),
                                                      __builtin_bit_cast(bf16x8_t, xb[xs][c]),
                                                      c_acc, 0, 0, 0);
    }
  };

#pragma unroll
  for (int q = 0; q < AHEAD; ++q) fetch_item(0, q);
  for (int j0 = 0; j0 < nsw; j0 += R) {
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
      if (j0 + jj >= nsw) break;                           // wave-uniform
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int q = jj * NT + t;
        if (q + AHEAD < R * NT) fetch_item(j0, q + AHEAD);
        else fetch_item(j0 + R, q + AHEAD - R * NT);
        compute(q % R, jj, acc[t]);
      }
    }
  }

  // acc[t][i] = sum over this wave's steps of W[row 16 t + 4 k4 + i] . x[m], m = n
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) part[t][wave - 1][lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0 || n >= M) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4_t sum = acc[t];
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) sum += part[t][w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = kRowsPerTile * t + 4 * k4 + i;
      if (r >= rows_here) continue;
      const int64_t o = (int64_t)n * a.y_stride + n0 + r;
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.y)[o] = f32_to_bf16(sum[i]);
      else
        reinterpret_cast<float*>(a.y)[o] = sum[i];
    }
  }
}

}  // namespace

int launch_qkv_gemv(const GemvArgs& a, hipStream_t s) {
  // one share of rows per CU (at most kMaxTiles tiles); the CU count is read
  // once per device
  static int cus_of[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_LAUNCH;
  int cus = dev >= 0 && dev < 64 ? cus_of[dev] : 0;
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    if (dev >= 0 && dev < 64) cus_of[dev] = cus;
  }
  int share = (a.N + cus - 1) / cus;
  share = share < kMaxTiles * kRowsPerTile ? share : kMaxTiles * kRowsPerTile;
  // A share that is not a whole number of tiles carries padding rows; with
  // one row of x (nothing to reuse across tiles) the 16-row grid, two to
  // four workgroups per CU balanced by the dispatcher, measured faster.
  if (a.M == 1 && share % kRowsPerTile != 0) share = kRowsPerTile;
  const int nt = (share + kRowsPerTile - 1) / kRowsPerTile;
  const dim3 grid((unsigned)((a.N + share - 1) / share)), block(kWaves * 64);
  switch (nt) {
    case 1: hipLaunchKernelGGL((qkv_gemv_kernel<1, kAhead>), grid, block, 0, s, a, share); break;
    case 2: hipLaunchKernelGGL((qkv_gemv_kernel<2, kAhead>), grid, block, 0, s, a, share); break;
    case 3: hipLaunchKernelGGL((qkv_gemv_kernel<3, kAhead>), grid, block, 0, s, a, share); break;
    default: hipLaunchKernelGGL((qkv_gemv_kernel<4, kAhead>), grid, block, 0, s, a, share); break;
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace gqa
