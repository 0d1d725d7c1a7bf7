// Attention of S query tokens per sequence over the KV cache on gfx950
// matrix cores: the prefill counterpart of the decode kernel.  Computes what
// the fusedtok 1.0.1 README ("Operators" row attention_prefill) describes --
// softmax attention of S query rows, causal or bidirectional -- with the GQA
// head mapping, per-sequence lengths and sliding window of its
// attention_decode row, over the same [B,Hkv,T,D] bf16 cache: the S tokens
// are the last S rows of each sequence's cache (a fresh sequence is the
// case lens = S), and token s sees
//   causal:        rows [lo_s, n_s), n_s = clamp(lens - (S-1-s), 0, T)
//   bidirectional: rows [lo, n),     n   = clamp(lens, 0, T)
// with lo = max(0, n - window) under a window, else 0.
//
// Here the contractions dominate: every cached row meets up to S*G query
// rows, so the kernel is bound by the matrix cores and the VALU softmax,
// not by HBM.  Work split: a workgroup of 4 waves owns 128 consecutive
// (token, head) rows of one (sequence, KV head) -- row r is token r / G,
// head r % G of the group, so the G heads of a token sit side by side -- and
// streams the K/V rows they need through LDS in tiles of 32 rows, shared by
// all 4 waves; each wave owns 32 rows (two blocks of 16).
//
// Lane l, with n = l % 16 and k4 = l / 16, per 16-row block (columns = query
// rows, so a row's softmax state stays in its own lanes):
//   QK: S^T[16 keys x 16 rows] += K[16 x 32] * q^T[32 x 16] per 32-wide slice
//       of D (v_mfma_f32_16x16x32_bf16).  The result leaves lane l holding
//       keys 4 k4 + i (i < 4) of query row n.  An fp32 q is split into bf16
//       hi + lo and takes two calls per slice; a bf16 q takes one.
//   PV: O^T[16 cols x 16 rows] += V^T[16 x 32] * P^T[32 x 16] per D/16 column
//       block, with the 16 keys as 32 k-indices k = 8 k4 + 2 i + x: x = 0 is
//       the bf16 hi part of P, x = 1 its lo part (P keeps ~16 mantissa bits),
//       and V appears at both k of its key.  Lane l's P operand is exactly
//       the four scores the QK step left in it.  Output column n of block b
//       stands for d = (D/16) n + b, so a lane reads one contiguous D/8-byte
//       piece of each V row from LDS for all blocks.
// Online softmax per row with a lazy rescale: the reference maximum only
// moves when a tile's maximum exceeds it by more than 2^8 (in exp2 units),
// so P stays below 256 and O is rarely rescaled.  Keys outside a row's
// range are masked only in tiles that are not wholly inside every range of
// the wave's rows.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;                  // two 16-row blocks
constexpr int kRows = kWaves * kRowsPerWave;      // query rows per workgroup
constexpr int kKeys = 32;                         // cache rows per LDS tile
constexpr float kRescaleLog2 = 8.0f;              // lazy-rescale threshold

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// x as a bf16 pair: hi = bf16(x) in the low half, lo = bf16(x - hi) above.
__device__ __forceinline__ uint32_t hi_lo_bf16(float x) {
  const __bf16 h = (__bf16)x;
  const bf16x2_t v = {h, (__bf16)(x - (float)h)};
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 element e of a packed slice, copied into both halves of a dword.
__device__ __forceinline__ uint32_t dup_half(uint32_t w, int e) {
  return __builtin_amdgcn_perm(w, w, (e & 1) ? 0x03020302u : 0x01000100u);
}

__device__ __forceinline__ int clampi(int64_t v, int lo, int hi) {
  return (int)(v < lo ? lo : v > hi ? hi : v);
}

template <int D, bool QF32>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void
attn_prefill_kernel(const PrefillArgs a) {
  constexpr int KC = D / 32;            // QK slices
  constexpr int VB = D / 16;            // PV column blocks
  constexpr int VW = D / 32;            // dwords of a lane's V piece (D/8 bytes)
  constexpr int ROW = D * 2 + 16;       // LDS row pitch in bytes (conflict-free reads)
  constexpr int CPR = D / 8;            // 16-byte chunks per cache row
  constexpr int FILL = kKeys * CPR / (kWaves * 64);   // chunks per thread per tile
  static_assert(FILL >= 1, "tile fill");

  __shared__ __attribute__((aligned(16))) unsigned char lds_k[kKeys * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[kKeys * ROW];

  const int Hq = a.Hq, Hkv = a.Hkv, S = a.S, T = a.T;
  const int G = Hq / Hkv;
  const int SG = S * G;
  const int nrb = a.row_blocks;
  const int npairs = a.B * Hkv;

  // Workgroup -> (sequence, KV head, row block).  Workgroup x runs on XCD
  // x % 8; when the pairs split evenly, every row block of a pair lands on
  // the same XCD so its K/V rows are reused from that XCD's L2.  Row blocks
  // run from the last (most keys under the causal mask) to the first.
  const int x = blockIdx.x;
  int pair, rbi;
  if ((npairs & 7) == 0) {
    const int slot = x >> 3;
    pair = (x & 7) + 8 * (slot / nrb);
    rbi = slot % nrb;
  } else {
    pair = x / nrb;
    rbi = x % nrb;
  }
  const int rb = nrb - 1 - rbi;
  const int b = pair / Hkv, g = pair % Hkv;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, k4 = lane >> 4;

  const int len = a.lens[b];
  const bool causal = a.causal != 0;
  const int window = a.window;
  auto n_of = [&](int t) -> int {
    return clampi(causal ? (int64_t)len - (S - 1 - t) : (int64_t)len, 0, T);
  };
  auto lo_of = [&](int nt) -> int { return window > 0 ? (nt > window ? nt - window : 0) : 0; };

  const int r0 = rb * kRows;
  const int rlast = (r0 + kRows < SG ? r0 + kRows : SG) - 1;
  const int kend = n_of(rlast / G);
  const int kbeg = lo_of(n_of(r0 / G));

  // This lane's two rows and their key ranges; rows past S*G see no key.
  int rlo[2], rhi[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = r0 + kRowsPerWave * wave + 16 * j + n;
    const int nt = row < SG ? n_of(row / G) : 0;
    rhi[j] = nt;
    rlo[j] = row < SG ? lo_of(nt) : 0;
  }
  // The wave's rows: keys every row sees ([free_lo, free_hi)) and keys any
  // row sees ([need_lo, need_hi)).
  const int wr0 = r0 + kRowsPerWave * wave;
  const bool wave_live = wr0 < SG;
  const int wr1 = (wr0 + kRowsPerWave < SG ? wr0 + kRowsPerWave : SG) - 1;
  int need_lo = 0, need_hi = 0, free_lo = 0, free_hi = 0;
  if (wave_live) {
    const int n0 = n_of(wr0 / G), n1 = n_of(wr1 / G);
    need_lo = lo_of(n0);
    need_hi = n1;
    free_lo = lo_of(n1);
    free_hi = n0;
  }

  // q operands (B of the QK calls): lane holds row n of block j, elements
  // 32c + 8 k4 .. + 8.
  u32x4_t qh[2][KC], ql[2][KC];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = r0 + kRowsPerWave * wave + 16 * j + n;
    const bool ok = row < SG;
    const int t = ok ? row / G : 0, h = ok ? row % G : 0;
    const int64_t qoff = (((int64_t)b * S + t) * Hq + (int64_t)g * G + h) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int e = 32 * c + 8 * k4;
      if constexpr (QF32) {
        const float* p = reinterpret_cast<const float*>(a.q) + qoff + e;
        float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (ok) {
          const float4 u = *reinterpret_cast<const float4*>(p);
          const float4 v = *reinterpret_cast<const float4*>(p + 4);
          f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
          f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
        }
        bf16x8_t hv, lv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hv[i] = (__bf16)f[i];
          lv[i] = (__bf16)(f[i] - (float)hv[i]);
        }
        qh[j][c] = __builtin_bit_cast(u32x4_t, hv);
        ql[j][c] = __builtin_bit_cast(u32x4_t, lv);
      } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(a.q) + qoff + e;
        qh[j][c] = ok ? *reinterpret_cast<const u32x4_t*>(p) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  f32x4_t o[2][VB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < VB; ++v) o[j][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};
  const float qscale = a.qscale;

  const int64_t slab = ((int64_t)b * Hkv + g) * T * D;
  const uint32_t slab_bytes = (uint32_t)((int64_t)T * D * 2);
  const __amdgpu_buffer_rsrc_t rk = slab_rsrc(a.k_cache + slab, slab_bytes);
  const __amdgpu_buffer_rsrc_t rv = slab_rsrc(a.v_cache + slab, slab_bytes);

  const int ntiles = kend > kbeg ? (kend - kbeg + kKeys - 1) / kKeys : 0;

  // Tile fill: thread t moves chunks t + 256 f of the tile (row-major, CPR
  // chunks per row).  Rows past the range are clamped into it (they are
  // masked below, and a row the workgroup attends holds finite values).
  u32x4_t fk[FILL], fv[FILL];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int f = 0; f < FILL; ++f) {
      const int ci = threadIdx.x + kWaves * 64 * f;
      const int rr = ci / CPR, cc = ci % CPR;
      int key = kbeg + kKeys * tile + rr;
      key = key < kend ? key : kend - 1;
      const uint32_t off = (uint32_t)key * (uint32_t)(D * 2) + 16u * cc;
      fk[f] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      fv[f] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int f = 0; f < FILL; ++f) {
      const int ci = threadIdx.x + kWaves * 64 * f;
      const int rr = ci / CPR, cc = ci % CPR;
      *reinterpret_cast<u32x4_t*>(lds_k + rr * ROW + 16 * cc) = fk[f];
      *reinterpret_cast<u32x4_t*>(lds_v + rr * ROW + 16 * cc) = fv[f];
    }
  };

  if (ntiles > 0) fetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();              // every wave is done with the previous tile
    stash();
    __syncthreads();
    if (tile + 1 < ntiles) fetch(tile + 1);   // in flight during the compute
    __builtin_amdgcn_sched_barrier(0);

    const int k0 = kbeg + kKeys * tile;
    if (!wave_live || k0 >= need_hi || k0 + kKeys <= need_lo) continue;   // wave-uniform
    const bool full = k0 >= free_lo && k0 + kKeys <= free_hi;

    // QK for both 16-key blocks and both row blocks.
    f32x4_t s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4_t ka =
            *reinterpret_cast<const u32x4_t*>(lds_k + (16 * kb + n) * ROW + 64 * c + 16 * k4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          s[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qh[j][c]), s[kb][j],
              0, 0, 0);
          if constexpr (QF32)
            s[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, ql[j][c]),
                s[kb][j], 0, 0, 0);
        }
      }
    }

    // Masks and the tile maximum of each row (raw scores; qscale > 0).
    float mnew[2];
    bool need[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 16 * kb + 4 * k4 + i;
            if (key < rlo[j] || key >= rhi[j]) s[kb][j][i] = -INFINITY;
          }
      }
      float t = fmaxf(fmaxf(fmaxf(s[0][j][0], s[0][j][1]), fmaxf(s[0][j][2], s[0][j][3])),
                      fmaxf(fmaxf(s[1][j][0], s[1][j][1]), fmaxf(s[1][j][2], s[1][j][3])));
      t = fmaxf(t, __shfl_xor(t, 16, 64));
      t = fmaxf(t, __shfl_xor(t, 32, 64));
      mnew[j] = fmaxf(m[j], t);
      // m = -inf with a finite maximum gives +inf (rescale); both -inf give
      // NaN (no rescale: the row has seen no key yet).
      need[j] = (mnew[j] - m[j]) * qscale > kRescaleLog2;
    }
    if (__any(need[0] || need[1])) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float alpha = need[j] ? __builtin_amdgcn_exp2f((m[j] - mnew[j]) * qscale) : 1.0f;
        if (need[j]) m[j] = mnew[j];
        l[j] *= alpha;
#pragma unroll
        for (int v = 0; v < VB; ++v) o[j][v] *= alpha;
      }
    }

    // P = exp2(s * qscale - m * qscale) as bf16 hi/lo pairs (the B operand).
    u32x4_t pb[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float mref = m[j] == -INFINITY ? 0.0f : m[j] * qscale;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j][i], qscale, -mref));
          ps += p;
          pb[j][kb][i] = hi_lo_bf16(p);
        }
      l[j] += ps;
    }

    // PV: V rows 16 kb + 4 k4 + i at columns (D/16) n .. + D/16.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t vw[4][VW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned char* src = lds_v + (16 * kb + 4 * k4 + i) * ROW + (D / 8) * n;
        if constexpr (VW == 4) {
          const u32x4_t t = *reinterpret_cast<const u32x4_t*>(src);
          vw[i][0] = t[0]; vw[i][1] = t[1]; vw[i][2] = t[2]; vw[i][3] = t[3];
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(src);
          vw[i][0] = t.x; vw[i][1] = t.y;
        }
      }
#pragma unroll
      for (int v = 0; v < VB; ++v) {
        u32x4_t va;
#pragma unroll
        for (int i = 0; i < 4; ++i) va[i] = dup_half(vw[i][v >> 1], v);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[j][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pb[j][kb]), o[j][v],
              0, 0, 0);
      }
    }
  }

  // Normalise and store.  Lane (n, k4) holds, for row n of block j,
  // columns d = (D/16)(4 k4 + i) + v of block v, i < 4: for each i the VB
  // columns from (D/16)(4 k4 + i) on are consecutive.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float lt = l[j];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int row = r0 + kRowsPerWave * wave + 16 * j + n;
    if (row >= SG) continue;
    const int t = row / G, h = row % G;
    const int64_t orow = ((int64_t)b * S + t) * Hq + (int64_t)g * G + h;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = VB * (4 * k4 + i);
      float y[VB];
#pragma unroll
      for (int v = 0; v < VB; ++v) y[v] = o[j][v][i] * inv;
      if (a.out_bf16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + orow * D + d0;
        uint32_t w[VB / 2];
#pragma unroll
        for (int v = 0; v < VB / 2; ++v)
          w[v] = (uint32_t)f32_to_bf16(y[2 * v]) | ((uint32_t)f32_to_bf16(y[2 * v + 1]) << 16);
        if constexpr (VB == 8)
          *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
        else
          *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
      } else {
        float* dst = reinterpret_cast<float*>(a.out) + orow * D + d0;
#pragma unroll
        for (int v = 0; v < VB; v += 4)
          *reinterpret_cast<float4*>(dst + v) = float4{y[v], y[v + 1], y[v + 2], y[v + 3]};
      }
    }
    if (a.lse_out != nullptr && k4 == 0)
      a.lse_out[orow] = lt > 0.0f ? (m[j] * qscale + log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, bool QF32>
int launch_t(const PrefillArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)a.B * a.Hkv * a.row_blocks);
  hipLaunchKernelGGL((attn_prefill_kernel<D, QF32>), dim3(blocks), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace

int prefill_rows_per_block() { return kRows; }

int launch_attn_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.D == 128) return a.in_bf16 ? launch_t<128, false>(a, s) : launch_t<128, true>(a, s);
  if (a.D == 64) return a.in_bf16 ? launch_t<64, false>(a, s) : launch_t<64, true>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
