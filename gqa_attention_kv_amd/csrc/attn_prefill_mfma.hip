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
// streams the K/V rows they need through LDS in tiles of 64 rows, shared by
// all 4 waves; each wave owns 32 rows (two blocks of 16).
//
// Lane l, with n = l % 16 and k4 = l / 16, per 16-row block (columns = query
// rows, so a row's softmax state stays in its own lanes):
//   QK: S^T[16 keys x 16 rows] += K[16 x 32] * q^T[32 x 16] per 32-wide slice
//       of D (v_mfma_f32_16x16x32_bf16), for both 16-key halves of the tile.
//       The results leave lane l holding keys 4 k4 + i and 16 + 4 k4 + i
//       (i < 4) of query row n.  An fp32 q is split into bf16 hi + lo and
//       takes two calls per slice; a bf16 q takes one.
//   PV: O^T[16 cols x 16 rows] += V^T[16 x 32] * P^T[32 x 16] per 16-column
//       block, the 32 keys of the tile as the k index in the order lane l's
//       P operand already holds them: k = 8 k4 + e is key 4 k4 + e (e < 4)
//       or 16 + 4 k4 + e - 4.  V stays row-major in LDS; lane l's V operand
//       comes from two transposed reads (ds_read_b64_tr_b16, four key rows
//       each).  P is rounded once to bf16 when the output is bf16 (a
//       relative error of at most 2^-8 per weight, so at most 2^-8 of
//       sum p|V| / sum p in the output, the order of the output's own
//       rounding); for an fp32 output P is carried as bf16 hi + lo (~16
//       mantissa bits) in two calls on the same V operand.
// K and V tiles go from the cache straight into LDS (buffer loads with the
// LDS destination) through two stages each, the next tile fetched while the
// current one is computed, with one barrier per tile.  Online softmax per
// row with a lazy rescale: the weights are formed against the current
// reference maximum, which moves only when a row has none yet or a lane's
// weights of the tile sum past 2^8, so P stays at most 256 and O is rarely
// rescaled.  Keys outside a row's range are masked only in tiles that are
// not wholly inside every range of the wave's rows.
#include <type_traits>

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
// Cache rows per LDS tile: 64 (two 32-key halves of the PV k index); 32
// measured 15% slower on the chunked-prefill workload.
constexpr int kKeys = 64;
constexpr int kKB = kKeys / 16;                   // 16-key blocks per tile
static_assert(kKeys == 32 || kKeys == 64, "tile of 32 or 64 keys");
constexpr float kSumLimit = 256.0f;               // lazy rescale: a lane's weight sum per tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int clampi(int64_t v, int lo, int hi) {
  return (int)(v < lo ? lo : v > hi ? hi : v);
}

// Maximum that propagates NaN (IEEE 754-2019 maximum, v_maximum3_f32 on
// gfx950).  Unlike fmaxf it needs no canonicalised inputs, which saves an
// instruction per matrix-core result.  The scores it sees are finite or
// -inf (masked); a NaN could only come from a NaN in an attended row, and
// that reaches the output through the exponential either way.
__device__ __forceinline__ float fmax_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 of a wave, in every lane:
// v_permlane32_swap exchanges the wave's halves and v_permlane16_swap the
// odd and even 16-lane rows (VALU ops, no LDS round trip).
__device__ __forceinline__ float max_over_rows(float t) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t),
                                                  false, false);
  t = fmax_nan(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t),
                                                  false, false);
  return fmax_nan(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Two floats as packed bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// QM: how q arrives -- 0 bf16 as given, 1 float32 as given, 2 / 3 raw
// bf16 / float32 that the kernel normalises and rotates itself (the q half
// of the prologue).  SPLIT: the launch shares each row block's keys among
// a.splits > 1 workgroups (the instances without it keep the plain loop and
// epilogue).  KG: key groups per workgroup -- with KG = 2 the workgroup has
// two groups of kWaves waves on the same rows, group g taking the tiles
// g, g + 2, ... of the range, combined through LDS at the end (for launches
// too small to give every CU two workgroups).
template <int D, int QM, bool PLO, bool SPLIT, int KG>
__global__ __launch_bounds__(kWaves * KG * 64) __attribute__((amdgpu_waves_per_eu(2))) void
attn_prefill_kernel(const PrefillArgs a) {
  static_assert(KG == 1 || KG == 2, "one or two key groups");
  constexpr int NTH = kWaves * KG * 64;   // threads
  constexpr bool QF32 = QM != 0;       // q carried as bf16 hi + lo
  constexpr bool PRO = QM >= 2;
  constexpr int KC = D / 32;            // QK slices
  constexpr int VB = D / 16;            // PV column blocks
  constexpr int RB = D * 2;             // bytes per cache row (unpadded in LDS)
  constexpr int SW = D / 8;             // 16-byte chunks per row
  constexpr int RPR = 256 / RB;         // rows per 256 bytes of LDS
  constexpr int RPB = 1024 / RB;        // rows per 1 KiB block (one wave's direct load)
  constexpr int KBYTES = kKeys * RB;    // one tile of K, and one of V
  constexpr int BPW = KBYTES / 1024 / kWaves;   // 1 KiB blocks per wave per tile, K and V each
  static_assert(BPW >= 1 && KBYTES % (1024 * kWaves) == 0, "tile fill");
  // The swizzle of a lane's row is the same in every block it fills.
  static_assert((4 * kWaves) % SW == 0, "block-invariant swizzle");
  // V operands read ahead in the PV loop (of its 2 D / 16 steps): fewer
  // when q or P take two register sets
  constexpr int VD = QF32 || PLO ? 3 : 6;

  // Two stages of V (lds_a*) and two of K (lds_b*) per key group, 64 KiB
  // per group for D = 128: two one-group workgroups per CU, or one
  // two-group workgroup (the second group's stages are lds_c*, lds_d*).
  // Separate variables, so the compiler can tell a read of one stage from a
  // fill of another in flight (with one array it makes every transposing
  // read wait for all fills); they are laid out in the order of their names.
  // The split instances' arrival flag reuses lds_b0 after the loop, and the
  // key groups' combine the first group's stages and lds_c0.
  constexpr int KB2 = KG == 2 ? KBYTES : 16;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a0[KBYTES], lds_a1[KBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b0[KBYTES], lds_b1[KBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_c0[KB2], lds_c1[KB2];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_d0[KB2], lds_d1[KB2];

  const int Hq = a.Hq, Hkv = a.Hkv, S = a.S, T = a.T;
  const int G = Hq / Hkv;
  const int SG = S * G;
  const int nrb = a.row_blocks;
  const int npairs = a.B * Hkv;

  // Workgroup -> (sequence, KV head, row block, key split).  Workgroup x
  // runs on XCD x % 8; when the pairs split evenly, every row block of a
  // pair lands on the same XCD so its K/V rows are reused from that XCD's
  // L2.  Row blocks run from the last (most keys under the causal mask) to
  // the first; the splits of a row block are adjacent.
  const int splits = SPLIT ? a.splits : 1;
  const int nunits = nrb * splits;
  const int x = blockIdx.x;
  int pair, ui;
  if ((npairs & 7) == 0) {
    const int slot = x >> 3;
    pair = (x & 7) + 8 * (slot / nunits);
    ui = slot % nunits;
  } else {
    pair = x / nunits;
    ui = x % nunits;
  }
  const int rb = nrb - 1 - ui / splits;
  const int sp = ui % splits;
  const int b = pair / Hkv, g = pair % Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index in a scalar register, so tests on the wave's rows (which
  // tiles it works on, which need masks) are scalar branches
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv / kWaves;    // key group
  const int wave = wv % kWaves;   // wave within the group: its rows and its share of the fills
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

  const int64_t slab = ((int64_t)b * Hkv + g) * T * D;
  const uint32_t slab_bytes = (uint32_t)((int64_t)T * D * 2);
  const __amdgpu_buffer_rsrc_t rk = slab_rsrc(a.k_cache + slab, slab_bytes);
  const __amdgpu_buffer_rsrc_t rv = slab_rsrc(a.v_cache + slab, slab_bytes);

  const int ntiles = kend > kbeg ? (kend - kbeg + kKeys - 1) / kKeys : 0;
  // This split's tiles [tb, te): the row block's tiles in `splits` nearly
  // equal runs (all of them with one split).
  const int per = (ntiles + splits - 1) / splits;
  const int tb = min(sp * per, ntiles);
  const int te = min(tb + per, ntiles);

  // Tile fill: K and V rows go from the cache straight into LDS (buffer
  // loads with the LDS destination, no register round trip).  One such load
  // writes 1 KiB of LDS, lane i the 16 bytes at 16 i: RPB rows.  Rows are
  // stored unpadded with their 16-byte chunks permuted -- chunk c of K row r
  // at position c ^ ksw(r), of V row r at c ^ vsw(r) -- so that the operand
  // reads below spread over all banks: a K read takes one chunk of 16
  // consecutive rows, a transposed V read two adjacent chunks of 8
  // consecutive rows per half-wave.  Lane i of wave w fills, in block
  // w + kWaves f of the tile, row RPB (w + kWaves f) + i / SW, position
  // i % SW, i.e. global chunk (i % SW) ^ swizzle; that swizzle does not
  // depend on f.  Keys past the range are clamped into it (they are masked
  // below, and a row the workgroup attends holds finite values).
  auto ksw = [](int r) { return (r / RPR) & (SW - 1); };
  auto vsw = [](int r) { return (2 * (r / RPR)) & (SW - 1); };
  const int frow = wave * RPB + lane / SW;        // the lane's row in its first block
  const uint32_t kfo = (uint32_t)(frow * RB + 16 * ((lane % SW) ^ ksw(frow)));
  const uint32_t vfo = (uint32_t)(frow * RB + 16 * ((lane % SW) ^ vsw(frow)));
  auto clamp_key = [&](int key) { return key < kend ? key : kend - 1; };
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  // One tile of K (V) into the stage at `st`: BPW loads per wave.
  auto issue = [&](int tile, unsigned char* st, uint32_t lane_off,
                   const __amdgpu_buffer_rsrc_t& rsrc) __attribute__((always_inline)) {
    const int base = kbeg + kKeys * tile;
    if (base + kKeys <= kend) {
      // wholly inside the range: the lane's part stays fixed, the tile and
      // the block go in the scalar offset
#pragma unroll
      for (int f = 0; f < BPW; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (lds_ptr_t)(st + 1024 * (wave + kWaves * f)), 16, lane_off,
            (uint32_t)base * (uint32_t)RB + (uint32_t)(kWaves * f * 1024), 0, 0);
    } else {
#pragma unroll
      for (int f = 0; f < BPW; ++f) {
        const int blk = wave + kWaves * f;
        const uint32_t vo = (uint32_t)clamp_key(base + blk * RPB + lane / SW) * (uint32_t)RB +
                            (lane_off & (uint32_t)(RB - 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(st + 1024 * blk), 16, vo, 0,
                                                 0, 0);
      }
    }
  };
  // stage S of key group GR
  auto kstage = [&](auto GR, auto S) __attribute__((always_inline)) -> unsigned char* {
    constexpr int gr = decltype(GR)::value, st = decltype(S)::value;
    if constexpr (gr == 0) return st == 0 ? lds_b0 : lds_b1;
    else return st == 0 ? lds_d0 : lds_d1;
  };
  auto vstage = [&](auto GR, auto S) __attribute__((always_inline)) -> unsigned char* {
    constexpr int gr = decltype(GR)::value, st = decltype(S)::value;
    if constexpr (gr == 0) return st == 0 ? lds_a0 : lds_a1;
    else return st == 0 ? lds_c0 : lds_c1;
  };
  // The first tile of each key group goes out before the q prologue, so
  // that its latency overlaps it: right away when q arrives ready, after the
  // q loads when the kernel normalises and rotates q (loads complete in
  // order, so the q arithmetic must not wait behind the tile).
  // The fill is issued even for a group without tiles (its rows are clamped
  // into the range, or read past the slab, which returns zeros): with the
  // same number of loads on every path the compiler can wait for the q
  // loads alone.
  const int nt = te - tb;
  auto first_fill = [&]() __attribute__((always_inline)) {
    if (KG == 1 || grp == 0) {
      issue(tb, lds_b0, kfo, rk);
      issue(tb, lds_a0, vfo, rv);
    } else {
      issue(tb + 1, lds_d0, kfo, rk);
      issue(tb + 1, lds_c0, vfo, rv);
    }
  };
  if constexpr (!PRO) first_fill();

  // q operands (B of the QK calls): lane holds row n of block j, elements
  // 32c + 8 k4 .. + 8.
  u32x4_t qh[2][KC], ql[2][KC];
  if constexpr (!PRO) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = r0 + kRowsPerWave * wave + 16 * j + n;
      const bool ok = row < SG;
      const int t = ok ? row / G : 0, h = ok ? row % G : 0;
      const int64_t qoff = (int64_t)b * a.q_bstride + ((int64_t)t * Hq + (int64_t)g * G + h) * D;
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
  } else {
    // The q half of the prologue for this lane's rows: RMSNorm over D (the
    // row's four lanes k4 hold a quarter each), then RoPE of token t at
    // position pos[b] + t -- the phase formed and reduced to [-1/2, 1/2]
    // turns in float64, sin and cos from v_sin_f32 / v_cos_f32, which take
    // turns.  NeoX pairs (i, i + D/2) sit in slices c and c + KC/2 of the
    // same lane; interleaved pairs (2i, 2i + 1) side by side in one slice.
    // With two key groups the work is shared: group g computes row block g
    // of its rows (slot 0 below) and the bf16 hi / lo operands are exchanged
    // through LDS, so each SIMD computes every row once.
    constexpr bool SQ = KG == 2;
    constexpr int NJ = SQ ? 1 : 2;        // row blocks computed by this wave
    auto jrow = [&](int jj) { return SQ ? grp : jj; };
    float f[NJ][KC][8];
    bool ok[NJ];
    int tk[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int row = r0 + kRowsPerWave * wave + 16 * jrow(jj) + n;
      ok[jj] = row < SG;
      tk[jj] = ok[jj] ? row / G : 0;
      const int h = ok[jj] ? row % G : 0;
      const int64_t qoff =
          (int64_t)b * a.q_bstride + ((int64_t)tk[jj] * Hq + (int64_t)g * G + h) * D;
      // Every load is issued unconditionally (a row past S*G reads token 0,
      // head 0 of the group and is zeroed below), so they are all in flight
      // together instead of one branch, and one wait, each.
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int e = 32 * c + 8 * k4;
        if constexpr (QM == 3) {
          const float* p = reinterpret_cast<const float*>(a.q) + qoff + e;
          const float4 u = *reinterpret_cast<const float4*>(p);
          const float4 v = *reinterpret_cast<const float4*>(p + 4);
          f[jj][c][0] = u.x; f[jj][c][1] = u.y; f[jj][c][2] = u.z; f[jj][c][3] = u.w;
          f[jj][c][4] = v.x; f[jj][c][5] = v.y; f[jj][c][6] = v.z; f[jj][c][7] = v.w;
        } else {
          const u32x4_t w = *reinterpret_cast<const u32x4_t*>(
              reinterpret_cast<const uint16_t*>(a.q) + qoff + e);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[jj][c][2 * i] = __uint_as_float(w[i] << 16);
            f[jj][c][2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
          }
        }
      }
    }
    // the norm weights and the rotary frequencies of the lane's pairs (NeoX:
    // pair 32 c + 8 k4 + i of slice c < KC/2; interleaved: pair
    // 16 c + 4 k4 + i/2 of slice c) are loaded with the q rows too
    float wv[KC][8];
    if (a.wq != nullptr) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const float4 u = *reinterpret_cast<const float4*>(a.wq + 32 * c + 8 * k4);
        const float4 v = *reinterpret_cast<const float4*>(a.wq + 32 * c + 8 * k4 + 4);
        wv[c][0] = u.x; wv[c][1] = u.y; wv[c][2] = u.z; wv[c][3] = u.w;
        wv[c][4] = v.x; wv[c][5] = v.y; wv[c][6] = v.z; wv[c][7] = v.w;
      }
    }
    constexpr int NFR = D / 8;   // rotary pairs per lane
    double fr[NFR];
    if (a.rope) {
      if (a.rope_interleaved) {
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int t = 0; t < 4; ++t) fr[4 * c + t] = a.inv_freq_rev[16 * c + 4 * k4 + t];
      } else {
#pragma unroll
        for (int c = 0; c < KC / 2; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) fr[8 * c + i] = a.inv_freq_rev[32 * c + 8 * k4 + i];
      }
    }
    first_fill();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) f[jj][c][i] = ok[jj] ? f[jj][c][i] : 0.0f;
    if (a.wq != nullptr) {
      float rs[NJ];
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) ss = fmaf(f[jj][c][i], f[jj][c][i], ss);
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        rs[jj] = ok[jj] ? 1.0f / sqrtf(ss / (float)D + a.eps) : 0.0f;
      }
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int i = 0; i < 8; ++i) f[jj][c][i] = f[jj][c][i] * rs[jj] * wv[c][i];
    }
    if (a.rope) {
      const float ms = a.rope_mscale;
      const int64_t p0 = a.pos[b];
      // element (c, i) of each row and its partner (c2, i2) rotate by the
      // lane's pair `slot` (indices stay compile-time: one loop per layout)
      auto rotate = [&](int c, int i, int c2, int i2, int slot) {
        const double fr_pair = fr[slot];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          const double rev = (double)(p0 + tk[jj]) * fr_pair;
          const float frac = (float)(rev - rint(rev));
          const float cs = __builtin_amdgcn_cosf(frac) * ms, sn = __builtin_amdgcn_sinf(frac) * ms;
          const float a1 = f[jj][c][i], a2 = f[jj][c2][i2];
          f[jj][c][i] = a1 * cs - a2 * sn;
          f[jj][c2][i2] = a2 * cs + a1 * sn;
        }
      };
      if (a.rope_interleaved) {
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int i = 0; i < 8; i += 2) rotate(c, i, c, i + 1, 4 * c + i / 2);
      } else {
#pragma unroll
        for (int c = 0; c < KC / 2; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) rotate(c, i, c + KC / 2, i, 8 * c + i);
      }
    }
    u32x4_t hq[NJ][KC], lq[NJ][KC];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      if (a.q_out != nullptr && sp == 0 && (SQ || grp == 0) && ok[jj]) {
        const int row = r0 + kRowsPerWave * wave + 16 * jrow(jj) + n;
        float* qo = a.q_out + (((int64_t)b * S + tk[jj]) * Hq + (int64_t)g * G + row % G) * D;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          *reinterpret_cast<float4*>(qo + 32 * c + 8 * k4) =
              float4{f[jj][c][0], f[jj][c][1], f[jj][c][2], f[jj][c][3]};
          *reinterpret_cast<float4*>(qo + 32 * c + 8 * k4 + 4) =
              float4{f[jj][c][4], f[jj][c][5], f[jj][c][6], f[jj][c][7]};
        }
      }
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        bf16x8_t hv, lv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hv[i] = (__bf16)f[jj][c][i];
          lv[i] = (__bf16)(f[jj][c][i] - (float)hv[i]);
        }
        hq[jj][c] = __builtin_bit_cast(u32x4_t, hv);
        lq[jj][c] = __builtin_bit_cast(u32x4_t, lv);
      }
    }
    if constexpr (!SQ) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          qh[j][c] = hq[j][c];
          ql[j][c] = lq[j][c];
        }
    } else {
      // Exchange through the second stages, which no fill has touched yet
      // (the first fills of the loop follow its opening barrier, and that
      // barrier waits for these reads): row block j's operands of wave w
      // sit at lane (16 B x 2 KC per lane) in the 8 KiB quarter w % 2 of
      // lds_a1 / lds_b1 (j = 0) or lds_c1 / lds_d1 (j = 1), the variable
      // chosen by w / 2.
      constexpr int QB = 2 * KC * 16;   // bytes per lane
      static_assert(2 * 64 * QB <= KB2, "exchange fits a stage");
      auto area = [&](int j) -> unsigned char* {
        unsigned char* v = j == 0 ? (wave < 2 ? lds_a1 : lds_b1) : (wave < 2 ? lds_c1 : lds_d1);
        return v + (wave & 1) * 64 * QB + lane * QB;
      };
      unsigned char* mine = area(grp);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        *reinterpret_cast<u32x4_t*>(mine + 16 * c) = hq[0][c];
        *reinterpret_cast<u32x4_t*>(mine + 16 * (KC + c)) = lq[0][c];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const unsigned char* src = area(j);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          qh[j][c] = *reinterpret_cast<const u32x4_t*>(src + 16 * c);
          ql[j][c] = *reinterpret_cast<const u32x4_t*>(src + 16 * (KC + c));
        }
      }
    }
  }

  // The q operands are complete before the loop: without this, the first
  // use inside the loop would wait for every load in flight (on each trip,
  // the prefetch of the tile after next as well).
  wait_vmem();

  f32x4_t o[2][VB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < VB; ++v) o[j][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  // the exponent's reference: m * qscale, or 0 while m = -inf; it changes
  // only with m, so it is kept rather than rebuilt every tile
  float mq[2] = {0.f, 0.f};
  float l[2] = {0.f, 0.f};
  const float qscale = a.qscale;

  auto tile_work = [&](int tile) __attribute__((always_inline)) {   // wave-uniform: does the wave attend any key of the tile
    const int k0 = kbeg + kKeys * tile;
    return wave_live && k0 < need_hi && k0 + kKeys > need_lo;
  };

  constexpr int NH = kKB / 2;
  f32x4_t s[kKB][2];              // scores of the tile whose softmax comes next
  u32x4_t ph[NH][2], pl[NH][2];   // P of the tile whose PV comes next

  // QK for every 16-key block and both row blocks of the tile in K stage
  // `cur`.  The K operands of block kb + 1 are read from LDS while block
  // kb's calls run (two register sets; the scheduling barriers keep the
  // reads ahead).
  auto qk = [&](const unsigned char* cur) __attribute__((always_inline)) {
    u32x4_t kbuf[2][KC];
    auto kread = [&](int kb, u32x4_t* dst) {
#pragma unroll
      for (int c = 0; c < KC; ++c)
        dst[c] = *reinterpret_cast<const u32x4_t*>(
            cur + 16 * kb * RB +
            ((uint32_t)(n * RB + 16 * ((4 * c + k4) ^ ksw(16 * kb + n))) &
             (uint32_t)(16 * RB - 1)));   // the lane's part masked as the V reads' is
    };
    kread(0, kbuf[0]);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      s[kb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (kb + 1 < kKB) kread(kb + 1, kbuf[(kb + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4_t ka = kbuf[kb & 1][c];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          s[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qh[j][c]),
              s[kb][j], 0, 0, 0);
          if constexpr (QF32)
            s[kb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, ql[j][c]),
                s[kb][j], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The online softmax of the tile starting at key k0: masks, row maxima,
  // lazy rescale, P = exp2(s * qscale - m * qscale) as the B operands of the
  // PV calls, one per 32-key half h: bf16 (hi) and, for an fp32 output, the
  // bf16 remainder (lo).  Word w of half h holds k = 2w, 2w + 1: keys
  // 32h + (4 k4 + 2w, + 1) for w < 2, 32h + (16 + 4 k4 + 2w - 4, + 1) for
  // w >= 2.
  auto softmax = [&](int k0) __attribute__((always_inline)) {
    const bool full = k0 >= free_lo && k0 + kKeys <= free_hi;
    if (!full) {
      // Key k0 + 4 k4 + x (x = 16 kb + i) is in row j's range iff
      // min(x - lo, hi - 1 - x) >= 0 with lo, hi taken relative to
      // k0 + 4 k4; the sign of that minimum, spread over the word, selects
      // -inf (v_bfi_b32).  Per-lane arithmetic: comparisons would each
      // leave a lane mask in scalar registers, more of them than there are.
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int lo = rlo[j] - (k0 + 4 * k4);
        const int hm1 = rhi[j] - 1 - (k0 + 4 * k4);
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int x = 16 * kb + i;
            const int d = min(x - lo, hm1 - x);
            const uint32_t out = (uint32_t)(d >> 31);   // all ones outside the range
            s[kb][j][i] = __uint_as_float((__float_as_uint(s[kb][j][i]) & ~out) |
                                          (0xff800000u & out));
          }
      }
    }
    // P against the current references and each lane's sum of them.
    float ps[2];
    auto weights = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float mref = mq[j];
        float p[kKB][4];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][j][i], qscale, -mref));
            ps[j] = kb == 0 && i == 0 ? p[0][0] : ps[j] + p[kb][i];
          }
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float pa = p[2 * hh + (w >> 1)][2 * (w & 1)];
            const float pb = p[2 * hh + (w >> 1)][2 * (w & 1) + 1];
            const uint32_t hw = pack_bf16(pa, pb);
            ph[hh][j][w] = hw;
            if constexpr (PLO)
              pl[hh][j][w] = pack_bf16(pa - __uint_as_float(hw << 16),
                                       pb - __uint_as_float(hw & 0xffff0000u));
          }
      }
    };
    weights();
    // The reference maximum moves only when a row has none yet (-inf: no
    // finite score seen) or a lane's weights of the tile sum past 2^8 (so
    // every accepted weight is at most 2^8).  Only then is the tile's exact
    // row maximum formed, the state rescaled and the weights recomputed;
    // the common tile takes no maximum at all.
    const bool need0 = m[0] == -INFINITY || ps[0] > kSumLimit;
    const bool need1 = m[1] == -INFINITY || ps[1] > kSumLimit;
    if (__any(need0 || need1)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float t = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
          t = fmax_nan(t, fmax_nan(fmax_nan(s[kb][j][0], s[kb][j][1]),
                                   fmax_nan(s[kb][j][2], s[kb][j][3])));
        t = max_over_rows(t);
        const float mnew = fmax_nan(m[j], t);
        // false for a NaN maximum (the NaN reaches the output through the
        // weights) and while the row has seen only -inf
        const bool move = mnew > m[j];
        const float alpha = move ? __builtin_amdgcn_exp2f((m[j] - mnew) * qscale) : 1.0f;
        if (move) {
          m[j] = mnew;
          mq[j] = m[j] * qscale;
        }
        l[j] *= alpha;
#pragma unroll
        for (int v = 0; v < VB; ++v) o[j][v] *= alpha;
      }
      weights();
    }
    l[0] += ps[0];
    l[1] += ps[1];
  };

  // PV with the tile in V stage `curv`: O^T[16 cols x 16 rows] +=
  // V^T[16 x 32] * P^T[32 x 16] per column block and 32-key half.  V
  // operands: column block v, lane row n is column 16 v + n of V, and its
  // eight k are keys 4 k4 + e and 16 + 4 k4 + e (e < 4) of the half, the
  // order P holds them in.  Each half comes from one transposed read
  // (ds_read_b64_tr_b16): in a group of 16 lanes, lane 4 e + q points at
  // columns 16 v + 4 q .. + 3 of key row 4 k4 + e, and lane n of the group
  // receives column 16 v + n of the four rows.
  // The lane's part of the V read offset for column block v (rows below
  // 16), masked to 16 rows: a no-op that lets the compiler see that a read
  // stays inside its stage (else it waits for the fills of the other stages
  // in flight).  Without the q prologue it is formed once, the empty asm
  // keeping it whole: left to itself the compiler rebuilt it from two parts
  // with an add before every read (the prologue instances, short of
  // registers, keep that).
  const int vq = lane & 3;
  const int vrow = 4 * k4 + ((lane & 15) >> 2);   // vsw(vrow + 16 m) == vsw(vrow)
  auto voff_of = [&](int v) -> uint32_t {
    const int col = 16 * v + 4 * vq;
    return (uint32_t)(vrow * RB + 16 * ((col / 8) ^ vsw(vrow)) + 2 * (col % 8));
  };
  uint32_t voff[VB];
  if constexpr (!PRO) {
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      uint32_t t = voff_of(v);
      asm volatile("" : "+v"(t));
      voff[v] = t & (uint32_t)(16 * RB - 1);
    }
  }
  auto pv = [&](const unsigned char* curv) __attribute__((always_inline)) {
    typedef __attribute__((ext_vector_type(4))) short s16x4_t;
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    auto vread = [&](int x) {
      const int hh = x / VB, v = x % VB;
      const uint32_t o0 = PRO ? voff_of(v) & (uint32_t)(16 * RB - 1) : voff[v];
      // the half and the second four-row group are constants
      const unsigned char* p0 = curv + o0 + 32 * hh * RB;
      const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
      const s16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p0 + 16 * RB));
      const auto a2 = __builtin_bit_cast(uint2, lo4);
      const auto b2 = __builtin_bit_cast(uint2, hi4);
      return u32x4_t{a2.x, a2.y, b2.x, b2.y};
    };
    // VD operands in flight: an LDS read takes longer than the two calls of
    // a step
    u32x4_t vbuf[VD];
#pragma unroll
    for (int x = 0; x < VD - 1; ++x) vbuf[x] = vread(x);
#pragma unroll
    for (int x = 0; x < NH * VB; ++x) {
      const int hh = x / VB, v = x % VB;
      if (x + VD - 1 < NH * VB) vbuf[(x + VD - 1) % VD] = vread(x + VD - 1);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t va = vbuf[x % VD];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        o[j][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, ph[hh][j]), o[j][v],
            0, 0, 0);
        if constexpr (PLO)
          o[j][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pl[hh][j]), o[j][v],
              0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };


  // Tile i (counted from this split's first tile) sits in K and V stage
  // i % 2.  At the top of trip i the K and V of tile i + 1 are fetched into
  // the other stages, which every wave finished reading before the barrier
  // that ended trip i - 1; the trip ends with each wave waiting for its own
  // fills and a barrier, after which every wave sees them.  The loop is
  // unrolled by two so that every LDS access names its stage variable.
  // Key group GR's share of the range: tiles tb + GR + KG it.  Its tile it
  // sits in the group's K and V stage it % 2 (tile 0 was fetched before the
  // q prologue); at the top of trip it the K
  // and V of its next tile are fetched into the other stages, which every
  // wave finished reading before the barrier that ended trip it - 1; the
  // trip ends with each wave waiting for its own fills and a barrier, after
  // which every wave sees them.  The loop is unrolled by two so that every
  // LDS access names its stage variable.  Both groups pass as many
  // barriers: the one with a tile less passes an extra one.
  auto run = [&](auto GR) __attribute__((always_inline)) {
    constexpr int gr = decltype(GR)::value;
    using ic0 = std::integral_constant<int, 0>;
    using ic1 = std::integral_constant<int, 1>;
    const int ng = nt > gr ? (nt - gr + KG - 1) / KG : 0;
    // (the group's first tile was fetched before the q prologue)
    wait_vmem();
    __syncthreads();
    auto trip = [&](int it, auto ST) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      const auto other = std::integral_constant<int, 1 - st>{};
      const int tile = tb + gr + KG * it;
      if (it + 1 < ng) {
        issue(tile + KG, kstage(GR, other), kfo, rk);
        issue(tile + KG, vstage(GR, other), vfo, rv);
      }
      if (tile_work(tile)) {
        // The two waves on a SIMD each alternate matrix-core blocks with
        // VALU softmax work: the one in a matrix-core block issues first, so
        // the other's VALU work fills the gaps instead of competing for the
        // same slots.
        __builtin_amdgcn_s_setprio(1);
        qk(kstage(GR, ST));
        __builtin_amdgcn_s_setprio(0);
        softmax(kbeg + kKeys * tile);
        __builtin_amdgcn_s_setprio(1);
        pv(vstage(GR, ST));
        __builtin_amdgcn_s_setprio(0);
      }
      wait_vmem();
      barrier_lds();
    };
    for (int it = 0; it < ng; it += 2) {
      trip(it, ic0{});
      if (it + 1 < ng) trip(it + 1, ic1{});
    }
    if (KG == 2 && ng < (nt + KG - 1) / KG) barrier_lds();
  };
  if constexpr (KG == 1) {
    run(std::integral_constant<int, 0>{});
  } else {
    if (grp == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
    // Combine the groups' states, row by row, into the first group's
    // registers: the second group's wave w leaves its o (16 KiB per wave),
    // reference maxima and sums in LDS; the first group's wave w holds the
    // same rows in the same lanes.  Every stage read has returned and no
    // fill is in flight (each group's last trip fetches nothing).
    float* om = reinterpret_cast<float*>(wave == 0 ? lds_a0 : wave == 1 ? lds_a1
                                         : wave == 2 ? lds_b0 : lds_b1);
    float* ml = reinterpret_cast<float*>(lds_c0) + 4 * 64 * wave;
    if (grp == 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < VB; ++v)
          *reinterpret_cast<f32x4_t*>(om + 4 * ((j * VB + v) * 64 + lane)) = o[j][v];
      *reinterpret_cast<f32x4_t*>(ml + 4 * lane) = f32x4_t{m[0], m[1], l[0], l[1]};
    }
    __syncthreads();
    if (grp == 0) {
      const f32x4_t o2 = *reinterpret_cast<const f32x4_t*>(ml + 4 * lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // both references are maxima (or -inf) of raw scores; the merged
        // one is the larger, and each side's weights scale by 2^((m - M) q)
        const float m2 = o2[j], l2 = o2[2 + j];
        const float M = fmax_nan(m[j], m2);
        const bool any = M != -INFINITY;
        const float a1 = any ? __builtin_amdgcn_exp2f((m[j] - M) * qscale) : 0.0f;
        const float a2 = any ? __builtin_amdgcn_exp2f((m2 - M) * qscale) : 0.0f;
        l[j] = l[j] * a1 + l2 * a2;
#pragma unroll
        for (int v = 0; v < VB; ++v) {
          const f32x4_t ov = *reinterpret_cast<const f32x4_t*>(om + 4 * ((j * VB + v) * 64 + lane));
          o[j][v] = o[j][v] * a1 + ov * a2;
        }
        m[j] = M;
      }
    }
  }

  // Normalise and store.  Lane (n, k4) holds, for row n of block j, columns
  // 16 v + 4 k4 + i (i < 4) of block v.  With key splits the normalised
  // rows and their lse are this split's partial.
  const int64_t team = (int64_t)pair * nrb + rb;
  constexpr int kCoherent = 0x10;   // sc1: write through to / read from the coherence point
  // this row block's partials (no records without splits)
  const __amdgpu_buffer_rsrc_t ro =
      SPLIT ? slab_rsrc(a.ws_o + team * splits * kRows * D, (uint32_t)(splits * kRows * D * 4))
            : slab_rsrc(nullptr, 0u);
  // (with two key groups the first one holds the combined rows)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float lt = l[j];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int rr = kRowsPerWave * wave + 16 * j + n;    // row within the block
    const int row = r0 + rr;
    if (row >= SG || grp != 0) continue;
    const int t = row / G, h = row % G;
    const int64_t orow = ((int64_t)b * S + t) * Hq + (int64_t)g * G + h;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const float lse = lt > 0.0f ? (m[j] * qscale + log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const int d0 = 16 * v + 4 * k4;
      const float y0 = o[j][v][0] * inv, y1 = o[j][v][1] * inv;
      const float y2 = o[j][v][2] * inv, y3 = o[j][v][3] * inv;
      if constexpr (SPLIT) {
        const uint32_t off = (uint32_t)(((sp * kRows + rr) * D + d0) * 4);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, float4{y0, y1, y2, y3}), ro, off, 0, kCoherent);
      } else if (a.out_bf16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + orow * D + d0;
        *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16(y0, y1), pack_bf16(y2, y3)};
      } else {
        float* dst = reinterpret_cast<float*>(a.out) + orow * D + d0;
        *reinterpret_cast<float4*>(dst) = float4{y0, y1, y2, y3};
      }
    }
    if (k4 == 0) {
      if constexpr (SPLIT)
        __hip_atomic_store(a.ws_lse + (team * splits + sp) * kRows + rr, lse, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else if (a.lse_out != nullptr)
        a.lse_out[orow] = lse;
    }
  }
  if constexpr (!SPLIT) return;

  // Arrival ticket (one per row block): the last split to arrive merges the
  // partials in split order, so reruns are bit-identical, and resets the
  // ticket.  No workgroup waits for another.  Every wave waits until its
  // write-through partial stores are complete before the barrier that
  // precedes the ticket (release), and the last arriver takes an
  // agent-scope acquire fence before it reads the partials back.
  wait_vmem();
  __syncthreads();
  // the tile stages are no longer read: their first word carries the flag
  int* s_last = reinterpret_cast<int*>(lds_b0);
  uint32_t* ticket = a.ws_cnt + team;
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (uint32_t)(splits - 1);
    // one wave invalidates before the barrier that the other waves' reads follow
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_last = last;
  }
  __syncthreads();
  if (!*s_last) return;
  // Thread tid owns float4 groups tid + NTH i of the block's rows x D: row
  // (tid + NTH i) / (D/4).  One memory round trip per split: M, W and A are
  // the running maximum lse, weight sum and weighted sum.
  constexpr int QD = D / 4;
  constexpr int GPT = kRows * QD / NTH;
  const int nvalid = SG - r0 < kRows ? SG - r0 : kRows;
  const float* lse_t = a.ws_lse + team * splits * kRows;
  float Mx[GPT], Wx[GPT];
  float4 Ax[GPT];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    Mx[i] = -INFINITY;
    Wx[i] = 0.0f;
    Ax[i] = float4{0.f, 0.f, 0.f, 0.f};
  }
  for (int q = 0; q < splits; ++q) {
    float lk[GPT];
    float4 ok[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int gi = tid + NTH * i;
      const int rr = gi / QD, d4 = gi % QD;
      lk[i] = -INFINITY;
      ok[i] = float4{0.f, 0.f, 0.f, 0.f};
      if (rr < nvalid) {
        lk[i] = __hip_atomic_load(lse_t + q * kRows + rr, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        ok[i] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(
                        ro, (uint32_t)(((q * kRows + rr) * D + 4 * d4) * 4), 0, kCoherent));
      }
    }
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      if (lk[i] == -INFINITY) continue;           // no key of this split for the row
      const float Mn = fmaxf(Mx[i], lk[i]);
      const float sc = __expf(Mx[i] - Mn);        // 0 while nothing was seen
      const float w = __expf(lk[i] - Mn);
      Wx[i] = Wx[i] * sc + w;
      Ax[i].x = fmaf(w, ok[i].x, Ax[i].x * sc);
      Ax[i].y = fmaf(w, ok[i].y, Ax[i].y * sc);
      Ax[i].z = fmaf(w, ok[i].z, Ax[i].z * sc);
      Ax[i].w = fmaf(w, ok[i].w, Ax[i].w * sc);
      Mx[i] = Mn;
    }
  }
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int gi = tid + NTH * i;
    const int rr = gi / QD, d4 = gi % QD;
    if (rr >= nvalid) continue;
    const int row = r0 + rr;
    const int t = row / G, h = row % G;
    const int64_t orow = ((int64_t)b * S + t) * Hq + (int64_t)g * G + h;
    const bool any = Wx[i] > 0.0f;
    const float inv = any ? 1.0f / Wx[i] : 0.0f;
    const float y0 = Ax[i].x * inv, y1 = Ax[i].y * inv, y2 = Ax[i].z * inv, y3 = Ax[i].w * inv;
    if (a.out_bf16) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + orow * D + 4 * d4;
      *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16(y0, y1), pack_bf16(y2, y3)};
    } else {
      float* dst = reinterpret_cast<float*>(a.out) + orow * D + 4 * d4;
      *reinterpret_cast<float4*>(dst) = float4{y0, y1, y2, y3};
    }
    if (d4 == 0 && a.lse_out != nullptr) a.lse_out[orow] = any ? Mx[i] + logf(Wx[i]) : -INFINITY;
  }
  if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compute units of the current device (0 if the attribute cannot be read),
// read once per device.
int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Unsplit launches with fewer workgroups than two per CU (one per CU at
// most, by LDS) run two key groups per workgroup: eight waves on a CU
// instead of four.
template <int D, int QM, bool PLO>
int launch_s(const PrefillArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.row_blocks * a.splits;
  if (a.splits > 1) {
    hipLaunchKernelGGL((attn_prefill_kernel<D, QM, PLO, true, 1>), dim3((unsigned)blocks),
                       dim3(kWaves * 64), 0, s, a);
  } else if (blocks < 2 * (int64_t)cu_count()) {
    hipLaunchKernelGGL((attn_prefill_kernel<D, QM, PLO, false, 2>), dim3((unsigned)blocks),
                       dim3(2 * kWaves * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_prefill_kernel<D, QM, PLO, false, 1>), dim3((unsigned)blocks),
                       dim3(kWaves * 64), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

template <int D, int QM>
int launch_t(const PrefillArgs& a, hipStream_t s) {
  return a.out_bf16 ? launch_s<D, QM, false>(a, s) : launch_s<D, QM, true>(a, s);
}

template <int D>
int launch_d(const PrefillArgs& a, hipStream_t s) {
  if (a.pro) return a.in_bf16 ? launch_t<D, 2>(a, s) : launch_t<D, 3>(a, s);
  return a.in_bf16 ? launch_t<D, 0>(a, s) : launch_t<D, 1>(a, s);
}

}  // namespace

int prefill_rows_per_block() { return kRows; }

int launch_attn_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.D == 128) return launch_d<128>(a, s);
  if (a.D == 64) return launch_d<64>(a, s);
  return GQA_ERR_UNSUPPORTED;
}

}  // namespace gqa
