// Device helpers shared by the gfx950 kernels: bf16 packing, DPP lane
// exchange, wave-level reductions and a float64 sin/cos of a reduced angle.
// Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bit pattern -> float32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two bf16 packed in one dword -> float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight bf16 in a 16-byte vector -> eight float32, element order preserved.
__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// float32 -> bf16 bits, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// DPP lane exchange within a 16-lane row (gfx9 encodings).
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <- lane 7-i inside each 8-lane half row
  kDppMirror = 0x140,     // lane i <- lane 15-i inside each 16-lane row
  kDppRowRor8 = 0x128,    // lane i <- lane i^8 inside each 16-lane row (rotate by 8)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 8 or 16), result in every lane of
// the group.  After the two quad steps each lane holds its quad's sum; the
// half-row mirror pairs quad 0 with quad 1, the row mirror pairs the halves.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (N == 16) v += dpp<kDppMirror>(v);
  return v;
}

// Sum over aligned groups of N lanes for any power of two N <= 64 (shuffles).
template <int N>
__device__ __forceinline__ float group_sum_shfl(float v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// sin and cos of |x| <= pi in float64, with few registers: x = k pi/2 + r
// (k = rint(2x/pi), pi/2 in two parts, |r| <= pi/4), then the Taylor series
// of sin r through r^17 and of cos r through r^16 (truncation below 1e-16
// on |r| <= pi/4, Horner form), and the quadrant k mod 4 swaps and signs.
__device__ __forceinline__ void sincos_pi_f64(double x, double* s, double* c) {
  constexpr double kHalfPi1 = 1.5707963267948966;      // fp64 nearest pi/2
  constexpr double kHalfPi2 = 6.123233995736766e-17;   // pi/2 - kHalfPi1
  const double k = rint(x * 0.6366197723675814);
  const double r = (x - k * kHalfPi1) - k * kHalfPi2;
  const double z = r * r;
  double ps = 1.0 / 355687428096000.0;                 // 1/17!
  ps = fma(ps, -z, 1.0 / 1307674368000.0);             // 1/15!
  ps = fma(ps, -z, 1.0 / 6227020800.0);                // 1/13!
  ps = fma(ps, -z, 1.0 / 39916800.0);                  // 1/11!
  ps = fma(ps, -z, 1.0 / 362880.0);                    // 1/9!
  ps = fma(ps, -z, 1.0 / 5040.0);                      // 1/7!
  ps = fma(ps, -z, 1.0 / 120.0);                       // 1/5!
  ps = fma(ps, -z, 1.0 / 6.0);                         // 1/3!
  const double sr = fma(-z * r, ps, r);
  double pc = 1.0 / 20922789888000.0;                  // 1/16!
  pc = fma(pc, -z, 1.0 / 87178291200.0);               // 1/14!
  pc = fma(pc, -z, 1.0 / 479001600.0);                 // 1/12!
  pc = fma(pc, -z, 1.0 / 3628800.0);                   // 1/10!
  pc = fma(pc, -z, 1.0 / 40320.0);                     // 1/8!
  pc = fma(pc, -z, 1.0 / 720.0);                       // 1/6!
  pc = fma(pc, -z, 1.0 / 24.0);                        // 1/4!
  pc = fma(pc, -z, 0.5);                               // 1/2!
  const double cr = fma(-z, pc, 1.0);
  const int q = (int)k & 3;
  const double sv = (q & 1) ? cr : sr, cv = (q & 1) ? sr : cr;
  *s = (q & 2) ? -sv : sv;
  *c = (q == 1 || q == 2) ? -cv : cv;
}

// Waits until every vector-memory access this wave has issued is complete
// (s_waitcnt vmcnt(0); the LDS and export counters are left unrestricted).
// A store's counter drops only once the store is acknowledged at the level
// its scope bits name, so after this wait a device-scope (write-through)
// store has reached the point where every XCD reads it.  A workgroup-scope
// release fence does not give this on gfx950: all waves of a workgroup share
// one CU, so it waits only for LDS traffic.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until at most N of this wave's vector memory operations are still
// outstanding (s_waitcnt vmcnt(N), N < 16): they complete in issue order,
// so everything but the N most recent ones is done.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier after this wave's LDS reads have returned, leaving
// vector memory alone.  __syncthreads() is a release/acquire fence plus the
// barrier, and the fence also waits for every load still in flight into
// LDS (buffer loads with the LDS destination count as vector memory), which
// would drain a tile prefetch at every barrier.  A caller that needs some
// of those loads complete waits for them itself beforehand.  The memory
// clobber keeps the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace gqa
