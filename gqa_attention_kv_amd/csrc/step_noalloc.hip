// gqa_decode_step_noalloc: the fused decode step (gqa_decode_step_multi)
// for callers that cannot allocate device memory -- code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation.  The
// step's workspace (arrival tickets and split-K partials) lives in a
// file-scope device array instead of a caller buffer.
//
// Layout of the array on each device:
//   [0, kTicketBytes)        uint32 arrival tickets, one per (sequence, KV
//                            head), always at offset 0 so every call finds
//                            them at zero whatever its shape (each call that
//                            completes leaves its tickets at zero);
//   [kTicketBytes, ...)      the lse partials [B,S,Hq,NP] fp32 (rounded up
//                            to 256 bytes), then the o partials
//                            [B,S,Hq,NP,D] fp32, rewritten by every call.
#include <mutex>

#include "launch.h"

namespace gqa {
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB per device
constexpr int kMaxTickets = 4096;                   // B * Hkv
constexpr size_t kTicketBytes = kMaxTickets * sizeof(uint32_t);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_setup;
char* g_scratch[kMaxDevices];   // device address of `scratch` on each device, after set-up

__global__ void clear_tickets(uint32_t* t, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) t[i] = 0u;
}

// The current device's copy of `scratch`.  The first call on a device looks
// up its address (the name itself is a host-side stand-in, not a device
// address) and clears the ticket region with a fill kernel on `stream`,
// ahead of the step.
int device_scratch(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_setup);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GQA_ERR_LAUNCH;
    hipLaunchKernelGGL(clear_tickets, dim3(kMaxTickets / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), kMaxTickets);
    if (hipGetLastError() != hipSuccess) return GQA_ERR_LAUNCH;
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return GQA_OK;
}

}  // namespace
}  // namespace gqa

extern "C" int gqa_decode_step_noalloc(
    const void* q, const void* k_new, const void* v_new, gqa_dtype_t in_dtype,
    int64_t q_bstride, int64_t kv_bstride, const float* q_norm_w, const float* k_norm_w,
    float eps, const double* inv_freq, double rope_mscale, int rope_layout, const int32_t* pos,
    int S, uint16_t* k_cache, uint16_t* v_cache, const int32_t* lens, int window, float scale,
    int part_tokens, void* out, gqa_dtype_t out_dtype, float* lse_out, float* q_out, int B,
    int Hq, int Hkv, int D, int T, hipStream_t stream) {
  gqa::KernelArgs a{};
  int rc = gqa::decode_step_args(q, k_new, v_new, in_dtype, q_bstride, kv_bstride, q_norm_w,
                                 k_norm_w, eps, inv_freq, rope_mscale, rope_layout, pos, S,
                                 k_cache, v_cache, lens, window, scale, part_tokens, out,
                                 out_dtype, lse_out, q_out, B, Hq, Hkv, D, T, &a);
  if (rc) return rc;
  // the shape must fit the static array
  const size_t lse = gqa::step_lse_bytes(B, S, Hq, a.num_parts);
  const size_t o = (size_t)B * S * Hq * a.num_parts * D * sizeof(float);
  if ((int64_t)B * Hkv > gqa::kMaxTickets || lse + o > gqa::kScratchBytes - gqa::kTicketBytes)
    return GQA_ERR_SCRATCH;
  char* ws = nullptr;
  if ((rc = gqa::device_scratch(stream, &ws))) return rc;
  a.ws_cnt = reinterpret_cast<uint32_t*>(ws);
  a.ws_lse = reinterpret_cast<float*>(ws + gqa::kTicketBytes);
  a.ws_o = reinterpret_cast<float*>(ws + gqa::kTicketBytes + lse);
  return gqa::launch_decode_step(a, stream);
}
