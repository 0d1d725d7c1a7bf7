// Streaming-read ceiling: the rate at which one launch reads a contiguous
// buffer once from HBM, with nothing else to do.  It is the bare form of
// what the decode kernels spend their time on (each K/V row read once,
// 16-byte non-temporal loads), so a decode step can be judged against what
// the part actually streams for the same number of bytes, not only against
// its nominal 8 TB/s.  Not part of the attention path.
//
// Workgroup w reads the w-th contiguous share of the buffer, lanes at
// consecutive 16-byte offsets, U loads in flight per lane.  The loaded words
// are folded into one value that is written only if it equals a constant no
// input here produces, which keeps every load alive without a store stream.
#include "device_common.h"
#include "launch.h"
#include "../../include/gqa_decode.h"

namespace gqa {

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kNonTemporal = 2;
constexpr uint32_t kNever = 0x9E3779B9u;

template <int U>
__global__ void stream_read_kernel(const void* base, uint32_t bytes, uint32_t share,
                                   uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  const uint32_t beg = blockIdx.x * share;
  const uint32_t end = min(beg + share, bytes);
  const uint32_t step = 16u * blockDim.x;
  uint32_t acc = 0;
  for (uint32_t off = beg + 16u * threadIdx.x; off < end; off += U * step) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)   // past the end the buffer returns zeros
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * step < end ? off + u * step : bytes,
                                                   0, kNonTemporal);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == kNever) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

int launch_stream_read(const void* buf, uint32_t bytes, int workgroups, int threads, int unroll,
                       uint32_t* sink, hipStream_t s) {
  // shares are whole multiples of one trip (threads * 16 bytes)
  const uint32_t trip = 16u * (uint32_t)threads;
  const uint64_t per = ((uint64_t)bytes + workgroups - 1) / workgroups;
  const uint32_t share = (uint32_t)((per + trip - 1) / trip * trip);
  const dim3 grid(workgroups), block(threads);
  switch (unroll) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, s, buf, bytes, share, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, s, buf, bytes, share, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, s, buf, bytes, share, sink); break;
    default: return GQA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace gqa
