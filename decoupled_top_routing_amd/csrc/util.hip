// Measurement aid: the read-only HBM streaming ceiling of the device.
//
// Every 16-byte chunk of a buffer is loaded exactly once with a streaming
// (non-temporal) load, as the expert kernels load their weights, and folded
// into an xor so the loads are live; each workgroup writes one word.  The
// time of a launch over a buffer far larger than the 256 MB Infinity Cache
// gives the rate a read-only kernel can reach, the ceiling against which the
// decode kernels' bandwidth is judged.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4 *__restrict__ p,
                                                                   uint64_t n16,
                                                                   uint32_t *__restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 q[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) q[u] = ld16_stream(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 q = ld16_stream(p + i);
    acc ^= q.x ^ q.y ^ q.z ^ q.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  __shared__ uint32_t s[kProbeThreads / kWave];
  if (lane_id() == 0) s[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace
}  // namespace moe

extern "C" int moe_hbm_read_probe(const void *buf, size_t bytes, uint32_t *out, int32_t blocks,
                                  void *stream) {
  if (!buf || !out || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536)
    return MOE_EINVAL;
  if ((uintptr_t)buf % 16 != 0 || (uintptr_t)out % 4 != 0) return MOE_EALIGN;
  moe::read_probe_kernel<<<dim3((unsigned)blocks), dim3(moe::kProbeThreads), 0,
                           (hipStream_t)stream>>>(static_cast<const uint4 *>(buf),
                                                  (uint64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
