// Device scratch of moe_forward_noalloc: a fixed array in place of the
// caller's workspace, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable, so each device the library
// runs on holds its own copy (at its own address) until the process ends.
// Its name is a host-side stand-in in host code: the device address comes
// from hipGetSymbolAddress, taken once per device on the first call there,
// and only that address is ever passed to kernels.  Every call on a device
// shares the device's array and finds the last call's contents; what must
// start at zero (the sync region and the one-token kernel's hand-over
// region, which later calls keep consistent themselves) is cleared once, by a
// fill kernel on the first call's stream.  Calls that overlap on one device
// race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace moe {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];  // device address per device, once taken

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void **ptr, size_t zero_prefix, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    const size_t n16 = (zero_prefix < kScratchBytes ? zero_prefix : kScratchBytes) / 16;
    zero_fill_kernel<<<dim3(64), dim3(256), 0, s>>>(static_cast<uint4 *>(p), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
