// Hand-over of values between workgroups of one kernel without fences or
// counters: a published value is a 64-bit word holding the value and the
// call's tag, written with a device-coherent store; a consumer re-reads the
// words it needs with device-coherent loads until each carries the current
// tag, so the data's arrival is the signal.  Device-coherent (agent scope)
// accesses bypass the caches that are not coherent across the chip; on
// gfx950 an agent-scope fence instead writes back or invalidates a whole L2,
// which takes microseconds.  Every wait is bounded: past its limit of
// re-reads (kSpinLimit unless the call lowers it) the wait gives up and sets
// an error word that the host can read, so a kernel always terminates.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kSyncThreads = 256;         // block size of the staging helper
constexpr uint32_t kSpinLimit = kDefaultSpinLimit;

template <typename T>
__device__ __forceinline__ void coh_st(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T coh_ld(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_inc(int32_t *p) {
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The tag of a call: 31 bits of the workspace's epoch with the low bit set,
// so a zero-filled word never carries a tag.  Tagged words live in a region
// of the workspace that only the hand-over uses, at fixed places that do not
// depend on the call's shapes, so a word can only carry the current tag if
// this call wrote it, or if 2^31 calls passed since it was last written.
__device__ __forceinline__ uint32_t call_tag(uint32_t epoch) { return (epoch << 1) | 1u; }

__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) {
  return ((uint64_t)tag << 32) | __float_as_uint(v);
}

// Re-read a tagged word until it carries `tag` (at most `limit` re-reads);
// returns its value.
__device__ __forceinline__ float await_tagged(const uint64_t *p, uint32_t tag, int32_t *err,
                                              uint32_t limit = kSpinLimit) {
  uint64_t w = coh_ld(p);
  uint32_t n = 0;
  while ((uint32_t)(w >> 32) != tag) {
    __builtin_amdgcn_s_sleep(1);
    if (++n > limit) {
      coh_st(err, 1);
      break;
    }
    w = coh_ld(p);
  }
  return __uint_as_float((uint32_t)w);
}

// Stage n tagged words into dst[0..n) (LDS; dst[0..2n) with two bf16 values
// per word when PACKED), n <= MAXW * kSyncThreads: each
// thread first issues the loads of all its words, then re-reads only those
// that do not carry `tag` yet, so the wait costs one round trip, not one per
// word.  At most `limit` rounds of re-reads.  Ends with a block barrier.
template <int MAXW, bool PACKED = false, typename AddrFn>
__device__ void stage_tagged(float *dst, int n, AddrFn addr, uint32_t tag, int32_t *err,
                             uint32_t limit = kSpinLimit) {
  uint64_t w[MAXW];
  const uint64_t done = (uint64_t)tag << 32;
#pragma unroll
  for (int k = 0; k < MAXW; ++k) {
    const int i = threadIdx.x + k * kSyncThreads;
    w[k] = i < n ? coh_ld(addr(i)) : done;
  }
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int k = 0; k < MAXW; ++k) ok &= (uint32_t)(w[k] >> 32) == tag;
    if (ok) break;
    if (++spins > limit) {
      coh_st(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int k = 0; k < MAXW; ++k) {
      const int i = threadIdx.x + k * kSyncThreads;
      if (i < n && (uint32_t)(w[k] >> 32) != tag) w[k] = coh_ld(addr(i));
    }
  }
#pragma unroll
  for (int k = 0; k < MAXW; ++k) {
    const int i = threadIdx.x + k * kSyncThreads;
    if (i < n) {
      if constexpr (PACKED) {
        dst[2 * i] = bf16_lo((uint32_t)w[k]);
        dst[2 * i + 1] = bf16_hi((uint32_t)w[k]);
      } else {
        dst[i] = __uint_as_float((uint32_t)w[k]);
      }
    }
  }
  __syncthreads();
}

}  // namespace moe
