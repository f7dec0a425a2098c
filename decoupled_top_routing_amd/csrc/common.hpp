// Device helpers shared by the kernels of libmoe.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
// bf16 is the upper half of an IEEE binary32; widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// f rounded to the nearest bf16 value (ties to even), kept as fp32.
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}

// Storage types: weights and activations are either float or bf16 (stored
// as uint16_t bit patterns).
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ void widen(const uint4 &q, float *f) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
  __device__ static __forceinline__ float load1(const float *p) { return *p; }
  __device__ static __forceinline__ void store1(float *p, float v) { *p = v; }
};
template <>
struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;
  __device__ static __forceinline__ void widen(const uint4 &q, float *f) {
    f[0] = bf16_lo(q.x);
    f[1] = bf16_hi(q.x);
    f[2] = bf16_lo(q.y);
    f[3] = bf16_hi(q.y);
    f[4] = bf16_lo(q.z);
    f[5] = bf16_hi(q.z);
    f[6] = bf16_lo(q.w);
    f[7] = bf16_hi(q.w);
  }
  __device__ static __forceinline__ float load1(const bf16_t *p) {
    return __uint_as_float(((uint32_t)p->bits) << 16);
  }
  __device__ static __forceinline__ void store1(bf16_t *p, float v) {
    p->bits = (uint16_t)f32_to_bf16_bits(v);
  }
};

// 16-byte global loads.
__device__ __forceinline__ uint4 ld16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}
// Streaming 16-byte load for data read exactly once (weights): non-temporal
// hint so it does not evict data that is reused.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t t = (uint32_t)__shfl_xor((int)v, o);
    v = t > v ? t : v;
  }
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// a.lo*b.lo + a.hi*b.hi + c for two packed bf16 pairs (v_dot2_f32_bf16):
// the bf16 products are exact in fp32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- DPP
// Wave-wide reductions with DPP lane moves (no LDS round trip).  The order
// is fixed: pairs (xor 1), quads (xor 2), half rows, rows of 16, then rows
// 0+1 and 2+3, then the two halves; the result is read from lane 63.  For
// a sum this is the pairwise tree over the 64 lanes.
namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // row_half_mirror
constexpr int kMirror = 0x140;     // row_mirror
constexpr int kBcast15 = 0x142;    // row_bcast:15
constexpr int kBcast31 = 0x143;    // row_bcast:31

template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t mov(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWMASK, 0xF, false);
}
}  // namespace dpp

__device__ __forceinline__ float wave_sum_dpp(float v) {
  using namespace dpp;
  auto step = [](float a, uint32_t b) { return a + __uint_as_float(b); };
  const uint32_t z = 0u;  // +0.0f
  v = step(v, mov<kXor1>(z, __float_as_uint(v)));
  v = step(v, mov<kXor2>(z, __float_as_uint(v)));
  v = step(v, mov<kHalfMirror>(z, __float_as_uint(v)));
  v = step(v, mov<kMirror>(z, __float_as_uint(v)));
  v = step(v, mov<kBcast15, 0xA>(z, __float_as_uint(v)));
  v = step(v, mov<kBcast31, 0xC>(z, __float_as_uint(v)));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  using namespace dpp;
  const uint32_t ninf = 0xFF800000u;
  v = fmaxf(v, __uint_as_float(mov<kXor1>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(mov<kXor2>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(mov<kHalfMirror>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(mov<kMirror>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(mov<kBcast15, 0xA>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(mov<kBcast31, 0xC>(ninf, __float_as_uint(v))));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  using namespace dpp;
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, mov<kXor1>(0u, v));
  v = mx(v, mov<kXor2>(0u, v));
  v = mx(v, mov<kHalfMirror>(0u, v));
  v = mx(v, mov<kMirror>(0u, v));
  v = mx(v, mov<kBcast15, 0xA>(0u, v));
  v = mx(v, mov<kBcast31, 0xC>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace moe
