// Channel top-k inside the activated experts ("Channel Selection for
// Mixture-of-Experts Decoding Needs No Calibration Data", section 5.2: the
// output-scaled score of a channel is its router weight times its down
// column's norm times its activation's magnitude, and the exact top-k over
// a token's channels across its experts is kept; section 2: a channel owns
// one gate row, one up row and one down column).
//
// down_column_norms_kernel: dn[e, c] = ||Wd[e, :, c]||_2 (fp32 sums of
// squares), once per weight set.
// channel_select_kernel: one workgroup per token, after the grouped gate/up
// kernel has stored a[t*k1 + r, c] = silu(g) * u * w_r.  Since w_r > 0,
// dn[e_r, c] * |a| is the channel's score.  The token's n = k1*I scores are
// sorted in LDS as 64-bit keys (score bits, then the complement of the flat
// index j = r*I + c, so equal scores put the lower j first), the first
// `keep` are marked, and every other activation is set to zero: the down
// kernel then sums the kept channels only.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kSelThreads = 1024;
constexpr int kSelMaxN = 8192;  // 64 KiB of keys in LDS

template <typename WT>
__global__ __launch_bounds__(256) void down_column_norms_kernel(const WT *__restrict__ Wd, int E,
                                                                int H, int I,
                                                                float *__restrict__ dn) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // e * I + c
  if (i >= (int64_t)E * I) return;
  const int64_t e = i / I, c = i - e * I;
  const WT *col = Wd + e * H * (int64_t)I + c;
  float s = 0.0f;
  for (int h = 0; h < H; ++h) {
    const float v = Elem<WT>::load1(col + (int64_t)h * I);
    s = __builtin_fmaf(v, v, s);
  }
  dn[i] = __builtin_sqrtf(s);
}

__global__ __launch_bounds__(kSelThreads) void channel_select_kernel(
    float *__restrict__ abuf, int k1, int I, const int32_t *__restrict__ ids,
    const float *__restrict__ dn, int keep, float *__restrict__ scores_out,
    uint8_t *__restrict__ kept_out) {
  __shared__ uint64_t keys[kSelMaxN];
  __shared__ uint32_t kept[kSelMaxN / 32];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = k1 * I;
  int P = 1;
  while (P < n) P <<= 1;
  float *a = abuf + t * (int64_t)n;
  for (int j = tid; j < P; j += kSelThreads) {
    uint64_t key = 0;  // padding sorts after every channel
    if (j < n) {
      const int r = j / I, c = j - r * I;
      const float s = dn[(int64_t)ids[t * k1 + r] * I + c] * fabsf(a[j]);
      if (scores_out) scores_out[t * (int64_t)n + j] = s;
      key = ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
    }
    keys[j] = key;
  }
  for (int j = tid; j < kSelMaxN / 32; j += kSelThreads) kept[j] = 0u;
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P; i += kSelThreads) {
        const int l = i ^ jj;
        if (l > i) {
          const uint64_t x = keys[i], y = keys[l];
          const bool desc = (i & k) == 0;
          if ((x < y) == desc) {
            keys[i] = y;
            keys[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < keep; i += kSelThreads) {
    const uint32_t j = 0xFFFFFFFFu - (uint32_t)keys[i];
    atomicOr(&kept[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  for (int j = tid; j < n; j += kSelThreads) {
    const bool on = (kept[j >> 5] >> (j & 31)) & 1u;
    if (!on) a[j] = 0.0f;
    if (kept_out) kept_out[t * (int64_t)n + j] = on ? 1 : 0;
  }
}

bool channel_select_supported(int k1, int I) { return (int64_t)k1 * I <= kSelMaxN; }

template <typename WT>
hipError_t launch_down_column_norms(const WT *Wd, int E, int H, int I, float *dn,
                                    hipStream_t s) {
  const int64_t n = (int64_t)E * I;
  down_column_norms_kernel<WT><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(Wd, E, H,
                                                                                      I, dn);
  return hipGetLastError();
}

hipError_t launch_channel_select(float *abuf, int64_t T, int k1, int I, const int32_t *ids,
                                 const float *dn, int keep, float *scores_out, uint8_t *kept_out,
                                 hipStream_t s) {
  if (!channel_select_supported(k1, I)) return hipErrorInvalidValue;
  channel_select_kernel<<<dim3((unsigned)T), dim3(kSelThreads), 0, s>>>(abuf, k1, I, ids, dn, keep,
                                                                       scores_out, kept_out);
  return hipGetLastError();
}

template hipError_t launch_down_column_norms<float>(const float *, int, int, int, float *,
                                                    hipStream_t);
template hipError_t launch_down_column_norms<bf16_t>(const bf16_t *, int, int, int, float *,
                                                     hipStream_t);

}  // namespace moe
