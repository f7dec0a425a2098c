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
// dn[e_r, c] * |a| is the channel's score.  An exact radix select over the
// token's n = k1*I scores keeps the `keep` highest (equal scores: the lower
// flat index j = r*I + c first) and sets every other activation to zero:
// the down kernel then sums the kept channels only.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kSelThreads = 1024;
constexpr int kSelMaxN = 8192;  // 8 channels per thread

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

// Exclusive prefix sum over the block's threads (kSelThreads, in thread
// order) of v; *total receives the sum.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *s_wave, uint32_t *total) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) s_wave[wv] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < kSelThreads / kWave; ++w) {
    const uint32_t t = s_wave[w];
    before += w < wv ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// One workgroup per token.  Thread i holds the scores of the flat channels
// j = 8i .. 8i+7: I is a multiple of 8, so they belong to one expert and
// come in with one id load and 16-byte loads of a and dn (scores are >= 0,
// so their bit patterns order like their values).  Four passes over 8-bit digits, most significant first, find the
// exact keep-th largest score tau: each pass counts the candidates (scores
// that share the digits found so far) per digit in per-wave LDS histograms,
// and the digit where the count from the top reaches the remaining rank is
// taken.  Scores above tau are kept, and of those equal to tau the
// remaining number with the lowest j (a block scan in j order).
constexpr int kSelPer = kSelMaxN / kSelThreads;  // 8 channels per thread
constexpr int kSelWaves = kSelThreads / kWave;

__global__ __launch_bounds__(kSelThreads) void channel_select_kernel(
    float *__restrict__ abuf, int k1, int I, const int32_t *__restrict__ ids,
    const float *__restrict__ dn, int keep, float *__restrict__ scores_out,
    uint8_t *__restrict__ kept_out) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t s_wave[kSelWaves];
  __shared__ uint32_t s_digit, s_rem;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int n = k1 * I;
  float *a = abuf + t * (int64_t)n;
  static_assert(kSelPer == 8, "two 16-byte loads per thread");
  const int j0 = tid * kSelPer;
  const bool mine = j0 < n;  // n and j0 are multiples of 8
  uint32_t key[kSelPer];
  float av[kSelPer];
  if (mine) {
    const int r = j0 / I, c0 = j0 - r * I;
    const float *dp = dn + (int64_t)ids[t * k1 + r] * I + c0;
    Elem<float>::widen(ld16(a + j0), av);
    Elem<float>::widen(ld16(a + j0 + 4), av + 4);
    float dv[kSelPer];
    Elem<float>::widen(ld16(dp), dv);
    Elem<float>::widen(ld16(dp + 4), dv + 4);
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) {
      const float sc = dv[q] * fabsf(av[q]);
      key[q] = __float_as_uint(sc);
    }
    if (scores_out) {
      float *so = scores_out + t * (int64_t)n + j0;
      *reinterpret_cast<float4 *>(so) = make_float4(__uint_as_float(key[0]), __uint_as_float(key[1]),
                                                    __uint_as_float(key[2]), __uint_as_float(key[3]));
      *reinterpret_cast<float4 *>(so + 4) =
          make_float4(__uint_as_float(key[4]), __uint_as_float(key[5]), __uint_as_float(key[6]),
                      __uint_as_float(key[7]));
    }
  } else {
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) key[q] = 0u;
  }
  uint32_t prefix = 0u, mask = 0u, rem = (uint32_t)keep;
  if (keep > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kSelPer; ++q) {
        const int j = tid * kSelPer + q;
        if (j < n && (key[q] & mask) == prefix) atomicAdd(&hist[wv][(key[q] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t c = 0;
        for (int w = 0; w < kSelWaves; ++w) c += hist[w][tid];
        tot[tid] = c;
      }
      __syncthreads();
      if (wv == 0) {
        // lane l holds digits 4l..4l+3; counts from the top (digit 255 down)
        uint32_t cnt[4], local = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          cnt[d] = tot[4 * lane + d];
          local += cnt[d];
        }
        // above[l] = candidates with a digit in a higher lane's range
        uint32_t incl = local;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t u = (uint32_t)__shfl_down((int)incl, o);
          if (lane + o < kWave) incl += u;
        }
        uint32_t above = incl - local;
        // the digit whose count from the top first reaches rem
#pragma unroll
        for (int d = 3; d >= 0; --d) {
          if (above < rem && rem <= above + cnt[d]) {
            s_digit = (uint32_t)(4 * lane + d);
            s_rem = rem - above;
          }
          above += cnt[d];
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      mask |= 255u << shift;
      rem = s_rem;
      __syncthreads();
    }
  }
  // prefix = tau; rem = how many scores equal to tau are kept, lowest j first
  uint32_t eq = 0;
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) eq += (tid * kSelPer + q < n && key[q] == prefix) ? 1u : 0u;
  uint32_t total;
  uint32_t before = block_exclusive_scan(eq, s_wave, &total);
  (void)total;
  if (!mine) return;
  uint32_t flags8[2] = {0u, 0u};
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) {
    bool on = false;
    if (keep > 0) {
      if (key[q] > prefix) {
        on = true;
      } else if (key[q] == prefix) {
        on = before < rem;
        ++before;
      }
    }
    if (!on) av[q] = 0.0f;
    flags8[q >> 2] |= (on ? 1u : 0u) << (8 * (q & 3));
  }
  *reinterpret_cast<float4 *>(a + j0) = make_float4(av[0], av[1], av[2], av[3]);
  *reinterpret_cast<float4 *>(a + j0 + 4) = make_float4(av[4], av[5], av[6], av[7]);
  if (kept_out)
    *reinterpret_cast<uint2 *>(kept_out + t * (int64_t)n + j0) = make_uint2(flags8[0], flags8[1]);
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
