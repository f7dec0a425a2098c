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
// the down kernel then sums the kept channels only.  With a kept list it
// also writes, in j order, each kept channel's row in the column copy of the
// down weights and its activation.
// down_columns_kernel: the column copy WdT[e, c, :] = Wd[e, :, c], once per
// weight set, so that a channel's down column is one contiguous row.
// kept_down_kernel + kept_combine_kernel: the down projection from the kept
// list, reading only the kept channels' columns (section 2: reading a
// channel means its gate row, up row and down column).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kSelThreads = 1024;
constexpr int kWaves4 = 4;  // waves of a 256-thread block
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
    uint8_t *__restrict__ kept_out, uint2 *__restrict__ kept_list) {
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
  int row0 = 0;  // row of channel j0 in the column copy: e * I + c
  if (mine) {
    const int r = j0 / I, c0 = j0 - r * I;
    row0 = ids[t * k1 + r] * I + c0;
    const float *dp = dn + (int64_t)row0;
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
  uint32_t flags8[2] = {0u, 0u};
  uint32_t nkept = 0;
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) {
    bool on = false;
    if (mine && keep > 0) {
      if (key[q] > prefix) {
        on = true;
      } else if (key[q] == prefix) {
        on = before < rem;
        ++before;
      }
    }
    if (!on) av[q] = 0.0f;
    flags8[q >> 2] |= (on ? 1u : 0u) << (8 * (q & 3));
    nkept += on ? 1u : 0u;
  }
  if (kept_list) {
    // the kept channels in j order: each thread's place from a block scan
    uint32_t kept_total;
    uint32_t pos = block_exclusive_scan(nkept, s_wave, &kept_total);
    (void)kept_total;
    uint2 *kl = kept_list + t * (int64_t)keep;
#pragma unroll
    for (int q = 0; q < kSelPer; ++q)
      if ((flags8[q >> 2] >> (8 * (q & 3))) & 1u)
        kl[pos++] = make_uint2((uint32_t)(row0 + q), __float_as_uint(av[q]));
  }
  if (!mine) return;
  *reinterpret_cast<float4 *>(a + j0) = make_float4(av[0], av[1], av[2], av[3]);
  *reinterpret_cast<float4 *>(a + j0 + 4) = make_float4(av[4], av[5], av[6], av[7]);
  if (kept_out)
    *reinterpret_cast<uint2 *>(kept_out + t * (int64_t)n + j0) = make_uint2(flags8[0], flags8[1]);
}

// Column copy of the down weights: WdT[e, c, h] = Wd[e, h, c], by 32 x 32
// tiles through LDS (coalesced reads along c, writes along h).
template <typename WT>
__global__ __launch_bounds__(256) void down_columns_kernel(const WT *__restrict__ Wd, int H,
                                                           int I, WT *__restrict__ WdT) {
  __shared__ WT tile[32][33];
  const int64_t e = blockIdx.z;
  const int c0 = blockIdx.x * 32, h0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8 threads
  const WT *src = Wd + e * H * (int64_t)I;
  WT *dst = WdT + e * I * (int64_t)H;
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int h = h0 + ty + k, c = c0 + tx;
    if (h < H && c < I) tile[ty + k][tx] = src[(int64_t)h * I + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int c = c0 + ty + k, h = h0 + tx;
    if (h < H && c < I) dst[(int64_t)c * H + h] = tile[tx][ty + k];
  }
}

// Kept-channel down projection.  Block (t, slice hs, group g) sums, over the
// 16-byte chunk of its h-slice that each lane holds, the kept channels of
// token t in list places [g*per, min(keep, (g+1)*per)): wave w takes every
// fourth of them, reads their list entries 64 at a time with one load per
// lane, and keeps up to kKeptBatch column reads in flight.  The four waves'
// sums are added in wave order; part[t, g, :] takes the block's sums.
constexpr int kKeptBatch = 8;

template <typename WT>
__global__ __launch_bounds__(256) void kept_down_kernel(const WT *__restrict__ WdT, int H,
                                                        const uint2 *__restrict__ list, int keep,
                                                        int per, int G, int n_hs,
                                                        float *__restrict__ part) {
  constexpr int NW = Elem<WT>::kPer16B;
  __shared__ float red[kWaves4][kWave * NW];
  const int b = blockIdx.x;
  const int g = b % G, hs = (b / G) % n_hs;
  const int64_t t = b / (G * n_hs);
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int h0 = (hs * kWave + lane) * NW;
  const bool live = h0 < H;
  const uint2 *kl = list + t * (int64_t)keep;
  const int lo = g * per, hi = min(keep, lo + per);
  float acc[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) acc[k] = 0.0f;
  // this wave's entries are lo + wv + 4 i; 64 of them per outer step
  for (int base = lo + wv; base < hi; base += 4 * kWave) {
    const int mine = base + 4 * lane;
    const uint2 ent = mine < hi ? kl[mine] : make_uint2(0u, 0u);
    const int n = min(kWave, (hi - base + 3) / 4);
    for (int i0 = 0; i0 < n; i0 += kKeptBatch) {
      uint4 q[kKeptBatch];
      float av[kKeptBatch];
#pragma unroll
      for (int k = 0; k < kKeptBatch; ++k) {
        const int i = min(i0 + k, n - 1);
        const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)ent.x, i);
        av[k] = i0 + k < n ? __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)ent.y, i))
                           : 0.0f;
        q[k] = live && i0 + k < n ? ld16_stream(WdT + (int64_t)row * H + h0)
                                  : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < kKeptBatch; ++k) {
        float wv8[NW];
        Elem<WT>::widen(q[k], wv8);
#pragma unroll
        for (int m = 0; m < NW; ++m) acc[m] = __builtin_fmaf(av[k], wv8[m], acc[m]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NW; ++k) red[wv][lane * NW + k] = acc[k];
  __syncthreads();
  if (wv == 0 && live) {
    float *dst = part + (t * G + g) * (int64_t)H + h0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int i = lane * NW + k;
      if (h0 + k < H) dst[k] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
    }
  }
}

// y[t, h] = the sum of the groups' partial sums, in a fixed order: block
// (t, 64 outputs h), wave w adds groups w, w + 4, ... (all its loads in
// flight, kCombineMaxG / 4 per lane at most), the four waves are added in
// wave order.
constexpr int kCombineMaxG = 64;

template <typename XT>
__global__ __launch_bounds__(256) void kept_combine_kernel(const float *__restrict__ part, int64_t T,
                                                           int H, int G, XT *__restrict__ y) {
  constexpr int PER = kCombineMaxG / kWaves4;
  __shared__ float red[kWaves4][kWave];
  const int n_hb = (H + kWave - 1) / kWave;
  const int64_t t = blockIdx.x / n_hb;
  const int h = (blockIdx.x % n_hb) * kWave + lane_id(), wv = threadIdx.x >> 6;
  const bool live = h < H;
  const float *p = part + t * G * (int64_t)H + h;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = wv + kWaves4 * i;
    v[i] = live && g < G ? p[(int64_t)g * H] : 0.0f;
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) s = s + v[i];
  red[wv][lane_id()] = s;
  __syncthreads();
  if (wv == 0 && live)
    Elem<XT>::store1(y + t * H + h, ((red[0][lane_id()] + red[1][lane_id()]) + red[2][lane_id()]) +
                                        red[3][lane_id()]);
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
                                 uint2 *kept_list, hipStream_t s) {
  if (!channel_select_supported(k1, I)) return hipErrorInvalidValue;
  channel_select_kernel<<<dim3((unsigned)T), dim3(kSelThreads), 0, s>>>(
      abuf, k1, I, ids, dn, keep, scores_out, kept_out, kept_list);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_down_columns(const WT *Wd, int E, int H, int I, WT *WdT, hipStream_t s) {
  const dim3 grid((unsigned)((I + 31) / 32), (unsigned)((H + 31) / 32), (unsigned)E);
  down_columns_kernel<WT><<<grid, dim3(256), 0, s>>>(Wd, H, I, WdT);
  return hipGetLastError();
}

// List groups per token: enough blocks (T * slices * groups, about 256) to
// keep every kept column read in flight at once, at most one group per four
// kept channels and kCombineMaxG in all.
int kept_groups(int64_t T, int H, int keep, int esz) {
  const int n_hs = kept_slices(H, esz);
  int64_t g = (256 + T * n_hs - 1) / (T * n_hs);
  const int64_t cap = (keep + 3) / 4;
  if (g > cap) g = cap;
  if (g > kCombineMaxG) g = kCombineMaxG;
  return (int)(g < 1 ? 1 : g);
}

int kept_slices(int H, int esz) {
  const int per_slice = kWave * 16 / esz;
  return (H + per_slice - 1) / per_slice;
}

template <typename WT, typename XT>
hipError_t launch_kept_down(const WT *WdT, int64_t T, int H, const uint2 *kept_list, int keep,
                            float *part, XT *y, hipStream_t s) {
  const int G = kept_groups(T, H, keep, sizeof(WT));
  const int n_hs = kept_slices(H, sizeof(WT));
  const int per = keep > 0 ? (keep + G - 1) / G : 0;
  kept_down_kernel<WT><<<dim3((unsigned)(T * n_hs * G)), dim3(256), 0, s>>>(
      WdT, H, kept_list, keep, per, G, n_hs, part);
  const int n_hb = (H + kWave - 1) / kWave;
  kept_combine_kernel<XT><<<dim3((unsigned)(T * n_hb)), dim3(256), 0, s>>>(part, T, H, G, y);
  return hipGetLastError();
}

template hipError_t launch_down_columns<float>(const float *, int, int, int, float *, hipStream_t);
template hipError_t launch_down_columns<bf16_t>(const bf16_t *, int, int, int, bf16_t *,
                                                hipStream_t);
template hipError_t launch_kept_down<float, float>(const float *, int64_t, int, const uint2 *, int,
                                                   float *, float *, hipStream_t);
template hipError_t launch_kept_down<bf16_t, bf16_t>(const bf16_t *, int64_t, int, const uint2 *,
                                                     int, float *, bf16_t *, hipStream_t);

template hipError_t launch_down_column_norms<float>(const float *, int, int, int, float *,
                                                    hipStream_t);
template hipError_t launch_down_column_norms<bf16_t>(const bf16_t *, int, int, int, float *,
                                                     hipStream_t);

}  // namespace moe
