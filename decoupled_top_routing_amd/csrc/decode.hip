// Expert path for small batches (decode): a grouped GEMV that streams only
// the activated experts' weights.
//
// An expert is a gated MLP whose channel c owns gate row Wg[e,c,:], up row
// Wu[e,c,:] and down column Wd[e,:,c] ("Channel Selection for Mixture-of-
// Experts Decoding Needs No Calibration Data", section 2 "Background").  The
// weights of Eq. 2 ("Paper of the Week #3 - Half the FLOPs Is Not Half the
// Time", section "The Receipt") scale each activated expert's output; here
// they are folded into the channel activations before the down projection.
//
//  plan_kernel   : unique experts of the batch and, per unique expert, the
//                  (token, slot) assignments routed to it (ascending);
//  gateup_kernel : one work item = (unique expert, block of channels): stream
//                  the gate and up rows once, dot with every token routed to
//                  the expert, a[t,r,c] = silu(g) * u * w[t,r];
//  down_kernel   : one work item = (token, block of output rows): y[t,h] =
//                  sum over the token's slots and channels of Wd[e,h,c] a[t,r,c].
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------- plan
// plan layout (int32): [0] = U, [1..3] unused, uniq[E] at 4, off[E+1] after
// it, list[T*k1] after that.  One workgroup of 1024 threads; T*k1 may be
// larger than the block (loops).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *__restrict__ ids, int64_t n_assign,
                                                    int E, int32_t *__restrict__ plan) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t uidx[kMaxExperts];
  __shared__ int32_t fill[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t s_U;
  int32_t *uniq = plan + 4;
  int32_t *off = uniq + E;
  int32_t *list = off + E + 1;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    cnt[e] = 0;
    fill[e] = 0;
  }
  __syncthreads();
  for (int64_t i = tid; i < n_assign; i += blockDim.x) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();
  // exclusive scans over experts of (cnt > 0) and cnt, E <= 1024 = one entry
  // per thread: wave-level inclusive scans, then across the 16 waves.
  const int lane = lane_id(), wv = tid >> 6;
  const int c = tid < E ? cnt[tid] : 0;
  int present = c > 0 ? 1 : 0;
  int sum_p = present, sum_c = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int tp = __shfl_up(sum_p, o), tc = __shfl_up(sum_c, o);
    if (lane >= o) {
      sum_p += tp;
      sum_c += tc;
    }
  }
  __shared__ int32_t wave_tot_c[16];
  if (lane == kWave - 1) {
    wave_tot[wv] = sum_p;
    wave_tot_c[wv] = sum_c;
  }
  __syncthreads();
  int base_p = 0, base_c = 0;
  for (int k = 0; k < wv; ++k) {
    base_p += wave_tot[k];
    base_c += wave_tot_c[k];
  }
  const int ex_p = base_p + sum_p - present;  // exclusive
  const int ex_c = base_c + sum_c - c;
  if (tid < E) {
    uidx[tid] = ex_p;
    if (present) {
      uniq[ex_p] = tid;
      off[ex_p] = ex_c;
      s_off[ex_p] = ex_c;
    }
  }
  if (tid == blockDim.x - 1) {
    const int U = base_p + sum_p;
    plan[0] = U;
    s_U = U;
    off[U] = (int32_t)n_assign;
    s_off[U] = (int32_t)n_assign;
  }
  __syncthreads();
  const int U = s_U;
  // scatter assignments to their expert's list
  for (int64_t i = tid; i < n_assign; i += blockDim.x) {
    const int e = ids[i];
    const int pos = atomicAdd(&fill[e], 1);
    list[s_off[uidx[e]] + pos] = (int32_t)i;
  }
  __threadfence_block();
  __syncthreads();
  // deterministic order inside each list: insertion sort (lists are short)
  for (int u = tid; u < U; u += blockDim.x) {
    const int b = s_off[u], n = s_off[u + 1] - b;
    for (int i = 1; i < n; ++i) {
      const int32_t v = list[b + i];
      int j = i - 1;
      while (j >= 0 && list[b + j] > v) {
        list[b + j + 1] = list[b + j];
        --j;
      }
      list[b + j + 1] = v;
    }
  }
}

hipError_t launch_plan(const int32_t *ids, int64_t n_assign, int E, int32_t *plan,
                       hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(ids, n_assign, E, plan);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gate/up
// A wave computes kCPW channels of one expert for every token routed to it.
// Lane L reads 16-byte chunks L, L+64, ... of each row, so a wave load
// instruction covers 1 KiB of contiguous weights.
constexpr int kGuWaves = 4;
constexpr int kCPW = 2;                       // channels per wave
constexpr int kGuCB = kGuWaves * kCPW;        // channels per workgroup
constexpr int kTokGroup = 4;                  // tokens held in registers at once

template <typename WT, typename XT>
__global__ __launch_bounds__(256) void gateup_kernel(const XT *__restrict__ x, int H,
                                                     const WT *__restrict__ Wg,
                                                     const WT *__restrict__ Wu, int I,
                                                     const int32_t *__restrict__ plan, int E,
                                                     int k1, const float *__restrict__ w,
                                                     float *__restrict__ abuf) {
  constexpr int NW = Elem<WT>::kPer16B;  // weights per 16-byte chunk
  const int n_cb = (I + kGuCB - 1) / kGuCB;
  const int u = blockIdx.x / n_cb;
  const int cb = blockIdx.x - u * n_cb;
  const int U = plan[0];
  if (u >= U) return;
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *list = off + E + 1;
  const int e = uniq[u];
  const int lb = off[u], ln = off[u + 1] - lb;
  const int lane = lane_id();
  const int c0 = cb * kGuCB + (threadIdx.x >> 6) * kCPW;
  const int n_chunks = H / NW;  // H % 8 == 0
  for (int ci = 0; ci < kCPW; ++ci) {
    const int c = c0 + ci;
    if (c >= I) break;
    const WT *grow = Wg + ((int64_t)e * I + c) * H;
    const WT *urow = Wu + ((int64_t)e * I + c) * H;
    for (int g0 = 0; g0 < ln; g0 += kTokGroup) {
      const int ng = min(kTokGroup, ln - g0);
      float ag[kTokGroup], au[kTokGroup];
      int tok[kTokGroup];
#pragma unroll
      for (int i = 0; i < kTokGroup; ++i) {
        ag[i] = 0.0f;
        au[i] = 0.0f;
        tok[i] = i < ng ? list[lb + g0 + i] / k1 : 0;
      }
      for (int ch = lane; ch < n_chunks; ch += kWave) {
        float gv[NW], uv[NW];
        Elem<WT>::widen(ld16_stream(grow + (int64_t)ch * NW), gv);
        Elem<WT>::widen(ld16_stream(urow + (int64_t)ch * NW), uv);
#pragma unroll
        for (int i = 0; i < kTokGroup; ++i) {
          if (i < ng) {
            const XT *xr = x + (int64_t)tok[i] * H + (int64_t)ch * NW;
#pragma unroll
            for (int k = 0; k < NW; ++k) {
              const float xv = Elem<XT>::load1(xr + k);
              ag[i] = __builtin_fmaf(gv[k], xv, ag[i]);
              au[i] = __builtin_fmaf(uv[k], xv, au[i]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kTokGroup; ++i) {
        if (i < ng) {
          const float g = wave_sum(ag[i]);
          const float uu = wave_sum(au[i]);
          if (lane == 0) {
            const int a = list[lb + g0 + i];
            abuf[(int64_t)a * I + c] = silu(g) * uu * w[a];
          }
        }
      }
    }
  }
}

template <typename WT, typename XT>
hipError_t launch_gateup(const XT *x, int H, const WT *Wg, const WT *Wu, int I,
                         const int32_t *plan, int E, int64_t n_assign, int k1, const float *w,
                         float *abuf, hipStream_t s) {
  const int64_t umax = n_assign < E ? n_assign : E;
  const int n_cb = (I + kGuCB - 1) / kGuCB;
  const dim3 grid((unsigned)(umax * n_cb)), block(256);
  gateup_kernel<WT, XT><<<grid, block, 0, s>>>(x, H, Wg, Wu, I, plan, E, k1, w, abuf);
  return hipGetLastError();
}

// ---------------------------------------------------------------- down
// A wave computes kRPW output rows of one token, summing over the token's
// k1 slots; lane L reads 16-byte chunks L, L+64, ... of each down row.
constexpr int kDnWaves = 4;
constexpr int kRPW = 2;
constexpr int kDnRB = kDnWaves * kRPW;

template <typename WT, typename XT>
__global__ __launch_bounds__(256) void down_kernel(const WT *__restrict__ Wd, int H, int I,
                                                   const int32_t *__restrict__ ids, int k1,
                                                   const float *__restrict__ abuf,
                                                   XT *__restrict__ y) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int n_hb = (H + kDnRB - 1) / kDnRB;
  const int64_t t = blockIdx.x / n_hb;
  const int hb = (int)(blockIdx.x - t * n_hb);
  const int lane = lane_id();
  const int h0 = hb * kDnRB + (threadIdx.x >> 6) * kRPW;
  const int n_chunks = I / NW;
  for (int hi = 0; hi < kRPW; ++hi) {
    const int h = h0 + hi;
    if (h >= H) break;
    float acc = 0.0f;
    for (int r = 0; r < k1; ++r) {
      const int e = ids[t * k1 + r];
      const WT *drow = Wd + ((int64_t)e * H + h) * I;
      const float *arow = abuf + (t * k1 + r) * (int64_t)I;
      for (int ch = lane; ch < n_chunks; ch += kWave) {
        float dv[NW];
        Elem<WT>::widen(ld16_stream(drow + (int64_t)ch * NW), dv);
#pragma unroll
        for (int k = 0; k < NW; ++k) acc = __builtin_fmaf(dv[k], arow[ch * NW + k], acc);
      }
    }
    const float sum = wave_sum(acc);
    if (lane == 0) Elem<XT>::store1(y + t * H + h, sum);
  }
}

template <typename WT, typename XT>
hipError_t launch_down(const WT *Wd, int64_t T, int H, int I, const int32_t *ids, int k1,
                       const float *abuf, XT *y, hipStream_t s) {
  const dim3 grid((unsigned)(((H + kDnRB - 1) / kDnRB) * T)), block(256);
  down_kernel<WT, XT><<<grid, block, 0, s>>>(Wd, H, I, ids, k1, abuf, y);
  return hipGetLastError();
}

#define MOE_INST_DECODE(WT, XT)                                                             \
  template hipError_t launch_gateup<WT, XT>(const XT *, int, const WT *, const WT *, int, \
                                            const int32_t *, int, int64_t, int,           \
                                            const float *, float *, hipStream_t);         \
  template hipError_t launch_down<WT, XT>(const WT *, int64_t, int, int, const int32_t *, \
                                          int, const float *, XT *, hipStream_t);
MOE_INST_DECODE(float, float)
MOE_INST_DECODE(bf16_t, bf16_t)

}  // namespace moe
