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
//  down_kernel   : one work item = (unique expert, block of output rows):
//                  stream the down rows once, z[t,r,h] = Wd[e,h,:] . a[t,r,:];
//  combine_kernel: y[t,h] = sum of z[t,r,h] over the token's slots, in order.
//
// Batches of at most kIdsMax assignments skip the plan: every gate/up and
// down block reads the batch's ids and finds its own expert and assignments.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "sync.hpp"

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

// ---------------------------------------------------------------- ids map
// Work items without a plan, for n <= kIdsMax = 64 assignments: there are
// min(n, E) keys per launch group, as many as a plan would have unique
// experts at most.  With n <= E key q is assignment q, and the item is live
// when q is the first assignment routed to its expert; otherwise key q is
// expert q, live when any assignment is routed to it.  Every wave reads the
// ids (one per lane) and one ballot marks the assignments of the item's
// expert, so a block finds its work in one round trip and no barrier.

// The assignments of a work item: n entries of lst, or the n set bits of
// mask (ascending) when lst is NULL.
struct Items {
  const int32_t *lst;
  uint64_t mask;
  int n;
  __device__ __forceinline__ int take(int i, uint64_t &rest) const {
    if (lst) return lst[i];
    const int a = __builtin_ctzll(rest);
    rest &= rest - 1ull;
    return a;
  }
};

// The item of `key` (n == 0: not live) and its expert in *e_out.
__device__ __forceinline__ Items ids_item(const int32_t *__restrict__ ids, int n, int E, int key,
                                          int *e_out) {
  const int lane = lane_id();
  const bool by_asg = n <= E;
  const int e = by_asg ? ids[key] : key;
  *e_out = e;
  const int ei = lane < n ? ids[lane] : -1;
  const uint64_t m = __ballot(ei == e);
  const bool live = by_asg ? __builtin_ctzll(m) == key : m != 0ull;
  return Items{nullptr, m, live ? (int)__popcll(m) : 0};
}

// The item of unique expert u of a plan (n == 0: u >= U).
__device__ __forceinline__ Items plan_item(const int32_t *__restrict__ plan, int E, int u,
                                           int *e_out) {
  if (u >= plan[0]) return Items{nullptr, 0ull, 0};
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  *e_out = uniq[u];
  const int lb = off[u];
  return Items{off + E + 1 + lb, 0ull, off[u + 1] - lb};
}

// ---------------------------------------------------------------- gate/up
// One workgroup = (unique expert u, block of 4*CPW channels); each wave owns
// CPW channels and issues the loads of all its gate and up rows (2*CPW*NCH
// 16-byte chunks per lane) before any arithmetic, then reuses them for every
// token routed to u: a[t,r,c] = silu(Wg[e,c,:] x_t) * (Wu[e,c,:] x_t) * w[t,r].
constexpr int kGuWaves = 4;

// The weights, plan and outputs of one group of experts in a gate/up launch.
// A launch takes the routed experts and, optionally, the shared expert as a
// one-expert layer over every token; blocks [0, n0) take group g0 and the
// rest g1.  The shared expert, when there is one, is g0: its blocks loop over
// every token, so they start first and overlap the routed blocks.
template <typename WT>
struct GuGroup {
  const WT *Wg, *Wu;
  int I;
  const int32_t *plan;
  int E, k1;
  const float *w;
  float *abuf;
  const int32_t *ids;  // non-NULL: work items from the ids (ids_item), no plan
  int n;               // assignments in ids
};

// NT assignments (list entries asg) against a wave's CPW gate and up rows
// already in registers: a[asg, c] = silu(g . x) * (u . x) * w[asg].
template <int NT, typename WT, typename XT, int NCH, int CPW>
__device__ __forceinline__ void gateup_tokens(const XT *__restrict__ x, int H, int I, int k1,
                                              const int32_t *__restrict__ asgs,
                                              const float *__restrict__ w,
                                              float *__restrict__ abuf,
                                              const uint4 (&gq)[CPW][NCH],
                                              const uint4 (&uq)[CPW][NCH], int c0) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int lane = lane_id();
  int asg[NT];
  const XT *xr[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    asg[q] = asgs[q];
    xr[q] = x + (int64_t)(asg[q] / k1) * H;
  }
  float ag[NT][CPW], au[NT][CPW];
#pragma unroll
  for (int q = 0; q < NT; ++q)
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci) ag[q][ci] = au[q][ci] = 0.0f;
  if constexpr (sizeof(WT) == 2 && sizeof(XT) == 2) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      uint4 xq[NT];
#pragma unroll
      for (int q = 0; q < NT; ++q) xq[q] = ld16(xr[q] + (j * kWave + lane) * NW);
#pragma unroll
      for (int q = 0; q < NT; ++q) {
#pragma unroll
        for (int ci = 0; ci < CPW; ++ci) {
          ag[q][ci] = dot2_bf16(gq[ci][j].x, xq[q].x, ag[q][ci]);
          ag[q][ci] = dot2_bf16(gq[ci][j].y, xq[q].y, ag[q][ci]);
          ag[q][ci] = dot2_bf16(gq[ci][j].z, xq[q].z, ag[q][ci]);
          ag[q][ci] = dot2_bf16(gq[ci][j].w, xq[q].w, ag[q][ci]);
          au[q][ci] = dot2_bf16(uq[ci][j].x, xq[q].x, au[q][ci]);
          au[q][ci] = dot2_bf16(uq[ci][j].y, xq[q].y, au[q][ci]);
          au[q][ci] = dot2_bf16(uq[ci][j].z, xq[q].z, au[q][ci]);
          au[q][ci] = dot2_bf16(uq[ci][j].w, xq[q].w, au[q][ci]);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float xv[NT][NW];
#pragma unroll
      for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int k = 0; k < NW; ++k) xv[q][k] = Elem<XT>::load1(xr[q] + (j * kWave + lane) * NW + k);
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        float gv[NW], uv[NW];
        Elem<WT>::widen(gq[ci][j], gv);
        Elem<WT>::widen(uq[ci][j], uv);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
#pragma unroll
          for (int k = 0; k < NW; ++k) {
            ag[q][ci] = __builtin_fmaf(gv[k], xv[q][k], ag[q][ci]);
            au[q][ci] = __builtin_fmaf(uv[k], xv[q][k], au[q][ci]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const float wt = w[asg[q]];
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci) {
      const float g = wave_sum_dpp(ag[q][ci]);
      const float uu = wave_sum_dpp(au[q][ci]);
      const int c = c0 + ci;
      if (lane == 0 && c < I) abuf[(int64_t)asg[q] * I + c] = silu(g) * uu * wt;
    }
  }
}

// The workspace epoch (source of the call tags of the router + route launch
// before this one, every block of which has ended) is advanced by block 0.
__device__ __forceinline__ void advance_epoch(int32_t *epoch) {
  if (epoch && blockIdx.x == 0 && threadIdx.x == 0) coh_st(epoch, coh_ld(epoch) + 1);
}

template <typename WT, typename XT, int NCH, int CPW>
__global__ __launch_bounds__(256) void gateup_kernel(const XT *__restrict__ x, int H,
                                                     GuGroup<WT> g0, GuGroup<WT> g1,
                                                     unsigned n0, int32_t *epoch) {
  advance_epoch(epoch);
  constexpr int NW = Elem<WT>::kPer16B;
  const bool second = blockIdx.x >= n0;
  const GuGroup<WT> G = second ? g1 : g0;
  const unsigned bid = second ? blockIdx.x - n0 : blockIdx.x;
  const WT *__restrict__ Wg = G.Wg;
  const WT *__restrict__ Wu = G.Wu;
  const int I = G.I, E = G.E, k1 = G.k1;
  const int32_t *__restrict__ plan = G.plan;
  const float *__restrict__ w = G.w;
  float *__restrict__ abuf = G.abuf;
  const int n_cb = (I + kGuWaves * CPW - 1) / (kGuWaves * CPW);
  const int u = bid / n_cb;
  const int cb = bid - u * n_cb;
  int e = 0;
  const Items it = G.ids ? ids_item(G.ids, G.n, E, u, &e) : plan_item(plan, E, u, &e);
  if (it.n == 0) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int c0 = (cb * kGuWaves + wv) * CPW;
  uint4 gq[CPW][NCH], uq[CPW][NCH];
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) {
    const int c = min(c0 + ci, I - 1);
    const WT *grow = Wg + ((int64_t)e * I + c) * H;
    const WT *urow = Wu + ((int64_t)e * I + c) * H;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      gq[ci][j] = ld16_stream(grow + (j * kWave + lane) * NW);
      uq[ci][j] = ld16_stream(urow + (j * kWave + lane) * NW);
    }
  }
  // one token at a time (two at a time measured slower: register pressure)
  uint64_t rest = it.mask;
  for (int i = 0; i < it.n; ++i) {
    const int32_t asg = it.take(i, rest);
    gateup_tokens<1, WT, XT, NCH, CPW>(x, H, I, k1, &asg, w, abuf, gq, uq, c0);
  }
}

// Any H (a multiple of 8): one channel per wave, chunks walked in a loop.
template <typename WT, typename XT>
__global__ __launch_bounds__(256) void gateup_any_kernel(const XT *__restrict__ x, int H,
                                                         GuGroup<WT> g0, GuGroup<WT> g1,
                                                         unsigned n0, int32_t *epoch) {
  advance_epoch(epoch);
  constexpr int NW = Elem<WT>::kPer16B;
  const bool second = blockIdx.x >= n0;
  const GuGroup<WT> G = second ? g1 : g0;
  const unsigned bid = second ? blockIdx.x - n0 : blockIdx.x;
  const WT *__restrict__ Wg = G.Wg;
  const WT *__restrict__ Wu = G.Wu;
  const int I = G.I, E = G.E, k1 = G.k1;
  const int32_t *__restrict__ plan = G.plan;
  const float *__restrict__ w = G.w;
  float *__restrict__ abuf = G.abuf;
  const int n_cb = (I + kGuWaves - 1) / kGuWaves;
  const int u = bid / n_cb;
  const int cb = bid - u * n_cb;
  if (u >= plan[0]) return;
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *list = off + E + 1;
  const int e = uniq[u];
  const int lb = off[u], ln = off[u + 1] - lb;
  const int lane = lane_id();
  const int c = cb * kGuWaves + (threadIdx.x >> 6);
  if (c >= I) return;
  const WT *grow = Wg + ((int64_t)e * I + c) * H;
  const WT *urow = Wu + ((int64_t)e * I + c) * H;
  const int n_chunks = H / NW;
  for (int i = 0; i < ln; ++i) {
    const int asg = list[lb + i];
    const XT *xr = x + (int64_t)(asg / k1) * H;
    float ag = 0.0f, au = 0.0f;
    for (int ch = lane; ch < n_chunks; ch += kWave) {
      float gv[NW], uv[NW];
      Elem<WT>::widen(ld16(grow + ch * NW), gv);
      Elem<WT>::widen(ld16(urow + ch * NW), uv);
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const float xv = Elem<XT>::load1(xr + ch * NW + k);
        ag = __builtin_fmaf(gv[k], xv, ag);
        au = __builtin_fmaf(uv[k], xv, au);
      }
    }
    const float g = wave_sum_dpp(ag), uu = wave_sum_dpp(au);
    if (lane == 0) abuf[(int64_t)asg * I + c] = silu(g) * uu * w[asg];
  }
}

template <typename WT, typename XT>
bool gateup_takes_ids(int H) {
  const int nch = (H * (int)sizeof(WT)) % (16 * kWave) == 0 ? (int)(H * sizeof(WT) / 16 / kWave) : 0;
  return nch == 1 || nch == 2 || nch == 4 || nch == 8;
}

template <typename WT, typename XT>
hipError_t launch_gateup(const XT *x, int H, const WT *Wg, const WT *Wu, int I,
                         const int32_t *plan, int E, int64_t n_assign, int k1, const float *w,
                         float *abuf, hipStream_t s, const WT *Sg, const WT *Su, int Is,
                         const int32_t *plan_s, const float *gs, float *abuf_s,
                         const int32_t *ids, int32_t *epoch) {
  const int64_t umax = n_assign < E ? n_assign : E;
  const int nch = (H * (int)sizeof(WT)) % (16 * kWave) == 0 ? (int)(H * sizeof(WT) / 16 / kWave) : 0;
  if (ids && (n_assign > kIdsMax || !gateup_takes_ids<WT, XT>(H))) return hipErrorInvalidValue;
  const GuGroup<WT> gr{Wg, Wu, I, plan, E, k1, w, abuf, ids, (int)(ids ? n_assign : 0)};
  const GuGroup<WT> gsh{Sg, Su, Is, plan_s, 1, 1, gs, abuf_s, nullptr, 0};
  const GuGroup<WT> g0 = Sg ? gsh : gr;
  auto go = [&](auto nch_c, auto cpw_c) {
    constexpr int NCH = decltype(nch_c)::value, CPW = decltype(cpw_c)::value;
    const unsigned n_r = (unsigned)(umax * ((I + kGuWaves * CPW - 1) / (kGuWaves * CPW)));
    const unsigned n_sh = Sg ? (unsigned)((Is + kGuWaves * CPW - 1) / (kGuWaves * CPW)) : 0u;
    gateup_kernel<WT, XT, NCH, CPW><<<dim3(n_r + n_sh), dim3(256), 0, s>>>(x, H, g0, gr,
                                                                           Sg ? n_sh : n_r, epoch);
  };
  using std::integral_constant;
  switch (nch) {
    case 1: go(integral_constant<int, 1>{}, integral_constant<int, 8>{}); break;
    case 2: go(integral_constant<int, 2>{}, integral_constant<int, 4>{}); break;
    case 4: go(integral_constant<int, 4>{}, integral_constant<int, 2>{}); break;
    case 8: go(integral_constant<int, 8>{}, integral_constant<int, 1>{}); break;
    default: {
      const unsigned n_r = (unsigned)(umax * ((I + kGuWaves - 1) / kGuWaves));
      const unsigned n_sh = Sg ? (unsigned)((Is + kGuWaves - 1) / kGuWaves) : 0u;
      gateup_any_kernel<WT, XT><<<dim3(n_r + n_sh), dim3(256), 0, s>>>(x, H, g0, gr,
                                                                        Sg ? n_sh : n_r, epoch);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- down
// One workgroup = (unique expert u, block of 4*RPW rows of Wd[e]); each wave
// loads its RPW rows (NCD 16-byte chunks per lane per row) up front, then for
// every assignment routed to u writes z[asg, h] = Wd[e,h,:] . a[asg,:].
// Four rows per wave measured faster than two and than eight from 2 to 64
// tokens (H=2048, I=768 bf16).
constexpr int kDnWaves = 4;
constexpr int kRPW = 4;
constexpr int kDnRB = kDnWaves * kRPW;

// One group of experts in a down launch (see GuGroup, whose block order it
// follows): Wd holds E experts' [H, I] down matrices; the shared expert's
// [H, Is] is one such expert.
template <typename WT>
struct DnGroup {
  const WT *Wd;
  int I;
  const int32_t *plan;
  int E;
  const float *abuf;
  float *zbuf;
  const int32_t *ids;  // non-NULL: work items from the ids (ids_item), no plan
  int n;               // assignments in ids
};

// NT assignments against a wave's kRPW down rows already in registers:
// z[asg, h] = Wd[e, h, :] . a[asg, :].
template <int NT, typename WT, int NCD>
__device__ __forceinline__ void down_tokens(int H, int I, const int32_t *__restrict__ asgs,
                                            const float *__restrict__ abuf,
                                            float *__restrict__ zbuf,
                                            const uint4 (&dq)[kRPW][NCD], int h0) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int lane = lane_id();
  const int nch = I / NW;
  int asg[NT];
  float av[NT][NCD][NW];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    asg[q] = asgs[q];
    const float *arow = abuf + (int64_t)asg[q] * I;
#pragma unroll
    for (int j = 0; j < NCD; ++j) {
      const int ch = j * kWave + lane;
      if (ch < nch) {
        Elem<float>::widen(ld16(arow + ch * NW), av[q][j]);
        if constexpr (NW == 8) Elem<float>::widen(ld16(arow + ch * NW + 4), av[q][j] + 4);
      } else {
#pragma unroll
        for (int k = 0; k < NW; ++k) av[q][j][k] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int ri = 0; ri < kRPW; ++ri) {
    float acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < NCD; ++j) {
      float dv[NW];
      Elem<WT>::widen(dq[ri][j], dv);
#pragma unroll
      for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int k = 0; k < NW; ++k) acc[q] = __builtin_fmaf(dv[k], av[q][j][k], acc[q]);
    }
    const int h = h0 + ri;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const float z = wave_sum_dpp(acc[q]);
      if (lane == 0 && h < H) zbuf[(int64_t)asg[q] * H + h] = z;
    }
  }
}

template <typename WT, int NCD>
__global__ __launch_bounds__(256) void down_kernel(int H, DnGroup<WT> g0, DnGroup<WT> g1,
                                                   unsigned n0) {
  constexpr int NW = Elem<WT>::kPer16B;
  const bool second = blockIdx.x >= n0;
  const DnGroup<WT> G = second ? g1 : g0;
  const unsigned bid = second ? blockIdx.x - n0 : blockIdx.x;
  const WT *__restrict__ Wd = G.Wd;
  const int I = G.I, E = G.E;
  const int32_t *__restrict__ plan = G.plan;
  const float *__restrict__ abuf = G.abuf;
  float *__restrict__ zbuf = G.zbuf;
  const int n_hb = (H + kDnRB - 1) / kDnRB;
  const int u = bid / n_hb;
  const int hb = bid - u * n_hb;
  int e = 0;
  const Items it = G.ids ? ids_item(G.ids, G.n, E, u, &e) : plan_item(plan, E, u, &e);
  if (it.n == 0) return;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int nch = I / NW;
  const int h0 = hb * kDnRB + wv * kRPW;
  uint4 dq[kRPW][NCD];
#pragma unroll
  for (int ri = 0; ri < kRPW; ++ri) {
    const WT *drow = Wd + ((int64_t)e * H + min(h0 + ri, H - 1)) * I;
#pragma unroll
    for (int j = 0; j < NCD; ++j) {
      const int ch = j * kWave + lane;
      dq[ri][j] = ch < nch ? ld16_stream(drow + ch * NW) : make_uint4(0, 0, 0, 0);
    }
  }
  // one token at a time (two at a time measured slower: register pressure)
  uint64_t rest = it.mask;
  for (int i = 0; i < it.n; ++i) {
    const int32_t asg = it.take(i, rest);
    down_tokens<1, WT, NCD>(H, I, &asg, abuf, zbuf, dq, h0);
  }
}

// Any I: one row per wave, chunks walked in a loop.
template <typename WT>
__global__ __launch_bounds__(256) void down_any_kernel(int H, DnGroup<WT> g0, DnGroup<WT> g1,
                                                       unsigned n0) {
  constexpr int NW = Elem<WT>::kPer16B;
  const bool second = blockIdx.x >= n0;
  const DnGroup<WT> G = second ? g1 : g0;
  const unsigned bid = second ? blockIdx.x - n0 : blockIdx.x;
  const WT *__restrict__ Wd = G.Wd;
  const int I = G.I, E = G.E;
  const int32_t *__restrict__ plan = G.plan;
  const float *__restrict__ abuf = G.abuf;
  float *__restrict__ zbuf = G.zbuf;
  const int n_hb = (H + kDnWaves - 1) / kDnWaves;
  const int u = bid / n_hb;
  const int hb = bid - u * n_hb;
  if (u >= plan[0]) return;
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *list = off + E + 1;
  const int e = uniq[u];
  const int lb = off[u], ln = off[u + 1] - lb;
  const int lane = lane_id();
  const int h = hb * kDnWaves + (threadIdx.x >> 6);
  if (h >= H) return;
  const WT *drow = Wd + ((int64_t)e * H + h) * I;
  const int nch = I / NW;
  for (int i = 0; i < ln; ++i) {
    const int asg = list[lb + i];
    const float *arow = abuf + (int64_t)asg * I;
    float acc = 0.0f;
    for (int ch = lane; ch < nch; ch += kWave) {
      float dv[NW];
      Elem<WT>::widen(ld16(drow + ch * NW), dv);
#pragma unroll
      for (int k = 0; k < NW; ++k) acc = __builtin_fmaf(dv[k], arow[ch * NW + k], acc);
    }
    acc = wave_sum_dpp(acc);
    if (lane == 0) zbuf[(int64_t)asg * H + h] = acc;
  }
}

template <typename WT>
static int down_ncd(int I, bool shared, int Is) {
  auto ncd_of = [](int i) { return (int)((i * sizeof(WT) / 16 + kWave - 1) / kWave); };
  // one NCD for both groups: the wider one (chunks past a row's end are masked)
  return shared ? max(ncd_of(I), ncd_of(Is)) : ncd_of(I);
}

template <typename WT>
bool down_takes_ids(int I, int Is) {
  const int ncd = down_ncd<WT>(I, Is > 0, Is);
  return ncd >= 1 && ncd <= 4;
}

template <typename WT>
hipError_t launch_down(const WT *Wd, int H, int I, const int32_t *plan, int E, int64_t n_assign,
                       const float *abuf, float *zbuf, hipStream_t s, const WT *Sd, int Is,
                       const int32_t *plan_s, const float *abuf_s, float *zbuf_s,
                       const int32_t *ids) {
  const int64_t umax = n_assign < E ? n_assign : E;
  const int n_hb = (H + kDnRB - 1) / kDnRB;
  const int ncd = down_ncd<WT>(I, Sd != nullptr, Is);
  if (ids && (n_assign > kIdsMax || !down_takes_ids<WT>(I, Sd ? Is : 0)))
    return hipErrorInvalidValue;
  const DnGroup<WT> gr{Wd, I, plan, E, abuf, zbuf, ids, (int)(ids ? n_assign : 0)};
  const DnGroup<WT> gsh{Sd, Is, plan_s, 1, abuf_s, zbuf_s, nullptr, 0};
  const DnGroup<WT> g0 = Sd ? gsh : gr;
  const unsigned n_r = (unsigned)(umax * n_hb), n_sh = Sd ? (unsigned)n_hb : 0u;
  const unsigned n0 = Sd ? n_sh : n_r;
  const dim3 grid(n_r + n_sh), block(256);
  switch (ncd) {
    case 1: down_kernel<WT, 1><<<grid, block, 0, s>>>(H, g0, gr, n0); break;
    case 2: down_kernel<WT, 2><<<grid, block, 0, s>>>(H, g0, gr, n0); break;
    case 3: down_kernel<WT, 3><<<grid, block, 0, s>>>(H, g0, gr, n0); break;
    case 4: down_kernel<WT, 4><<<grid, block, 0, s>>>(H, g0, gr, n0); break;
    default: {
      const int n_hb1 = (H + kDnWaves - 1) / kDnWaves;
      const unsigned m_r = (unsigned)(umax * n_hb1), m_sh = Sd ? (unsigned)n_hb1 : 0u;
      down_any_kernel<WT><<<dim3(m_r + m_sh), block, 0, s>>>(H, g0, gr, Sd ? m_sh : m_r);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- down, T = 1
// One token: each wave owns one output row and sums over every unique
// expert directly, y[h] = sum_u Wd[e_u,h,:] . a[u,:] (ascending expert order,
// per-lane partial sums, one wave reduction), so no partials and no combine.
// The rows of the first kPF experts are loaded before any arithmetic.
constexpr int kPF1 = 8;

template <typename WT, typename XT, int NCD>
__global__ __launch_bounds__(256) void down_one_token_kernel(const WT *__restrict__ Wd, int H,
                                                             int I, const int32_t *__restrict__ plan,
                                                             int E, const float *__restrict__ abuf,
                                                             XT *__restrict__ y) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (h >= H) return;
  const int lane = lane_id();
  const int U = plan[0];
  const int32_t *uniq = plan + 4;
  const int32_t *off = uniq + E;
  const int32_t *list = off + E + 1;
  const int nch = I / NW;
  uint4 dq[kPF1][NCD];
  auto issue = [&](int u, uint4 (&dst)[NCD]) {
    const WT *drow = Wd + ((int64_t)uniq[u] * H + h) * I;
#pragma unroll
    for (int j = 0; j < NCD; ++j) {
      const int ch = j * kWave + lane;
      dst[j] = ch < nch ? ld16_stream(drow + ch * NW) : make_uint4(0, 0, 0, 0);
    }
  };
#pragma unroll
  for (int s = 0; s < kPF1; ++s)
    if (s < U) issue(s, dq[s]);
  float acc = 0.0f;
  for (int ub = 0; ub < U; ub += kPF1) {
#pragma unroll
    for (int s = 0; s < kPF1; ++s) {
      const int u = ub + s;
      if (u < U) {
        const float *arow = abuf + (int64_t)list[off[u]] * I;
#pragma unroll
        for (int j = 0; j < NCD; ++j) {
          const int ch = j * kWave + lane;
          if (ch < nch) {
            float av[NW], dv[NW];
            Elem<float>::widen(ld16(arow + ch * NW), av);
            if constexpr (NW == 8) Elem<float>::widen(ld16(arow + ch * NW + 4), av + 4);
            Elem<WT>::widen(dq[s][j], dv);
#pragma unroll
            for (int k = 0; k < NW; ++k) acc = __builtin_fmaf(dv[k], av[k], acc);
          }
        }
        if (u + kPF1 < U) issue(u + kPF1, dq[s]);
      }
    }
  }
  acc = wave_sum_dpp(acc);
  if (lane == 0) Elem<XT>::store1(y + h, acc);
}

template <typename WT, typename XT>
hipError_t launch_down_one_token(const WT *Wd, int H, int I, const int32_t *plan, int E,
                                 const float *abuf, XT *y, hipStream_t s) {
  const int ncd = (int)((I * sizeof(WT) / 16 + kWave - 1) / kWave);
  const dim3 grid((unsigned)((H + 3) / 4)), block(256);
  switch (ncd) {
    case 1: down_one_token_kernel<WT, XT, 1><<<grid, block, 0, s>>>(Wd, H, I, plan, E, abuf, y); break;
    case 2: down_one_token_kernel<WT, XT, 2><<<grid, block, 0, s>>>(Wd, H, I, plan, E, abuf, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// y[t,h] = sum over the token's k1 slots of z[t*k1 + r, h], in slot order,
// then the shared expert's term zs[t, h] if there is one.
template <typename XT>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ zbuf,
                                                      const float *__restrict__ zs, int64_t T,
                                                      int H, int k1, XT *__restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * H) return;
  const int64_t t = i / H, h = i - t * H;
  // eight slots' loads in flight at once, summed in slot order
  constexpr int kU = 8;
  const float *zt = zbuf + t * k1 * H + h;
  const float sh = zs ? zs[i] : 0.0f;
  float s = 0.0f;
  for (int r0 = 0; r0 < k1; r0 += kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = r0 + u < k1 ? zt[(int64_t)(r0 + u) * H] : 0.0f;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (r0 + u < k1) s = s + v[u];
  }
  if (zs) s = s + sh;
  Elem<XT>::store1(y + i, s);
}

template <typename XT>
hipError_t launch_combine(const float *zbuf, const float *zs, int64_t T, int H, int k1, XT *y,
                          hipStream_t s) {
  const int64_t n = T * H;
  combine_kernel<XT><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(zbuf, zs, T, H, k1,
                                                                             y);
  return hipGetLastError();
}

// ---------------------------------------------------------------- shared expert
// The shared expert ("Channel Selection for Mixture-of-Experts Decoding Needs
// No Calibration Data", appendix B: shared experts always run in full) runs
// as a one-expert layer over every token.  This kernel writes its plan in
// the layout above for E = 1 (one unique expert holding assignments 0..T-1
// in order), zero ids for the prefill plan (either may be NULL), and the
// factor gs[t] = sigmoid(x[t] . sg), or 1 without sg.  One wave per token.
template <typename XT>
__global__ __launch_bounds__(256) void shared_prep_kernel(const XT *__restrict__ x, int64_t T,
                                                          int H, const float *__restrict__ sgw,
                                                          int32_t *__restrict__ plan,
                                                          int32_t *__restrict__ ids0,
                                                          float *__restrict__ gs) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (plan && blockIdx.x == 0 && threadIdx.x == 0) {
    plan[0] = 1;             // U
    plan[4] = 0;             // uniq[0]
    plan[5] = 0;             // off[0]
    plan[6] = (int32_t)T;    // off[1]
  }
  if (t >= T) return;
  const int lane = lane_id();
  float g = 1.0f;
  if (sgw) {
    // x rows are 16-byte aligned (H % 8 == 0): one 16-byte chunk of x per
    // step, several steps' loads in flight; sgate is only 4-byte aligned
    constexpr int n = Elem<XT>::kPer16B;
    const XT *xr = x + t * H;
    const int nc = H / n;
    float z = 0.0f;
#pragma unroll 4
    for (int c = lane; c < nc; c += kWave) {
      float xv[n];
      Elem<XT>::widen(ld16(xr + (int64_t)c * n), xv);
      const float *wp = sgw + (int64_t)c * n;
#pragma unroll
      for (int q = 0; q < n; ++q) z = __builtin_fmaf(xv[q], wp[q], z);
    }
    z = wave_sum_dpp(z);
    g = 1.0f / (1.0f + __expf(-z));
  }
  if (lane == 0) {
    if (plan) plan[7 + t] = (int32_t)t;  // list
    if (ids0) ids0[t] = 0;
    gs[t] = g;
  }
}

size_t shared_plan_words(int64_t T) { return 7 + (size_t)T; }

template <typename XT>
hipError_t launch_shared_prep(const XT *x, int64_t T, int H, const float *sgw, int32_t *plan,
                              int32_t *ids0, float *gs, hipStream_t s) {
  shared_prep_kernel<XT><<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s>>>(x, T, H, sgw, plan,
                                                                             ids0, gs);
  return hipGetLastError();
}

#define MOE_INST_DECODE(WT, XT)                                                             \
  template hipError_t launch_gateup<WT, XT>(const XT *, int, const WT *, const WT *, int, \
                                            const int32_t *, int, int64_t, int,           \
                                            const float *, float *, hipStream_t,          \
                                            const WT *, const WT *, int, const int32_t *, \
                                            const float *, float *, const int32_t *,      \
                                            int32_t *);                                   \
  template hipError_t launch_down<WT>(const WT *, int, int, const int32_t *, int, int64_t,  \
                                      const float *, float *, hipStream_t, const WT *, int, \
                                      const int32_t *, const float *, float *,              \
                                      const int32_t *);                                     \
  template bool gateup_takes_ids<WT, XT>(int);                                              \
  template bool down_takes_ids<WT>(int, int);                                               \
  template hipError_t launch_combine<XT>(const float *, const float *, int64_t, int, int, XT *, \
                                         hipStream_t);                                        \
  template hipError_t launch_shared_prep<XT>(const XT *, int64_t, int, const float *, int32_t *, \
                                             int32_t *, float *, hipStream_t);                \
  template hipError_t launch_down_one_token<WT, XT>(const WT *, int, int, const int32_t *, int, \
                                                    const float *, XT *, hipStream_t);
MOE_INST_DECODE(float, float)
MOE_INST_DECODE(bf16_t, bf16_t)

}  // namespace moe
