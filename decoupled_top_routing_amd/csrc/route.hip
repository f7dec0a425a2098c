// Router logits, fp32 softmax, top-k2 ranking and the Eq. 2 weights.
//
// "Paper of the Week #3 - Half the FLOPs Is Not Half the Time":
//  - section "Ship It - Code of the Week": logits from a linear router,
//    probabilities from an fp32 softmax, the min(k2, E) most probable experts
//    in descending order, the first k1 of them activated;
//  - section "The Receipt", Eq. 2: w_i = p_i / (sum of the top-k2 p) for the
//    top-k1 experts; k2 >= E means the weights are the probabilities.
//
// One workgroup routes one token (route_device.hpp).  The softmax arithmetic
// is pinned down so that the ids and weights are reproducible bit for bit.
#include "common.hpp"
#include "kernels.hpp"
#include "route_device.hpp"
#include "sync.hpp"

#pragma clang fp contract(off)

namespace moe {

// One workgroup per token.  With `plan`, the last block to finish (ticket)
// also builds the batch plan (T*k1 <= 64); the ids it reads were stored
// device-coherently by the other blocks.  The ticket word is zero before
// and after the kernel.  wbf16 rounds the weights to bf16.
template <int V>
__global__ __launch_bounds__(256) void route_plan_kernel(const float *__restrict__ logits,
                                                         int64_t T, int E, int k1, int k2,
                                                         int32_t *__restrict__ ids,
                                                         float *__restrict__ w,
                                                         int32_t *__restrict__ ids2,
                                                         float *__restrict__ w2,
                                                         int32_t *__restrict__ plan,
                                                         int32_t *__restrict__ ticket,
                                                         bool wbf16) {
  __shared__ float sl[kBlockThreads];
  __shared__ int32_t s_ids[kMaxExperts];
  __shared__ float s_w[kMaxExperts];
  __shared__ BlockRoute S;
  __shared__ int s_last;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const float *lrow = logits + t * E;
  if (E <= kBlockThreads) {
    if (tid < E) sl[tid] = lrow[tid];
    __syncthreads();
    route_into_lds<V>(sl, E, k1, k2, s_ids, s_w, S, wbf16);
  } else {
    route_into_lds<V>(lrow, E, k1, k2, s_ids, s_w, S, wbf16);
  }
  const int64_t o = t * k1;
  for (int r = tid; r < k1; r += kBlockThreads) {
    if (plan)
      coh_st(ids + o + r, s_ids[r]);
    else
      ids[o + r] = s_ids[r];
    w[o + r] = s_w[r];
    if (ids2) ids2[o + r] = s_ids[r];
    if (w2) w2[o + r] = s_w[r];
  }
  if (!plan) return;
  if (!last_of(ticket, (int)T, &s_last) || tid >= kWave) return;
  const int n = (int)T * k1;
  wave_plan(tid < n ? coh_ld(ids + tid) : 0x7FFFFFFF, n, E, plan);
}

hipError_t launch_route_plan(const float *logits, int64_t T, int E, int k1, int k2,
                             int32_t *ids, float *w, int32_t *ids2, float *w2, int32_t *plan,
                             int32_t *ticket, bool wbf16, hipStream_t s) {
  const dim3 grid((unsigned)T), block(256);
  if (E <= 64)
    route_plan_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2, plan, ticket, wbf16);
  else if (E <= 128)
    route_plan_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2, plan, ticket, wbf16);
  else if (E <= 256)
    route_plan_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2, plan, ticket, wbf16);
  else if (E <= 512)
    route_plan_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2, plan, ticket, wbf16);
  else
    route_plan_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2, plan, ticket, wbf16);
  return hipGetLastError();
}

// ---------------------------------------------------------------- router
// logits[t, e] = sum_h x[t, h] Wr[e, h] (+ br[e]), fp32 accumulation.
// One wave per (expert, group of 8 tokens); each lane walks h in steps of
// 4 floats (16-byte loads of Wr), the wave reduces at the end.
template <typename XT>
__global__ __launch_bounds__(256) void router_kernel(const XT *__restrict__ x, int64_t T, int H,
                                                     const float *__restrict__ Wr,
                                                     const float *__restrict__ br, int E,
                                                     float *__restrict__ logits,
                                                     float *__restrict__ logits2) {
  const int n_eb = (E + 3) / 4;
  const int64_t tb = blockIdx.x / n_eb;
  const int e = (int)(blockIdx.x - tb * n_eb) * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int lane = lane_id();
  const int64_t t0 = tb * 8;
  const int nt = (int)min<int64_t>(8, T - t0);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  const float *wrow = Wr + (int64_t)e * H;
  for (int h = lane * 4; h < H; h += 4 * kWave) {
    const uint4 wq = ld16(wrow + h);
    float wv[4];
    Elem<float>::widen(wq, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nt) {
        const XT *xr = x + (t0 + i) * (int64_t)H + h;
        float xv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) xv[k] = Elem<XT>::load1(xr + k);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i] = __builtin_fmaf(wv[k], xv[k], acc[i]);
      }
    }
  }
  const float b = br ? br[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < nt) {
      const float sum = wave_sum(acc[i]) + b;
      if (lane == 0) {
        logits[(t0 + i) * E + e] = sum;
        if (logits2) logits2[(t0 + i) * E + e] = sum;
      }
    }
  }
}

// Small batches: one wave per (expert, group of kRowsTok tokens) loads the
// expert's whole router row (NCHR 16-byte chunks per lane, all in flight at
// once), then dots it with the group's tokens, four at a time (x read 4
// elements per load).
template <typename XT>
__device__ __forceinline__ void load4(const XT *p, float (&v)[4]) {
  if constexpr (sizeof(XT) == 2) {
    const uint2 q = *reinterpret_cast<const uint2 *>(p);
    v[0] = bf16_lo(q.x);
    v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y);
    v[3] = bf16_hi(q.y);
  } else {
    Elem<float>::widen(ld16(p), v);
  }
}

constexpr int kRowsTok = 16;

// Block `bid` of the router: experts 4*(bid % n_eb) .. +3, tokens of group
// bid / n_eb.  With tl, each logit is also published as a tagged word
// tl[t * kMaxExperts + e] (read by other workgroups of the same kernel).
template <typename XT, int NCHR>
__device__ __forceinline__ void router_rows(const XT *__restrict__ x, int64_t T, int H,
                                            const float *__restrict__ Wr,
                                            const float *__restrict__ br, int E,
                                            float *__restrict__ logits,
                                            float *__restrict__ logits2, int bid,
                                            uint64_t *__restrict__ tl = nullptr,
                                            uint32_t tag = 0u) {
  const int n_eb = (E + 3) / 4;
  const int tg = bid / n_eb;
  const int e = (bid - tg * n_eb) * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int lane = lane_id();
  const float *wrow = Wr + (int64_t)e * H;
  float wv[NCHR][4];
#pragma unroll
  for (int j = 0; j < NCHR; ++j) Elem<float>::widen(ld16_stream(wrow + (j * kWave + lane) * 4), wv[j]);
  const float b = br ? br[e] : 0.0f;
  const int64_t t_end = min<int64_t>(T, (int64_t)(tg + 1) * kRowsTok);
  for (int64_t t0 = (int64_t)tg * kRowsTok; t0 < t_end; t0 += 4) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = min<int64_t>(t0 + q, t_end - 1);
      const XT *xr = x + t * H;
#pragma unroll
      for (int j = 0; j < NCHR; ++j) {
        float xv[4];
        load4(xr + (j * kWave + lane) * 4, xv);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[q] = __builtin_fmaf(wv[j][k], xv[k], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sum = wave_sum_dpp(acc[q]) + b;
      const int64_t t = t0 + q;
      if (lane == 0 && t < t_end) {
        if (tl) coh_st(tl + t * kMaxExperts + e, tagged(tag, sum));
        logits[t * E + e] = sum;
        if (logits2) logits2[t * E + e] = sum;
      }
    }
  }
}

// Block `bid` of the small-batch router when a lane holds at least four
// 16-byte chunks of a router row: expert bid % E, tokens of group bid / E;
// each wave takes a quarter of the row, the four partial dot products of
// each token are added in a fixed order, and the logits are published as
// tagged words tl[t * kMaxExperts + e].  A block per expert spreads the
// router's loads over E compute units (four experts per block left most of
// them idle).
// With WB the router weight is bf16 (the router method on a bf16 model): the
// products are exact in fp32, the sum is rounded once to bf16, no bias.
template <typename XT, int NCHR, bool WB>
__device__ __forceinline__ void router_rows_split(const XT *__restrict__ x, int64_t T, int H,
                                                  const void *__restrict__ Wr,
                                                  const float *__restrict__ br, int E,
                                                  float *__restrict__ logits,
                                                  float *__restrict__ logits2, int bid,
                                                  uint64_t *__restrict__ tl, uint32_t tag) {
  constexpr int NCW = NCHR / 4;
  static_assert(NCHR % 4 == 0, "a row in four quarters");
  __shared__ float part[4][kRowsTok];
  const int tg = bid / E;
  const int e = bid - tg * E;
  const int lane = lane_id(), wq = threadIdx.x >> 6;
  const int j0 = wq * NCW;
  float wv[NCW][4];
  if constexpr (WB) {
    const uint16_t *wrow = static_cast<const uint16_t *>(Wr) + (int64_t)e * H;
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const uint2 q = *reinterpret_cast<const uint2 *>(wrow + ((j0 + j) * kWave + lane) * 4);
      wv[j][0] = bf16_lo(q.x);
      wv[j][1] = bf16_hi(q.x);
      wv[j][2] = bf16_lo(q.y);
      wv[j][3] = bf16_hi(q.y);
    }
  } else {
    const float *wrow = static_cast<const float *>(Wr) + (int64_t)e * H;
#pragma unroll
    for (int j = 0; j < NCW; ++j)
      Elem<float>::widen(ld16_stream(wrow + ((j0 + j) * kWave + lane) * 4), wv[j]);
  }
  const int64_t t_begin = (int64_t)tg * kRowsTok;
  const int64_t t_end = min<int64_t>(T, t_begin + kRowsTok);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 4) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = min<int64_t>(t0 + q, t_end - 1);
      const XT *xr = x + t * H;
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        float xv[4];
        load4(xr + ((j0 + j) * kWave + lane) * 4, xv);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[q] = __builtin_fmaf(wv[j][k], xv[k], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sum = wave_sum_dpp(acc[q]);
      if (lane == 0 && t0 + q < t_end) part[wq][t0 + q - t_begin] = sum;
    }
  }
  __syncthreads();
  const int i = (int)threadIdx.x;
  if (i < t_end - t_begin) {
    const int64_t t = t_begin + i;
    float sum = (part[0][i] + part[1][i]) + (part[2][i] + part[3][i]);
    if constexpr (WB)
      sum = round_bf16(sum);
    else
      sum = sum + (br ? br[e] : 0.0f);
    coh_st(tl + t * kMaxExperts + e, tagged(tag, sum));
    logits[t * E + e] = sum;
    if (logits2) logits2[t * E + e] = sum;
  }
}

template <typename XT, int NCHR>
__global__ __launch_bounds__(256) void router_rows_kernel(const XT *__restrict__ x, int64_t T,
                                                          int H, const float *__restrict__ Wr,
                                                          const float *__restrict__ br, int E,
                                                          float *__restrict__ logits,
                                                          float *__restrict__ logits2) {
  router_rows<XT, NCHR>(x, T, H, Wr, br, E, logits, logits2, blockIdx.x);
}

// Small batches (2 <= T <= kRouteBatchMax): router and route in one launch,
// with the one-token layer's hand-over (sync.hpp) instead of a barrier: the
// first n_router blocks compute the logits and publish each as a tagged word
// of the call (tl); the last T blocks of the grid each stage one token's E
// tagged words (one round trip, then re-reads of the missing ones) and route
// it.  Only those T <= 64 blocks ever wait and every other block runs to its
// end, so the waiters cannot keep the blocks they wait for from running; the
// wait is bounded and sets the error word when it gives up.  No counter or word of
// the sync region changes, so nothing has to return to zero; the epoch that
// makes the tag is advanced by the gate/up launch that follows.  `withhold`
// (a test hook) makes the route blocks wait for a tag no word carries, so
// every wait gives up; they route the finite values they read (this call's
// or an earlier call's logits, or zero), so the ids stay in range; the
// outputs are unspecified.
template <typename XT, int NCHR, int V, bool WB>
__global__ __launch_bounds__(256) void router_route_batch_kernel(
    const XT *__restrict__ x, int T, int H, const void *__restrict__ Wr,
    const float *__restrict__ br, int E, int k1, int k2, float *__restrict__ logits,
    float *__restrict__ logits2, int32_t *__restrict__ ids, float *__restrict__ w,
    int32_t *__restrict__ ids2, float *__restrict__ w2, int32_t *__restrict__ sync,
    uint64_t *__restrict__ tl, uint32_t spin_limit, bool withhold, int n_router) {
  __shared__ float sl[kMaxExperts];
  __shared__ int32_t s_ids[kMaxExperts];
  __shared__ float s_w[kMaxExperts];
  __shared__ BlockRoute S;
  const uint32_t tag = call_tag((uint32_t)coh_ld(sync + kEpochWord));
  if ((int)blockIdx.x < n_router) {
    if constexpr (NCHR % 4 == 0)
      router_rows_split<XT, NCHR, WB>(x, T, H, Wr, br, E, logits, logits2, blockIdx.x, tl, tag);
    else if constexpr (!WB)
      router_rows<XT, NCHR>(x, T, H, static_cast<const float *>(Wr), br, E, logits, logits2,
                            blockIdx.x, tl, tag);
  }
  const int t = (int)blockIdx.x - ((int)gridDim.x - T);
  if (t < 0) return;
  // 2: not a call tag (their low bit is set) and not the zero fill
  const uint32_t want = withhold ? 2u : tag;
  const uint64_t *trow = tl + (int64_t)t * kMaxExperts;
  stage_tagged<kMaxExperts / kSyncThreads>(sl, E, [&](int i) { return trow + i; }, want,
                                           sync + kErrorWord, spin_limit);
  route_into_lds<V>(sl, E, k1, k2, s_ids, s_w, S, WB);
  const int64_t o = (int64_t)t * k1;
  for (int r = (int)threadIdx.x; r < k1; r += kBlockThreads) {
    ids[o + r] = s_ids[r];
    w[o + r] = s_w[r];
    if (ids2) ids2[o + r] = s_ids[r];
    if (w2) w2[o + r] = s_w[r];
  }
}

bool router_route_batch_supported(int64_t T, int H, bool wr_bf16) {
  // the bf16 router weight only with a row in four quarters (H % 1024 == 0)
  return T >= 2 && T <= kRouteBatchMax && router_route_supported(H) &&
         (!wr_bf16 || (H / (4 * kWave)) % 4 == 0);
}

template <typename XT, int NCHR, bool WB>
static void launch_rrb_v(const XT *x, int T, int H, const void *Wr, const float *br, int E,
                         int k1, int k2, float *logits, float *logits2, int32_t *ids, float *w,
                         int32_t *ids2, float *w2, int32_t *sync, uint64_t *tl,
                         uint32_t spin_limit, bool withhold, hipStream_t s) {
  const int n_router =
      (NCHR % 4 == 0 ? E : (E + 3) / 4) * ((T + kRowsTok - 1) / kRowsTok);
  const dim3 grid((unsigned)max(n_router, T)), block(256);
#define RRB(V)                                                                               \
  router_route_batch_kernel<XT, NCHR, V, WB><<<grid, block, 0, s>>>(                        \
      x, T, H, Wr, br, E, k1, k2, logits, logits2, ids, w, ids2, w2, sync, tl, spin_limit, withhold, \
      n_router)
  if (E <= 64) RRB(1);
  else if (E <= 128) RRB(2);
  else if (E <= 256) RRB(4);
  else if (E <= 512) RRB(8);
  else RRB(16);
#undef RRB
}

template <typename XT>
hipError_t launch_router_route_batch(const XT *x, int64_t T, int H, const void *Wr, bool wr_bf16,
                                     const float *br, int E, int k1, int k2, float *logits,
                                     float *logits2, int32_t *ids, float *w, int32_t *ids2,
                                     float *w2, int32_t *sync, uint64_t *tl, uint32_t spin_limit,
                                     bool withhold, hipStream_t s) {
  if (!router_route_batch_supported(T, H, wr_bf16)) return hipErrorInvalidValue;
  const int t = (int)T;
#define GO(N, WB) launch_rrb_v<XT, N, WB>(x, t, H, Wr, br, E, k1, k2, logits, logits2, ids, w, \
                                          ids2, w2, sync, tl, spin_limit, withhold, s)
  if (wr_bf16) {
    if constexpr (sizeof(XT) == 2) {
      switch (H / (4 * kWave)) {
        case 4: GO(4, true); break;
        case 8: GO(8, true); break;
        default: GO(16, true); break;
      }
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    switch (H / (4 * kWave)) {
      case 1: GO(1, false); break;
      case 2: GO(2, false); break;
      case 4: GO(4, false); break;
      case 8: GO(8, false); break;
      default: GO(16, false); break;
    }
  }
#undef GO
  return hipGetLastError();
}

template hipError_t launch_router_route_batch<float>(const float *, int64_t, int, const void *,
                                                     bool, const float *, int, int, int, float *,
                                                     float *, int32_t *, float *, int32_t *,
                                                     float *, int32_t *, uint64_t *, uint32_t,
                                                     bool, hipStream_t);
template hipError_t launch_router_route_batch<bf16_t>(const bf16_t *, int64_t, int,
                                                      const void *, bool, const float *, int, int,
                                                      int, float *, float *, int32_t *, float *,
                                                      int32_t *, float *, int32_t *, uint64_t *,
                                                      uint32_t, bool, hipStream_t);

// bf16 router (the router method on a bf16 model): logits[t, e] =
// bf16(sum_h x[t, h] Wr[e, h]) with bf16 x and Wr, the products exact and the
// sum in fp32, rounded once to bf16 (kept as fp32 values).  One wave per
// (expert, group of kRowsTok tokens); lanes take 16-byte chunks of the row
// and of x, four tokens per pass.
__global__ __launch_bounds__(256) void router_bf16_kernel(const bf16_t *__restrict__ x, int64_t T,
                                                          int H, const bf16_t *__restrict__ Wr,
                                                          int E, float *__restrict__ logits,
                                                          float *__restrict__ logits2) {
  const int n_eb = (E + 3) / 4;
  const int64_t tg = blockIdx.x / n_eb;
  const int e = (int)(blockIdx.x - tg * n_eb) * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int lane = lane_id();
  const bf16_t *wrow = Wr + (int64_t)e * H;
  const int nch = H / 8;
  const int64_t t_end = min<int64_t>(T, (tg + 1) * kRowsTok);
  for (int64_t t0 = tg * kRowsTok; t0 < t_end; t0 += 4) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = lane; c < nch; c += kWave) {
      const uint4 wq = ld16(wrow + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t t = min<int64_t>(t0 + q, t_end - 1);
        const uint4 xq = ld16(x + t * H + c * 8);
        acc[q] = dot2_bf16(wq.x, xq.x, acc[q]);
        acc[q] = dot2_bf16(wq.y, xq.y, acc[q]);
        acc[q] = dot2_bf16(wq.z, xq.z, acc[q]);
        acc[q] = dot2_bf16(wq.w, xq.w, acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float l = round_bf16(wave_sum_dpp(acc[q]));
      const int64_t t = t0 + q;
      if (lane == 0 && t < t_end) {
        logits[t * E + e] = l;
        if (logits2) logits2[t * E + e] = l;
      }
    }
  }
}

hipError_t launch_router_bf16(const bf16_t *x, int64_t T, int H, const bf16_t *Wr, int E,
                              float *logits, float *logits2, hipStream_t s) {
  const dim3 grid((unsigned)(((E + 3) / 4) * ((T + kRowsTok - 1) / kRowsTok))), block(256);
  router_bf16_kernel<<<grid, block, 0, s>>>(x, T, H, Wr, E, logits, logits2);
  return hipGetLastError();
}

// One token: router, route and plan in one launch.  Wave e computes logit
// e (its router row in flight at once, NCHR 16-byte chunks per lane) and
// stores it device-coherently; the block that takes the last ticket reads
// every logit back, routes the token, writes ids and w and, for k1 <= 64,
// the plan.
template <typename XT, int NCHR, int V>
__global__ __launch_bounds__(256) void router_route_kernel(
    const XT *__restrict__ x, int H, const float *__restrict__ Wr, const float *__restrict__ br,
    int E, int k1, int k2, float *__restrict__ logits, float *__restrict__ logits2,
    int32_t *__restrict__ ids, float *__restrict__ w, int32_t *__restrict__ ids2,
    float *__restrict__ w2, int32_t *__restrict__ plan, int32_t *__restrict__ ticket) {
  __shared__ float sl[kMaxExperts];
  __shared__ int32_t s_ids[kMaxExperts];
  __shared__ float s_w[kMaxExperts];
  __shared__ BlockRoute S;
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = lane_id();
  const int e = blockIdx.x * 4 + (tid >> 6);
  if (e < E) {
    const float *wrow = Wr + (int64_t)e * H;
    float wv[NCHR][4];
#pragma unroll
    for (int j = 0; j < NCHR; ++j)
      Elem<float>::widen(ld16_stream(wrow + (j * kWave + lane) * 4), wv[j]);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NCHR; ++j) {
      const int h = (j * kWave + lane) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(wv[j][k], Elem<XT>::load1(x + h + k), acc);
    }
    const float sum = wave_sum_dpp(acc) + (br ? br[e] : 0.0f);
    if (lane == 0) {
      coh_st(logits + e, sum);
      if (logits2) logits2[e] = sum;
    }
  }
  if (!last_of(ticket, (int)gridDim.x, &s_last)) return;
  for (int i = tid; i < E; i += kBlockThreads) sl[i] = coh_ld(logits + i);
  __syncthreads();
  route_into_lds<V>(sl, E, k1, k2, s_ids, s_w, S);
  for (int r = tid; r < k1; r += kBlockThreads) {
    ids[r] = s_ids[r];
    w[r] = s_w[r];
    if (ids2) ids2[r] = s_ids[r];
    if (w2) w2[r] = s_w[r];
  }
  if (plan && k1 <= kWave && tid < kWave) wave_plan(tid < k1 ? s_ids[tid] : 0x7FFFFFFF, k1, E, plan);
}

template <typename XT, int NCHR>
static void launch_rr_v(const XT *x, int H, const float *Wr, const float *br, int E, int k1,
                        int k2, float *logits, float *logits2, int32_t *ids, float *w,
                        int32_t *ids2, float *w2, int32_t *plan, int32_t *ticket, hipStream_t s) {
  const dim3 grid((unsigned)((E + 3) / 4)), block(256);
#define RR(V) router_route_kernel<XT, NCHR, V><<<grid, block, 0, s>>>(x, H, Wr, br, E, k1, k2, \
                                                                      logits, logits2, ids, w, \
                                                                      ids2, w2, plan, ticket)
  if (E <= 64) RR(1);
  else if (E <= 128) RR(2);
  else if (E <= 256) RR(4);
  else if (E <= 512) RR(8);
  else RR(16);
#undef RR
}

bool router_route_supported(int H) {
  const int nchr = (H % (4 * kWave) == 0) ? H / (4 * kWave) : 0;
  return nchr == 1 || nchr == 2 || nchr == 4 || nchr == 8 || nchr == 16;
}

template <typename XT>
hipError_t launch_router_route(const XT *x, int H, const float *Wr, const float *br, int E,
                               int k1, int k2, float *logits, float *logits2, int32_t *ids,
                               float *w, int32_t *ids2, float *w2, int32_t *plan, int32_t *ticket,
                               hipStream_t s) {
  switch (H / (4 * kWave)) {
    case 1: launch_rr_v<XT, 1>(x, H, Wr, br, E, k1, k2, logits, logits2, ids, w, ids2, w2, plan, ticket, s); break;
    case 2: launch_rr_v<XT, 2>(x, H, Wr, br, E, k1, k2, logits, logits2, ids, w, ids2, w2, plan, ticket, s); break;
    case 4: launch_rr_v<XT, 4>(x, H, Wr, br, E, k1, k2, logits, logits2, ids, w, ids2, w2, plan, ticket, s); break;
    case 8: launch_rr_v<XT, 8>(x, H, Wr, br, E, k1, k2, logits, logits2, ids, w, ids2, w2, plan, ticket, s); break;
    default: launch_rr_v<XT, 16>(x, H, Wr, br, E, k1, k2, logits, logits2, ids, w, ids2, w2, plan, ticket, s); break;
  }
  return hipGetLastError();
}

template hipError_t launch_router_route<float>(const float *, int, const float *, const float *,
                                               int, int, int, float *, float *, int32_t *, float *,
                                               int32_t *, float *, int32_t *, int32_t *,
                                               hipStream_t);
template hipError_t launch_router_route<bf16_t>(const bf16_t *, int, const float *, const float *,
                                                int, int, int, float *, float *, int32_t *,
                                                float *, int32_t *, float *, int32_t *, int32_t *,
                                                hipStream_t);

template <typename XT>
hipError_t launch_router(const XT *x, int64_t T, int H, const float *Wr, const float *br, int E,
                         float *logits, float *logits2, hipStream_t s) {
  const int nchr = (H % (4 * kWave) == 0) ? H / (4 * kWave) : 0;
  if (T <= 64 && (nchr == 1 || nchr == 2 || nchr == 4 || nchr == 8 || nchr == 16)) {
    const dim3 grid((unsigned)(((E + 3) / 4) * ((T + kRowsTok - 1) / kRowsTok))), block(256);
    switch (nchr) {
      case 1: router_rows_kernel<XT, 1><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2); break;
      case 2: router_rows_kernel<XT, 2><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2); break;
      case 4: router_rows_kernel<XT, 4><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2); break;
      case 8: router_rows_kernel<XT, 8><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2); break;
      default: router_rows_kernel<XT, 16><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2); break;
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(((E + 3) / 4) * ((T + 7) / 8))), block(256);
  router_kernel<XT><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2);
  return hipGetLastError();
}

template hipError_t launch_router<float>(const float *, int64_t, int, const float *,
                                         const float *, int, float *, float *, hipStream_t);
template hipError_t launch_router<bf16_t>(const bf16_t *, int64_t, int, const float *,
                                          const float *, int, float *, float *, hipStream_t);

}  // namespace moe
