// Device-side route of one token: fp32 softmax with a specified exp, ranking
// and the Eq. 2 weights ("Paper of the Week #3 - Half the FLOPs Is Not Half
// the Time", section "The Receipt", Eq. 2; section "Ship It - Code of the
// Week").  Used by the route kernels and by the one-token layer kernel.
#pragma once

#include "common.hpp"
#include "sync.hpp"

namespace moe {

namespace expc {
// Constants of the exp below, derived from ln 2 at compile time.
constexpr double kLn2 = 0.693147180559945309417232121458176568;
__host__ __device__ constexpr uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ constexpr float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }
// log2(e) rounded to float
constexpr float kLog2e = (float)(1.0 / kLn2);
// ln 2 rounded to float with its 8 low significand bits cleared (16
// significant bits, so n * hi is exact for |n| < 256) and the rounded rest.
constexpr float kLn2Hi = bitsf(fbits((float)kLn2) & 0xFFFFFF00u);
constexpr float kLn2Lo = (float)(kLn2 - (double)kLn2Hi);
// 1/k!, k = 0..7, rounded to float
constexpr float kC0 = 1.0f, kC1 = 1.0f, kC2 = (float)(1.0 / 2.0), kC3 = (float)(1.0 / 6.0),
                kC4 = (float)(1.0 / 24.0), kC5 = (float)(1.0 / 120.0),
                kC6 = (float)(1.0 / 720.0), kC7 = (float)(1.0 / 5040.0);
}  // namespace expc

// e^d for d <= 0 by Cody & Waite's reduction (Software Manual for the
// Elementary Functions, 1980): n = rint(d log2 e), r = d - n ln2 with ln2
// split in two parts, e^d = 2^n e^r, e^r by its degree-7 Taylor polynomial
// in Horner form with fused multiply-adds.  Zero below -80, so every nonzero
// result is a normal float.
__device__ __forceinline__ float exp_nonpos(float d) {
#pragma clang fp contract(off)
  using namespace expc;
  if (d < -80.0f) return 0.0f;
  float t = d * kLog2e;
  float n = __builtin_rintf(t);
  float r = __builtin_fmaf(-n, kLn2Hi, d);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float q = kC7;
  q = __builtin_fmaf(q, r, kC6);
  q = __builtin_fmaf(q, r, kC5);
  q = __builtin_fmaf(q, r, kC4);
  q = __builtin_fmaf(q, r, kC3);
  q = __builtin_fmaf(q, r, kC2);
  q = __builtin_fmaf(q, r, kC1);
  q = __builtin_fmaf(q, r, kC0);
  return __builtin_ldexpf(q, (int)n);
}

// The route of one token, shared by every route below:
//  1. m = max of the logits (exact);
//  2. e = exp_nonpos(l - m), 0 for the padding;
//  3. S = pairwise sum of e over the next power of two >= E (zero padded):
//     each 64-expert chunk by the wave sum (wave_sum_dpp is the pairwise
//     tree over the lanes in order), then the pairwise tree over the chunk
//     sums.  fp32 addition is commutative, so the order inside a node does
//     not matter, and zero padding leaves a power-of-two tree's sum
//     unchanged;
//  4. p = e / S (IEEE division);
//  5. ranking by (p descending, index ascending) with key = bits of p + 1
//     (p >= 0, so the bits order like the values; padding has key 0), packed
//     with the index so that one unsigned compare orders the experts; only
//     the first R = min(k2, E) ranks are needed (k1 when k2 >= E: no mass);
//  6. M = p_(0) + p_(1) + ... left to right over the min(k2, E) ranked values;
//     w_r = p_(r) / M, or p_(r) when k2 >= E;
//  7. with wbf16 (the router run on a bf16 model, where the method casts the
//     weights to the logits' dtype), w_r is then rounded to bf16.

constexpr int kBlockThreads = 256;
constexpr int kBlockWaves = kBlockThreads / kWave;

// LDS of a block route.
struct BlockRoute {
  alignas(16) uint64_t KL[kMaxExperts];  // the candidates' packed keys
  uint32_t key[kMaxExperts];             // E > 256: every expert's key
  float red[kBlockWaves];
  float chunk[kMaxExperts / kWave];
  int32_t n;
  float M;
};

// The route from nc candidates in S.KL (packed keys, the R largest among
// them) by the whole block: each candidate's rank counted against the
// others, the first R ranks stored (w holding p), the mass summed in rank
// order by thread 0, then w = p / M (or p), rounded to bf16 with wbf16.
__device__ __forceinline__ void block_rank(BlockRoute &S, int nc, int R, int k1, bool renorm,
                                           bool wbf16, int32_t *ids, float *w) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  for (int i = tid; i < nc; i += kBlockThreads) {
    const uint64_t Ki = S.KL[i];
    int r = 0;
    for (int q = 0; q < nc; ++q) r += S.KL[q] > Ki ? 1 : 0;
    if (r < R) {
      w[r] = __uint_as_float((uint32_t)(Ki >> 11) - 1u);
      ids[r] = 2047 - (int)(Ki & 2047u);
    }
  }
  __syncthreads();
  if (tid == 0) {
    float M = 0.0f;
    if (renorm) {
      int r = 0;
      for (; r + 8 <= R; r += 8) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = w[r + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) M = M + v[q];
      }
      for (; r < R; ++r) M = M + w[r];
    }
    S.M = M;
  }
  __syncthreads();
  for (int r = tid; r < k1; r += kBlockThreads) {
    float wr = renorm ? w[r] / S.M : w[r];
    if (wbf16) wr = round_bf16(wr);
    w[r] = wr;
  }
  __syncthreads();
}

constexpr int kTauBits = 12;

template <int V>
__device__ void route_token_block_large(const float *l, int E, int k1, int k2, int32_t *ids,
                                        float *w, BlockRoute &S, bool wbf16 = false) {
#pragma clang fp contract(off)
  constexpr int J = kMaxExperts / kBlockThreads;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  // thread t holds experts t, t + 256, t + 512, t + 768
  float lv[J];
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = j * kBlockThreads + tid;
    lv[j] = e < E ? l[e] : -INFINITY;
    tmax = fmaxf(tmax, lv[j]);
  }
  const float wm = wave_max_dpp(tmax);
  if (lane == 0) S.red[wv] = wm;
  __syncthreads();
  const float m = fmaxf(fmaxf(S.red[0], S.red[1]), fmaxf(S.red[2], S.red[3]));
  float ex[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = j * kBlockThreads + tid;
    ex[j] = e < E ? exp_nonpos(lv[j] - m) : 0.0f;
    // chunk 4j + wv is experts [64 (4j + wv), +64), one per lane in order
    const float cs = wave_sum_dpp(ex[j]);
    if (lane == 0) S.chunk[j * kBlockWaves + wv] = cs;
  }
  __syncthreads();
  float c8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) c8[q] = S.chunk[2 * q] + S.chunk[2 * q + 1];
  const float sum = ((c8[0] + c8[1]) + (c8[2] + c8[3])) + ((c8[4] + c8[5]) + (c8[6] + c8[7]));
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = j * kBlockThreads + tid;
    S.key[e] = e < E ? __float_as_uint(ex[j] / sum) + 1u : 0u;
  }
  __syncthreads();
  const bool renorm = k2 < E;
  const int R = renorm ? k2 : k1;
  if (wv == 0) {
    // the first wave holds expert q * 64 + lane in key[q]
    uint32_t key[V];
#pragma unroll
    for (int q = 0; q < V; ++q) key[q] = S.key[q * kWave + lane];
    // all V compares are issued before the first scalar popcount reads a
    // result (interleaved, each popcount stalled the wave on its compare)
    auto count_ge = [&](uint32_t c) {
      uint64_t bal[V];
#pragma unroll
      for (int q = 0; q < V; ++q) bal[q] = __ballot(key[q] >= c);
      __builtin_amdgcn_sched_barrier(0);
      int n = 0;
#pragma unroll
      for (int q = 0; q < V; ++q) n += __popcll(bal[q]);
      return n;
    };
    // keys are at most bits(1.0f) + 1 < 2^30: the top kTauBits bits of the
    // R-th largest key, from the top
    uint32_t tau = 0u;
    for (int b = 29; b >= 30 - kTauBits; --b) {
      const uint32_t c = tau | (1u << b);
      if (count_ge(c) >= R) tau = c;
    }
    // the candidates: every key >= tau (at least R of them, every one of
    // the R largest among them)
    const uint64_t below = (1ull << lane) - 1ull;
    int pos = 0;
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const bool cand = key[q] >= tau;
      const uint64_t cm = __ballot(cand);
      if (cand)
        S.KL[pos + __popcll(cm & below)] =
            ((uint64_t)key[q] << 11) | (uint64_t)(2047 - (q * kWave + lane));
      pos += __popcll(cm);
    }
    if (lane == 0) S.n = pos;
  }
  __syncthreads();
  block_rank(S, S.n, R, k1, renorm, wbf16, ids, w);
}

// Every store of this block is complete (s_waitcnt), then thread 0 takes a
// ticket; true in the whole block that takes the last of n tickets, which
// also puts the ticket word back to zero.
__device__ inline bool last_of(int32_t *ticket, int n, int *s_last) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = old == n - 1;
    if (old == n - 1) coh_st(ticket, 0);
  }
  __syncthreads();
  return *s_last;
}

// The batch plan from ids [n] (n <= 64), built by one wave: U, the unique
// experts ascending, and per unique expert its assignments (t*k1 + r)
// ascending.  Lane i holds assignment i.
__device__ inline void wave_plan(int e, int n, int E, int32_t *plan) {
  const int i = lane_id();
  int cnt_less = 0, same_before = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    cnt_less += ej < e;
    same_before += (ej == e) & (j < i);
  }
  const uint64_t first = __ballot(i < n && same_before == 0);
  int uniq_less = 0;
  for (int j = 0; j < n; ++j)
    if ((first >> j) & 1ull) uniq_less += __builtin_amdgcn_readlane(e, j) < e;
  int32_t *uniq = plan + 4;
  int32_t *off = uniq + E;
  int32_t *list = off + E + 1;
  if (i < n) {
    if (same_before == 0) {
      uniq[uniq_less] = e;
      off[uniq_less] = cnt_less;
    }
    list[cnt_less + same_before] = i;
  }
  if (i == 0) {
    const int U = __popcll(first);
    plan[0] = U;
    off[U] = n;
  }
}

// The keys of the experts held by one wave (E <= V * 64): lane L holds
// experts q * 64 + L in slot q < V (index order (q, L), so a ballot's lower
// lanes are the lower indices).  Exact max; e = exp_nonpos(l - max); S =
// the pairwise tree (each chunk q by the wave sum, then the tree over the V
// chunk sums); p = e / S; key = bits of p + 1, 0 for the padding.
template <int V>
__device__ __forceinline__ void wave_keys(const float *l, int E, uint32_t (&key)[V]) {
#pragma clang fp contract(off)
  const int lane = lane_id();
  float ex[V];
  float tmax = -INFINITY;
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = q * kWave + lane;
    ex[q] = e < E ? l[e] : -INFINITY;
    tmax = fmaxf(tmax, ex[q]);
  }
  const float m = wave_max_dpp(tmax);
  float cs[V];
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = q * kWave + lane;
    ex[q] = e < E ? exp_nonpos(ex[q] - m) : 0.0f;
    cs[q] = wave_sum_dpp(ex[q]);
  }
#pragma unroll
  for (int step = 1; step < V; step <<= 1)
#pragma unroll
    for (int q = 0; q + step < V; q += 2 * step) cs[q] = cs[q] + cs[q + step];
  const float sum = cs[0];
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = q * kWave + lane;
    key[q] = e < E ? __float_as_uint(ex[q] / sum) + 1u : 0u;
  }
}

// The top kTauBits bits of the R-th largest of the wave's keys (one ballot
// count per bit, from the top; keys are at most bits(1.0f) + 1 < 2^30).
template <int V>
__device__ __forceinline__ uint32_t wave_tau(const uint32_t (&key)[V], int R) {
  // all V compares are issued before the first scalar popcount reads a
  // result (interleaved, each popcount stalled the wave on its compare)
  auto count_ge = [&](uint32_t c) {
    uint64_t bal[V];
#pragma unroll
    for (int q = 0; q < V; ++q) bal[q] = __ballot(key[q] >= c);
    __builtin_amdgcn_sched_barrier(0);
    int n = 0;
#pragma unroll
    for (int q = 0; q < V; ++q) n += __popcll(bal[q]);
    return n;
  };
  uint32_t tau = 0u;
  for (int b = 29; b >= 30 - kTauBits; --b) {
    const uint32_t c = tau | (1u << b);
    if (count_ge(c) >= R) tau = c;
  }
  return tau;
}

// The candidates, every key >= tau (at least R of them when tau is the
// prefix of the R-th largest, every one of the R largest among them),
// packed with their index (key << 11 | 2047 - index, so that one unsigned
// compare orders by (p descending, index ascending)) into S.KL in index
// order; returns their number (in every lane).
template <int V>
__device__ __forceinline__ int wave_candidates(const uint32_t (&key)[V], uint32_t tau,
                                               BlockRoute &S) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
  int nc = 0;
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const bool cand = key[q] >= tau;
    const uint64_t cm = __ballot(cand);
    if (cand)
      S.KL[nc + __popcll(cm & below)] =
          ((uint64_t)key[q] << 11) | (uint64_t)(2047 - (q * kWave + lane));
    nc += __popcll(cm);
  }
  return nc;
}

// Rank of packed key K among the nc candidates in S.KL (LDS reads at one
// address for the whole wave; measured faster than broadcasting the keys
// from the lanes with readlane).
__device__ __forceinline__ int wave_rank(const BlockRoute &S, uint64_t K, int nc) {
  int r = 0;
  for (int q = 0; q < nc; ++q) r += S.KL[q] > K ? 1 : 0;
  return r;
}

// One token (E <= 256) routed by one wave, with the arithmetic above: the
// keys (wave_keys), then the candidates at or above the top kTauBits bits of
// the R-th largest key, ranked against each other, the mass summed in rank
// order.  With at most 64 candidates the wave ranks them itself (one per
// lane) and ids and w (LDS, kMaxExperts entries) receive the route in rank
// order, with no barrier (the wave's LDS accesses are ordered by waiting for
// them); with more, the candidates stay in S.KL for block_rank.  Returns the
// number of candidates (in every lane).
//
// With EARLY, the activated set is found first, before the ranks that the
// mass needs: the candidates of the k1-th key are ranked and top_set(sel,
// index) is called in every lane of the wave, sel true in exactly the k1
// lanes that hold an activated expert's index; it is not called (and false
// is stored in *early_done) when those candidates are more than 64.
template <int V, bool EARLY = false, typename TopSet>
__device__ int route_token_wave_ex(const float *l, int E, int k1, int k2, int32_t *ids, float *w,
                                   BlockRoute &S, bool wbf16, TopSet &&top_set,
                                   bool *early_done) {
#pragma clang fp contract(off)
  const int lane = lane_id();
  uint32_t key[V];
  wave_keys<V>(l, E, key);
  const bool renorm = k2 < E;
  const int R = renorm ? k2 : k1;
  uint32_t tau = 0u;
  int nc = -1;
  if constexpr (EARLY) {
    const uint32_t tau1 = wave_tau<V>(key, k1);
    const int nc1 = wave_candidates<V>(key, tau1, S);
    *early_done = nc1 <= kWave;
    if (nc1 <= kWave) {
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      const uint64_t K = lane < nc1 ? S.KL[lane] : 0ull;
      const int r = lane < nc1 ? wave_rank(S, K, nc1) : kWave;
      top_set(r < k1, 2047 - (int)(K & 2047u));
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
    }
    if (R == k1) {
      tau = tau1;
      nc = nc1;
    }
  }
  if (nc < 0) {
    tau = wave_tau<V>(key, R);
    nc = wave_candidates<V>(key, tau, S);
  }
  if (lane == 0) S.n = nc;
  if (nc > kWave) return nc;  // ranked by the block
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // lane i ranks candidate i against the others
  if (lane < nc) {
    const uint64_t K = S.KL[lane];
    const int r = wave_rank(S, K, nc);
    if (r < R) {
      w[r] = __uint_as_float((uint32_t)(K >> 11) - 1u);
      ids[r] = 2047 - (int)(K & 2047u);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  float M = 0.0f;
  if (renorm) {
    // every lane sums the same values in the same order
    int q = 0;
    for (; q + 8 <= R; q += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = w[q + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) M = M + v[u];
    }
    for (; q < R; ++q) M = M + w[q];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  for (int q = lane; q < k1; q += kWave) {
    float wr = renorm ? w[q] / M : w[q];
    if (wbf16) wr = round_bf16(wr);
    w[q] = wr;
  }
  return nc;
}

template <int V>
__device__ int route_token_wave(const float *l, int E, int k1, int k2, int32_t *ids, float *w,
                                BlockRoute &S, bool wbf16 = false) {
  return route_token_wave_ex<V, false>(l, E, k1, k2, ids, w, S, wbf16, [](bool, int) {},
                                       nullptr);
}

// Route one token into LDS (s_ids, s_w: rank order, kMaxExperts entries
// each) with the whole block; wbf16 rounds the weights to bf16.  V = E / 64
// rounded up to a power of two: V <= 4 routes in one wave, V = 8 and 16 with
// the block.
template <int V>
__device__ void route_into_lds(const float *l, int E, int k1, int k2, int32_t *s_ids, float *s_w,
                               BlockRoute &S, bool wbf16 = false) {
  if constexpr (V * kWave <= kBlockThreads) {
    if (threadIdx.x < kWave) route_token_wave<V>(l, E, k1, k2, s_ids, s_w, S, wbf16);
    __syncthreads();
    if (S.n > kWave) {
      const bool renorm = k2 < E;
      block_rank(S, S.n, renorm ? k2 : k1, k1, renorm, wbf16, s_ids, s_w);
    }
  } else {
    route_token_block_large<V>(l, E, k1, k2, s_ids, s_w, S, wbf16);
  }
}

}  // namespace moe
