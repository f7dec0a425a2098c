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

// Route one token with the calling wavefront.  V = values per lane, with
// 64 * V >= E; lane L holds experts [L*V, L*V + V) ("blocked" layout, so a
// lower lane always holds lower indices).
//
//  1. m = max of the logits (exact);
//  2. e = exp_nonpos(l - m), 0 for the padding;
//  3. S = pairwise sum of e over 64*V slots: a lane-local adjacent-pair tree,
//     then the pairwise tree over lanes (wave_sum_dpp).  fp32 addition is
//     commutative, so the lane order inside a node does not matter, and zero
//     padding of a power-of-two tree leaves its sum unchanged: S equals the
//     pairwise sum over the next power of two >= E;
//  4. p = e / S (IEEE division);
//  5. ranking by (p descending, index ascending) with key = bits of p + 1
//     (p >= 0, so the bits order like the values; padding has key 0): for
//     E <= 256 every expert's rank is counted directly, otherwise R rounds
//     take the largest remaining key (lowest lane, lowest slot on ties).
//     Only the first R = min(k2, E) ranks are read (k1 when k2 >= E: no mass
//     needed);
//  6. M = p_(0) + p_(1) + ... left to right over the min(k2, E) ranked values;
//     w_r = p_(r) / M, or p_(r) when k2 >= E;
//  7. with wbf16 (the router run on a bf16 model, where the method casts the
//     weights to the logits' dtype), w_r is then rounded to bf16.
// Rank r is held by lane r % 64 in slot r / 64 until the end.
// COHERENT: read the logits with device-coherent loads (they were written by
// other workgroups of the same kernel).  ids and w may point to LDS.
template <int V, bool COHERENT = false>
__device__ void route_token(const float *__restrict__ l, int E, int k1, int k2,
                            int32_t *__restrict__ ids, float *__restrict__ w,
                            int32_t *__restrict__ ids2, float *__restrict__ w2,
                            bool wbf16 = false) {
#pragma clang fp contract(off)
  const int lane = lane_id();
  float ex[V];
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane * V + j;
    float lv = -INFINITY;
    if (e < E)
      lv = COHERENT ? __hip_atomic_load(const_cast<float *>(l + e), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT)
                    : l[e];
    ex[j] = lv;
    lmax = fmaxf(lmax, ex[j]);
  }
  const float m = wave_max_dpp(lmax);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane * V + j;
    ex[j] = e < E ? exp_nonpos(ex[j] - m) : 0.0f;
  }
  float s[V];
#pragma unroll
  for (int j = 0; j < V; ++j) s[j] = ex[j];
#pragma unroll
  for (int step = 1; step < V; step <<= 1) {
#pragma unroll
    for (int j = 0; j + step < V; j += 2 * step) s[j] = s[j] + s[j + step];
  }
  // the DPP sum is the pairwise tree over the 64 lanes (see wave_sum_dpp)
  const float S = wave_sum_dpp(s[0]);

  uint32_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane * V + j;
    key[j] = e < E ? __float_as_uint(ex[j] / S) + 1u : 0u;
  }

  const bool renorm = k2 < E;
  const int R = renorm ? k2 : k1;
  float M = 0.0f;
  int32_t my_id[V];
  float my_p[V];
#pragma unroll
  for (int q = 0; q < V; ++q) {
    my_id[q] = 0;
    my_p[q] = 0.0f;
  }
  auto keep = [&](int r, int id, float pr) {
    if (r < k1 && lane == (r & (kWave - 1))) {
      const int q = r / kWave;
#pragma unroll
      for (int qq = 0; qq < V; ++qq)
        if (qq == q) {
          my_id[qq] = id;
          my_p[qq] = pr;
        }
    }
  };
  if constexpr (V <= 4) {
    // Rank of each expert = number of experts ahead of it in the order (p
    // descending, index ascending); keys are distinct, so the ranks are a
    // permutation.  Each lane counts against every key, broadcast with
    // readlane: independent instructions instead of a chain of reductions.
    // key and index packed so one unsigned compare orders by (p desc, index
    // asc): padding (key 0) sorts after every expert (key >= 1)
    uint64_t K[V];
    int rank[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      K[j] = ((uint64_t)key[j] << 11) | (uint64_t)(2047 - (lane * V + j));
      rank[j] = 0;
    }
#pragma unroll 4
    for (int L = 0; L < kWave; ++L) {
#pragma unroll
      for (int s2 = 0; s2 < V; ++s2) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)K[s2], L);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(K[s2] >> 32), L);
        const uint64_t kk = ((uint64_t)hi << 32) | lo;
#pragma unroll
        for (int j = 0; j < V; ++j) rank[j] += kk > K[j] ? 1 : 0;
      }
    }
    // walk the ranks in order: the lane holding rank r hands over its expert
    for (int r = 0; r < R; ++r) {
      int sid = -1;
      uint32_t skey = 0u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const bool m = rank[j] == r;
        sid = m ? lane * V + j : sid;
        skey = m ? key[j] : skey;
      }
      const uint64_t mask = __ballot(sid >= 0);
      const int win = __ffsll((unsigned long long)mask) - 1;
      const int id = __builtin_amdgcn_readlane(sid, win);
      const float pr = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)skey, win) - 1u);
      if (renorm) M = M + pr;
      keep(r, id, pr);
    }
  } else {
    // R rounds: each lane offers its best untaken expert, the wave takes the
    // largest key, and the lowest lane holding it wins.
    for (int r = 0; r < R; ++r) {
      uint32_t best = 0u;
      int bj = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        if (key[j] > best) {
          best = key[j];
          bj = j;
        }
      }
      const uint32_t kmax = wave_max_u32_dpp(best);
      const uint64_t mask = __ballot(best == kmax);
      const int win = __ffsll((unsigned long long)mask) - 1;
      if (lane == win) {
#pragma unroll
        for (int j = 0; j < V; ++j)
          if (j == bj) key[j] = 0u;
      }
      const int id = __builtin_amdgcn_readlane(lane * V + bj, win);
      const float pr = __uint_as_float(kmax - 1u);
      if (renorm) M = M + pr;
      keep(r, id, pr);
    }
  }
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int r = q * kWave + lane;
    if (r < k1) {
      float wr = renorm ? my_p[q] / M : my_p[q];
      if (wbf16) wr = round_bf16(wr);
      ids[r] = my_id[q];
      w[r] = wr;
      if (ids2) ids2[r] = my_id[q];
      if (w2) w2[r] = wr;
    }
  }
}

constexpr int kBlockThreads = 256;
constexpr int kBlockWaves = kBlockThreads / kWave;

// One token (E <= 256) routed by the whole block, with the arithmetic of
// route_token: exact max; e = exp_nonpos(l - max); S = the pairwise tree
// (each wave's 64 experts, then (w0 + w1) + (w2 + w3)); p = e / S; ranks by
// (p descending, index ascending) counted in parallel (element e by
// min(256 / P, P) threads, P = next_pow2(E), each over a slice of the keys);
// the mass summed in rank order by one thread; w = p / M or p, rounded to
// bf16 with wbf16.

struct BlockRoute {
  alignas(16) uint64_t K[kBlockThreads];
  int32_t rank[kBlockThreads];
  float sp[kBlockThreads];
  int32_t sid[kBlockThreads];
  float red[kBlockWaves];
  float M;
};

// Rank counting over keys in LDS (16-byte aligned, read at the same address
// by every lane, so each read is a broadcast).  With kBatch16 the reads go in
// batches of 16 keys issued together, one LDS round trip per batch instead
// of one per 8 keys; each batch keeps 16 compare masks live in scalar
// registers, so it is used only where the kernel has them to spare (a spill
// to scratch on this path costs more than the batching saves).
__device__ __forceinline__ void load16(const uint64_t *K, ulonglong2 (&q)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = *reinterpret_cast<const ulonglong2 *>(K + 2 * i);
}
__device__ __forceinline__ int above16(const ulonglong2 (&q)[8], uint64_t Ke) {
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    c0 += (q[i].x > Ke) + (q[i].y > Ke);
    c1 += (q[i + 1].x > Ke) + (q[i + 1].y > Ke);
  }
  return c0 + c1;
}
// How many of the n keys at K exceed Ke (n a multiple of 8, or 16 with
// kBatch16).
template <bool kBatch16>
__device__ __forceinline__ int count_above(const uint64_t *K, int n, uint64_t Ke) {
  int c = 0;
  if constexpr (kBatch16) {
#pragma unroll 1
    for (int j = 0; j < n; j += 16) {
      ulonglong2 q[8];
      load16(K + j, q);
      c += above16(q, Ke);
    }
  } else {
    int c1 = 0;
    for (int j = 0; j < n; j += 8) {
      const ulonglong2 q0 = *reinterpret_cast<const ulonglong2 *>(K + j);
      const ulonglong2 q1 = *reinterpret_cast<const ulonglong2 *>(K + j + 2);
      const ulonglong2 q2 = *reinterpret_cast<const ulonglong2 *>(K + j + 4);
      const ulonglong2 q3 = *reinterpret_cast<const ulonglong2 *>(K + j + 6);
      c += (q0.x > Ke) + (q0.y > Ke) + (q1.x > Ke) + (q1.y > Ke);
      c1 += (q2.x > Ke) + (q2.y > Ke) + (q3.x > Ke) + (q3.y > Ke);
    }
    c += c1;
  }
  return c;
}

template <bool kBatch16 = false>
__device__ void route_token_block(const float *l, int E, int k1, int k2, int32_t *ids, float *w,
                                  int32_t *ids_out, float *w_out, BlockRoute &S,
                                  bool wbf16 = false) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const bool valid = tid < E;
  const float lv = valid ? l[tid] : -INFINITY;
  const float wm = wave_max_dpp(lv);
  if (lane == 0) S.red[wv] = wm;
  __syncthreads();
  const float m = fmaxf(fmaxf(S.red[0], S.red[1]), fmaxf(S.red[2], S.red[3]));
  const float ex = valid ? exp_nonpos(lv - m) : 0.0f;
  const float ws = wave_sum_dpp(ex);
  __syncthreads();
  if (lane == 0) S.red[wv] = ws;
  __syncthreads();
  const float sum = (S.red[0] + S.red[1]) + (S.red[2] + S.red[3]);
  const float p = ex / sum;
  const uint32_t key = valid ? __float_as_uint(p) + 1u : 0u;
  S.K[tid] = ((uint64_t)key << 11) | (uint64_t)(2047 - tid);
  S.rank[tid] = 0;
  __syncthreads();
  int epow = 1, lg = 0;
  while (epow < E) {
    epow <<= 1;
    ++lg;
  }
  // element e is ranked by `split` threads, each over `chunk` keys of the
  // padded key array (keys past E are below every valid key, so they never
  // count)
  const int split = min(kBlockThreads / epow, epow);
  const int e = tid & (epow - 1), part = tid >> lg;
  const int chunk = epow / split;
  if (e < E && part < split) {
    const uint64_t Ke = S.K[e];
    const uint64_t *Kp = S.K + part * chunk;
    int cnt;
    if (chunk >= 16) {
      cnt = count_above<kBatch16>(Kp, chunk, Ke);
    } else {
      cnt = 0;
      for (int j = 0; j < chunk; ++j) cnt += Kp[j] > Ke ? 1 : 0;
    }
    if (cnt) atomicAdd(&S.rank[e], cnt);
  }
  __syncthreads();
  const bool renorm = k2 < E;
  const int R = renorm ? k2 : k1;
  if (valid) {
    const int r = S.rank[tid];
    if (r < R) {
      S.sp[r] = p;
      S.sid[r] = tid;
    }
  }
  __syncthreads();
  if (tid == 0) {
    // left to right in rank order; the loads run ahead of the adds
    float M = 0.0f;
    if (renorm) {
      int r = 0;
      for (; r + 8 <= R; r += 8) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = S.sp[r + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) M = M + v[q];
      }
      for (; r < R; ++r) M = M + S.sp[r];
    }
    S.M = M;
  }
  __syncthreads();
  if (tid < k1) {
    float wr = renorm ? S.sp[tid] / S.M : S.sp[tid];
    if (wbf16) wr = round_bf16(wr);
    ids[tid] = S.sid[tid];
    w[tid] = wr;
    if (ids_out) ids_out[tid] = S.sid[tid];
    if (w_out) w_out[tid] = wr;
  }
  __syncthreads();
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

// Route one token into LDS (s_ids, s_w: rank order), by the whole block
// (E <= 256, k1 <= 256) or by its first wave; wbf16 rounds the weights to
// bf16.
template <int V>
__device__ void route_into_lds(const float *l, int E, int k1, int k2, int32_t *s_ids, float *s_w,
                               BlockRoute &S, bool wbf16 = false) {
  // V = 8 and 16 serve E > 256 only, so their kernels carry no block route
  if constexpr (V * kWave <= kBlockThreads) {
    if (E <= kBlockThreads && k1 <= kBlockThreads) {
      route_token_block<(V <= 2)>(l, E, k1, k2, s_ids, s_w, nullptr, nullptr, S, wbf16);
      return;
    }
  }
  if (threadIdx.x < kWave) route_token<V>(l, E, k1, k2, s_ids, s_w, nullptr, nullptr, wbf16);
  __syncthreads();
}

}  // namespace moe
