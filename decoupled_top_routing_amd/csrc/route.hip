// Router logits, fp32 softmax, top-k2 ranking and the Eq. 2 weights.
//
// "Paper of the Week #3 - Half the FLOPs Is Not Half the Time":
//  - section "Ship It - Code of the Week": logits from a linear router,
//    probabilities from an fp32 softmax, the min(k2, E) most probable experts
//    in descending order, the first k1 of them activated;
//  - section "The Receipt", Eq. 2: w_i = p_i / (sum of the top-k2 p) for the
//    top-k1 experts; k2 >= E means the weights are the probabilities.
//
// One wavefront routes one token.  The softmax arithmetic is pinned down so
// that the ids and weights are reproducible bit for bit (see route_token).
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

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
//     then a butterfly over lanes (xor 1, 2, ..., 32).  Both halves of every
//     node are added in the same order on every lane, and zero padding of a
//     power-of-two tree leaves its sum unchanged, so S equals the pairwise
//     sum over the next power of two >= E;
//  4. p = e / S (IEEE division);
//  5. R rounds of selection: each lane offers its best untaken expert (key =
//     bits of p + 1, larger p first, lower index first within the lane), the
//     wave takes the maximum key, and the lowest lane holding it wins; this
//     ranks by p descending, then index ascending.  R = min(k2, E), or k1 when
//     k2 >= E (no mass needed);
//  6. M = p_(0) + p_(1) + ... left to right over the min(k2, E) ranked values;
//     w_r = p_(r) / M, or p_(r) when k2 >= E.
// Rank r is held by lane r % 64 in slot r / 64 until the end.
template <int V>
__device__ void route_token(const float *__restrict__ l, int E, int k1, int k2,
                            int32_t *__restrict__ ids, float *__restrict__ w,
                            int32_t *__restrict__ ids2, float *__restrict__ w2) {
  const int lane = lane_id();
  float ex[V];
  float lmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane * V + j;
    ex[j] = e < E ? l[e] : -INFINITY;
    lmax = fmaxf(lmax, ex[j]);
  }
  const float m = wave_max(lmax);
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
  float S = s[0];
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) S = S + __shfl_xor(S, o);

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
    const uint32_t kmax = wave_max_u32(best);
    const uint64_t mask = __ballot(best == kmax);
    const int win = __ffsll((unsigned long long)mask) - 1;
    if (lane == win) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (j == bj) key[j] = 0u;
    }
    const int id = __shfl(lane * V + bj, win);
    const float pr = __uint_as_float(kmax - 1u);
    if (renorm) M = M + pr;
    if (r < k1 && lane == (r & (kWave - 1))) {
      const int q = r / kWave;
#pragma unroll
      for (int qq = 0; qq < V; ++qq)
        if (qq == q) {
          my_id[qq] = id;
          my_p[qq] = pr;
        }
    }
  }
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int r = q * kWave + lane;
    if (r < k1) {
      const float wr = renorm ? my_p[q] / M : my_p[q];
      ids[r] = my_id[q];
      w[r] = wr;
      if (ids2) ids2[r] = my_id[q];
      if (w2) w2[r] = wr;
    }
  }
}

template <int V>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int64_t T,
                                                    int E, int k1, int k2,
                                                    int32_t *__restrict__ ids,
                                                    float *__restrict__ w,
                                                    int32_t *__restrict__ ids2,
                                                    float *__restrict__ w2) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<V>(logits + t * E, E, k1, k2, ids + t * k1, w + t * k1,
                 ids2 ? ids2 + t * k1 : nullptr, w2 ? w2 + t * k1 : nullptr);
}

hipError_t launch_route(const float *logits, int64_t T, int E, int k1, int k2, int32_t *ids,
                        float *w, int32_t *ids2, float *w2, hipStream_t s) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2);
  else if (E <= 512)
    route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k1, k2, ids, w, ids2, w2);
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

template <typename XT>
hipError_t launch_router(const XT *x, int64_t T, int H, const float *Wr, const float *br, int E,
                         float *logits, float *logits2, hipStream_t s) {
  const dim3 grid((unsigned)(((E + 3) / 4) * ((T + 7) / 8))), block(256);
  router_kernel<XT><<<grid, block, 0, s>>>(x, T, H, Wr, br, E, logits, logits2);
  return hipGetLastError();
}

template hipError_t launch_router<float>(const float *, int64_t, int, const float *,
                                         const float *, int, float *, float *, hipStream_t);
template hipError_t launch_router<bf16_t>(const bf16_t *, int64_t, int, const float *,
                                          const float *, int, float *, float *, hipStream_t);

}  // namespace moe
