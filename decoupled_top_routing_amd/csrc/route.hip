// Router logits, fp32 softmax, top-k2 ranking and the Eq. 2 weights.
//
// "Paper of the Week #3 - Half the FLOPs Is Not Half the Time":
//  - section "Ship It - Code of the Week": logits from a linear router,
//    probabilities from an fp32 softmax, the min(k2, E) most probable experts
//    in descending order, the first k1 of them activated;
//  - section "The Receipt", Eq. 2: w_i = p_i / (sum of the top-k2 p) for the
//    top-k1 experts; k2 >= E means the weights are the probabilities.
//
// One wavefront routes one token (route_device.hpp).  The softmax arithmetic
// is pinned down so that the ids and weights are reproducible bit for bit.
#include "common.hpp"
#include "kernels.hpp"
#include "route_device.hpp"

#pragma clang fp contract(off)

namespace moe {

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
