// The routed MoE layer for ONE token (batch-1 decode) in two launches.
//
// What it computes: router logits, the fp32 softmax / top-k2 / Eq. 2 route
// of "Paper of the Week #3 - Half the FLOPs Is Not Half the Time" (section
// "The Receipt", Eq. 2; section "Ship It - Code of the Week"), and for each
// activated expert the gated MLP of "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data" (section 2 "Background"), weighted and
// summed.
//
// Launch 1 (front), workgroups in block-index order:
//   R   [0, n_r)        wave e computes logit e and publishes it as a tagged
//                       word (sync.hpp);
//   P   n_r             stages the E tagged logits, routes the token, writes
//                       ids, w and the plan, and publishes (expert, weight)
//                       of the activated experts, ascending by expert, as
//                       tagged words in kRepP copies;
//   GU  [n_r+1, ..)     (activated expert u, block of channels): waits for
//                       the two words of u, streams the gate and up rows once
//                       and writes a[u, c] = silu(g) * up * w_u.
// A block only waits for blocks of smaller index, which the hardware
// dispatched before it.  Launch 2 (down) computes each output row over every
// activated expert, y[h] = sum_u Wd[e_u, h, :] . a[u, :], in ascending expert
// order, and advances the workspace's epoch: the tags of launch 1 are made
// from the epoch, and launch 2 starts only after every block of launch 1 has
// finished with them.
#include "common.hpp"
#include "kernels.hpp"
#include "route_device.hpp"
#include "sync.hpp"

namespace moe {
namespace b1 {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRepP = 16;  // copies of the published route

struct Args {
  const void *x;
  const float *Wr;
  const float *br;
  const void *Wg;
  const void *Wu;
  float *logits_out;
  int32_t *ids_out;
  float *w_out;
  int32_t *sync;
  uint64_t *tl;     // E tagged logits
  uint64_t *tp;     // kRepP copies of 2*k1 tagged words (expert, weight)
  int64_t tp_rep;   // copy stride in words
  int32_t *ids;
  float *w;
  int32_t *plan;
  float *abuf;      // [k1, I]: row u = activated expert u (ascending)
  int H, E, I, k1, k2, n_r, n_cb;
};

// gate and up rows of CPW channels per wave (NCH 16-byte chunks per lane of
// a row, all 2*CPW*NCH loads in flight before any arithmetic), dotted with x.
template <typename WT, typename XT, int NCH, int CPW>
__device__ void gateup_rows(const Args &a, int u, int e, float wt, int c0) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int lane = lane_id();
  const WT *Wg = static_cast<const WT *>(a.Wg);
  const WT *Wu = static_cast<const WT *>(a.Wu);
  const XT *x = static_cast<const XT *>(a.x);
  uint4 gq[CPW][NCH], uq[CPW][NCH];
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) {
    const int c = min(c0 + ci, a.I - 1);
    const WT *grow = Wg + ((int64_t)e * a.I + c) * a.H;
    const WT *urow = Wu + ((int64_t)e * a.I + c) * a.H;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      gq[ci][j] = ld16_stream(grow + (j * kWave + lane) * NW);
      uq[ci][j] = ld16_stream(urow + (j * kWave + lane) * NW);
    }
  }
  float ag[CPW], au[CPW];
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) ag[ci] = au[ci] = 0.0f;
  if constexpr (sizeof(WT) == 2 && sizeof(XT) == 2) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const uint4 xq = ld16(x + (j * kWave + lane) * NW);
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        ag[ci] = dot2_bf16(gq[ci][j].x, xq.x, ag[ci]);
        ag[ci] = dot2_bf16(gq[ci][j].y, xq.y, ag[ci]);
        ag[ci] = dot2_bf16(gq[ci][j].z, xq.z, ag[ci]);
        ag[ci] = dot2_bf16(gq[ci][j].w, xq.w, ag[ci]);
        au[ci] = dot2_bf16(uq[ci][j].x, xq.x, au[ci]);
        au[ci] = dot2_bf16(uq[ci][j].y, xq.y, au[ci]);
        au[ci] = dot2_bf16(uq[ci][j].z, xq.z, au[ci]);
        au[ci] = dot2_bf16(uq[ci][j].w, xq.w, au[ci]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float xv[NW];
#pragma unroll
      for (int k = 0; k < NW; ++k) xv[k] = Elem<XT>::load1(x + (j * kWave + lane) * NW + k);
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        float gv[NW], uv[NW];
        Elem<WT>::widen(gq[ci][j], gv);
        Elem<WT>::widen(uq[ci][j], uv);
#pragma unroll
        for (int k = 0; k < NW; ++k) {
          ag[ci] = __builtin_fmaf(gv[k], xv[k], ag[ci]);
          au[ci] = __builtin_fmaf(uv[k], xv[k], au[ci]);
        }
      }
    }
  }
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) {
    const float g = wave_sum_dpp(ag[ci]);
    const float up = wave_sum_dpp(au[ci]);
    const int c = c0 + ci;
    if (lane == 0 && c < a.I) a.abuf[(int64_t)u * a.I + c] = silu(g) * up * wt;
  }
}

template <typename WT, typename XT, int NCHR, int V, int NCH, int CPW>
__global__ __launch_bounds__(kThreads) void front_kernel(Args a) {
  __shared__ float sl[kMaxExperts];
  __shared__ int32_t s_ids[kMaxExperts];
  __shared__ float s_w[kMaxExperts];
  __shared__ BlockRoute S;
  __shared__ int s_e;
  __shared__ float s_wt;
  const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const uint32_t tag = call_tag((uint32_t)coh_ld(a.sync + kEpochWord));
  int32_t *err = a.sync + kErrorWord;
  if (b < a.n_r) {
    // ---- router: one expert per wave
    const int e = b * kWaves + wv;
    if (e >= a.E) return;
    const XT *x = static_cast<const XT *>(a.x);
    const float *wrow = a.Wr + (int64_t)e * a.H;
    float wr[NCHR][4];
#pragma unroll
    for (int j = 0; j < NCHR; ++j)
      Elem<float>::widen(ld16_stream(wrow + (j * kWave + lane) * 4), wr[j]);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NCHR; ++j) {
      const int h = (j * kWave + lane) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(wr[j][k], Elem<XT>::load1(x + h + k), acc);
    }
    const float s = wave_sum_dpp(acc) + (a.br ? a.br[e] : 0.0f);
    if (lane == 0) {
      coh_st(a.tl + e, tagged(tag, s));
      if (a.logits_out) a.logits_out[e] = s;
    }
    return;
  }
  if (b == a.n_r) {
    // ---- route and plan
    stage_tagged<kMaxExperts / kSyncThreads>(sl, a.E, [&](int i) { return a.tl + i; }, tag, err);
    route_into_lds<V>(sl, a.E, a.k1, a.k2, s_ids, s_w, S);
    for (int r = tid; r < a.k1; r += kThreads) {
      a.ids[r] = s_ids[r];
      a.w[r] = s_w[r];
      if (a.ids_out) a.ids_out[r] = s_ids[r];
      if (a.w_out) a.w_out[r] = s_w[r];
    }
    if (tid < kWave) {
      // lane r holds slot r; u = its expert's place among the activated ones
      const int n = a.k1;
      const int e = lane < n ? s_ids[lane] : 0x7FFFFFFF;
      // lane L writes slot L % n into copy L / n, then the next copies
      const int r = lane % n;
      const int er = s_ids[r];
      int u = 0;
      for (int j = 0; j < n; ++j) u += __builtin_amdgcn_readlane(e, j) < er;
      const uint64_t we = tagged(tag, __int_as_float(er));
      const uint64_t ww = tagged(tag, s_w[r]);
      const int per = kWave / n;
      if (lane < per * n) {
        for (int c = lane / n; c < kRepP; c += per) {
          coh_st(a.tp + c * a.tp_rep + 2 * u, we);
          coh_st(a.tp + c * a.tp_rep + 2 * u + 1, ww);
        }
      }
      wave_plan(e, n, a.E, a.plan);
    }
    return;
  }
  // ---- gate/up of (activated expert u, block of channels)
  const int item = b - a.n_r - 1;
  const int u = item / a.n_cb, cb = item - u * a.n_cb;
  if (tid < kWave) {
    const uint64_t *tp = a.tp + (item % kRepP) * a.tp_rep + 2 * u;
    uint64_t we = coh_ld(tp), ww = coh_ld(tp + 1);
    uint32_t spins = 0;
    while ((uint32_t)(we >> 32) != tag || (uint32_t)(ww >> 32) != tag) {
      if (++spins > kSpinLimit) {
        if (lane == 0) coh_st(err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      if ((uint32_t)(we >> 32) != tag) we = coh_ld(tp);
      if ((uint32_t)(ww >> 32) != tag) ww = coh_ld(tp + 1);
    }
    if (lane == 0) {
      // a timed-out wait leaves any value here: keep the index in range
      s_e = min(max(__float_as_int(__uint_as_float((uint32_t)we)), 0), a.E - 1);
      s_wt = __uint_as_float((uint32_t)ww);
    }
  }
  __syncthreads();
  gateup_rows<WT, XT, NCH, CPW>(a, u, s_e, s_wt, (cb * kWaves + wv) * CPW);
}

// ---- launch 2: y[h] = sum_u Wd[e_u, h, :] . a[u, :]; one row per wave, in
// rounds of kPF experts: the block loads the round's a rows (issued first,
// so waiting for them does not wait for the down rows), then every wave
// issues its kPF down rows, stages a in LDS and accumulates.
constexpr int kPF = 8;
constexpr int kMaxI = 1024;

template <typename WT, typename XT, int NCD>
__global__ __launch_bounds__(kThreads) void down_kernel(const WT *__restrict__ Wd, int H, int I,
                                                        const int32_t *__restrict__ plan, int U,
                                                        const float *__restrict__ abuf,
                                                        XT *__restrict__ y,
                                                        int32_t *__restrict__ sync) {
  constexpr int NW = Elem<WT>::kPer16B;
  constexpr int kA4 = kPF * kMaxI / 4 / kThreads;  // float4 of a per thread per round
  __shared__ float s_a[kPF * kMaxI];
  if (blockIdx.x == 0 && threadIdx.x == 0) coh_st(sync + kEpochWord, coh_ld(sync + kEpochWord) + 1);
  const int tid = threadIdx.x, lane = lane_id();
  const int h = min(blockIdx.x * kWaves + (tid >> 6), H - 1);
  const int32_t *uniq = plan + 4;
  const int nch = I / NW;
  float acc = 0.0f;
  for (int ub = 0; ub < U; ub += kPF) {
    const int nu = min(kPF, U - ub);
    const int n4 = nu * I / 4;
    const float *ab = abuf + (int64_t)ub * I;
    uint4 aq[kA4];
#pragma unroll
    for (int k = 0; k < kA4; ++k) {
      const int i = tid + k * kThreads;
      if (i < n4) aq[k] = ld16(ab + 4 * i);
    }
    uint4 dq[kPF][NCD];
#pragma unroll
    for (int s = 0; s < kPF; ++s) {
      if (s < nu) {
        const WT *drow = Wd + ((int64_t)uniq[ub + s] * H + h) * I;
#pragma unroll
        for (int j = 0; j < NCD; ++j) {
          const int ch = j * kWave + lane;
          dq[s][j] = ch < nch ? ld16_stream(drow + ch * NW) : make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kA4; ++k) {
      const int i = tid + k * kThreads;
      if (i < n4) *reinterpret_cast<uint4 *>(&s_a[4 * i]) = aq[k];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kPF; ++s) {
      if (s < nu) {
        const float *arow = s_a + s * I;
#pragma unroll
        for (int j = 0; j < NCD; ++j) {
          const int ch = j * kWave + lane;
          if (ch < nch) {
            float av[NW], dv[NW];
            Elem<float>::widen(*reinterpret_cast<const uint4 *>(arow + ch * NW), av);
            if constexpr (NW == 8)
              Elem<float>::widen(*reinterpret_cast<const uint4 *>(arow + ch * NW + 4), av + 4);
            Elem<WT>::widen(dq[s][j], dv);
#pragma unroll
            for (int k = 0; k < NW; ++k) acc = __builtin_fmaf(dv[k], av[k], acc);
          }
        }
      }
    }
    __syncthreads();
  }
  acc = wave_sum_dpp(acc);
  if (lane == 0 && blockIdx.x * kWaves + (tid >> 6) < H) Elem<XT>::store1(y + h, acc);
}

}  // namespace b1

// Shapes the two-launch path takes: the router row and the gate/up row in
// 1..16 / 1..8 chunks of 16 bytes per lane, the down row in at most 2 per
// lane, k1 <= 64.
bool decode_b1_supported(int H, int I, int k1, bool bf16) {
  const int esz = bf16 ? 2 : 4;
  if (k1 > kWave || H % (4 * kWave) != 0 || (H * esz) % (16 * kWave) != 0) return false;
  const int nchr = H / (4 * kWave), nch = H * esz / (16 * kWave);
  if (!(nchr == 1 || nchr == 2 || nchr == 4 || nchr == 8 || nchr == 16)) return false;
  if (!(nch == 1 || nch == 2 || nch == 4 || nch == 8)) return false;
  return I * esz / 16 <= 2 * kWave && I <= b1::kMaxI;
}

size_t decode_b1_tagged_bytes(int E, int k1, int64_t *tp_offset, int64_t *tp_rep_words) {
  const size_t tl = ((size_t)E * 8 + 255) & ~(size_t)255;
  const size_t rep = ((((size_t)2 * k1 * 8 + 4095) & ~(size_t)4095) + 1280);
  *tp_offset = (int64_t)tl;
  *tp_rep_words = (int64_t)(rep / 8);
  return tl + b1::kRepP * rep;
}

template <typename WT, typename XT, int NCHR, int V>
static void launch_front_nch(b1::Args &a, int nch, hipStream_t s) {
  // 4 gate/up row pairs... 16 chunk loads per lane in flight
  auto go = [&](auto kern, int cpw) {
    a.n_cb = (a.I + b1::kWaves * cpw - 1) / (b1::kWaves * cpw);
    const int grid = a.n_r + 1 + a.k1 * a.n_cb;
    kern<<<dim3((unsigned)grid), dim3(b1::kThreads), 0, s>>>(a);
  };
  if (nch == 1) go(b1::front_kernel<WT, XT, NCHR, V, 1, 8>, 8);
  else if (nch == 2) go(b1::front_kernel<WT, XT, NCHR, V, 2, 4>, 4);
  else if (nch == 4) go(b1::front_kernel<WT, XT, NCHR, V, 4, 2>, 2);
  else go(b1::front_kernel<WT, XT, NCHR, V, 8, 1>, 1);
}

template <typename WT, typename XT, int V>
static void launch_front_v(b1::Args &a, int nchr, int nch, hipStream_t s) {
  switch (nchr) {
    case 1: launch_front_nch<WT, XT, 1, V>(a, nch, s); break;
    case 2: launch_front_nch<WT, XT, 2, V>(a, nch, s); break;
    case 4: launch_front_nch<WT, XT, 4, V>(a, nch, s); break;
    case 8: launch_front_nch<WT, XT, 8, V>(a, nch, s); break;
    default: launch_front_nch<WT, XT, 16, V>(a, nch, s); break;
  }
}

template <typename WT, typename XT>
hipError_t launch_decode_b1_front(const XT *x, int H, const float *Wr, const float *br, int E,
                                  const WT *Wg, const WT *Wu, int I, int k1, int k2,
                                  float *logits_out, int32_t *ids_out, float *w_out,
                                  int32_t *sync, char *tagged, int32_t *ids, float *w,
                                  int32_t *plan, float *abuf, hipStream_t s) {
  b1::Args a;
  int64_t tp_off = 0, tp_rep = 0;
  decode_b1_tagged_bytes(E, k1, &tp_off, &tp_rep);
  a.x = x;
  a.Wr = Wr;
  a.br = br;
  a.Wg = Wg;
  a.Wu = Wu;
  a.logits_out = logits_out;
  a.ids_out = ids_out;
  a.w_out = w_out;
  a.sync = sync;
  a.tl = reinterpret_cast<uint64_t *>(tagged);
  a.tp = reinterpret_cast<uint64_t *>(tagged + tp_off);
  a.tp_rep = tp_rep;
  a.ids = ids;
  a.w = w;
  a.plan = plan;
  a.abuf = abuf;
  a.H = H;
  a.E = E;
  a.I = I;
  a.k1 = k1;
  a.k2 = k2;
  a.n_r = (E + b1::kWaves - 1) / b1::kWaves;
  a.n_cb = 0;
  constexpr int esz = sizeof(WT);
  const int nchr = H / (4 * kWave), nch = H * esz / (16 * kWave);
  if (E <= 64) launch_front_v<WT, XT, 1>(a, nchr, nch, s);
  else if (E <= 128) launch_front_v<WT, XT, 2>(a, nchr, nch, s);
  else if (E <= 256) launch_front_v<WT, XT, 4>(a, nchr, nch, s);
  else if (E <= 512) launch_front_v<WT, XT, 8>(a, nchr, nch, s);
  else launch_front_v<WT, XT, 16>(a, nchr, nch, s);
  return hipGetLastError();
}

template <typename WT, typename XT>
hipError_t launch_decode_b1_down(const WT *Wd, int H, int I, int k1, const int32_t *plan,
                                 const float *abuf, XT *y, int32_t *sync, hipStream_t s) {
  constexpr int esz = sizeof(WT);
  const int ncd = (I * esz / 16 + kWave - 1) / kWave;
  const dim3 grid((unsigned)((H + b1::kWaves - 1) / b1::kWaves)), block(b1::kThreads);
  if (ncd == 1)
    b1::down_kernel<WT, XT, 1><<<grid, block, 0, s>>>(Wd, H, I, plan, k1, abuf, y, sync);
  else
    b1::down_kernel<WT, XT, 2><<<grid, block, 0, s>>>(Wd, H, I, plan, k1, abuf, y, sync);
  return hipGetLastError();
}

#define MOE_INST_B1(WT, XT)                                                                    \
  template hipError_t launch_decode_b1_front<WT, XT>(                                         \
      const XT *, int, const float *, const float *, int, const WT *, const WT *, int, int, int, \
      float *, int32_t *, float *, int32_t *, char *, int32_t *, float *, int32_t *, float *,    \
      hipStream_t);                                                                            \
  template hipError_t launch_decode_b1_down<WT, XT>(const WT *, int, int, int, const int32_t *, \
                                                    const float *, XT *, int32_t *, hipStream_t);
MOE_INST_B1(float, float)
MOE_INST_B1(bf16_t, bf16_t)

}  // namespace moe
