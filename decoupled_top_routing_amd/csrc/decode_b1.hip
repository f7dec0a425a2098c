// The routed MoE layer for ONE token (batch-1 decode) in one launch.
//
// What it computes: router logits, the fp32 softmax / top-k2 / Eq. 2 route
// of "Paper of the Week #3 - Half the FLOPs Is Not Half the Time" (section
// "The Receipt", Eq. 2; section "Ship It - Code of the Week"), and for each
// activated expert the gated MLP of "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data" (section 2 "Background"), weighted and
// summed in ascending expert order.
//
// Workgroups, in block-index order (a block only waits for blocks of smaller
// index, which the hardware dispatched before it, so the kernel cannot
// deadlock whatever the occupancy):
//   R   [0, n_r)          logit e, published as a tagged word (sync.hpp):
//                         block e's four waves each take a quarter of the
//                         router row when a lane holds at least four 16-byte
//                         chunks of it (the loads spread over E compute
//                         units), else wave e of the range takes the row;
//   P   n_r               sets the activated experts' completion counters to
//                         (tag, 0), stages the E tagged logits and routes the
//                         token; it publishes the activated experts,
//                         ascending by expert, in kRepP copies as soon as
//                         the top-k1 set is known (one wave, E <= 256), then
//                         their Eq. 2 weights once the top-k2 mass is
//                         summed;
//   GU  [.., +(k1+m)*n_cb) (expert u, block of channels): the first m*n_cb
//                         blocks are the shared expert's, its Is = m*I
//                         channels as m pieces u = k1..k1+m-1 of I channels
//                         (each channel owns a gate row, an up row and a down
//                         column, so the pieces add up to the whole); they
//                         need no route and stream while it is computed.
//                         A routed block waits for the expert of its u.
//                         Each streams the gate and up rows once, stores
//                         a[u, c] = silu(g) * up (times the gate factor for
//                         a shared piece) device-coherently, then adds 1 to
//                         u's counter (a shared block first waits for the
//                         route, which is published after the counters are
//                         set); the block that completes the count
//                         publishes "u complete" in every copy;
//   D   [.., +n_d)        (block of four output rows): marks itself started,
//                         waits for the activated experts, issues their down
//                         rows and the shared pieces' (they stream while
//                         gate/up runs), reads the Eq. 2 weights w_u, waits
//                         until every slot is complete, stages a in LDS and
//                         writes y[h] = sum_u w_u (Wd[e_u, h, :] . a[u, :])
//                         (+ the shared pieces' Sd[h, piece] . a[u, :]).
// The shared expert ("Channel Selection for Mixture-of-Experts Decoding Needs
// No Calibration Data", appendix B: shared experts always run in full) is
// added with the factor sigmoid(x . sg), or 1 without a gate vector sg.
// The gate/up block that completes the last expert advances the workspace
// epoch, the source of the call's tags, once every D block has marked itself
// started (by then every block of the call has read the epoch).
// With the bf16 router (the router method on a bf16 model) Wr is bf16, the
// R blocks round each logit to bf16 and P rounds each weight to bf16.
// The channel activations a are stored as bf16 when the weights are bf16
// (the down projection reads bf16 weights; a relative rounding of 2^-9) and
// as fp32 otherwise.
#include "common.hpp"
#include "kernels.hpp"
#include "route_device.hpp"
#include "sync.hpp"

namespace moe {
namespace b1 {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRepP = kB1RepP;    // copies of the published route
constexpr int kPF = 8;            // activated experts whose down rows are in flight per wave
constexpr int kCntStride = kB1CntStride;  // 64-bit words between two counters (128 B)
constexpr int kLdsBytes = 24576;  // staged channel activations of one D block
// waves that share one router row (NCHR 16-byte chunks of fp32 per lane):
// a block per expert spreads the router's loads over E compute units
template <int NCHR>
constexpr int kRouterRowSplit = NCHR % kWaves == 0 ? kWaves : 1;

struct Args {
  const void *x;
  const void *Wr;     // fp32, or bf16 with router_bf16
  const float *br;
  const void *Wg;
  const void *Wu;
  const void *Wd;
  void *y;
  float *logits_out;
  int32_t *ids_out;
  float *w_out;
  int32_t *sync;
  uint64_t *tl;       // E tagged logits
  uint64_t *tp;       // kRepP copies of 3*k1 tagged words: the activated
                      // experts, their weights, then one "complete" word each
  int64_t tp_rep;     // copy stride in words
  uint64_t *cnt;      // k1 + m + 1 counters (tag << 32 | count), kCntStride
                      // apart: blocks done per expert u, then experts complete
  uint64_t *started;  // n_d tagged words
  void *abuf;         // [k1 + m, I] channel activations (bf16 or fp32), row u
  const void *Sg, *Su, *Sd;  // shared expert [Is, H], [Is, H], [H, Is] (m > 0)
  const float *sgw;   // shared gate vector [H], or NULL (factor 1)
  int m, Is;          // shared pieces (Is / I, 0 without a shared expert)
  int H, E, I, k1, k2, n_r, n_cb, n_gu, n_d;
  uint32_t spin_limit;  // re-reads before a wait gives up
  bool router_bf16;   // bf16 router: bf16 Wr, logits and weights rounded to bf16
  bool withhold_route;  // test hook: the route is never published, so every
                        // wait for it gives up (outputs unspecified, error set)
};

// LDS of a block: the route block's arrays or a D block's staged activations
union Lds {
  struct {
    float sl[kMaxExperts];
    int32_t s_ids[kMaxExperts];
    float s_w[kMaxExperts];
    BlockRoute S;
  } r;
  uint64_t a[kLdsBytes / 8];
};

// bytes of one stored channel activation
template <typename WT>
constexpr int kABytes = sizeof(WT) == 2 ? 2 : 4;

// Wait until the tagged words p[0..n) (n <= kWave, one per lane) carry tag;
// lane i returns word i.  At most `limit` re-reads; SLEEP is the pause
// between two of them.
template <int SLEEP = 1>
__device__ uint64_t await_lane(const uint64_t *p, int n, uint32_t tag, int32_t *err,
                               uint32_t limit) {
  const int lane = lane_id();
  uint64_t w = lane < n ? coh_ld(p + lane) : ((uint64_t)tag << 32);
  uint32_t spins = 0;
  while (__ballot((uint32_t)(w >> 32) != tag)) {
    if (++spins > limit) {
      if (lane == 0) coh_st(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(SLEEP);
    if ((uint32_t)(w >> 32) != tag) w = coh_ld(p + lane);
  }
  return w;
}

// gate and up rows of CPW channels per wave (NCH 16-byte chunks per lane of
// a row, all 2*CPW*NCH loads in flight before any arithmetic), dotted with x;
// the activations, scaled by weight() (called once the dot products are
// done), are stored device-coherently.  Wg and Wu point at the first of the
// I rows of expert (or shared piece) u.
template <typename WT, typename XT, int NCH, int CPW, typename WeightFn>
__device__ void gateup_rows(const Args &a, int u, const WT *Wg, const WT *Wu, int c0,
                            WeightFn &&weight) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int lane = lane_id();
  const XT *x = static_cast<const XT *>(a.x);
  uint4 gq[CPW][NCH], uq[CPW][NCH];
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) {
    const int c = min(c0 + ci, a.I - 1);
    const WT *grow = Wg + (int64_t)c * a.H;
    const WT *urow = Wu + (int64_t)c * a.H;
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
  const float wt = weight();
  float av[CPW];
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) av[ci] = silu(wave_sum_dpp(ag[ci])) * wave_sum_dpp(au[ci]) * wt;
  if (lane != 0) return;
  if constexpr (sizeof(WT) == 2) {
    uint16_t *ab = static_cast<uint16_t *>(a.abuf) + (int64_t)u * a.I;
    if constexpr (CPW % 2 == 0) {
#pragma unroll
      for (int ci = 0; ci < CPW; ci += 2)
        if (c0 + ci < a.I)
          coh_st(reinterpret_cast<uint32_t *>(ab + c0 + ci),
                 f32_to_bf16_bits(av[ci]) | (f32_to_bf16_bits(av[ci + 1]) << 16));
    } else {
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci)
        if (c0 + ci < a.I) coh_st(ab + c0 + ci, (uint16_t)f32_to_bf16_bits(av[ci]));
    }
  } else {
    float *ab = static_cast<float *>(a.abuf) + (int64_t)u * a.I;
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci)
      if (c0 + ci < a.I) coh_st(ab + c0 + ci, av[ci]);
  }
}

// One output row per wave: y[h] = sum over the activated experts, ascending,
// of Wd[e_u, h, :] . a[u, :].
template <typename WT, typename XT, int NCD>
__device__ void down_rows(const Args &a, Lds &L, int *s_uniq, float *s_ws, uint32_t *s_new,
                          uint32_t tag, int d) {
  constexpr int NW = Elem<WT>::kPer16B;
  constexpr int AB = kABytes<WT>;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  int32_t *err = a.sync + kErrorWord;
  // mark this block started (it has read the epoch)
  if (tid == 0) coh_st(a.started + d, (uint64_t)tag << 32);
  // the activated experts, ascending, then the shared pieces
  if (wv == 0) {
    const uint64_t w = await_lane(a.tp + (d % kRepP) * a.tp_rep, a.k1, tag, err, a.spin_limit);
    if (lane < a.k1)
      s_uniq[lane] = min(max(__float_as_int(__uint_as_float((uint32_t)w)), 0), a.E - 1);
    if (lane < a.m) s_uniq[a.k1 + lane] = lane;
  }
  __syncthreads();
  const int h = min(d * kWaves + wv, a.H - 1);
  const WT *Wd = static_cast<const WT *>(a.Wd);
  const WT *Sd = static_cast<const WT *>(a.Sd);
  const int nch = a.I / NW;
  const int U = a.k1 + a.m;
  // the slots' Eq. 2 weights (1 for the shared pieces, whose factor is in
  // their activations), read by wave 0 once its down rows are issued; the
  // barriers of the loops below publish them to the block
  auto await_weights = [&]() {
    if (wv == 0) {
      const uint64_t w =
          await_lane(a.tp + (d % kRepP) * a.tp_rep + a.k1, a.k1, tag, err, a.spin_limit);
      if (lane < a.k1) s_ws[lane] = __uint_as_float((uint32_t)w);
      if (lane < a.m) s_ws[a.k1 + lane] = 1.0f;
    }
  };
  float acc = 0.0f;
  // Wd[e_s, h, :] . a[s, :] from the staged activations of slot s (one lane's share)
  auto dot_slot = [&](const uint4 (&dqs)[NCD], int s, float v) {
    const char *sa = reinterpret_cast<const char *>(L.a);
#pragma unroll
    for (int j = 0; j < NCD; ++j) {
      const int ch = j * kWave + lane;
      if (ch < nch) {
        if constexpr (sizeof(WT) == 2) {
          const uint4 aq = *reinterpret_cast<const uint4 *>(sa + ((int64_t)s * a.I + ch * NW) * AB);
          v = dot2_bf16(dqs[j].x, aq.x, v);
          v = dot2_bf16(dqs[j].y, aq.y, v);
          v = dot2_bf16(dqs[j].z, aq.z, v);
          v = dot2_bf16(dqs[j].w, aq.w, v);
        } else {
          float dv[NW], av[NW];
          Elem<WT>::widen(dqs[j], dv);
          Elem<float>::widen(
              *reinterpret_cast<const uint4 *>(sa + ((int64_t)s * a.I + ch * NW) * AB), av);
#pragma unroll
          for (int k = 0; k < NW; ++k) v = __builtin_fmaf(dv[k], av[k], v);
        }
      }
    }
    return v;
  };
  if (U <= kPF) {
    // One round: each expert (or shared piece) is staged and multiplied as
    // soon as it completes, so only the last one to complete is left when it
    // does.  Per-slot partial sums are added in slot order at the end, so y
    // does not depend on the order of completion.
    uint4 dq[kPF][NCD];
#pragma unroll
    for (int s = 0; s < kPF; ++s) {
      if (s < U) {
        const WT *drow = s < a.k1 ? Wd + ((int64_t)s_uniq[s] * a.H + h) * a.I
                                  : Sd + (int64_t)h * a.Is + (int64_t)s_uniq[s] * a.I;
#pragma unroll
        for (int j = 0; j < NCD; ++j) {
          const int ch = j * kWave + lane;
          dq[s][j] = ch < nch ? ld16_stream(drow + ch * NW) : make_uint4(0, 0, 0, 0);
        }
      }
    }
    await_weights();
    float part[kPF];
#pragma unroll
    for (int s = 0; s < kPF; ++s) part[s] = 0.0f;
    const uint64_t *cw = a.tp + (d % kRepP) * a.tp_rep + 2 * a.k1;
    const uint32_t all = (1u << U) - 1u;
    const int row8 = a.I * AB / 8;  // 8-byte words of one slot's activations
    uint32_t done = 0u;
    while (done != all) {
      if (wv == 0) {
        // wait until at least one more of the slots not yet done is complete
        const bool open = lane < U && !((done >> lane) & 1u);
        uint64_t ready = 0;
        uint32_t spins = 0;
        while (true) {
          const uint64_t w = open ? coh_ld(cw + lane) : 0ull;
          ready = __ballot(open && (uint32_t)(w >> 32) == tag);
          if (ready) break;
          if (++spins > a.spin_limit) {
            if (lane == 0) coh_st(err, 1);
            ready = all & ~done;  // give up waiting; the call reports an error
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        if (lane == 0) *s_new = (uint32_t)ready;
      }
      __syncthreads();
      const uint32_t nw = *s_new;
      // stage the newly complete slots' activations (device-coherent loads)
      for (uint32_t m = nw; m; m &= m - 1) {
        const int s = __builtin_ctz(m);
        const uint64_t *src = reinterpret_cast<const uint64_t *>(
            static_cast<const char *>(a.abuf) + (int64_t)s * a.I * AB);
        for (int i = tid; i < row8; i += kThreads) L.a[s * row8 + i] = coh_ld(src + i);
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kPF; ++s)
        if ((nw >> s) & 1u) part[s] = dot_slot(dq[s], s, part[s]);
      done |= nw;
      __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < kPF; ++s)
      if (s < U) acc = acc + s_ws[s] * part[s];
  }
  for (int ub = 0; U > kPF && ub < U; ub += kPF) {
    const int nu = min(kPF, U - ub);
    uint4 dq[kPF][NCD];
#pragma unroll
    for (int s = 0; s < kPF; ++s) {
      if (s < nu) {
        const int uu = ub + s;
        const WT *drow = uu < a.k1 ? Wd + ((int64_t)s_uniq[uu] * a.H + h) * a.I
                                   : Sd + (int64_t)h * a.Is + (int64_t)s_uniq[uu] * a.I;
#pragma unroll
        for (int j = 0; j < NCD; ++j) {
          const int ch = j * kWave + lane;
          dq[s][j] = ch < nch ? ld16_stream(drow + ch * NW) : make_uint4(0, 0, 0, 0);
        }
      }
    }
    if (ub == 0) {
      await_weights();
      // every activated expert's and shared piece's activations are stored
      if (wv == 0) await_lane<4>(a.tp + (d % kRepP) * a.tp_rep + 2 * a.k1, U, tag, err, a.spin_limit);
      __syncthreads();
    }
    // stage this round's activations (device-coherent 8-byte loads)
    const int nw8 = nu * a.I * AB / 8;
    const uint64_t *src = reinterpret_cast<const uint64_t *>(
        static_cast<const char *>(a.abuf) + (int64_t)ub * a.I * AB);
    for (int i = tid; i < nw8; i += kThreads) L.a[i] = coh_ld(src + i);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kPF; ++s)
      if (s < nu) acc = acc + s_ws[ub + s] * dot_slot(dq[s], s, 0.0f);
    __syncthreads();
  }
  acc = wave_sum_dpp(acc);
  if (lane == 0 && d * kWaves + wv < a.H) Elem<XT>::store1(static_cast<XT *>(a.y) + h, acc);
}

template <typename WT, typename XT, int NCHR, int V, int NCH, int CPW, int NCD>
__global__ __launch_bounds__(kThreads) void layer_kernel(Args a) {
  __shared__ Lds L;
  __shared__ int s_uniq[kWave];
  __shared__ float s_ws[kWave];
  __shared__ int s_e, s_last;
  __shared__ float s_wt;
  __shared__ float s_red[kWaves];
  __shared__ uint32_t s_new;
  const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const uint32_t tag_epoch = (uint32_t)coh_ld(a.sync + kEpochWord);
  const uint32_t tag = call_tag(tag_epoch);
  int32_t *err = a.sync + kErrorWord;
  if (b < a.n_r) {
    // ---- router: one expert per block, each wave a quarter of its row (a
    // row of at least 4 chunks per lane), else one expert per wave
    constexpr int RS = kRouterRowSplit<NCHR>;
    constexpr int NCW = NCHR / RS;  // 16-byte (fp32) chunks per lane
    const int e = RS > 1 ? b : b * kWaves + wv;
    if (e >= a.E) return;  // uniform across the block when RS > 1
    const int j0 = RS > 1 ? wv * NCW : 0;
    const XT *x = static_cast<const XT *>(a.x);
    float wr[NCW][4];
    if (a.router_bf16) {
      const uint16_t *wrow = static_cast<const uint16_t *>(a.Wr) + (int64_t)e * a.H;
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        const uint2 q = *reinterpret_cast<const uint2 *>(wrow + ((j0 + j) * kWave + lane) * 4);
        wr[j][0] = bf16_lo(q.x);
        wr[j][1] = bf16_hi(q.x);
        wr[j][2] = bf16_lo(q.y);
        wr[j][3] = bf16_hi(q.y);
      }
    } else {
      const float *wrow = static_cast<const float *>(a.Wr) + (int64_t)e * a.H;
#pragma unroll
      for (int j = 0; j < NCW; ++j)
        Elem<float>::widen(ld16_stream(wrow + ((j0 + j) * kWave + lane) * 4), wr[j]);
    }
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const int h = ((j0 + j) * kWave + lane) * 4;
      float xv[4];
      if constexpr (sizeof(XT) == 2) {
        const uint2 q = *reinterpret_cast<const uint2 *>(x + h);
        xv[0] = bf16_lo(q.x);
        xv[1] = bf16_hi(q.x);
        xv[2] = bf16_lo(q.y);
        xv[3] = bf16_hi(q.y);
      } else {
        Elem<float>::widen(ld16(x + h), xv);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(wr[j][k], xv[k], acc);
    }
    float s = wave_sum_dpp(acc);
    if constexpr (RS > 1) {
      static_assert(RS == 4 && kWaves == 4, "a row in four quarters");
      if (lane == 0) s_red[wv] = s;
      __syncthreads();
      if (wv != 0) return;
      s = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    }
    s = s + (a.br ? a.br[e] : 0.0f);
    if (a.router_bf16) s = round_bf16(s);
    if (lane == 0) {
      coh_st(a.tl + e, tagged(tag, s));
      if (a.logits_out) a.logits_out[e] = s;
    }
    return;
  }
  if (b == a.n_r) {
    // ---- route.  The counters (k1 per-expert ones and the count of complete
    // experts) are set to (tag, 0) first, and each thread waits for its
    // stores to complete (while the router runs), so they are in place
    // before any route word is published.
    if (tid <= a.k1 + a.m) coh_st(a.cnt + tid * kCntStride, (uint64_t)tag << 32);
    __builtin_amdgcn_s_waitcnt(0);
    stage_tagged<kMaxExperts / kSyncThreads>(L.r.sl, a.E, [&](int i) { return a.tl + i; }, tag,
                                             err, a.spin_limit);
    // publish the activated experts: the selected lanes (exactly k1), each
    // at its place u among them in ascending expert order, in every copy
    const bool publish = !a.withhold_route;
    auto publish_experts = [&](bool sel, int idx) {
      const uint64_t smask = __ballot(sel);
      int u = 0;
      for (uint64_t mm = smask; mm; mm &= mm - 1)
        u += __builtin_amdgcn_readlane(idx, __builtin_ctzll(mm)) < idx;
      if (sel && publish) {
        const uint64_t we = tagged(tag, __int_as_float(idx));
        for (int c = 0; c < kRepP; ++c) coh_st(a.tp + c * a.tp_rep + u, we);
      }
    };
    bool early = false;
    if constexpr (V * kWave <= kBlockThreads) {
      // one wave: the activated set is published as soon as it is known,
      // before the ranks and the mass that the weights need
      if (tid < kWave)
        route_token_wave_ex<V, true>(L.r.sl, a.E, a.k1, a.k2, L.r.s_ids, L.r.s_w, L.r.S,
                                     a.router_bf16, publish_experts, &early);
      __syncthreads();
      if (L.r.S.n > kWave) {
        const bool renorm = a.k2 < a.E;
        block_rank(L.r.S, L.r.S.n, renorm ? a.k2 : a.k1, a.k1, renorm, a.router_bf16,
                   L.r.s_ids, L.r.s_w);
      }
    } else {
      route_token_block_large<V>(L.r.sl, a.E, a.k1, a.k2, L.r.s_ids, L.r.s_w, L.r.S,
                                 a.router_bf16);
    }
    if (tid < kWave) {
      // lane r < k1 holds rank r; u = its expert's place among the activated
      const int n = a.k1;
      const int er = lane < n ? L.r.s_ids[lane] : 0x7FFFFFFF;
      const float wr = lane < n ? L.r.s_w[lane] : 0.0f;
      if (!early) publish_experts(lane < n, er);
      int u = 0;
      for (int j = 0; j < n; ++j) u += __builtin_amdgcn_readlane(er, j) < er;
      if (lane < n && publish) {
        const uint64_t ww = tagged(tag, wr);
        for (int c = 0; c < kRepP; ++c) coh_st(a.tp + c * a.tp_rep + n + u, ww);
      }
      if (lane < n) {
        if (a.ids_out) a.ids_out[lane] = er;
        if (a.w_out) a.w_out[lane] = wr;
      }
    }
    return;
  }
  if (b < a.n_r + 1 + a.n_gu) {
    // ---- gate/up of (expert or shared piece u, block of channels); the
    // shared pieces' blocks come first
    const int item = b - a.n_r - 1;
    const int n_sh = a.m * a.n_cb;
    const bool shared = item < n_sh;
    const int u = shared ? a.k1 + item / a.n_cb : (item - n_sh) / a.n_cb;
    const int cb = shared ? item % a.n_cb : (item - n_sh) % a.n_cb;
    const WT *gbase, *ubase;
    if (shared) {
      // factor sigmoid(x . sg), or 1
      if (a.sgw) {
        const XT *x = static_cast<const XT *>(a.x);
        float z = 0.0f;
        for (int h = tid; h < a.H; h += kThreads) z = __builtin_fmaf(Elem<XT>::load1(x + h), a.sgw[h], z);
        z = wave_sum_dpp(z);
        if (lane == 0) s_red[wv] = z;
        __syncthreads();
        if (tid == 0) s_wt = 1.0f / (1.0f + __expf(-((s_red[0] + s_red[1]) + (s_red[2] + s_red[3]))));
      } else if (tid == 0) {
        s_wt = 1.0f;
      }
      __syncthreads();
      const int64_t off = (int64_t)(u - a.k1) * a.I * a.H;
      gbase = static_cast<const WT *>(a.Sg) + off;
      ubase = static_cast<const WT *>(a.Su) + off;
    } else {
      if (wv == 0) {
        const uint64_t we = await_lane(a.tp + (item % kRepP) * a.tp_rep + u, 1, tag, err,
                                       a.spin_limit);
        // a timed-out wait leaves any value here: keep the index in range
        if (lane == 0) s_e = min(max(__float_as_int(__uint_as_float((uint32_t)we)), 0), a.E - 1);
      }
      __syncthreads();
      const int64_t off = (int64_t)s_e * a.I * a.H;
      gbase = static_cast<const WT *>(a.Wg) + off;
      ubase = static_cast<const WT *>(a.Wu) + off;
    }
    // a routed expert's Eq. 2 weight is applied by the down blocks
    gateup_rows<WT, XT, NCH, CPW>(a, u, gbase, ubase, (cb * kWaves + wv) * CPW,
                                  [&]() { return shared ? s_wt : 1.0f; });
    // a shared block counts itself only once the route is published: the
    // route block sets the counters before it publishes
    if (shared && wv == 0) await_lane(a.tp + (item % kRepP) * a.tp_rep, 1, tag, err, a.spin_limit);
    // every activation store of the block is complete, then count the block
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      s_last = 0;
      const uint64_t old = __hip_atomic_fetch_add(a.cnt + u * kCntStride, (uint64_t)1,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (((uint64_t)tag << 32) | (uint32_t)(a.n_cb - 1))) {
        // the last block of expert u: every block of u counted itself after
        // its stores were complete; publish "u complete" in every copy
        for (int c = 0; c < kRepP; ++c) coh_st(a.tp + c * a.tp_rep + 2 * a.k1 + u, (uint64_t)tag << 32);
        const int n_exp = a.k1 + a.m;
        const uint64_t done = __hip_atomic_fetch_add(a.cnt + n_exp * kCntStride, (uint64_t)1,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = done == (((uint64_t)tag << 32) | (uint32_t)(n_exp - 1));
      }
    }
    __syncthreads();
    if (s_last) {
      // the block completing the last expert advances the epoch once every D
      // block has marked itself started: then no block of this call reads the
      // epoch any more (R and P blocks read it before the route existed, every
      // gate/up block before it counted itself)
      for (int i = tid; i < a.n_d; i += kThreads) {
        uint32_t spins = 0;
        while (coh_ld(a.started + i) != ((uint64_t)tag << 32)) {
          if (++spins > a.spin_limit) {
            coh_st(err, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
      if (tid == 0) coh_st(a.sync + kEpochWord, (int32_t)(tag_epoch + 1u));
    }
    return;
  }
  down_rows<WT, XT, NCD>(a, L, s_uniq, s_ws, &s_new, tag, b - a.n_r - 1 - a.n_gu);
}

}  // namespace b1

static int b1_nch(int H, int esz) { return H * esz / (16 * kWave); }

// Shapes the one-launch path takes: the router row in 1..16 and the gate/up
// row in 1..8 chunks of 16 bytes per lane, the down row in at most 2, k1 <=
// 32 (two published words per activated expert, one per lane), k1 + m <= 64
// (one completion word per lane), and one round of activations within a D
// block's LDS.  m = shared pieces (Is / I).
bool decode_b1_supported(int H, int I, int k1, bool bf16, int m) {
  const int esz = bf16 ? 2 : 4;
  if (2 * k1 > kWave || k1 + m > kWave || H % (4 * kWave) != 0 ||
      (H * esz) % (16 * kWave) != 0)
    return false;
  const int nchr = H / (4 * kWave), nch = b1_nch(H, esz);
  if (!(nchr == 1 || nchr == 2 || nchr == 4 || nchr == 8 || nchr == 16)) return false;
  if (!(nch == 1 || nch == 2 || nch == 4 || nch == 8)) return false;
  const int ab = bf16 ? 2 : 4;
  const int round_bytes = (k1 + m < b1::kPF ? k1 + m : b1::kPF) * I * ab;
  // the fixed tagged region holds every word of these shapes
  static_assert(3 * (kWave / 2) + kWave / 2 <= kB1TpRepWords, "route copy too small");
  static_assert(kWave + 1 <= kB1MaxCounters, "too few counters");
  if ((H + b1::kWaves - 1) / b1::kWaves > kB1MaxDownBlocks) return false;
  return I * esz / 16 <= 2 * kWave && round_bytes <= b1::kLdsBytes && (I * ab) % 8 == 0;
}

size_t decode_b1_abuf_bytes(int I, int k1, bool bf16, int m) {
  return (((size_t)(k1 + m) * I * (bf16 ? 2 : 4)) + 255) & ~(size_t)255;
}

// The gate/up row's 16-byte chunks per lane follow from the router row's
// (NCHR, fp32) and the weight dtype, so only those kernels are built; each
// wave takes CPW = 8 / NCH channels, 8 chunks of each row in flight per lane.
template <typename WT, typename XT, int NCHR, int V>
static void launch_nch(b1::Args &a, int ncd, hipStream_t s) {
  constexpr int NCH = sizeof(WT) == 2 ? NCHR / 2 : NCHR;
  static_assert(NCH >= 1 && NCH <= 8, "gate/up chunks per lane out of range");
  constexpr int CPW = 8 / NCH;
  a.n_r = b1::kRouterRowSplit<NCHR> > 1 ? a.E : (a.E + b1::kWaves - 1) / b1::kWaves;
  a.n_cb = (a.I + b1::kWaves * CPW - 1) / (b1::kWaves * CPW);
  a.n_gu = (a.k1 + a.m) * a.n_cb;
  const int grid = a.n_r + 1 + a.n_gu + a.n_d;
  if (ncd == 1)
    b1::layer_kernel<WT, XT, NCHR, V, NCH, CPW, 1><<<dim3((unsigned)grid), dim3(b1::kThreads), 0, s>>>(a);
  else
    b1::layer_kernel<WT, XT, NCHR, V, NCH, CPW, 2><<<dim3((unsigned)grid), dim3(b1::kThreads), 0, s>>>(a);
}

template <typename WT, typename XT, int V>
static void launch_v(b1::Args &a, int nchr, int ncd, hipStream_t s) {
  if constexpr (sizeof(WT) == 2) {
    switch (nchr) {
      case 2: launch_nch<WT, XT, 2, V>(a, ncd, s); break;
      case 4: launch_nch<WT, XT, 4, V>(a, ncd, s); break;
      case 8: launch_nch<WT, XT, 8, V>(a, ncd, s); break;
      default: launch_nch<WT, XT, 16, V>(a, ncd, s); break;
    }
  } else {
    switch (nchr) {
      case 1: launch_nch<WT, XT, 1, V>(a, ncd, s); break;
      case 2: launch_nch<WT, XT, 2, V>(a, ncd, s); break;
      case 4: launch_nch<WT, XT, 4, V>(a, ncd, s); break;
      default: launch_nch<WT, XT, 8, V>(a, ncd, s); break;
    }
  }
}

template <typename WT, typename XT>
hipError_t launch_decode_b1(const XT *x, int H, const void *Wr, bool router_bf16, const float *br,
                            int E, const WT *Wg, const WT *Wu, const WT *Wd, int I, int k1,
                            int k2, const WT *Sg, const WT *Su, const WT *Sd, int Is,
                            const float *sgw, XT *y, float *logits_out, int32_t *ids_out,
                            float *w_out, int32_t *sync, char *region, void *abuf,
                            uint32_t spin_limit, bool withhold_route, hipStream_t s) {
  constexpr int esz = sizeof(WT);
  const int m = Sg ? Is / I : 0;
  b1::Args a;
  a.x = x;
  a.Wr = Wr;
  a.router_bf16 = router_bf16;
  a.br = br;
  a.Wg = Wg;
  a.Wu = Wu;
  a.Wd = Wd;
  a.Sg = Sg;
  a.Su = Su;
  a.Sd = Sd;
  a.sgw = sgw;
  a.m = m;
  a.Is = Is;
  a.y = y;
  a.logits_out = logits_out;
  a.ids_out = ids_out;
  a.w_out = w_out;
  a.sync = sync;
  a.tl = reinterpret_cast<uint64_t *>(region + kB1Tl);
  a.tp = reinterpret_cast<uint64_t *>(region + kB1Tp);
  a.tp_rep = kB1TpRepWords;
  a.cnt = reinterpret_cast<uint64_t *>(region + kB1Cnt);
  a.started = reinterpret_cast<uint64_t *>(region + kB1Started);
  a.abuf = abuf;
  a.spin_limit = spin_limit;
  a.withhold_route = withhold_route;
  a.H = H;
  a.E = E;
  a.I = I;
  a.k1 = k1;
  a.k2 = k2;
  a.n_r = (E + b1::kWaves - 1) / b1::kWaves;
  a.n_d = (H + b1::kWaves - 1) / b1::kWaves;
  a.n_cb = a.n_gu = 0;
  const int nchr = H / (4 * kWave);
  const int ncd = (I * esz / 16 + kWave - 1) / kWave;
  if (E <= 64) launch_v<WT, XT, 1>(a, nchr, ncd, s);
  else if (E <= 128) launch_v<WT, XT, 2>(a, nchr, ncd, s);
  else if (E <= 256) launch_v<WT, XT, 4>(a, nchr, ncd, s);
  else if (E <= 512) launch_v<WT, XT, 8>(a, nchr, ncd, s);
  else launch_v<WT, XT, 16>(a, nchr, ncd, s);
  return hipGetLastError();
}

#define MOE_INST_B1(WT, XT)                                                                 \
  template hipError_t launch_decode_b1<WT, XT>(const XT *, int, const void *, bool,           \
                                               const float *, int, const WT *, const WT *,    \
                                               const WT *, int, int, int, const WT *,         \
                                               const WT *, const WT *, int, const float *,    \
                                               XT *, float *, int32_t *, float *, int32_t *,  \
                                               char *, void *, uint32_t, bool, hipStream_t);
MOE_INST_B1(float, float)
MOE_INST_B1(bf16_t, bf16_t)

}  // namespace moe
