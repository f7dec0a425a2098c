// The whole routed MoE layer for small batches (decode, T <= 8 tokens) in ONE
// kernel launch.
//
// What it computes: router logits, the fp32 softmax / top-k2 / Eq. 2 route of
// "Paper of the Week #3 - Half the FLOPs Is Not Half the Time" (section "The
// Receipt", Eq. 2; section "Ship It - Code of the Week"), then for every
// activated expert the gated MLP of "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data" (section 2 "Background": channel c owns
// gate row Wg[e,c,:], up row Wu[e,c,:] and down column Wd[e,:,c]), weighted
// and summed per token.
//
// Why one launch: at batch 1 the activated experts of an H=2048, E=128,
// I=768 layer are 38 MB, under 5 us of HBM time, while a kernel boundary
// costs about 1.7 us even inside a HIP graph.
//
// Workgroups, in block-index order (the hardware dispatches blocks in
// increasing index order within each XCD, so a block only waits for blocks
// with smaller indices, which were dispatched before it):
//   R  [0, nR)            router: each wave computes the logits of `epw`
//                         experts for every token.
//   GU [nR, nR+nGU)       (unique expert u, block of channels): route every
//                         token itself (T <= 8: cheap, identical in every
//                         block), stream the gate and up rows of expert u
//                         once, and for each token routed to u publish
//                         a[t,r,c] = silu(g) u w[t,r].
//   D  [.., +nHB)         (block of output rows): route the tokens, load the
//                         down rows of the first kPF unique experts (before
//                         any gate/up result exists), then for each unique
//                         expert stage its a vectors in LDS and accumulate
//                         y[t,h] += Wd[e,h,:] . a[t,r,:] in ascending expert
//                         order, prefetching the rows of expert u+kPF.
// Hand-over without counters: every published value (logit, a) is a 64-bit
// word holding the value and the call's tag, written with a device-coherent
// store; a consumer re-reads the words it needs with coherent loads until
// every tag is the current one, so the data's arrival is the signal.  There
// are no fences (on gfx950 an agent-scope fence writes back or invalidates a
// whole XCD's L2, which takes microseconds) and no hot counters (same-address
// atomics serialize at about 10 ns each).  The tag is a NaN pattern made
// from the workspace's epoch (call_tag); the last block to finish (a
// two-level count) advances the epoch, so stale words never match.  Every wait is bounded: a
// timeout sets the error word and the block moves on, so the kernel always
// terminates.
#include "common.hpp"
#include "kernels.hpp"
#include "route_device.hpp"
#include "sync.hpp"

namespace moe {
namespace fused {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxTok = 8;        // tokens each block routes itself
constexpr int kMaxAssign = 512;   // T * k1 held in LDS
constexpr int kPF = 6;            // down rows prefetched for this many experts
constexpr int kRPW = 1;           // down rows per wave
constexpr int kRB = kWaves * kRPW;
constexpr int kSub = 32;          // sub-counters of the done count
constexpr int kStage = 2048;      // a values staged in LDS per round (floats)
// Published words are written to several copies spread over memory channels
// (copy stride = a multiple of 4 KiB plus 1280 B), and each consumer block
// reads the copy of its index, so that hundreds of blocks do not poll the
// same few lines of one channel.
constexpr int kRepL = 16;         // copies of the logits
constexpr int kRepA = 8;          // copies of the channel activations

// int32 word offsets in the sync region; counters are 16 words (64 B) apart
constexpr int kLine = 16;
constexpr int kEpoch = kEpochWord;
constexpr int kDoneTop = kLine;
constexpr int kError = kErrorWord;
static_assert(kErrorWord == 2 * kLine, "error word is a line of its own");
constexpr int kDoneSub0 = 4 * kLine;  // kSub lines
constexpr int kSyncWords = kDoneSub0 + kSub * kLine;
constexpr int kMaxLogits = 2048;      // T * E staged in LDS

struct Args {
  const void *x;
  const float *Wr;
  const float *br;
  const void *Wg;
  const void *Wu;
  const void *Wd;
  void *y;
  float *logits_out;
  int32_t *ids_out;
  float *w_out;
  int32_t *sync;
  uint64_t *logits;  // kRepL copies of [T, E], tagged
  uint64_t *abuf;    // kRepA copies of [T*k1, I], tagged
  int64_t rep_l, rep_a;  // copy strides in words
  int T, H, E, I, k1, k2;
  int n_r, epw, umax, n_cb, n_gu, n_hb, n_blocks;
};

// Thread 0 adds 1 to *ctr once the whole block is here; the old value is
// returned to every thread of the block.
__device__ int block_count(int32_t *ctr, int *s_old) {
  __syncthreads();
  if (threadIdx.x == 0) *s_old = atomic_inc(ctr);
  __syncthreads();
  return *s_old;
}

// ------------------------------------------------------------- router
template <typename XT, int NCHR>
__device__ void router_block(const Args &a, int rb, uint32_t tag) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const XT *x = static_cast<const XT *>(a.x);
  for (int q = 0; q < a.epw; ++q) {
    const int e = (rb * kWaves + wv) * a.epw + q;
    if (e >= a.E) break;
    const float *wrow = a.Wr + (int64_t)e * a.H;
    float wv4[NCHR][4];
#pragma unroll
    for (int j = 0; j < NCHR; ++j) Elem<float>::widen(ld16_stream(wrow + (j * kWave + lane) * 4), wv4[j]);
    const float b = a.br ? a.br[e] : 0.0f;
    for (int t = 0; t < a.T; ++t) {
      const XT *xr = x + (int64_t)t * a.H;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NCHR; ++j) {
        const int h = (j * kWave + lane) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(wv4[j][k], Elem<XT>::load1(xr + h + k), acc);
      }
      const float s = wave_sum_dpp(acc) + b;  // the same on every lane
      if (lane < kRepL) coh_st(a.logits + lane * a.rep_l + (int64_t)t * a.E + e, tagged(tag, s));
      if (lane == 0 && a.logits_out) a.logits_out[(int64_t)t * a.E + e] = s;
    }
  }
}

// ------------------------------------------------------------- local plan
// The route of every token and the unique experts of the batch, in LDS:
// uniq[u] ascending, list[off[u] .. off[u+1]) = assignments (t*k1 + r) routed
// to uniq[u], ascending.  Built identically by every block.

struct Plan {
  float logits[kMaxLogits];
  int32_t ids[kMaxAssign];
  float w[kMaxAssign];
  int32_t uniq[kMaxAssign];
  int32_t off[kMaxAssign + 1];
  int32_t list[kMaxAssign];
  uint32_t bits[kMaxExperts / 32];
  int32_t pre[kMaxExperts / 32];
  int32_t U;
  BlockRoute br;
};

__device__ __forceinline__ int uidx_of(const Plan &P, int e) {
  return P.pre[e >> 5] + __popc(P.bits[e >> 5] & ((1u << (e & 31)) - 1u));
}

template <int V>
__device__ void build_plan(const Args &a, Plan &P, uint32_t tag, bool write_out) {
  const int n = a.T * a.k1;
  const int nw = (a.E + 31) >> 5;
  for (int i = threadIdx.x; i < nw; i += kThreads) P.bits[i] = 0u;
  // the router's logits, as soon as each one carries this call's tag
  const uint64_t *lg = a.logits + (blockIdx.x % kRepL) * a.rep_l;
  stage_tagged<kMaxLogits / kThreads>(P.logits, a.T * a.E, [&](int i) { return lg + i; }, tag,
                                      a.sync + kError);
  if (a.T == 1 && a.E <= kThreads && a.k1 <= kThreads) {
    route_token_block(P.logits, a.E, a.k1, a.k2, P.ids, P.w, write_out ? a.ids_out : nullptr,
                      write_out ? a.w_out : nullptr, P.br);
  } else {
    const int wv = threadIdx.x >> 6;
    for (int t = wv; t < a.T; t += kWaves) {
      const int o = t * a.k1;
      route_token<V>(P.logits + t * a.E, a.E, a.k1, a.k2, P.ids + o, P.w + o,
                     write_out && a.ids_out ? a.ids_out + o : nullptr,
                     write_out && a.w_out ? a.w_out + o : nullptr);
    }
    __syncthreads();
  }
  if (n <= kWave) {
    // one wave builds the plan: lane i holds assignment i
    if (threadIdx.x < kWave) {
      const int i = threadIdx.x;
      const int e = i < n ? P.ids[i] : 0x7FFFFFFF;
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
      if (i < n) {
        if (same_before == 0) {
          P.uniq[uniq_less] = e;
          P.off[uniq_less] = cnt_less;
        }
        P.list[cnt_less + same_before] = i;
      }
      if (i == 0) {
        const int U = __popcll(first);
        P.U = U;
        P.off[U] = n;
      }
    }
    __syncthreads();
    return;
  }
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int e = P.ids[i];
    atomicOr(&P.bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int k = 0; k < nw; ++k) {
      P.pre[k] = s;
      s += __popc(P.bits[k]);
    }
    P.U = s;
  }
  __syncthreads();
  const int U = P.U;
  // unique experts in ascending order
  for (int k = threadIdx.x; k < nw; k += kThreads) {
    uint32_t m = P.bits[k];
    int u = P.pre[k];
    while (m) {
      const int bit = __ffs(m) - 1;
      P.uniq[u++] = k * 32 + bit;
      m &= m - 1u;
    }
  }
  // off[u] = assignments whose expert ranks below u
  for (int u = threadIdx.x; u <= U; u += kThreads) {
    int c = 0;
    for (int j = 0; j < n; ++j) c += uidx_of(P, P.ids[j]) < u;
    P.off[u] = c;
  }
  __syncthreads();
  // assignment i goes after the earlier tokens routed to the same expert
  // (a token never lists an expert twice, so assignment order = token order)
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int e = P.ids[i];
    int r = 0;
    for (int j = 0; j < i; ++j) r += P.ids[j] == e;
    P.list[P.off[uidx_of(P, e)] + r] = i;
  }
  __syncthreads();
}

// ------------------------------------------------------------- gate/up
// NCH = 16-byte chunks per lane of one gate (or up) row; CPW channels per
// wave; all 2*CPW*NCH loads are issued before any arithmetic.
template <typename WT, typename XT, int NCH, int CPW>
__device__ void gateup_block(const Args &a, const Plan &P, int item, uint32_t tag) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int u = item / a.n_cb, cb = item - u * a.n_cb;
  const int e = P.uniq[u];
  const int lb = P.off[u], ln = P.off[u + 1] - lb;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int c0 = (cb * kWaves + wv) * CPW;
  const WT *Wg = static_cast<const WT *>(a.Wg);
  const WT *Wu = static_cast<const WT *>(a.Wu);
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
  const XT *x = static_cast<const XT *>(a.x);
  for (int i = 0; i < ln; ++i) {
    const int asg = P.list[lb + i];
    const XT *xr = x + (int64_t)(asg / a.k1) * a.H;
    const float wt = P.w[asg];
    if constexpr (sizeof(WT) == 2 && sizeof(XT) == 2) {
      // bf16 x bf16: packed dot products (v_dot2_f32_bf16), x kept packed
      uint4 xq[NCH];
#pragma unroll
      for (int j = 0; j < NCH; ++j) xq[j] = ld16(xr + (j * kWave + lane) * NW);
      float av[CPW];
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          ag = dot2_bf16(gq[ci][j].x, xq[j].x, ag);
          ag = dot2_bf16(gq[ci][j].y, xq[j].y, ag);
          ag = dot2_bf16(gq[ci][j].z, xq[j].z, ag);
          ag = dot2_bf16(gq[ci][j].w, xq[j].w, ag);
          au = dot2_bf16(uq[ci][j].x, xq[j].x, au);
          au = dot2_bf16(uq[ci][j].y, xq[j].y, au);
          au = dot2_bf16(uq[ci][j].z, xq[j].z, au);
          au = dot2_bf16(uq[ci][j].w, xq[j].w, au);
        }
        av[ci] = silu(wave_sum_dpp(ag)) * wave_sum_dpp(au) * wt;
      }
      if constexpr (CPW % 2 == 0) {
        // two channels per word, as bf16 (the down projection reads bf16
        // weights; a 2^-9 relative rounding of a)
#pragma unroll
        for (int ci = 0; ci < CPW; ci += 2) {
          const int c = c0 + ci;
          const uint64_t word = ((uint64_t)tag << 32) | (f32_to_bf16_bits(av[ci + 1]) << 16) |
                                f32_to_bf16_bits(av[ci]);
          if (lane < kRepA && c < a.I)
            coh_st(a.abuf + lane * a.rep_a + ((int64_t)asg * a.I + c) / 2, word);
        }
      } else {
#pragma unroll
        for (int ci = 0; ci < CPW; ++ci) {
          const int c = c0 + ci;
          if (lane < kRepA && c < a.I)
            coh_st(a.abuf + lane * a.rep_a + (int64_t)asg * a.I + c, tagged(tag, av[ci]));
        }
      }
    } else {
      float xv[NCH][NW];
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int k = 0; k < NW; ++k) xv[j][k] = Elem<XT>::load1(xr + (j * kWave + lane) * NW + k);
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          float gv[NW], uv[NW];
          Elem<WT>::widen(gq[ci][j], gv);
          Elem<WT>::widen(uq[ci][j], uv);
#pragma unroll
          for (int k = 0; k < NW; ++k) {
            ag = __builtin_fmaf(gv[k], xv[j][k], ag);
            au = __builtin_fmaf(uv[k], xv[j][k], au);
          }
        }
        ag = wave_sum_dpp(ag);
        au = wave_sum_dpp(au);
        const int c = c0 + ci;
        if (lane < kRepA && c < a.I)
          coh_st(a.abuf + lane * a.rep_a + (int64_t)asg * a.I + c, tagged(tag, silu(ag) * au * wt));
      }
    }
  }
}

// ------------------------------------------------------------- down
// Each wave owns kRPW rows; lane L holds 16-byte chunks L and L+64 of a row
// (NCD = 1 or 2 chunks per lane, I*sizeof(WT)/16 <= 128).
template <typename WT, typename XT, int NCD, bool PACKED>
__device__ void down_block(const Args &a, const Plan &P, int hb, float *s_a, float *s_y,
                           uint32_t tag) {
  constexpr int NW = Elem<WT>::kPer16B;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int U = P.U;
  const int nch = a.I / NW;
  const int h = min(hb * kRB + wv, a.H - 1);  // kRPW = 1
  const WT *Wd = static_cast<const WT *>(a.Wd);
  for (int i = threadIdx.x; i < a.T * kRB; i += kThreads) s_y[i] = 0.0f;
  uint4 dq[kPF][NCD];
  auto issue = [&](int slot_u, uint4 (&dst)[NCD]) {
    const WT *drow = Wd + ((int64_t)P.uniq[slot_u] * a.H + h) * a.I;
#pragma unroll
    for (int j = 0; j < NCD; ++j) {
      const int ch = j * kWave + lane;
      dst[j] = ch < nch ? ld16_stream(drow + ch * NW) : make_uint4(0, 0, 0, 0);
    }
  };
#pragma unroll
  for (int s = 0; s < kPF; ++s)
    if (s < U) issue(s, dq[s]);
  const uint64_t *ab = a.abuf + (blockIdx.x % kRepA) * a.rep_a;
  // assignments staged per round (I <= 1024)
  const int per_round = (PACKED ? 2 * kStage : kStage) / a.I;
  for (int ub = 0; ub < U; ub += kPF) {
    const int ue = min(U, ub + kPF);
    const int g0 = P.off[ub], g1 = P.off[ue];
    for (int r0 = g0; r0 < g1; r0 += per_round) {
      const int r1 = min(g1, r0 + per_round);
      // stage the a vectors of assignments list[r0 .. r1) as they are published
      if constexpr (PACKED) {
        const int half = a.I / 2;
        stage_tagged<kStage / kThreads, true>(
            s_a, (r1 - r0) * half,
            [&](int idx) {
              const int i = r0 + idx / half, c2 = idx - (idx / half) * half;
              return ab + ((int64_t)P.list[i] * a.I) / 2 + c2;
            },
            tag, a.sync + kError);
      } else {
        stage_tagged<kStage / kThreads>(
            s_a, (r1 - r0) * a.I,
            [&](int idx) {
              const int i = r0 + idx / a.I, c = idx - (idx / a.I) * a.I;
              return ab + (int64_t)P.list[i] * a.I + c;
            },
            tag, a.sync + kError);
      }
#pragma unroll
      for (int s = 0; s < kPF; ++s) {
        const int u = ub + s;
        if (u < ue) {
          const int lb = max(P.off[u], r0), le = min(P.off[u + 1], r1);
          for (int i = lb; i < le; ++i) {
            const float *av = s_a + (i - r0) * a.I;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < NCD; ++j) {
              const int ch = j * kWave + lane;
              if (ch < nch) {
                float dv[NW];
                Elem<WT>::widen(dq[s][j], dv);
#pragma unroll
                for (int k = 0; k < NW; ++k) acc = __builtin_fmaf(dv[k], av[ch * NW + k], acc);
              }
            }
            acc = wave_sum_dpp(acc);
            if (lane == 0) s_y[(P.list[i] / a.k1) * kRB + wv] += acc;
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < kPF; ++s)
      if (ub + kPF + s < U) issue(ub + kPF + s, dq[s]);
  }
  __syncthreads();
  XT *y = static_cast<XT *>(a.y);
  for (int i = threadIdx.x; i < a.T * kRB; i += kThreads) {
    const int t = i / kRB, r = i - t * kRB;
    const int hh = hb * kRB + r;
    if (hh < a.H) Elem<XT>::store1(y + (int64_t)t * a.H + hh, s_y[i]);
  }
}

// ------------------------------------------------------------- kernel
template <typename WT, typename XT, int V, int NCHR, int NCH, int CPW, int NCD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void fused_decode_kernel(Args a) {
  __shared__ Plan P;
  __shared__ float s_a[2 * kStage];
  __shared__ float s_y[kMaxTok * kRB];
  __shared__ int s_old;
  const int b = blockIdx.x;
  int32_t *sync = a.sync;
  const uint32_t epoch = (uint32_t)coh_ld(sync + kEpoch);
  const uint32_t tag = call_tag(epoch);
  if (b < a.n_r) {
    router_block<XT, NCHR>(a, b, tag);
    return;
  }
  const bool is_gu = b < a.n_r + a.n_gu;
  const int item = is_gu ? b - a.n_r : b - a.n_r - a.n_gu;
  build_plan<V>(a, P, tag, !is_gu && item == 0);
  if (is_gu) {
    if (item / a.n_cb < P.U) gateup_block<WT, XT, NCH, CPW>(a, P, item, tag);
  } else {
    down_block<WT, XT, NCD, sizeof(WT) == 2 && CPW % 2 == 0>(a, P, item, s_a, s_y, tag);
  }
  // done count over the non-router blocks (kSub sub-counters, then the top);
  // the last one advances the epoch and clears the counters
  const int sub = b % kSub;
  auto upto = [&](int lim) { return lim > sub ? (lim - sub + kSub - 1) / kSub : 0; };
  const int n_sub = upto(a.n_blocks) - upto(a.n_r);
  if (block_count(sync + kDoneSub0 + sub * kLine, &s_old) == n_sub - 1) {
    const int n_top = min(kSub, a.n_blocks - a.n_r);
    if (block_count(sync + kDoneTop, &s_old) == n_top - 1) {
      for (int k = threadIdx.x; k < kSub; k += kThreads) coh_st(sync + kDoneSub0 + k * kLine, 0);
      if (threadIdx.x == 0) {
        coh_st(sync + kDoneTop, 0);
        coh_st(sync + kEpoch, (int32_t)(epoch + 1u));
      }
    }
  }
}

}  // namespace fused

bool fused_decode_supported(int64_t T, int H, int E, int I, int k1, bool bf16) {
  const int esz = bf16 ? 2 : 4;
  if (T < 1 || T > fused::kMaxTok || T * k1 > fused::kMaxAssign) return false;
  if (T * E > fused::kMaxLogits) return false;
  if (E > kMaxExperts || I > 1024) return false;
  if ((H * 4) % (16 * kWave) != 0 || (H * esz) % (16 * kWave) != 0) return false;
  const int nchr = H * 4 / 16 / kWave;
  const int nch = H * esz / 16 / kWave;
  if (!(nchr == 1 || nchr == 2 || nchr == 4 || nchr == 8 || nchr == 16)) return false;
  if (!(nch == 1 || nch == 2 || nch == 4 || nch == 8)) return false;
  return I * esz / 16 <= 2 * kWave;
}

// bytes between two copies of a published buffer
static size_t fused_copy_stride(size_t bytes) { return ((bytes + 4095) & ~(size_t)4095) + 1280; }

size_t fused_decode_workspace(int64_t T, int H, int E, int I, int k1, DecodeLayout *L) {
  (void)H;
  static_assert(fused::kSyncWords <= kRouteTicketWord, "sync words overlap the route ticket");
  static_assert(fused::kSyncWords * 4 <= kSyncRegionBytes, "sync region too small");
  L->sync = 0;
  size_t o = kSyncRegionBytes;
  L->logits = o;
  o += fused::kRepL * fused_copy_stride((size_t)T * E * 8);
  L->abuf = o;
  o += fused::kRepA * fused_copy_stride((size_t)T * k1 * (size_t)I * 8);
  L->total = o;
  return o;
}

template <typename WT, typename XT, int V, int NCHR, int NCH, int CPW, int NCD>
static hipError_t launch_fused_t(fused::Args &a, hipStream_t s) {
  a.n_cb = (a.I + fused::kWaves * CPW - 1) / (fused::kWaves * CPW);
  a.n_gu = a.umax * a.n_cb;
  a.n_hb = (a.H + fused::kRB - 1) / fused::kRB;
  a.n_blocks = a.n_r + a.n_gu + a.n_hb;
  fused::fused_decode_kernel<WT, XT, V, NCHR, NCH, CPW, NCD>
      <<<dim3((unsigned)a.n_blocks), dim3(fused::kThreads), 0, s>>>(a);
  return hipGetLastError();
}

// 16 chunk loads per lane in flight in the gate/up phase
template <typename WT, typename XT, int V, int NCHR>
static hipError_t launch_fused_nch(fused::Args &a, int nch, int ncd, hipStream_t s) {
  if (ncd == 1) {
    if (nch == 1) return launch_fused_t<WT, XT, V, NCHR, 1, 8, 1>(a, s);
    if (nch == 2) return launch_fused_t<WT, XT, V, NCHR, 2, 4, 1>(a, s);
    if (nch == 4) return launch_fused_t<WT, XT, V, NCHR, 4, 2, 1>(a, s);
    return launch_fused_t<WT, XT, V, NCHR, 8, 1, 1>(a, s);
  }
  if (nch == 1) return launch_fused_t<WT, XT, V, NCHR, 1, 8, 2>(a, s);
  if (nch == 2) return launch_fused_t<WT, XT, V, NCHR, 2, 4, 2>(a, s);
  if (nch == 4) return launch_fused_t<WT, XT, V, NCHR, 4, 2, 2>(a, s);
  return launch_fused_t<WT, XT, V, NCHR, 8, 1, 2>(a, s);
}

template <typename WT, typename XT, int V>
static hipError_t launch_fused_v(fused::Args &a, int nchr, int nch, int ncd, hipStream_t s) {
  switch (nchr) {
    case 1: return launch_fused_nch<WT, XT, V, 1>(a, nch, ncd, s);
    case 2: return launch_fused_nch<WT, XT, V, 2>(a, nch, ncd, s);
    case 4: return launch_fused_nch<WT, XT, V, 4>(a, nch, ncd, s);
    case 8: return launch_fused_nch<WT, XT, V, 8>(a, nch, ncd, s);
    default: return launch_fused_nch<WT, XT, V, 16>(a, nch, ncd, s);
  }
}

template <typename WT, typename XT>
hipError_t launch_fused_decode(const XT *x, int64_t T, int H, const float *Wr, const float *br,
                               int E, const WT *Wg, const WT *Wu, const WT *Wd, int I, int k1,
                               int k2, XT *y, float *logits_out, int32_t *ids_out, float *w_out,
                               char *ws, hipStream_t s) {
  DecodeLayout L;
  fused_decode_workspace(T, H, E, I, k1, &L);
  fused::Args a;
  a.x = x;
  a.Wr = Wr;
  a.br = br;
  a.Wg = Wg;
  a.Wu = Wu;
  a.Wd = Wd;
  a.y = y;
  a.logits_out = logits_out;
  a.ids_out = ids_out;
  a.w_out = w_out;
  a.sync = reinterpret_cast<int32_t *>(ws + L.sync);
  a.logits = reinterpret_cast<uint64_t *>(ws + L.logits);
  a.abuf = reinterpret_cast<uint64_t *>(ws + L.abuf);
  a.rep_l = (int64_t)(fused_copy_stride((size_t)T * E * 8) / 8);
  a.rep_a = (int64_t)(fused_copy_stride((size_t)T * k1 * (size_t)I * 8) / 8);
  a.T = (int)T;
  a.H = H;
  a.E = E;
  a.I = I;
  a.k1 = k1;
  a.k2 = k2;
  a.umax = (int)(T * k1 < E ? T * k1 : E);
  // at most 32 router blocks; each wave takes epw experts
  a.n_r = (E + fused::kWaves - 1) / fused::kWaves;
  if (a.n_r > 32) a.n_r = 32;
  a.epw = (E + a.n_r * fused::kWaves - 1) / (a.n_r * fused::kWaves);
  constexpr int esz = sizeof(WT);
  const int nchr = H * 4 / 16 / kWave;
  const int nch = H * esz / 16 / kWave;
  const int ncd = (I * esz / 16 + kWave - 1) / kWave;
  if (E <= 64) return launch_fused_v<WT, XT, 1>(a, nchr, nch, ncd, s);
  if (E <= 128) return launch_fused_v<WT, XT, 2>(a, nchr, nch, ncd, s);
  if (E <= 256) return launch_fused_v<WT, XT, 4>(a, nchr, nch, ncd, s);
  if (E <= 512) return launch_fused_v<WT, XT, 8>(a, nchr, nch, ncd, s);
  return launch_fused_v<WT, XT, 16>(a, nchr, nch, ncd, s);
}

template hipError_t launch_fused_decode<float, float>(const float *, int64_t, int, const float *,
                                                      const float *, int, const float *,
                                                      const float *, const float *, int, int,
                                                      int, float *, float *, int32_t *, float *,
                                                      char *, hipStream_t);
template hipError_t launch_fused_decode<bf16_t, bf16_t>(const bf16_t *, int64_t, int,
                                                        const float *, const float *, int,
                                                        const bf16_t *, const bf16_t *,
                                                        const bf16_t *, int, int, int, bf16_t *,
                                                        float *, int32_t *, float *, char *,
                                                        hipStream_t);

}  // namespace moe
