// Internal launchers of libmoe.so (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

constexpr int kMaxExperts = 1024;

// Every workspace starts with a fixed 16 KiB region of synchronisation words
// (an epoch word, then counters that are zero whenever no call is running).
// Its size and place do not depend on the call's shapes, so one workspace can
// serve calls of different shapes.
constexpr size_t kSyncRegionBytes = 16384;
// int32 words of the sync region shared by the paths that hand values over
// between workgroups: the workspace's epoch (source of the call tags) and an
// error word set by a wait that timed out
constexpr int kEpochWord = 0;
constexpr int kErrorWord = 32;
// re-reads before a hand-over wait gives up (and sets the error word)
constexpr uint32_t kDefaultSpinLimit = 1u << 20;

template <typename XT>
hipError_t launch_router(const XT *x, int64_t T, int H, const float *Wr, const float *br, int E,
                         float *logits, float *logits2, hipStream_t s);

hipError_t launch_plan(const int32_t *ids, int64_t n_assign, int E, int32_t *plan,
                       hipStream_t s);

// Route with one workgroup per token; with plan != NULL (T*k1 <= 64) the last
// block also builds the plan.  `ticket` is a zero word of the sync region.
// wbf16 rounds the weights to bf16.
hipError_t launch_route_plan(const float *logits, int64_t T, int E, int k1, int k2,
                             int32_t *ids, float *w, int32_t *ids2, float *w2, int32_t *plan,
                             int32_t *ticket, bool wbf16, hipStream_t s);

// bf16 router: bf16 x and Wr, logits rounded to bf16 (stored as fp32)
hipError_t launch_router_bf16(const bf16_t *x, int64_t T, int H, const bf16_t *Wr, int E,
                              float *logits, float *logits2, hipStream_t s);

template <typename WT, typename XT>
hipError_t launch_down_one_token(const WT *Wd, int H, int I, const int32_t *plan, int E,
                                 const float *abuf, XT *y, hipStream_t s);

// one token: router, route and plan (k1 <= 64) in one launch
bool router_route_supported(int H);
template <typename XT>
hipError_t launch_router_route(const XT *x, int H, const float *Wr, const float *br, int E,
                               int k1, int k2, float *logits, float *logits2, int32_t *ids,
                               float *w, int32_t *ids2, float *w2, int32_t *plan, int32_t *ticket,
                               hipStream_t s);

// ---- one token in one launch (router, route, gate/up and down)
// Its tagged hand-over words sit at fixed places of a region of fixed size
// that follows the sync region in every workspace (no other path writes
// there): E tagged logits (up to kMaxExperts), kB1RepP copies of the
// published route (kB1TpRepWords apart: 4 KiB + 1280 B, so that pollers
// spread over memory channels), up to kB1MaxCounters completion counters
// (kB1CntStride words apart) and a started word per down block (up to
// kB1MaxDownBlocks).
constexpr int kB1RepP = 16;
constexpr int64_t kB1TpRepWords = (4096 + 1280) / 8;
constexpr int kB1MaxCounters = 65;
constexpr int kB1CntStride = 16;
constexpr int kB1MaxDownBlocks = 1024;
constexpr size_t kB1Tl = 0;
constexpr size_t kB1Tp = kB1Tl + (size_t)kMaxExperts * 8;
constexpr size_t kB1Cnt = kB1Tp + (size_t)kB1RepP * kB1TpRepWords * 8;
constexpr size_t kB1Started = kB1Cnt + (size_t)kB1MaxCounters * kB1CntStride * 8;
constexpr size_t kB1RegionBytes = (kB1Started + (size_t)kB1MaxDownBlocks * 8 + 255) & ~(size_t)255;
// m = pieces of I channels of the shared expert (0 without one)
bool decode_b1_supported(int H, int I, int k1, bool bf16, int m);
// bytes of the channel activations [k1 + m, I] (bf16 or fp32)
size_t decode_b1_abuf_bytes(int I, int k1, bool bf16, int m);
// region: the fixed tagged region; abuf: decode_b1_abuf_bytes bytes.  A wait
// gives up after spin_limit re-reads; withhold_route is a test hook that
// keeps the route from being published, so the waits for it give up.
template <typename WT, typename XT>
hipError_t launch_decode_b1(const XT *x, int H, const void *Wr, bool router_bf16, const float *br,
                            int E, const WT *Wg, const WT *Wu, const WT *Wd, int I, int k1,
                            int k2, const WT *Sg, const WT *Su, const WT *Sd, int Is,
                            const float *sgw, XT *y, float *logits_out, int32_t *ids_out,
                            float *w_out, int32_t *sync, char *region, void *abuf,
                            uint32_t spin_limit, bool withhold_route, hipStream_t s);

// ---- prefill (bf16 MFMA) path
bool prefill_supported(int H, int I, bool bf16);
size_t prefill_plan_words(int64_t n, int E);
hipError_t launch_split_router(const float *Wr, int E, int H, uint16_t *w3, hipStream_t s);
// logits = x Wr^T from nterms bf16 terms of the router weight in one
// workgroup per tile: three (the split fp32 weight) added in a fixed order,
// plus br; one (the bf16 router) rounded to bf16, no bias
hipError_t launch_router_mma(const uint16_t *x, int64_t T, int H, const uint16_t *w3, int E,
                             int nterms, const float *br, float *logits, float *logits2,
                             hipStream_t s);
hipError_t launch_prefill_plan(const int32_t *ids, int64_t n, int E, int32_t *plan,
                               hipStream_t s);
hipError_t launch_gateup_mma(const uint16_t *x, int H, const uint16_t *Wg, const uint16_t *Wu,
                             int I, const int32_t *plan, int E, int64_t n, int k1, const float *w,
                             uint16_t *abf, hipStream_t s);
hipError_t launch_down_mma(const uint16_t *abf, int H, const uint16_t *Wd, int I,
                           const int32_t *plan, int E, int64_t n, uint16_t *zbf, hipStream_t s);
// zs: the shared expert's bf16 term [T, H], or NULL
hipError_t launch_combine_bf16(const uint16_t *zbf, const uint16_t *zs, int64_t T, int H, int k1,
                               uint16_t *y, hipStream_t s);

// ---- channel top-k inside the activated experts
bool channel_select_supported(int k1, int I);
template <typename WT>
hipError_t launch_down_column_norms(const WT *Wd, int E, int H, int I, float *dn, hipStream_t s);
// zeroes every activation of abuf [T*k1, I] outside each token's top-keep
// channels by score dn[e, c] * |a|; optional scores and kept flags [T, k1*I],
// and the kept list [T, keep] of (row e*I + c of the column copy, activation)
// in flat-channel order
hipError_t launch_channel_select(float *abuf, int64_t T, int k1, int I, const int32_t *ids,
                                 const float *dn, int keep, float *scores_out, uint8_t *kept_out,
                                 uint2 *kept_list, hipStream_t s);
// the column copy WdT [E, I, H] of Wd [E, H, I]
template <typename WT>
hipError_t launch_down_columns(const WT *Wd, int E, int H, int I, WT *WdT, hipStream_t s);
// h-slices (one 16-byte chunk per lane) and list groups of the kept-channel
// down projection; its partial sums take T * groups * H floats
int kept_slices(int H, int esz);
int kept_groups(int64_t T, int H, int keep, int esz);
// y = the kept channels' columns scaled by their activations, from the list
template <typename WT, typename XT>
hipError_t launch_kept_down(const WT *WdT, int64_t T, int H, const uint2 *kept_list, int keep,
                            float *part, XT *y, hipStream_t s);

// ---- the device scratch of moe_forward_noalloc (noalloc.hip)
size_t noalloc_scratch_bytes();
// The current device's scratch address; the first call on a device takes it
// with hipGetSymbolAddress and zero-fills its first zero_prefix bytes on s.
hipError_t noalloc_scratch(void **ptr, size_t zero_prefix, hipStream_t s);

// word of the sync region used as the route kernel's ticket
constexpr int kRouteTicketWord = 1024;
// Small batches: router and route in one launch (router_route_supported(H),
// 2 <= T <= kRouteBatchMax; a bf16 router weight (wr_bf16, bf16 x) when H is
// a multiple of 1024: logits rounded to bf16, no bias, weights rounded to
// bf16).  The router blocks
// publish the logits as tagged words in tl, a fixed region of
// kRouteBatchTlBytes after the one-token layer's (token t's E logits at
// word t * kMaxExperts); the call's tag comes from the epoch word of sync,
// which the gate/up launch that follows advances (launch_gateup's epoch
// argument).  A route block's wait for its token's logits gives up after
// spin_limit re-reads and sets the error word (withhold: every wait gives
// up, a test hook).
constexpr int kRouteBatchMax = 64;
constexpr size_t kRouteBatchTlBytes = (size_t)kRouteBatchMax * kMaxExperts * 8;
bool router_route_batch_supported(int64_t T, int H, bool wr_bf16);
template <typename XT>
hipError_t launch_router_route_batch(const XT *x, int64_t T, int H, const void *Wr, bool wr_bf16,
                                     const float *br, int E, int k1, int k2, float *logits,
                                     float *logits2, int32_t *ids, float *w, int32_t *ids2,
                                     float *w2, int32_t *sync, uint64_t *tl, uint32_t spin_limit,
                                     bool withhold, hipStream_t s);
// Batches of at most kIdsMax assignments (T*k1) need no plan: the gate/up
// and down blocks find their work from the ids.
constexpr int kIdsMax = 64;

// Grouped gate/up and down over the plan's experts, or with ids != NULL
// (n_assign <= kIdsMax, where gateup_takes_ids / down_takes_ids) over the
// experts the ids name, without a plan; with Sg (Sd) the same launch also
// runs the shared expert as a one-expert layer (plan_s, factors gs,
// activations abuf_s [T, Is], outputs zbuf_s [T, H]).
template <typename WT, typename XT>
bool gateup_takes_ids(int H);
template <typename WT>
bool down_takes_ids(int I, int Is);

template <typename WT, typename XT>
hipError_t launch_gateup(const XT *x, int H, const WT *Wg, const WT *Wu, int I,
                         const int32_t *plan, int E, int64_t n_assign, int k1, const float *w,
                         float *abuf, hipStream_t s, const WT *Sg = nullptr,
                         const WT *Su = nullptr, int Is = 0, const int32_t *plan_s = nullptr,
                         const float *gs = nullptr, float *abuf_s = nullptr,
                         const int32_t *ids = nullptr, int32_t *epoch = nullptr);

template <typename WT>
hipError_t launch_down(const WT *Wd, int H, int I, const int32_t *plan, int E, int64_t n_assign,
                       const float *abuf, float *zbuf, hipStream_t s, const WT *Sd = nullptr,
                       int Is = 0, const int32_t *plan_s = nullptr,
                       const float *abuf_s = nullptr, float *zbuf_s = nullptr,
                       const int32_t *ids = nullptr);

// zs: the shared expert's term [T, H], or NULL
template <typename XT>
hipError_t launch_combine(const float *zbuf, const float *zs, int64_t T, int H, int k1, XT *y,
                          hipStream_t s);

// ---- shared expert as a one-expert layer: its plan (grouped layout, E = 1),
// zero ids for the prefill plan, and the per-token factor
size_t shared_plan_words(int64_t T);
template <typename XT>
hipError_t launch_shared_prep(const XT *x, int64_t T, int H, const float *sgw, int32_t *plan,
                              int32_t *ids0, float *gs, hipStream_t s);


}  // namespace moe
