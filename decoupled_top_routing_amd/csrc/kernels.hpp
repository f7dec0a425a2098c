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

// Byte offsets of the fused decode kernel's buffers in the workspace.
struct DecodeLayout {
  size_t sync, logits, abuf, total;
};
size_t fused_decode_workspace(int64_t T, int H, int E, int I, int k1, DecodeLayout *L);
bool fused_decode_supported(int64_t T, int H, int E, int I, int k1, bool bf16);

template <typename WT, typename XT>
hipError_t launch_fused_decode(const XT *x, int64_t T, int H, const float *Wr, const float *br,
                               int E, const WT *Wg, const WT *Wu, const WT *Wd, int I, int k1,
                               int k2, XT *y, float *logits_out, int32_t *ids_out, float *w_out,
                               char *ws, hipStream_t s);

hipError_t launch_route(const float *logits, int64_t T, int E, int k1, int k2, int32_t *ids,
                        float *w, int32_t *ids2, float *w2, hipStream_t s);

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
struct B1Layout {
  size_t tl, tp, cnt, started, abuf, total;  // byte offsets in the path's region
  int64_t tp_rep_words;
};
// m = pieces of I channels of the shared expert (0 without one)
bool decode_b1_supported(int H, int I, int k1, bool bf16, int m);
B1Layout decode_b1_layout(int H, int E, int I, int k1, bool bf16, int m);
template <typename WT, typename XT>
hipError_t launch_decode_b1(const XT *x, int H, const void *Wr, bool router_bf16, const float *br,
                            int E, const WT *Wg, const WT *Wu, const WT *Wd, int I, int k1,
                            int k2, const WT *Sg, const WT *Su, const WT *Sd, int Is,
                            const float *sgw, XT *y, float *logits_out, int32_t *ids_out,
                            float *w_out, int32_t *sync, char *region, hipStream_t s);

// ---- prefill (bf16 MFMA) path
bool prefill_supported(int H, int I, bool bf16);
size_t prefill_plan_words(int64_t n, int E);
hipError_t launch_split_router(const float *Wr, int E, int H, uint16_t *w3, hipStream_t s);
// nterms bf16 terms of the router weight; with one term the logits are
// written directly, rounded to bf16 (the bf16 router), else the partial sums
hipError_t launch_router_mma(const uint16_t *x, int64_t T, int H, const uint16_t *w3, int E,
                             int nterms, float *part, float *logits, float *logits2,
                             hipStream_t s);
hipError_t launch_router_sum(const float *part, int64_t T, int E, const float *br, float *logits,
                             float *logits2, hipStream_t s);
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
// channels by score dn[e, c] * |a|; optional scores and kept flags [T, k1*I]
hipError_t launch_channel_select(float *abuf, int64_t T, int k1, int I, const int32_t *ids,
                                 const float *dn, int keep, float *scores_out, uint8_t *kept_out,
                                 hipStream_t s);

// word of the sync region used as the route kernel's ticket
constexpr int kRouteTicketWord = 1024;

// Grouped gate/up and down over the plan's experts; with Sg (Sd) the same
// launch also runs the shared expert as a one-expert layer (plan_s, factors
// gs, activations abuf_s [T, Is], outputs zbuf_s [T, H]).
template <typename WT, typename XT>
hipError_t launch_gateup(const XT *x, int H, const WT *Wg, const WT *Wu, int I,
                         const int32_t *plan, int E, int64_t n_assign, int k1, const float *w,
                         float *abuf, hipStream_t s, const WT *Sg = nullptr,
                         const WT *Su = nullptr, int Is = 0, const int32_t *plan_s = nullptr,
                         const float *gs = nullptr, float *abuf_s = nullptr);

template <typename WT>
hipError_t launch_down(const WT *Wd, int H, int I, const int32_t *plan, int E, int64_t n_assign,
                       const float *abuf, float *zbuf, hipStream_t s, const WT *Sd = nullptr,
                       int Is = 0, const int32_t *plan_s = nullptr,
                       const float *abuf_s = nullptr, float *zbuf_s = nullptr);

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
