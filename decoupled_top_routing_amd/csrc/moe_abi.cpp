// C ABI of libmoe.so: argument checks, workspace layout and dispatch.
// The declarations and the contract of each entry point are in include/moe.h.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(MOE_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// The shared expert of moe_forward_shared (Sg == NULL: none).
struct Shared {
  const void *Sg = nullptr, *Su = nullptr, *Sd = nullptr;
  int32_t Is = 0;
  const float *sgw = nullptr;
};

// Channel top-k of moe_forward_channel_topk (dn == NULL: off).
struct ChannelTopk {
  const float *dn = nullptr;
  int32_t keep = 0;
  float *scores_out = nullptr;
  uint8_t *kept_out = nullptr;
  const void *cols = nullptr;  // column copy of the down weights, or NULL
};

// Extra workspace of channel top-k with the column copy: the kept list
// [T, keep] of 8-byte entries and the kept-down partial sums [T, groups, H].
struct TopkLayout {
  size_t list, part, total;
};
TopkLayout topk_layout(size_t base, int64_t T, int32_t H, int32_t I, int32_t k1, int esz) {
  TopkLayout L;
  size_t o = base;
  L.list = o;
  o += round256((size_t)T * k1 * I * 8);
  L.part = o;
  const int G = moe::kept_groups(T, H, k1 * I, esz);
  o += round256((size_t)T * G * H * 4);
  L.total = o;
  return L;
}

// pieces of I channels the one-launch kernel splits the shared expert into
// (0: none, or Is not a multiple of I)
int shared_pieces(int32_t I, int32_t Is) { return Is > 0 && Is % I == 0 ? Is / I : 0; }

// Workspace layout of moe_forward (each segment 256-byte aligned).
struct Layout {
  size_t logits, ids, w, plan, abuf, zbuf, abuf_b1, plan_s, gs, abuf_s, zbuf_s, total;
};

// Every workspace starts with the sync region, then the one-token kernel's
// fixed tagged region; the per-call buffers follow.
constexpr size_t kFixedBytes =
    moe::kSyncRegionBytes + moe::kB1RegionBytes + moe::kRouteBatchTlBytes;

Layout layout(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1, int32_t Is) {
  Layout L;
  size_t o = kFixedBytes;
  const size_t n_assign = (size_t)T * (size_t)k1;
  L.logits = o;
  o += round256((size_t)T * E * 4);
  L.ids = o;
  o += round256(n_assign * 4);
  L.w = o;
  o += round256(n_assign * 4);
  L.plan = o;
  o += round256((4 + (size_t)E + (size_t)E + 1 + n_assign) * 4);
  L.abuf = o;
  o += round256(n_assign * (size_t)I * 4);
  L.zbuf = o;
  o += round256(n_assign * (size_t)H * 4);
  L.abuf_b1 = o;
  o += moe::decode_b1_abuf_bytes(I, k1, false, shared_pieces(I, Is));
  L.plan_s = L.gs = L.abuf_s = L.zbuf_s = o;
  if (Is > 0) {
    L.plan_s = o;
    o += round256(moe::shared_plan_words(T) * 4);
    L.gs = o;
    o += round256((size_t)T * 4);
    L.abuf_s = o;
    o += round256((size_t)T * Is * 4);
    L.zbuf_s = o;
    o += round256((size_t)T * H * 4);
  }
  L.total = o;
  return L;
}

// Workspace layout of the prefill path.
struct PrefillLayout {
  size_t logits, ids, w, plan, w3, abf, zbf, ids_s, plan_s, gs, abf_s, zbf_s, total;
};

PrefillLayout prefill_layout(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1, int32_t Is) {
  PrefillLayout L;
  size_t o = kFixedBytes;
  const size_t n = (size_t)T * (size_t)k1;
  L.logits = o;
  o += round256((size_t)T * E * 4);
  L.ids = o;
  o += round256(n * 4);
  L.w = o;
  o += round256(n * 4);
  L.plan = o;
  o += round256(moe::prefill_plan_words((int64_t)n, E) * 4);
  L.w3 = o;
  o += round256((size_t)3 * E * H * 2);
  L.abf = o;
  o += round256(n * (size_t)I * 2);
  L.zbf = o;
  o += round256(n * (size_t)H * 2);
  L.ids_s = L.plan_s = L.gs = L.abf_s = L.zbf_s = o;
  if (Is > 0) {
    L.ids_s = o;
    o += round256((size_t)T * 4);
    L.plan_s = o;
    o += round256(moe::prefill_plan_words(T, 1) * 4);
    L.gs = o;
    o += round256((size_t)T * 4);
    L.abf_s = o;
    o += round256((size_t)T * Is * 2);
    L.zbf_s = o;
    o += round256((size_t)T * H * 2);
  }
  L.total = o;
  return L;
}

// Largest T accepted.  With the size limits of check_sizes, every launch of
// every path stays inside the hardware's 32-bit grid size (work-items per
// launch < 2^32) and every element index inside int64.
constexpr int64_t kMaxT = int64_t(1) << 18;

int check_route_args(int64_t T, int32_t E, int32_t k1, int32_t k2) {
  if (T < 0 || T > kMaxT) return fail(MOE_EINVAL, "T=%lld out of [0, %lld]", (long long)T, (long long)kMaxT);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "E=%d out of [1, %d]", E, MOE_MAX_EXPERTS);
  if (k1 < 1 || k1 > E) return fail(MOE_EINVAL, "k1=%d out of [1, E=%d]", k1, E);
  if (k2 < k1) return fail(MOE_EINVAL, "k2=%d < k1=%d", k2, k1);
  return MOE_OK;
}

// Work-items of the largest MFMA launch of the prefill path (a grouped GEMM
// over n assignments of at most E experts, N columns of width 64 or 128).
int64_t prefill_grid_items(int64_t n, int32_t E, int32_t N) {
  const int64_t u = n < E ? n : E;
  return ((n + 127) / 128 + u + 8) * ((N + 63) / 64) * 256;
}

// Size limits beyond the per-argument ranges: the per-expert launches
// (E*H and E*I work-items, a few per element), the elementwise ones (T*H)
// and the prefill GEMMs.
int check_sizes(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1, int32_t Is) {
  constexpr int64_t kGrid = int64_t(1) << 32;
  if ((int64_t)E * H > (int64_t(1) << 25) || (int64_t)E * I > (int64_t(1) << 25))
    return fail(MOE_EINVAL, "E*H=%lld and E*I=%lld must not exceed 2^25", (long long)E * H,
                (long long)E * I);
  if (T * H > (int64_t(1) << 28) || T * Is > (int64_t(1) << 28) || T * E > (int64_t(1) << 28))
    return fail(MOE_EINVAL, "T*H, T*E and T*Is must not exceed 2^28 (T=%lld H=%d E=%d Is=%d)",
                (long long)T, H, E, Is);
  const int32_t N = H > I ? H : I;
  if (prefill_grid_items(T * k1, E, N) >= kGrid ||
      (Is > 0 && prefill_grid_items(T, 1, H > Is ? H : Is) >= kGrid))
    return fail(MOE_EINVAL, "T*k1=%lld is too large for one call at H=%d I=%d", (long long)(T * k1),
                H, I);
  return MOE_OK;
}

enum class Path { Single, Grouped, Prefill };

// The expert projections run as MFMA GEMMs from kPrefillMinAssign
// assignments (T * k1) on, when the experts get two rows each on average;
// below that the grouped GEMV path reads the same weights faster (measured:
// the H=2048/E=128/I=768 layer crosses over between 384 and 512 assignments,
// and the E=512 layer at 640 assignments stays faster on the GEMV path).
constexpr int64_t kPrefillMinAssign = 512;

// The grouped multi-kernel path is the default below the prefill rule; one
// token takes the single-launch kernel (decided by the caller).
int choose_path(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1, int32_t Is, bool bf16,
                uint32_t flags, Path *path) {
  const bool prefill_ok =
      moe::prefill_supported(H, I, bf16) && (Is == 0 || moe::prefill_supported(H, Is, bf16));
  if (flags & MOE_FLAG_FORCE_PREFILL) {
    if (!prefill_ok)
      return fail(MOE_ENOTSUP,
                  "the prefill path takes bf16, H % 128 == 0 and I % 64 == 0 (and Is % 64 == 0)");
    *path = Path::Prefill;
    return MOE_OK;
  }
  if (flags & MOE_FLAG_FORCE_GROUPED) {
    *path = Path::Grouped;
    return MOE_OK;
  }
  const int64_t n = T * k1;
  *path = (prefill_ok && n >= kPrefillMinAssign && n >= 2 * (int64_t)E) ? Path::Prefill
                                                                        : Path::Grouped;
  return MOE_OK;
}

size_t workspace_bytes_for(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1, int32_t Is) {
  const size_t b = layout(T, H, E, I, k1, Is).total;
  const size_t c = prefill_layout(T, H, E, I, k1, Is).total;
  return c > b ? c : b;
}

// ---- launches of one moe_forward call, with the profiling aid of
// moe_profile_launch: the armed launch is bracketed by two events.
thread_local int g_prof_launch = -1;
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
thread_local char g_prof_name[64] = "";
// test hook of moe_debug_withhold_route: one-token calls left on this thread
// that withhold their route, and the wait limit they use
thread_local int g_withhold_calls = 0;
thread_local uint32_t g_withhold_spin = 0;

struct Launches {
  hipStream_t s;
  int n, prof;
  hipEvent_t start, stop;
  uint32_t spin_limit = moe::kDefaultSpinLimit;
  bool withhold_route = false;
  explicit Launches(hipStream_t st) : s(st), n(0), prof(g_prof_launch), start(g_prof_start),
                                      stop(g_prof_stop) {
    g_prof_launch = -1;  // one call only
    g_prof_name[0] = 0;
  }
  template <typename F>
  int operator()(const char *name, F &&launch) {
    const bool p = n == prof && start && stop;
    if (p && hipEventRecord(start, s) != hipSuccess) return hip_fail(hipGetLastError(), "event");
    const hipError_t e = launch();
    if (p) {
      if (hipEventRecord(stop, s) != hipSuccess) return hip_fail(hipGetLastError(), "event");
      snprintf(g_prof_name, sizeof g_prof_name, "%s", name);
    }
    ++n;
    return e == hipSuccess ? MOE_OK : hip_fail(e, name);
  }
};

#define RUN(name, expr)                               \
  do {                                                \
    const int rc_ = run(name, [&] { return (expr); }); \
    if (rc_ != MOE_OK) return rc_;                    \
  } while (0)

int forward_prefill(const uint16_t *x, int64_t T, int32_t H, const void *Wr, bool router_bf16,
                    const float *br, int32_t E, const uint16_t *Wg, const uint16_t *Wu,
                    const uint16_t *Wd, int32_t I, int32_t k1, int32_t k2, const Shared &sh,
                    uint16_t *y, float *logits_out, int32_t *ids_out, float *w_out, char *ws,
                    Launches &run) {
  const PrefillLayout L = prefill_layout(T, H, E, I, k1, sh.Is);
  float *logits = reinterpret_cast<float *>(ws + L.logits);
  int32_t *ids = reinterpret_cast<int32_t *>(ws + L.ids);
  float *w = reinterpret_cast<float *>(ws + L.w);
  int32_t *plan = reinterpret_cast<int32_t *>(ws + L.plan);
  uint16_t *abf = reinterpret_cast<uint16_t *>(ws + L.abf);
  uint16_t *zbf = reinterpret_cast<uint16_t *>(ws + L.zbf);
  const int64_t n = T * k1;
  const hipStream_t s = run.s;
  if (router_bf16) {
    RUN("router_mma", moe::launch_router_mma(x, T, H, static_cast<const uint16_t *>(Wr), E, 1,
                                             nullptr, logits, logits_out, s));
  } else {
    uint16_t *w3 = reinterpret_cast<uint16_t *>(ws + L.w3);
    RUN("split_router", moe::launch_split_router(static_cast<const float *>(Wr), E, H, w3, s));
    RUN("router_mma", moe::launch_router_mma(x, T, H, w3, E, 3, br, logits, logits_out, s));
  }
  RUN("route", moe::launch_route_plan(logits, T, E, k1, k2, ids, w, ids_out, w_out, nullptr,
                                      nullptr, router_bf16, s));
  RUN("prefill_plan", moe::launch_prefill_plan(ids, n, E, plan, s));
  RUN("gateup_mma", moe::launch_gateup_mma(x, H, Wg, Wu, I, plan, E, n, k1, w, abf, s));
  RUN("down_mma", moe::launch_down_mma(abf, H, Wd, I, plan, E, n, zbf, s));
  uint16_t *zbf_s = nullptr;
  if (sh.Sg) {
    // the shared expert as a one-expert layer over every token
    int32_t *ids_s = reinterpret_cast<int32_t *>(ws + L.ids_s);
    int32_t *plan_s = reinterpret_cast<int32_t *>(ws + L.plan_s);
    float *gs = reinterpret_cast<float *>(ws + L.gs);
    uint16_t *abf_s = reinterpret_cast<uint16_t *>(ws + L.abf_s);
    zbf_s = reinterpret_cast<uint16_t *>(ws + L.zbf_s);
    RUN("shared_prep", moe::launch_shared_prep<moe::bf16_t>(
                           reinterpret_cast<const moe::bf16_t *>(x), T, H, sh.sgw, nullptr, ids_s,
                           gs, s));
    RUN("shared_plan", moe::launch_prefill_plan(ids_s, T, 1, plan_s, s));
    RUN("shared_gateup_mma",
        moe::launch_gateup_mma(x, H, static_cast<const uint16_t *>(sh.Sg),
                               static_cast<const uint16_t *>(sh.Su), sh.Is, plan_s, 1, T, 1, gs,
                               abf_s, s));
    RUN("shared_down_mma", moe::launch_down_mma(abf_s, H, static_cast<const uint16_t *>(sh.Sd),
                                                sh.Is, plan_s, 1, T, zbf_s, s));
  }
  RUN("combine", moe::launch_combine_bf16(zbf, zbf_s, T, H, k1, y, s));
  return MOE_OK;
}

template <typename WT, typename XT>
int forward_typed(const XT *x, int64_t T, int32_t H, const void *Wr, bool router_bf16,
                  const float *br, int32_t E, const WT *Wg, const WT *Wu, const WT *Wd, int32_t I,
                  int32_t k1, int32_t k2, const Shared &sh, const ChannelTopk &ck, XT *y,
                  float *logits_out, int32_t *ids_out, float *w_out, Path path, char *ws,
                  const Layout &L, Launches &run) {
  const hipStream_t s = run.s;
  const float *Wr32 = static_cast<const float *>(Wr);  // meaningful without router_bf16
  if constexpr (sizeof(WT) == 2) {
    if (path == Path::Prefill)
      return forward_prefill(reinterpret_cast<const uint16_t *>(x), T, H, Wr, router_bf16, br, E,
                             reinterpret_cast<const uint16_t *>(Wg),
                             reinterpret_cast<const uint16_t *>(Wu),
                             reinterpret_cast<const uint16_t *>(Wd), I, k1, k2, sh,
                             reinterpret_cast<uint16_t *>(y), logits_out, ids_out, w_out, ws, run);
  }
  float *logits = reinterpret_cast<float *>(ws + L.logits);
  int32_t *ids = reinterpret_cast<int32_t *>(ws + L.ids);
  float *w = reinterpret_cast<float *>(ws + L.w);
  int32_t *plan = reinterpret_cast<int32_t *>(ws + L.plan);
  float *abuf = reinterpret_cast<float *>(ws + L.abuf);
  float *zbuf = reinterpret_cast<float *>(ws + L.zbuf);
  int32_t *sync = reinterpret_cast<int32_t *>(ws);
  const int64_t n_assign = T * k1;
  int32_t *ticket = sync + moe::kRouteTicketWord;
  const WT *Sg = static_cast<const WT *>(sh.Sg), *Su = static_cast<const WT *>(sh.Su),
           *Sd = static_cast<const WT *>(sh.Sd);
  // the launches with a bounded wait inside: the one-token kernel and the
  // small-batch router + route
  const bool batch_route = path != Path::Single && (!router_bf16 || sizeof(XT) == 2) &&
                           moe::router_route_batch_supported(T, H, router_bf16);
  if ((path == Path::Single || batch_route) && g_withhold_calls > 0) {
    --g_withhold_calls;
    run.withhold_route = true;
    run.spin_limit = g_withhold_spin;
  }
  if (path == Path::Single) {
    RUN("b1_layer", (moe::launch_decode_b1<WT, XT>(x, H, Wr, router_bf16, br, E, Wg, Wu, Wd, I,
                                                   k1, k2, Sg, Su, Sd, sh.Is, sh.sgw, y,
                                                   logits_out, ids_out, w_out, sync,
                                                   ws + moe::kSyncRegionBytes, ws + L.abuf_b1,
                                                   run.spin_limit, run.withhold_route, s)));
    return MOE_OK;
  }
  // 2..kIdsMax assignments of two or more tokens: no plan; up to
  // kRouteBatchMax tokens: router and route in one launch
  const bool by_ids = T >= 2 && n_assign <= moe::kIdsMax && moe::gateup_takes_ids<WT, XT>(H) &&
                      moe::down_takes_ids<WT>(I, Sg ? sh.Is : 0);
  if (batch_route) {
    RUN("router_route",
        moe::launch_router_route_batch<XT>(
            x, T, H, Wr, router_bf16, br, E, k1, k2, logits, logits_out, ids, w, ids_out, w_out, sync,
            reinterpret_cast<uint64_t *>(ws + moe::kSyncRegionBytes + moe::kB1RegionBytes),
            run.spin_limit, run.withhold_route, s));
    if (!by_ids) RUN("plan", moe::launch_plan(ids, n_assign, E, plan, s));
  } else if (by_ids) {
    if (router_bf16) {
      if constexpr (sizeof(XT) == 2)
        RUN("router", moe::launch_router_bf16(x, T, H, static_cast<const moe::bf16_t *>(Wr), E,
                                              logits, logits_out, s));
    } else {
      RUN("router", moe::launch_router<XT>(x, T, H, Wr32, br, E, logits, logits_out, s));
    }
    RUN("route", moe::launch_route_plan(logits, T, E, k1, k2, ids, w, ids_out, w_out, nullptr,
                                        nullptr, router_bf16, s));
  } else if (T == 1 && !router_bf16 && moe::router_route_supported(H)) {
    RUN("router_route", moe::launch_router_route<XT>(x, H, Wr32, br, E, k1, k2, logits,
                                                     logits_out, ids, w, ids_out, w_out, plan,
                                                     ticket, s));
    if (n_assign > 64) RUN("plan", moe::launch_plan(ids, n_assign, E, plan, s));
  } else {
    if (router_bf16) {
      if constexpr (sizeof(XT) == 2)
        RUN("router", moe::launch_router_bf16(x, T, H, static_cast<const moe::bf16_t *>(Wr), E,
                                              logits, logits_out, s));
    } else {
      RUN("router", moe::launch_router<XT>(x, T, H, Wr32, br, E, logits, logits_out, s));
    }
    if (n_assign <= 64) {
      RUN("route_plan", moe::launch_route_plan(logits, T, E, k1, k2, ids, w, ids_out, w_out, plan,
                                               ticket, router_bf16, s));
    } else {
      RUN("route", moe::launch_route_plan(logits, T, E, k1, k2, ids, w, ids_out, w_out, nullptr,
                                          nullptr, router_bf16, s));
      RUN("plan", moe::launch_plan(ids, n_assign, E, plan, s));
    }
  }
  // the shared expert runs as a one-expert layer over every token, inside
  // the routed gate/up and down launches
  int32_t *plan_s = nullptr;
  float *gs = nullptr, *abuf_s = nullptr, *zbuf_s = nullptr;
  if (Sg) {
    plan_s = reinterpret_cast<int32_t *>(ws + L.plan_s);
    gs = reinterpret_cast<float *>(ws + L.gs);
    abuf_s = reinterpret_cast<float *>(ws + L.abuf_s);
    zbuf_s = reinterpret_cast<float *>(ws + L.zbuf_s);
    RUN("shared_prep", moe::launch_shared_prep<XT>(x, T, H, sh.sgw, plan_s, nullptr, gs, s));
  }
  RUN("gateup", (moe::launch_gateup<WT, XT>(x, H, Wg, Wu, I, plan, E, n_assign, k1, w, abuf, s,
                                            Sg, Su, sh.Is, plan_s, gs, abuf_s,
                                            by_ids ? ids : nullptr,
                                            batch_route ? sync + moe::kEpochWord : nullptr)));
  if (ck.dn) {
    uint2 *kept_list = nullptr;
    float *part = nullptr;
    if (ck.cols) {
      const TopkLayout K = topk_layout(L.total, T, H, I, k1, (int)sizeof(WT));
      kept_list = reinterpret_cast<uint2 *>(ws + K.list);
      part = reinterpret_cast<float *>(ws + K.part);
    }
    RUN("channel_select", moe::launch_channel_select(abuf, T, k1, I, ids, ck.dn, ck.keep,
                                                     ck.scores_out, ck.kept_out, kept_list, s));
    if (ck.cols) {
      // the down projection reads only the kept channels' columns
      RUN("kept_down", (moe::launch_kept_down<WT, XT>(static_cast<const WT *>(ck.cols), T, H,
                                                      kept_list, ck.keep, part, y, s)));
      return MOE_OK;
    }
  }
  const int ncd = (int)((I * sizeof(WT) / 16 + 63) / 64);
  if (T == 1 && ncd <= 2 && !Sg) {
    RUN("down_one_token", (moe::launch_down_one_token<WT, XT>(Wd, H, I, plan, E, abuf, y, s)));
    return MOE_OK;
  }
  RUN("down", moe::launch_down<WT>(Wd, H, I, plan, E, n_assign, abuf, zbuf, s, Sd, sh.Is, plan_s,
                                   abuf_s, zbuf_s, by_ids ? ids : nullptr));
  RUN("combine", moe::launch_combine<XT>(zbuf, zbuf_s, T, H, k1, y, s));
  return MOE_OK;
}

#undef RUN

// MOE_DEBUG set (and not "0") in the environment: every forward call waits
// for its work and checks the device status word (not under graph capture).
bool debug_checks() {
  static const bool on = [] {
    const char *v = getenv("MOE_DEBUG");
    return v != nullptr && *v != 0 && strcmp(v, "0") != 0;
  }();
  return on;
}

// Wait for the stream, read the error word of the workspace's sync region
// and reset it: MOE_EDEVICE if a hand-over wait gave up since the last check.
// A wait that gave up can leave a count of the sync region off zero, so the
// reset clears every word of the region but the epoch.
int take_device_status(char *ws, hipStream_t s) {
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws + 4 * moe::kErrorWord, sizeof v, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "read of the device status word");
  if (v == 0) return MOE_OK;
  static const int32_t zeros[moe::kSyncRegionBytes / 4] = {};
  e = hipMemcpyAsync(ws + 4, zeros, moe::kSyncRegionBytes - 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reset of the device status word");
  return fail(MOE_EDEVICE,
              "a hand-over wait inside the layer kernel gave up: the outputs of a call on this "
              "workspace since the last check are unspecified");
}

// moe_forward and moe_forward_shared: argument checks, then the path.
int forward_impl(const void *x, int32_t act_dtype, int64_t T, int32_t H, const void *Wr,
                 const float *br, int32_t E, const void *Wgate, const void *Wup,
                 const void *Wdown, int32_t w_dtype, int32_t I, int32_t k1, int32_t k2,
                 const Shared &sh, const ChannelTopk &ck, void *y, float *logits_out,
                 int32_t *ids_out, float *w_out, uint32_t flags, void *workspace,
                 size_t workspace_bytes, void *stream) {
  int rc = check_route_args(T, E, k1, k2);
  if (rc != MOE_OK) return rc;
  if (H < 8 || H % 8 != 0) return fail(MOE_EINVAL, "H=%d must be a positive multiple of 8", H);
  if (I < 8 || I % 8 != 0) return fail(MOE_EINVAL, "I=%d must be a positive multiple of 8", I);
  if ((int64_t)H * I > (int64_t(1) << 31))
    return fail(MOE_EINVAL, "H*I=%lld exceeds 2^31", (long long)H * I);
  if (sh.Sg && (sh.Is < 8 || sh.Is % 8 != 0 || (int64_t)H * sh.Is > (int64_t(1) << 31)))
    return fail(MOE_EINVAL, "Is=%d must be a positive multiple of 8 with H*Is <= 2^31", sh.Is);
  if ((rc = check_sizes(T, H, E, I, k1, sh.Sg ? sh.Is : 0)) != MOE_OK) return rc;
  const uint32_t paths = MOE_FLAG_FORCE_GROUPED | MOE_FLAG_FORCE_PREFILL;
  if (flags & ~(paths | MOE_FLAG_ROUTER_BF16))
    return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
  if (__builtin_popcount(flags & paths) > 1)
    return fail(MOE_EINVAL, "more than one path flag set");
  const bool router_bf16 = (flags & MOE_FLAG_ROUTER_BF16) != 0;
  const bool f32 = act_dtype == MOE_F32 && w_dtype == MOE_F32;
  const bool b16 = act_dtype == MOE_BF16 && w_dtype == MOE_BF16;
  if (!f32 && !b16)
    return fail(MOE_ENOTSUP, "dtype pair (act=%d, w=%d) not supported", act_dtype, w_dtype);
  if (router_bf16 && !b16)
    return fail(MOE_ENOTSUP, "the bf16 router takes bf16 activations and weights");
  if (router_bf16 && br)
    return fail(MOE_EINVAL, "the bf16 router takes no bias (br must be NULL)");
  if (ck.dn) {
    if (!moe::channel_select_supported(k1, I))
      return fail(MOE_ENOTSUP, "channel top-k takes k1*I <= 8192 (got %lld)", (long long)k1 * I);
    if (ck.keep < 0 || (int64_t)ck.keep > (int64_t)k1 * I)
      return fail(MOE_EINVAL, "keep=%d out of [0, k1*I=%lld]", ck.keep, (long long)k1 * I);
    if (flags & MOE_FLAG_FORCE_PREFILL)
      return fail(MOE_ENOTSUP, "channel top-k runs on the grouped path only");
  }
  if (T == 0) return MOE_OK;
  if (!x || !Wr || !Wgate || !Wup || !Wdown || !y) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(Wgate, 16) || !aligned(Wup, 16) ||
      !aligned(Wdown, 16) || !aligned(y, 16))
    return fail(MOE_EALIGN, "x, Wr, Wgate, Wup, Wdown and y need 16-byte alignment");
  if (sh.Sg && (!aligned(sh.Sg, 16) || !aligned(sh.Su, 16) || !aligned(sh.Sd, 16)))
    return fail(MOE_EALIGN, "Sgate, Sup and Sdown need 16-byte alignment");
  if ((br && !aligned(br, 4)) || (logits_out && !aligned(logits_out, 4)) ||
      (ids_out && !aligned(ids_out, 4)) || (w_out && !aligned(w_out, 4)) ||
      (sh.sgw && !aligned(sh.sgw, 4)))
    return fail(MOE_EALIGN, "br, sgate and the route outputs need 4-byte alignment");
  if (ck.cols && !aligned(ck.cols, 16))
    return fail(MOE_EALIGN, "Wdown_cols needs 16-byte alignment");
  if ((ck.dn && !aligned(ck.dn, 16)) || (ck.scores_out && !aligned(ck.scores_out, 16)) ||
      (ck.kept_out && !aligned(ck.kept_out, 8)))
    return fail(MOE_EALIGN, "dnorm and scores_out need 16-byte, kept_out 8-byte alignment");
  const Layout L = layout(T, H, E, I, k1, sh.Is);
  size_t need = workspace_bytes_for(T, H, E, I, k1, sh.Is);
  if (ck.cols) {
    const size_t t = topk_layout(L.total, T, H, I, k1, f32 ? 4 : 2).total;
    if (t > need) need = t;
  }
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu at %p)",
                need, workspace_bytes, workspace);
  Path path;
  if (ck.dn) {
    path = Path::Grouped;
  } else if ((rc = choose_path(T, H, E, I, k1, sh.Is, b16, flags, &path)) != MOE_OK) {
    return rc;
  }
  // one token takes the one-launch kernel unless a path is forced
  const int m = shared_pieces(I, sh.Is);
  if (path == Path::Grouped && !(flags & MOE_FLAG_FORCE_GROUPED) && T == 1 && !ck.dn &&
      (!sh.Sg || m > 0) && moe::decode_b1_supported(H, I, k1, b16, m))
    path = Path::Single;
  Launches run((hipStream_t)stream);
  char *ws = static_cast<char *>(workspace);
  if (f32)
    rc = forward_typed<float, float>(
        static_cast<const float *>(x), T, H, Wr, false, br, E, static_cast<const float *>(Wgate),
        static_cast<const float *>(Wup), static_cast<const float *>(Wdown), I, k1, k2, sh, ck,
        static_cast<float *>(y), logits_out, ids_out, w_out, path, ws, L, run);
  else
    rc = forward_typed<moe::bf16_t, moe::bf16_t>(
        static_cast<const moe::bf16_t *>(x), T, H, Wr, router_bf16, br, E,
        static_cast<const moe::bf16_t *>(Wgate), static_cast<const moe::bf16_t *>(Wup),
        static_cast<const moe::bf16_t *>(Wdown), I, k1, k2, sh, ck,
        static_cast<moe::bf16_t *>(y), logits_out, ids_out, w_out, path, ws, L, run);
  if (rc == MOE_OK && debug_checks()) rc = take_device_status(ws, (hipStream_t)stream);
  return rc;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EALIGN: return "misaligned pointer";
    case MOE_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ENOTSUP: return "unsupported dtype combination";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_EDEVICE: return "a device-side wait gave up; outputs unspecified";
    default: return "unknown status";
  }
}

const char *moe_last_error_str(void) { return g_err; }

int moe_route(const float *logits, int64_t T, int32_t E, int32_t k1, int32_t k2, int32_t *ids,
              float *weights, void *stream) {
  int rc = check_route_args(T, E, k1, k2);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !weights) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4))
    return fail(MOE_EALIGN, "logits, ids and weights need 4-byte alignment");
  hipError_t e = moe::launch_route_plan(logits, T, E, k1, k2, ids, weights, nullptr, nullptr,
                                        nullptr, nullptr, false, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "route kernel");
  return MOE_OK;
}

size_t moe_forward_workspace(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1,
                             int32_t act_dtype, int32_t w_dtype) {
  return moe_forward_shared_workspace(T, H, E, I, k1, 0, act_dtype, w_dtype);
}

size_t moe_forward_shared_workspace(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1,
                                    int32_t Is, int32_t act_dtype, int32_t w_dtype) {
  (void)act_dtype;
  (void)w_dtype;
  if (T < 0 || T > kMaxT || E < 1 || E > MOE_MAX_EXPERTS || k1 < 1 || k1 > E || H < 8 ||
      I < 8 || Is < 0 || (Is > 0 && Is < 8) || check_sizes(T, H, E, I, k1, Is) != MOE_OK)
    return 0;
  return workspace_bytes_for(T, H, E, I, k1, Is);
}

int moe_forward(const void *x, int32_t act_dtype, int64_t T, int32_t H, const void *Wr,
                const float *br, int32_t E, const void *Wgate, const void *Wup,
                const void *Wdown, int32_t w_dtype, int32_t I, int32_t k1, int32_t k2, void *y,
                float *logits_out, int32_t *ids_out, float *w_out, uint32_t flags,
                void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(x, act_dtype, T, H, Wr, br, E, Wgate, Wup, Wdown, w_dtype, I, k1, k2,
                      Shared{}, ChannelTopk{}, y, logits_out, ids_out, w_out, flags, workspace,
                      workspace_bytes, stream);
}

int moe_forward_shared(const void *x, int32_t act_dtype, int64_t T, int32_t H, const void *Wr,
                       const float *br, int32_t E, const void *Wgate, const void *Wup,
                       const void *Wdown, int32_t w_dtype, int32_t I, int32_t k1, int32_t k2,
                       const void *Sgate, const void *Sup, const void *Sdown, int32_t Is,
                       const float *sgate, void *y, float *logits_out, int32_t *ids_out,
                       float *w_out, uint32_t flags, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (!Sgate || !Sup || !Sdown) return fail(MOE_EINVAL, "NULL shared expert pointer");
  Shared sh;
  sh.Sg = Sgate;
  sh.Su = Sup;
  sh.Sd = Sdown;
  sh.Is = Is;
  sh.sgw = sgate;
  return forward_impl(x, act_dtype, T, H, Wr, br, E, Wgate, Wup, Wdown, w_dtype, I, k1, k2, sh,
                      ChannelTopk{}, y, logits_out, ids_out, w_out, flags, workspace,
                      workspace_bytes, stream);
}

int moe_down_column_norms(const void *Wdown, int32_t w_dtype, int32_t E, int32_t H, int32_t I,
                          float *dnorm, void *stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || H < 1 || I < 1 || (int64_t)H * I > (int64_t(1) << 31))
    return fail(MOE_EINVAL, "E=%d H=%d I=%d out of range", E, H, I);
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16)
    return fail(MOE_ENOTSUP, "weight dtype %d not supported", w_dtype);
  if (!Wdown || !dnorm) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned(Wdown, 16) || !aligned(dnorm, 4))
    return fail(MOE_EALIGN, "Wdown needs 16-byte and dnorm 4-byte alignment");
  const hipStream_t s = (hipStream_t)stream;
  const hipError_t e =
      w_dtype == MOE_F32
          ? moe::launch_down_column_norms(static_cast<const float *>(Wdown), E, H, I, dnorm, s)
          : moe::launch_down_column_norms(static_cast<const moe::bf16_t *>(Wdown), E, H, I,
                                          dnorm, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "down column norms");
}

int moe_down_columns(const void *Wdown, int32_t w_dtype, int32_t E, int32_t H, int32_t I,
                     void *Wdown_cols, void *stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || H < 1 || I < 1 || (int64_t)H * I > (int64_t(1) << 31))
    return fail(MOE_EINVAL, "E=%d H=%d I=%d out of range", E, H, I);
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16)
    return fail(MOE_ENOTSUP, "weight dtype %d not supported", w_dtype);
  if (!Wdown || !Wdown_cols) return fail(MOE_EINVAL, "NULL pointer");
  if (!aligned(Wdown, 16) || !aligned(Wdown_cols, 16))
    return fail(MOE_EALIGN, "Wdown and Wdown_cols need 16-byte alignment");
  const hipStream_t s = (hipStream_t)stream;
  const hipError_t e =
      w_dtype == MOE_F32
          ? moe::launch_down_columns(static_cast<const float *>(Wdown), E, H, I,
                                     static_cast<float *>(Wdown_cols), s)
          : moe::launch_down_columns(static_cast<const moe::bf16_t *>(Wdown), E, H, I,
                                     static_cast<moe::bf16_t *>(Wdown_cols), s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "down columns");
}

size_t moe_forward_channel_topk_workspace(int64_t T, int32_t H, int32_t E, int32_t I, int32_t k1,
                                          int32_t act_dtype, int32_t w_dtype) {
  const size_t base = moe_forward_workspace(T, H, E, I, k1, act_dtype, w_dtype);
  if (base == 0) return 0;
  const Layout L = layout(T, H, E, I, k1, 0);
  const size_t t = topk_layout(L.total, T, H, I, k1, w_dtype == MOE_F32 ? 4 : 2).total;
  return t > base ? t : base;
}

int moe_forward_channel_topk(const void *x, int32_t act_dtype, int64_t T, int32_t H,
                             const void *Wr, const float *br, int32_t E, const void *Wgate,
                             const void *Wup, const void *Wdown, int32_t w_dtype, int32_t I,
                             int32_t k1, int32_t k2, const float *dnorm, int32_t keep,
                             const void *Wdown_cols, void *y, float *logits_out,
                             int32_t *ids_out, float *w_out, float *scores_out,
                             uint8_t *kept_out, uint32_t flags, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (!dnorm) return fail(MOE_EINVAL, "NULL dnorm");
  ChannelTopk ck;
  ck.dn = dnorm;
  ck.keep = keep;
  ck.scores_out = scores_out;
  ck.kept_out = kept_out;
  ck.cols = Wdown_cols;
  return forward_impl(x, act_dtype, T, H, Wr, br, E, Wgate, Wup, Wdown, w_dtype, I, k1, k2,
                      Shared{}, ck, y, logits_out, ids_out, w_out, flags, workspace,
                      workspace_bytes, stream);
}

int moe_profile_launch(int32_t launch, void *start, void *stop) {
  if (launch < 0) return fail(MOE_EINVAL, "launch=%d < 0", launch);
  g_prof_launch = launch;
  g_prof_start = static_cast<hipEvent_t>(start);
  g_prof_stop = static_cast<hipEvent_t>(stop);
  return MOE_OK;
}

const char *moe_profile_launch_name(void) { return g_prof_name; }

int moe_forward_noalloc(const void *x, int32_t act_dtype, int64_t T, int32_t H, const void *Wr,
                        const float *br, int32_t E, const void *Wgate, const void *Wup,
                        const void *Wdown, int32_t w_dtype, int32_t I, int32_t k1, int32_t k2,
                        void *y, float *logits_out, int32_t *ids_out, float *w_out,
                        uint32_t flags, void *stream) {
  // argument errors (and T = 0) are returned by moe_forward's checks before
  // the scratch is touched: those sizes need no workspace
  const size_t need = moe_forward_workspace(T, H, E, I, k1, act_dtype, w_dtype);
  if (T == 0 || need == 0)
    return forward_impl(x, act_dtype, T, H, Wr, br, E, Wgate, Wup, Wdown, w_dtype, I, k1, k2,
                        Shared{}, ChannelTopk{}, y, logits_out, ids_out, w_out, flags, nullptr, 0,
                        stream);
  const size_t have = moe::noalloc_scratch_bytes();
  if (need > have)
    return fail(MOE_EWORKSPACE,
                "these sizes need %zu bytes of scratch; moe_forward_noalloc holds %zu "
                "(call moe_forward with a workspace)", need, have);
  void *ws = nullptr;
  const hipError_t e = moe::noalloc_scratch(&ws, kFixedBytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "device scratch of moe_forward_noalloc");
  return forward_impl(x, act_dtype, T, H, Wr, br, E, Wgate, Wup, Wdown, w_dtype, I, k1, k2,
                      Shared{}, ChannelTopk{}, y, logits_out, ids_out, w_out, flags, ws, have,
                      stream);
}

size_t moe_noalloc_scratch_bytes(void) { return moe::noalloc_scratch_bytes(); }

int moe_workspace_status(void *workspace, void *stream) {
  if (!workspace) return fail(MOE_EINVAL, "NULL workspace");
  if (!aligned(workspace, 256)) return fail(MOE_EWORKSPACE, "workspace must be 256-byte aligned");
  return take_device_status(static_cast<char *>(workspace), (hipStream_t)stream);
}

int moe_debug_withhold_route(int32_t calls, uint32_t spin_limit) {
  if (calls < 0 || spin_limit < 1)
    return fail(MOE_EINVAL, "calls=%d must be >= 0 and spin_limit=%u >= 1", calls, spin_limit);
  g_withhold_calls = calls;
  g_withhold_spin = spin_limit;
  return MOE_OK;
}

}  // extern "C"
