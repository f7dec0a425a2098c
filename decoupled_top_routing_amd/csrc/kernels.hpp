// Internal launchers of libmoe.so (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

constexpr int kMaxExperts = 1024;

hipError_t launch_route(const float *logits, int64_t T, int E, int k1, int k2, int32_t *ids,
                        float *w, int32_t *ids2, float *w2, hipStream_t s);

template <typename XT>
hipError_t launch_router(const XT *x, int64_t T, int H, const float *Wr, const float *br, int E,
                         float *logits, float *logits2, hipStream_t s);

hipError_t launch_plan(const int32_t *ids, int64_t n_assign, int E, int32_t *plan,
                       hipStream_t s);

template <typename WT, typename XT>
hipError_t launch_gateup(const XT *x, int H, const WT *Wg, const WT *Wu, int I,
                         const int32_t *plan, int E, int64_t n_assign, int k1, const float *w,
                         float *abuf, hipStream_t s);

template <typename WT, typename XT>
hipError_t launch_down(const WT *Wd, int64_t T, int H, int I, const int32_t *ids, int k1,
                       const float *abuf, XT *y, hipStream_t s);

}  // namespace moe
