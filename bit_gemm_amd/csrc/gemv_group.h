// Several layers in one decode launch (gemv.hip, k_gemv_r_group).
#pragma once

#include "mq_internal.h"

namespace mq {

// Up to kGroupMax layers with K = 4096, one group size, no block residual,
// and inputs of 1..16 tokens (up to 4 tokens: every layer's densest row block
// within 80 residual chunks of 32 entries) run in one launch; each output
// equals that layer's own launch bit for bit.
constexpr int kGroupMax = 8;
bool gemv_group_takes(const mq_packed* const* p, int n, int64_t M);
hipError_t launch_gemv_group(const mq_packed* const* p, const uint16_t* const* X, int64_t M, uint16_t* const* Y,
                             int n, hipStream_t s);

}  // namespace mq
