// Host-side argument check of dmq_layer_prefill (dmq_api.cpp).
#pragma once

#include "../../include/dmq.h"

#include <stdint.h>

namespace dmq {

// DMQ_OK, or the status the first failing requirement of the layer's single
// calls (for all M rows) or an overlap of a written buffer would produce.
int check_layer(const dmq_layer_weights* w, const dmq_layer_buffers* b, int64_t M, int64_t pos0, int32_t D,
                int32_t F, int32_t hq, int32_t hkv, int64_t cache_len, double theta, float eps);

}  // namespace dmq
