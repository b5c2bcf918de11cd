// Launchers of the attention side of a decoder layer (attention.hip): RoPE +
// KV-cache append, grouped-query attention over the cache, residual add fused
// with RMSNorm.  Head dimension 128.  Arguments are validated on the host
// (dmq_api.cpp) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmq {

hipError_t launch_rope_kv(const float* q, const float* k, const float* v, const float* ff, void* q_out, void* k_cache,
                          void* v_cache, double theta, int64_t cache_len, int64_t M, int64_t pos0, int hq, int hkv,
                          hipStream_t s);
hipError_t launch_attention(const void* q, const void* k_cache, const void* v_cache, void* out, int64_t cache_len,
                            int64_t M, int64_t pos0, int hq, int hkv, hipStream_t s);
hipError_t launch_residual_rmsnorm(const float* h_in, const float* y, const float* g, float eps, float* h_out,
                                   void* xn, int64_t M, int64_t K, hipStream_t s);

}  // namespace dmq
