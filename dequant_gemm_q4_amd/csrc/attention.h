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
// RoPE + cache append (launch_rope_kv) followed by attention
// (launch_attention), with the same results bit for bit; at M = 1 on the
// split path both run in the pieces' kernel (no RoPE launch).
hipError_t launch_rope_attention(const float* q, const float* k, const float* v, const float* ff, void* q_out,
                                 void* k_cache, void* v_cache, void* out, double theta, int64_t cache_len, int64_t M,
                                 int64_t pos0, int hq, int hkv, hipStream_t s);
// ws: NULL, or a device buffer of at least attention_scratch_bytes(M, pos0,
// hq) bytes for the decode path's partial softmax states; NULL takes the
// stream's workspace (workspace.cpp).
hipError_t launch_attention(const void* q, const void* k_cache, const void* v_cache, void* out, int64_t cache_len,
                            int64_t M, int64_t pos0, int hq, int hkv, hipStream_t s, float* ws = nullptr);
// Bytes of partial states the decode path of these sizes writes (0: the call
// runs a path that takes no workspace).
size_t attention_scratch_bytes(int64_t M, int64_t pos0, int hq);
// This device's fixed scratch for callers that cannot allocate: its device
// address (looked up once per device) and size.
hipError_t noalloc_scratch(float** ptr, size_t* bytes);
hipError_t launch_residual_rmsnorm(const float* h_in, const float* y, const float* g, float eps, float* h_out,
                                   void* xn, int64_t M, int64_t K, hipStream_t s);

}  // namespace dmq
