// RMSNorm of prefill activations, ahead of the Q|K|V or gate|up GEMMs: each
// decoder layer normalizes its input before the QKV projections and again
// before the feed-forward network (article "Building DAMASCUS", layer
// description; overview "[04] one decode step").  The normalized rows are
// written once as fp16, the operand type of the MFMA kernels that read them.
// (The decode kernel instead normalizes x while it stages it in LDS.)
#include "dmq_common.h"

namespace dmq {

// One workgroup per row: the sum of squares over the row (fp32, then the
// workgroup's fixed-order reduction), then x * g * r rounded to fp16.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const half_t* x, const float* g, float eps, half_t* xn,
                                                       int K) {
  __shared__ float red4[4];
  const int64_t m = blockIdx.x;
  const half_t* row = x + m * K;
  const float r = rms_inv(row, K, eps, red4);
  const uint4* xr = (const uint4*)row;
  uint4* out = (uint4*)(xn + m * K);
  for (int i = (int)threadIdx.x; i < K / 8; i += 256) out[i] = norm8(xr[i], g + 8 * i, r);
}

hipError_t launch_rmsnorm(const void* x, const float* g, float eps, void* xn, int64_t M, int64_t K, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, s, (const half_t*)x, g, eps, (half_t*)xn,
                     (int)K);
  return hipGetLastError();
}

}  // namespace dmq
