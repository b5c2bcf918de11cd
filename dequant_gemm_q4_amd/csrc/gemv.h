// Decode-kernel (M = 1) launcher with the residual connection fused into the
// staging of x (gemv.hip).  Arguments are validated on the host (dmq_api.cpp)
// before it is called.
#pragma once

#include "dmq_common.h"

namespace dmq {

// As launch_gemv with every problem's g and eps set, but x = h_in + h_add in
// fp32 (x of the problems is not read): each workgroup forms the sum and its
// RMSNorm while it stages x, and one workgroup writes the sum to h_out (fp32)
// and, where problem 0 has xn set, the normalized fp16 row.  h_out must not
// overlap h_in or h_add: other workgroups still read them.
hipError_t launch_gemv_residual(const GemmProblem* probs, int count, const float* h_in, const float* h_add,
                                float* h_out, hipStream_t s);

}  // namespace dmq
