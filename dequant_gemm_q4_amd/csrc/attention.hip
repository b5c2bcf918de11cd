// The attention side of a decoder layer, around the projection GEMMs: RoPE on
// the Q and K projections with the KV-cache append, grouped-query attention
// over the cache, and the residual add fused with the next RMSNorm.  The
// overview page's "[04] one decode step" chains RMSNorm -> QKV projection ->
// RoPE -> attention over the KV cache (GQA) -> residual add -> RMSNorm ->
// SwiGLU FFN -> residual add; its model table gives 24 query heads, 8 KV
// heads, head dimension 128 and RoPE theta 500000.  These kernels move a few
// MB per layer against the GEMMs' tens; they are bound by memory latency and
// bandwidth, not by the matrix units.
#include "attention.h"
#include "dmq_common.h"

#include <math.h>

namespace dmq {

constexpr int HEAD_DIM = 128;

// ------------------------------------------------------------ RoPE + cache --
// One workgroup per token.  Pair i (dims 2i, 2i+1) of every head turns by
// pos * theta^(-2i/128) / f_i: the angle is formed and reduced modulo 2 pi in
// fp64 (positions reach 10^5 and more, where an fp32 angle would be off by a
// large fraction of an fp16 step), its cosine and sine rounded to fp32, the
// rotation done in fp32 and the result rounded once to fp16.
struct RopeArgs {
  const float* q;          // [M, Hq*128] fp32 (the Q projection's y)
  const float* k;          // [M, Hkv*128]
  const float* v;          // [M, Hkv*128]
  const float* ff;         // 64 frequency factors, or NULL
  half_t* q_out;           // [M, Hq*128] fp16
  half_t* k_cache;         // [Hkv, cache_len, 128] fp16
  half_t* v_cache;
  double theta;
  int64_t cache_len;
  int32_t pos0, hq, hkv;
};

__global__ __launch_bounds__(256) void rope_kv_kernel(RopeArgs a) {
  __shared__ float cs[HEAD_DIM / 2], sn[HEAD_DIM / 2];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int64_t pos = (int64_t)a.pos0 + m;
  if (tid < HEAD_DIM / 2) {
    double inv = pow(a.theta, -2.0 * tid / HEAD_DIM);
    if (a.ff) inv /= (double)a.ff[tid];
    const double ang = remainder((double)pos * inv, 2.0 * M_PI);
    cs[tid] = (float)cos(ang);
    sn[tid] = (float)sin(ang);
  }
  __syncthreads();
  auto rot = [&](const float* src, half_t* dst, int pairs) {
    for (int p = tid; p < pairs; p += 256) {
      const int i = p & (HEAD_DIM / 2 - 1);
      const float2 x = ((const float2*)src)[p];
      const float c = cs[i], s = sn[i];
      const h2 o = {(half_t)(x.x * c - x.y * s), (half_t)(x.x * s + x.y * c)};
      ((h2*)dst)[p] = o;
    }
  };
  rot(a.q + (int64_t)m * a.hq * HEAD_DIM, a.q_out + (int64_t)m * a.hq * HEAD_DIM, a.hq * HEAD_DIM / 2);
  // K (rotated) and V go to row `pos` of each KV head's cache
  for (int h = 0; h < a.hkv; ++h) {
    const int64_t row = ((int64_t)h * a.cache_len + pos) * HEAD_DIM;
    rot(a.k + ((int64_t)m * a.hkv + h) * HEAD_DIM, a.k_cache + row, HEAD_DIM / 2);
    const float* vs = a.v + ((int64_t)m * a.hkv + h) * HEAD_DIM;
    for (int d = tid; d < HEAD_DIM / 2; d += 256) {
      const float2 x = ((const float2*)vs)[d];
      const h2 o = {(half_t)x.x, (half_t)x.y};
      ((h2*)(a.v_cache + row))[d] = o;
    }
  }
}

hipError_t launch_rope_kv(const float* q, const float* k, const float* v, const float* ff, void* q_out, void* k_cache,
                          void* v_cache, double theta, int64_t cache_len, int64_t M, int64_t pos0, int hq, int hkv,
                          hipStream_t s) {
  RopeArgs a{q, k, v, ff, (half_t*)q_out, (half_t*)k_cache, (half_t*)v_cache, theta, cache_len,
             (int32_t)pos0, hq, hkv};
  hipLaunchKernelGGL(rope_kv_kernel, dim3((unsigned)M), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- attention --
// One workgroup per (query, KV head): the G = Hq/Hkv query heads of the group
// share every K and V row the workgroup reads.  Positions 0..n-1 (n = pos0 +
// m + 1) are taken in chunks of CH with an online softmax:
//  * scores: thread t dots the keys of positions t, t + 256, ... with the G
//    queries (fp32, queries pre-scaled by 1/sqrt(128), read from LDS as
//    broadcasts);
//  * the chunk maximum and the rescaling of the running sums (workgroup
//    reductions through LDS, in a fixed order);
//  * values: thread (d, half) adds p_t * v_t[d] over the even (half 0) or odd
//    (half 1) positions of the chunk, for all G heads; V rows are read as
//    256 contiguous bytes by 128 threads.
// The two halves are added at the end and o / sum is rounded to fp16.
constexpr int ATT_CH = 512;

struct AttnArgs {
  const half_t* q;         // [M, Hq*128] fp16 (after RoPE)
  const half_t* k_cache;   // [Hkv, cache_len, 128] fp16
  const half_t* v_cache;
  half_t* out;             // [M, Hq*128] fp16
  int64_t cache_len;
  int32_t pos0, hq, hkv;
};

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();   // red is reused: earlier readers are done
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

template <int G>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[G][HEAD_DIM];
  __shared__ float ps[G][ATT_CH];
  __shared__ float red[4];
  __shared__ float ohalf[G][HEAD_DIM];
  const int m = blockIdx.x, kv = blockIdx.y, tid = threadIdx.x;
  const int n = a.pos0 + m + 1;
  const float scale = 0.08838834764831845f;   // 1 / sqrt(128)
  for (int i = tid; i < G * HEAD_DIM; i += 256)
    qs[i / HEAD_DIM][i % HEAD_DIM] = (float)a.q[((int64_t)m * a.hq + kv * G) * HEAD_DIM + i] * scale;
  const half_t* kc = a.k_cache + (int64_t)kv * a.cache_len * HEAD_DIM;
  const half_t* vc = a.v_cache + (int64_t)kv * a.cache_len * HEAD_DIM;
  const int d = tid & (HEAD_DIM - 1), half = tid >> 7;
  float mx[G], sum[G], o[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mx[g] = -INFINITY;
    sum[g] = 0.0f;
    o[g] = 0.0f;
  }
  __syncthreads();
  for (int c0 = 0; c0 < n; c0 += ATT_CH) {
    const int cn = n - c0 < ATT_CH ? n - c0 : ATT_CH;
    // scores of this chunk
    float lmax[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lmax[g] = -INFINITY;
    for (int t = tid; t < cn; t += 256) {
      const uint4* kr = (const uint4*)(kc + (int64_t)(c0 + t) * HEAD_DIM);
      float s[G];
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = 0.0f;
#pragma unroll 2
      for (int i = 0; i < HEAD_DIM / 8; ++i) {
        const uint4 kw = kr[i];
        const uint32_t w4[4] = {kw.x, kw.y, kw.z, kw.w};
        float kf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h2 kp = as_h2(w4[e]);
          kf[2 * e] = (float)kp.x;
          kf[2 * e + 1] = (float)kp.y;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float4 qa = *(const float4*)&qs[g][8 * i];
          const float4 qb = *(const float4*)&qs[g][8 * i + 4];
          float acc = s[g];
          acc = __builtin_fmaf(qa.x, kf[0], acc);
          acc = __builtin_fmaf(qa.y, kf[1], acc);
          acc = __builtin_fmaf(qa.z, kf[2], acc);
          acc = __builtin_fmaf(qa.w, kf[3], acc);
          acc = __builtin_fmaf(qb.x, kf[4], acc);
          acc = __builtin_fmaf(qb.y, kf[5], acc);
          acc = __builtin_fmaf(qb.z, kf[6], acc);
          acc = __builtin_fmaf(qb.w, kf[7], acc);
          s[g] = acc;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        ps[g][t] = s[g];
        lmax[g] = fmaxf(lmax[g], s[g]);
      }
    }
    // running maxima, rescaled sums and accumulators
    float fac[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float cm = block_reduce(lmax[g], true, red);
      const float nm = fmaxf(mx[g], cm);
      fac[g] = __expf(mx[g] - nm);   // 0 on the first chunk (mx = -inf)
      mx[g] = nm;
    }
    float lsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lsum[g] = 0.0f;
    for (int t = tid; t < cn; t += 256)   // the scores this thread wrote
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = __expf(ps[g][t] - mx[g]);
        ps[g][t] = p;
        lsum[g] += p;
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float cs = block_reduce(lsum[g], false, red);
      sum[g] = sum[g] * fac[g] + cs;
      o[g] *= fac[g];
    }
    __syncthreads();   // probabilities visible
    for (int t = half; t < cn; t += 2) {
      const float vv = (float)vc[(int64_t)(c0 + t) * HEAD_DIM + d];
#pragma unroll
      for (int g = 0; g < G; ++g) o[g] = __builtin_fmaf(ps[g][t], vv, o[g]);
    }
    __syncthreads();   // ps is rewritten by the next chunk
  }
  if (half == 1)
#pragma unroll
    for (int g = 0; g < G; ++g) ohalf[g][d] = o[g];
  __syncthreads();
  if (half == 0)
#pragma unroll
    for (int g = 0; g < G; ++g)
      a.out[((int64_t)m * a.hq + kv * G + g) * HEAD_DIM + d] = (half_t)((o[g] + ohalf[g][d]) / sum[g]);
}

hipError_t launch_attention(const void* q, const void* k_cache, const void* v_cache, void* out, int64_t cache_len,
                            int64_t M, int64_t pos0, int hq, int hkv, hipStream_t s) {
  AttnArgs a{(const half_t*)q, (const half_t*)k_cache, (const half_t*)v_cache, (half_t*)out, cache_len,
             (int32_t)pos0, hq, hkv};
  const dim3 grid((unsigned)M, (unsigned)hkv);
  switch (hq / hkv) {
    case 1: hipLaunchKernelGGL(attention_kernel<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attention_kernel<2>, grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(attention_kernel<3>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attention_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL(attention_kernel<5>, grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL(attention_kernel<6>, grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL(attention_kernel<7>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(attention_kernel<8>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

// ----------------------------------------------------- residual + RMSNorm --
// One workgroup per row: h = h_in + y in fp32 (written to h_out; h_in may be
// h_out), then, with g, xn = fp16(h * g / sqrt(mean(h^2) + eps)) as in the
// RMSNorm kernel but from the fp32 sum.
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(const float* h_in, const float* y, const float* g,
                                                                float eps, float* h_out, half_t* xn, int K) {
  __shared__ float red[4];
  const int64_t base = (int64_t)blockIdx.x * K;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < K / 4; i += 256) {
    const float4 a = ((const float4*)(h_in + base))[i];
    const float4 b = ((const float4*)(y + base))[i];
    const float4 h = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    ((float4*)(h_out + base))[i] = h;
    ss += (h.x * h.x + h.y * h.y) + (h.z * h.z + h.w * h.w);
  }
  if (!g) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / __builtin_sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)K + eps);
  for (int i = threadIdx.x; i < K / 4; i += 256) {
    const float4 h = ((const float4*)(h_out + base))[i];   // this thread's own writes
    const float4 gg = ((const float4*)g)[i];
    const h2 lo = {(half_t)((h.x * gg.x) * r), (half_t)((h.y * gg.y) * r)};
    const h2 hi = {(half_t)((h.z * gg.z) * r), (half_t)((h.w * gg.w) * r)};
    ((uint2*)(xn + base))[i] = make_uint2(as_u32(lo), as_u32(hi));
  }
}

hipError_t launch_residual_rmsnorm(const float* h_in, const float* y, const float* g, float eps, float* h_out,
                                   void* xn, int64_t M, int64_t K, hipStream_t s) {
  hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, s, h_in, y, g, eps, h_out,
                     (half_t*)xn, (int)K);
  return hipGetLastError();
}

}  // namespace dmq
