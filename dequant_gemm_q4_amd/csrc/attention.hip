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
#include "dmq.h"
#include "dmq_common.h"

#include <math.h>

#include <algorithm>
#include <mutex>

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

// cos and sin of pair i's angle at position pos (fp64 angle, reduced modulo
// 2 pi, each rounded to fp32).  The RoPE kernel and the fused decode
// attention kernel both take their angles from here, so they agree bit for bit.
__device__ __forceinline__ void rope_angle(double theta, const float* ff, int64_t pos, int i, float& c, float& s) {
  double inv = pow(theta, -2.0 * i / HEAD_DIM);
  if (ff) inv /= (double)ff[i];
  const double ang = remainder((double)pos * inv, 2.0 * M_PI);
  c = (float)cos(ang);
  s = (float)sin(ang);
}

// (a, b) -> (a cos - b sin, a sin + b cos) in fp32, each rounded once to
// fp16; the fused multiply-adds are written out so that every kernel using
// this rounds the same way.
__device__ __forceinline__ h2 rope_pair(float2 x, float c, float s) {
  const h2 o = {(half_t)__builtin_fmaf(x.x, c, -(x.y * s)), (half_t)__builtin_fmaf(x.x, s, x.y * c)};
  return o;
}

// grid: (token, unit): units 0 .. ceil(Hq/8)-1 take 8 query heads each, the
// following ones 8 KV heads (K and V) each.
constexpr int ROPE_UNIT = 8;
__global__ __launch_bounds__(256) void rope_kv_kernel(RopeArgs a) {
  __shared__ float cs[HEAD_DIM / 2], sn[HEAD_DIM / 2];
  const int m = blockIdx.x, unit = blockIdx.y, tid = threadIdx.x;
  const int uq = (a.hq + ROPE_UNIT - 1) / ROPE_UNIT;
  const int64_t pos = (int64_t)a.pos0 + m;
  if (tid < HEAD_DIM / 2) rope_angle(a.theta, a.ff, pos, tid, cs[tid], sn[tid]);
  __syncthreads();
  auto rot = [&](const float* src, half_t* dst, int pairs) {
    for (int p = tid; p < pairs; p += 256) {
      const int i = p & (HEAD_DIM / 2 - 1);
      ((h2*)dst)[p] = rope_pair(((const float2*)src)[p], cs[i], sn[i]);
    }
  };
  if (unit < uq) {
    const int h0 = unit * ROPE_UNIT, nh = a.hq - h0 < ROPE_UNIT ? a.hq - h0 : ROPE_UNIT;
    const int64_t off = ((int64_t)m * a.hq + h0) * HEAD_DIM;
    rot(a.q + off, a.q_out + off, nh * HEAD_DIM / 2);
    return;
  }
  // K (rotated) and V go to row `pos` of each KV head's cache
  const int k0 = (unit - uq) * ROPE_UNIT, k1 = k0 + ROPE_UNIT < a.hkv ? k0 + ROPE_UNIT : a.hkv;
  for (int p = tid; p < (k1 - k0) * (HEAD_DIM / 2); p += 256) {
    const int h = k0 + p / (HEAD_DIM / 2), i = p % (HEAD_DIM / 2);
    const int64_t src = ((int64_t)m * a.hkv + h) * HEAD_DIM + 2 * i;
    const int64_t row = ((int64_t)h * a.cache_len + pos) * HEAD_DIM + 2 * i;
    *(h2*)(a.k_cache + row) = rope_pair(*(const float2*)(a.k + src), cs[i], sn[i]);
    const float2 v = *(const float2*)(a.v + src);
    const h2 vo = {(half_t)v.x, (half_t)v.y};
    *(h2*)(a.v_cache + row) = vo;
  }
}

hipError_t launch_rope_kv(const float* q, const float* k, const float* v, const float* ff, void* q_out, void* k_cache,
                          void* v_cache, double theta, int64_t cache_len, int64_t M, int64_t pos0, int hq, int hkv,
                          hipStream_t s) {
  RopeArgs a{q, k, v, ff, (half_t*)q_out, (half_t*)k_cache, (half_t*)v_cache, theta, cache_len,
             (int32_t)pos0, hq, hkv};
  const unsigned units = (unsigned)((hq + ROPE_UNIT - 1) / ROPE_UNIT + (hkv + ROPE_UNIT - 1) / ROPE_UNIT);
  hipLaunchKernelGGL(rope_kv_kernel, dim3((unsigned)M, units), dim3(256), 0, s, a);
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
constexpr int ATT_SPLIT_MAX_M = 16;   // up to this many queries: the split (decode) path

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

// Few queries (decode): the positions are split into pieces of SPLIT_S, one
// workgroup per (piece, KV head, query), so that a decode step has hundreds
// of workgroups instead of one per KV head.  Each piece writes its partial
// softmax state (maximum, sum of weights, weighted sum of V) for each query
// head to a workspace; a second kernel merges the pieces in piece order.
constexpr int SPLIT_S = 64;
constexpr int MERGE_MAX_PIECES = 4096;    // pieces the merge stages in LDS (262144 positions)
constexpr int SPLIT_REC = HEAD_DIM + 2;   // floats per (query head, piece): o[128], max, sum

// The RoPE inputs of the fused decode variant (ROPE): the Q, K and V
// projections' fp32 rows, and where the rotated queries and the new cache
// rows go.
struct RopeIn {
  const float* q;          // [1, Hq*128]
  const float* k;          // [1, Hkv*128]
  const float* v;          // [1, Hkv*128]
  const float* ff;         // 64 frequency factors, or NULL
  half_t* q_out;           // [1, Hq*128] fp16: the rotated queries
  half_t* k_cache;         // the caches of AttnArgs, written at row pos0
  half_t* v_cache;
  double theta;
};

// ROPE (one query, M = 1): the workgroup rotates the queries of its KV group
// itself, with the angles of position pos0 (the RoPE kernel's arithmetic),
// instead of reading them rotated; piece 0 also stores them to q_out.  The
// piece that holds position pos0 (the last one) rotates K and rounds V of
// that position, writes them to the cache row pos0 and reads them back from
// there after the barrier that follows, like every other row; no other piece
// reads that row.  So the results are those of the RoPE kernel followed by
// this kernel, bit for bit, without the RoPE launch in between.
template <int G, bool ROPE>
__global__ __launch_bounds__(256) void attention_split_kernel(AttnArgs a, RopeIn r, float* ws, int nsplit) {
  __shared__ __attribute__((aligned(16))) float qs[G][HEAD_DIM];
  __shared__ float ps[G][SPLIT_S];
  __shared__ float st[G][2];
  __shared__ float vsl[8][G][HEAD_DIM];
  __shared__ float rcs[ROPE ? HEAD_DIM / 2 : 1], rsn[ROPE ? HEAD_DIM / 2 : 1];
  const int sp = blockIdx.x, kv = blockIdx.y, m = blockIdx.z, tid = threadIdx.x;
  const int n = a.pos0 + m + 1;
  const int c0 = sp * SPLIT_S;
  if (c0 >= n) return;   // no positions: the merge reads pieces < ceil(n / SPLIT_S) only
  const int cn = n - c0 < SPLIT_S ? n - c0 : SPLIT_S;
  const float scale = 0.08838834764831845f;   // 1 / sqrt(128)
  if constexpr (ROPE) {
    const int64_t pos = (int64_t)a.pos0 + m;
    if (tid < HEAD_DIM / 2) rope_angle(r.theta, r.ff, pos, tid, rcs[tid], rsn[tid]);
    __syncthreads();
    for (int p = tid; p < G * HEAD_DIM / 2; p += 256) {
      const int g = p / (HEAD_DIM / 2), i = p % (HEAD_DIM / 2);
      const int64_t off = ((int64_t)m * a.hq + kv * G + g) * HEAD_DIM + 2 * i;
      const h2 o = rope_pair(*(const float2*)(r.q + off), rcs[i], rsn[i]);
      if (sp == 0) *(h2*)(r.q_out + off) = o;
      qs[g][2 * i] = (float)o.x * scale;
      qs[g][2 * i + 1] = (float)o.y * scale;
    }
    if (pos >= c0 && pos < c0 + cn && tid < HEAD_DIM / 2) {
      const int64_t src = ((int64_t)m * a.hkv + kv) * HEAD_DIM + 2 * tid;
      const int64_t row = ((int64_t)kv * a.cache_len + pos) * HEAD_DIM + 2 * tid;
      *(h2*)(r.k_cache + row) = rope_pair(*(const float2*)(r.k + src), rcs[tid], rsn[tid]);
      const float2 vv = *(const float2*)(r.v + src);
      const h2 vo = {(half_t)vv.x, (half_t)vv.y};
      *(h2*)(r.v_cache + row) = vo;
    }
  } else {
    for (int i = tid; i < G * HEAD_DIM; i += 256)
      qs[i / HEAD_DIM][i % HEAD_DIM] = (float)a.q[((int64_t)m * a.hq + kv * G) * HEAD_DIM + i] * scale;
  }
  const half_t* kc = a.k_cache + (int64_t)kv * a.cache_len * HEAD_DIM;
  const half_t* vc = a.v_cache + (int64_t)kv * a.cache_len * HEAD_DIM;
  // (with ROPE, also orders the new cache row's stores before its loads
  // below: a workgroup barrier carries a workgroup-scope release and acquire)
  __syncthreads();
  // scores: 4 threads per position, 32 dimensions each, summed across the quad
  {
    const int t = tid >> 2, part = tid & 3;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.0f;
    if (t < cn) {
      const uint4* kr = (const uint4*)(kc + (int64_t)(c0 + t) * HEAD_DIM + 32 * part);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
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
          const float* qg = &qs[g][32 * part + 8 * i];
          float acc = s[g];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qg[e], kf[e], acc);
          s[g] = acc;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s[g] += __shfl_xor(s[g], 1, 64);
      s[g] += __shfl_xor(s[g], 2, 64);
      if (part == 0 && t < cn) ps[g][t] = s[g];
    }
  }
  __syncthreads();
  // the piece's softmax state per head: wave 0, one lane per position
  if (tid < 64) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = tid < cn ? ps[g][tid] : -INFINITY;
      float mx = v;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      const float p = tid < cn ? __expf(v - mx) : 0.0f;
      float sum = p;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
      if (tid < cn) ps[g][tid] = p;
      if (tid == 0) {
        st[g][0] = mx;
        st[g][1] = sum;
      }
    }
  }
  __syncthreads();
  // weighted sum of V: thread (slice, q4) takes dims 4 q4 .. +3 of positions
  // slice, slice + 8, ... (8 loads in flight), the 8 slices summed in order
  const int q4 = tid & 31, slice = tid >> 5;
  float o[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[g][e] = 0.0f;
  uint2 vr[SPLIT_S / 8];
#pragma unroll
  for (int u = 0; u < SPLIT_S / 8; ++u) {
    const int t = slice + 8 * u;
    vr[u] = t < cn ? *(const uint2*)(vc + (int64_t)(c0 + t) * HEAD_DIM + 4 * q4) : make_uint2(0, 0);
  }
#pragma unroll
  for (int u = 0; u < SPLIT_S / 8; ++u) {
    const int t = slice + 8 * u;
    if (t < cn) {
      const h2 v01 = as_h2(vr[u].x), v23 = as_h2(vr[u].y);
      const float vv[4] = {(float)v01.x, (float)v01.y, (float)v23.x, (float)v23.y};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = ps[g][t];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[g][e] = __builtin_fmaf(p, vv[e], o[g][e]);
      }
    }
  }
  __syncthreads();   // ps no longer read: reuse ohalf as the slices' staging
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) vsl[slice][g][4 * q4 + e] = o[g][e];
  __syncthreads();
  for (int i = tid; i < G * HEAD_DIM; i += 256) {
    const int g = i / HEAD_DIM, dd = i % HEAD_DIM;
    float acc = vsl[0][g][dd];
#pragma unroll
    for (int sl = 1; sl < 8; ++sl) acc += vsl[sl][g][dd];
    float* rec = ws + (((int64_t)m * a.hq + kv * G + g) * nsplit + sp) * SPLIT_REC;
    rec[dd] = acc;
    if (dd == 0) {
      rec[HEAD_DIM] = st[g][0];
      rec[HEAD_DIM + 1] = st[g][1];
    }
  }
}

// Merge of the pieces of one (query, query head), in piece order: rescale
// each piece's sums to the overall maximum and divide.  The pieces' maxima
// and sums are read in parallel into LDS first; the weighted sums of V are
// then read 8 pieces at a time, so the loads overlap.
__global__ __launch_bounds__(128) void attention_merge_kernel(AttnArgs a, const float* ws, int nsplit) {
  __shared__ float fac[MERGE_MAX_PIECES];
  __shared__ float red[2];
  const int h = blockIdx.x, m = blockIdx.y, d = threadIdx.x;
  const int n = a.pos0 + m + 1;
  const int np = (n + SPLIT_S - 1) / SPLIT_S;
  const float* rec = ws + ((int64_t)m * a.hq + h) * nsplit * SPLIT_REC;
  float mx = -INFINITY;
  for (int i = d; i < np; i += 128) {
    fac[i] = rec[i * SPLIT_REC + HEAD_DIM];
    mx = fmaxf(mx, fac[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((d & 63) == 0) red[d >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  for (int i = d; i < np; i += 128) fac[i] = __expf(fac[i] - mx);   // the thread's own entries
  __syncthreads();
  float sum = 0.0f, o = 0.0f;
  int i = 0;
  for (; i + 8 <= np; i += 8) {
    float ov[8], sv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ov[u] = rec[(i + u) * SPLIT_REC + d];
      sv[u] = rec[(i + u) * SPLIT_REC + HEAD_DIM + 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sum = __builtin_fmaf(sv[u], fac[i + u], sum);
      o = __builtin_fmaf(ov[u], fac[i + u], o);
    }
  }
  for (; i < np; ++i) {
    sum = __builtin_fmaf(rec[i * SPLIT_REC + HEAD_DIM + 1], fac[i], sum);
    o = __builtin_fmaf(rec[i * SPLIT_REC + d], fac[i], o);
  }
  a.out[((int64_t)m * a.hq + h) * HEAD_DIM + d] = (half_t)(o / sum);
}

// Many queries (prefill): MFMA flash attention.  One workgroup = 8 waves =
// 128 consecutive queries of one query head, in two halves of 4 waves that
// take the even and the odd key blocks and merge their softmax states in LDS
// at the end (two independent chains per SIMD).  Wave w of a half owns
// queries 32w .. 32w+31 of the block and keeps them as MFMA operands for the
// whole key loop.  Keys go in blocks of 32, staged in LDS by each half (K
// row-major with 16-byte chunks XOR-swizzled by the key; V transposed to
// [dim][key pair], packed 32-bit words on conflict-free banks), double-
// buffered, with the global loads of later blocks in flight during the
// current block's compute.  A half's iteration forms the scores of its next
// block while the current block's softmax runs (software pipeline).  Per key
// block and wave, with v_mfma_f32_32x32x16_f16 (D = A B^T):
//  * S^T = K Q^T (A = K rows, B = Q rows, 8 MFMAs over the 128 dims): an
//    accumulator lane holds one query (its lane % 32) and 16 of the 32 keys,
//    the lane 32 away the other 16, so a query's maximum and sum need one
//    exchange between the two lanes;
//  * online softmax in fp32 on exp2 with log2(e)/sqrt(128) folded into the
//    exponent; keys past a query's position are masked to -inf (only in
//    blocks that cross the wave's diagonal); the reference maximum moves
//    lazily (only by more than 2^8), so O is rarely rescaled;
//  * O^T += V^T P^T (A = V^T rows, B = P rows, 2 key steps x 4 dim blocks):
//    the key order inside a 16-key step is permuted the same way for both
//    operands so that P's B fragment is 8 consecutive accumulator registers,
//    converted to fp16.
// The 128 dims of O^T stay in 64 accumulator registers per lane; at the end
// O / sum is rounded to fp16 and stored.
constexpr int FA_KB = 32;                 // keys per block
constexpr int FA_QB = 128;                // queries per workgroup
constexpr float FA_RESCALE = 8.0f;        // log2 headroom of the lazy softmax rescale
constexpr int FA_MERGE_STRIDE = HEAD_DIM / 2 + 4;   // floats per lane in the merge: O^T, m, l, pad
constexpr int FA_VT_WORDS = 18;           // 32-bit words per V^T row (16 key pairs + pad)
// V^T word swizzle: rows 32..63 and 96..127 swap the two 8-word halves
__device__ __forceinline__ int fa_vt_swz(int row) { return 8 * ((row >> 5) & 1); }

typedef float f16acc __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void attention_mfma_kernel(AttnArgs a, int M, int nqb) {
  // per half: K double buffer, V^T double buffer; reused for the final merge
  constexpr int KS_BYTES = 2 * FA_KB * HEAD_DIM * 2, VT_BYTES = 2 * HEAD_DIM * FA_VT_WORDS * 4;
  constexpr int HALF_BYTES = KS_BYTES + VT_BYTES;
  static_assert(2 * HALF_BYTES >= 4 * 64 * FA_MERGE_STRIDE * 4, "merge staging must fit");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * HALF_BYTES];
  const int hf = threadIdx.x >> 8;            // half: key blocks hf, hf + 2, hf + 4, ...
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
  half_t (*ks)[FA_KB * HEAD_DIM] = (half_t (*)[FA_KB * HEAD_DIM])(lds + hf * HALF_BYTES);
  half_t (*vt)[HEAD_DIM * 2 * FA_VT_WORDS] = (half_t (*)[HEAD_DIM * 2 * FA_VT_WORDS])(lds + hf * HALF_BYTES + KS_BYTES);
  const int li = lane & 31, g = lane >> 5;
  // work item t = (KV head, query block from the last, query head of the
  // group).  Workgroups are dealt to the 8 XCDs round-robin; XCD x takes the
  // items x*per .. x*per+per-1, so the queries of one KV head share an L2 and
  // its K and V are read from HBM about once.  Longest blocks first.
  const int G = a.hq / a.hkv;
  const int nitems = nqb * a.hq, per = (nitems + 7) / 8;
  const int t = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (t >= nitems) return;
  const int kvh = t / (nqb * G);
  const int rem = t - kvh * nqb * G;
  const int qb = nqb - 1 - rem / G;
  const int h = kvh * G + rem % G;
  const int q0 = qb * FA_QB;                  // first query (row of q) of the block
  const int qw = q0 + 32 * wave;              // first query of this wave
  const int64_t pos_q = (int64_t)a.pos0 + qw + li;   // this lane's query position
  const half_t* kc = a.k_cache + (int64_t)kvh * a.cache_len * HEAD_DIM;
  const half_t* vc = a.v_cache + (int64_t)kvh * a.cache_len * HEAD_DIM;

  // Q fragments (B operand of S^T): query qw + li, dims 16 kk + 8 g .. +7
  h8 qf[HEAD_DIM / 16];
  {
    const bool ok = qw + li < M;
    const half_t* qr = a.q + ((int64_t)(qw + li) * a.hq + h) * HEAD_DIM + 8 * g;
#pragma unroll
    for (int kk = 0; kk < HEAD_DIM / 16; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *(const uint4*)(qr + 16 * kk);
      qf[kk] = __builtin_bit_cast(h8, v);
    }
  }
  // keys needed: positions 0 .. last query position of the workgroup
  const int qlast = (q0 + FA_QB < M ? q0 + FA_QB : M) - 1;
  const int64_t nkeys = (int64_t)a.pos0 + qlast + 1;
  const int nkb = (int)((nkeys + FA_KB - 1) / FA_KB);
  const int64_t wave_first_pos = (int64_t)a.pos0 + qw;

  // staging of a key block (32 keys x 128 dims of K and of V).  K: thread t
  // holds 16-byte chunks t and t + 256 (key = chunk / 16, dims 8 (chunk % 16)
  // ..+7).  V: thread t holds keys 2 jp, 2 jp + 1 at dims 8 cv .. +7 and
  // writes them as 8 key pairs (one 32-bit word per dim) of V^T; a wave's
  // lanes take 8 key pairs x 8 dim chunks, which the row stride of 18 words and
  // the swizzle keep on 64 distinct banks.  A block's loads are issued before
  // an iteration's compute and written to LDS after it (K two blocks ahead of
  // the softmax, V one); rows past the last key re-read the last one and are
  // zeroed when stored, so the load addresses need no branch.
  uint4 kr0, kr1, va, vb;
  const int ck0 = tid >> 4, ck1 = (tid + 256) >> 4, cch = tid & 15;
  const int jp = (tid & 7) + 8 * ((tid >> 6) & 1), cv = ((tid >> 3) & 7) + 8 * (tid >> 7);
  auto load_k = [&](int kb) {
    const int64_t k0 = (int64_t)kb * FA_KB;
    const int64_t r0 = k0 + ck0 < nkeys ? k0 + ck0 : nkeys - 1;
    const int64_t r1 = k0 + ck1 < nkeys ? k0 + ck1 : nkeys - 1;
    kr0 = *(const uint4*)(kc + r0 * HEAD_DIM + 8 * cch);
    kr1 = *(const uint4*)(kc + r1 * HEAD_DIM + 8 * cch);
  };
  auto load_v = [&](int kb) {
    const int64_t k0 = (int64_t)kb * FA_KB;
    const int64_t ra = k0 + 2 * jp < nkeys ? k0 + 2 * jp : nkeys - 1;
    const int64_t rb = k0 + 2 * jp + 1 < nkeys ? k0 + 2 * jp + 1 : nkeys - 1;
    va = *(const uint4*)(vc + ra * HEAD_DIM + 8 * cv);
    vb = *(const uint4*)(vc + rb * HEAD_DIM + 8 * cv);
  };
  // component-wise masks: a select of whole uint4 values goes through scratch
  auto store_k = [&](int kb, int b) {
    const int64_t k0 = (int64_t)kb * FA_KB;
    const uint32_t m0 = k0 + ck0 < nkeys ? 0xffffffffu : 0u;
    const uint32_t m1 = k0 + ck1 < nkeys ? 0xffffffffu : 0u;
    *(uint4*)(&ks[b][ck0 * HEAD_DIM + 8 * (cch ^ (ck0 & 15))]) =
        make_uint4(kr0.x & m0, kr0.y & m0, kr0.z & m0, kr0.w & m0);
    *(uint4*)(&ks[b][ck1 * HEAD_DIM + 8 * (cch ^ (ck1 & 15))]) =
        make_uint4(kr1.x & m1, kr1.y & m1, kr1.z & m1, kr1.w & m1);
  };
  auto store_v = [&](int kb, int b) {
    const int64_t k0 = (int64_t)kb * FA_KB;
    const uint32_t ma = k0 + 2 * jp < nkeys ? 0xffffffffu : 0u;
    const uint32_t mb = k0 + 2 * jp + 1 < nkeys ? 0xffffffffu : 0u;
    const uint32_t wa[4] = {va.x & ma, va.y & ma, va.z & ma, va.w & ma};
    const uint32_t wb[4] = {vb.x & mb, vb.y & mb, vb.z & mb, vb.w & mb};
    uint32_t* vrow = (uint32_t*)vt[b];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 8 * cv + e;
      const uint32_t x = wa[e >> 1], y = wb[e >> 1];
      const uint32_t pair = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      vrow[row * FA_VT_WORDS + (jp ^ fa_vt_swz(row))] = pair;
    }
  };

  f16acc o[HEAD_DIM / 32];
#pragma unroll
  for (int db = 0; db < HEAD_DIM / 32; ++db) o[db] = (f16acc){};
  float mrun = -INFINITY, lrun = 0.0f;
  const float c = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)

  // S^T = K Q^T of the key block in K buffer kbuf
  auto scores = [&](int kbuf) {
    f16acc sacc = (f16acc){};
#pragma unroll
    for (int kk = 0; kk < HEAD_DIM / 16; ++kk) {
      const int ch = 2 * kk + g;
      const h8 kf = *(const h8*)(&ks[kbuf][li * HEAD_DIM + 8 * (ch ^ (li & 15))]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], sacc, 0, 0, 0);
    }
    return sacc;
  };
  // causal mask of the block at key k0, only where it reaches past the
  // wave's first query (a wave-uniform test: most blocks lie wholly below
  // the diagonal); a block wholly past the wave's queries masks to -inf and
  // then adds nothing
  auto mask = [&](f16acc& sacc, int64_t k0) {
    if (k0 + FA_KB - 1 > wave_first_pos) {
      const int64_t dd = pos_q - k0 - 4 * g;   // key k0 + 4g + j is visible iff j <= dd
      const int d = dd < -1 ? -1 : (dd > FA_KB ? FA_KB : (int)dd);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > d) sacc[r] = -INFINITY;
    }
  };
  // online softmax of one block's scores: P (fp16, as the MFMA operand),
  // the rescale factor alpha and whether any lane's reference moved
  auto softmax = [&](const f16acc& sacc, h8 (&pf)[2], float& alpha, bool& move) {
    // block maximum of this lane's query (raw scores; the scale c > 0 keeps the order)
    float bm = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bm = fmaxf(bm, sacc[r]);
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    // lazy rescaling: the reference m of the running sums moves only when
    // the block maximum exceeds it by more than FA_RESCALE (so p <= 2^8 in
    // fp16), which after the first blocks is rare; O and l share m, so the
    // result does not depend on it.  A query with no visible key yet keeps
    // m = -inf, l = 0, O = 0 (reference point 0: p = 0).
    const float bmc = bm * c;
    move = bmc > mrun + FA_RESCALE;
    const float mnew = move ? bmc : mrun;
    const float mref = mnew == -INFINITY ? 0.0f : mnew;
    alpha = move ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
    float sv[16];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -mref));
      sv[r] = p;
      ps += p;
    }
    ps += __shfl_xor(ps, 32, 64);
    lrun = lrun * alpha + ps;
    mrun = mnew;
#pragma unroll
    for (int e = 0; e < 16; ++e) pf[e >> 3][e & 7] = (half_t)sv[e];
  };
  // O^T = alpha O^T + V^T P^T with V^T from buffer vbuf
  auto update = [&](const h8 (&pf)[2], float alpha, bool move, int vbuf) {
    if (__any(move)) {
#pragma unroll
      for (int db = 0; db < HEAD_DIM / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    // O^T += V^T P^T, two 16-key steps
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int db = 0; db < HEAD_DIM / 32; ++db) {
        const int row = 32 * db + li;
        const uint32_t* vr = (const uint32_t*)vt[vbuf] + row * FA_VT_WORDS;
        const int sw = fa_vt_swz(row);
        const uint2 lo = *(const uint2*)(vr + ((8 * kk + 2 * g) ^ sw));       // keys 16kk + 4g + 0..3
        const uint2 hi = *(const uint2*)(vr + ((8 * kk + 4 + 2 * g) ^ sw));   // keys 16kk + 8 + 4g + 0..3
        const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, w), pf[kk], o[db], 0, 0, 0);
      }
    }
  };

  // Software pipeline over this half's blocks j = 0, 1, ... (key blocks
  // 2j + hf): iteration j computes the scores of block j+1 while it runs
  // block j's softmax and O update, so the MFMA pipe and the VALU overlap.
  // K is staged two blocks ahead (buffer j&1 is free once block j's scores
  // exist), V one block ahead.  Both halves run the same number of
  // iterations: the barriers are shared.
  const int nloc = hf < nkb ? (nkb - hf + 1) / 2 : 0;
  const int niter = (nkb + 1) / 2;
  if (nloc > 0) {
    load_k(hf);
    load_v(hf);
    store_k(hf, 0);
    store_v(hf, 0);
  }
  if (nloc > 1) {
    load_k(2 + hf);
    store_k(2 + hf, 1);
  }
  __syncthreads();
  f16acc scur = (f16acc){};
  if (nloc > 0) {
    scur = scores(0);
    mask(scur, (int64_t)hf * FA_KB);
  }
  __syncthreads();   // K buffer 0 is rewritten in iteration 0
  for (int j = 0; j < niter; ++j) {
    if (j + 1 < nloc) {
      const int jk = j + 2 < nloc ? j + 2 : nloc - 1;   // clamped: the loads stay unconditional
      load_k(2 * jk + hf);
      load_v(2 * (j + 1) + hf);
      f16acc snext = scores((j + 1) & 1);
      h8 pf[2];
      float alpha;
      bool move;
      softmax(scur, pf, alpha, move);
      // interleave: each MFMA of the next block's scores followed by this
      // block's softmax VALU work, which runs while the MFMA executes
#pragma unroll
      for (int i = 0; i < HEAD_DIM / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read (K fragment)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // eight VALU
      }
      update(pf, alpha, move, j & 1);
      if (j + 2 < nloc) store_k(2 * (j + 2) + hf, j & 1);
      store_v(2 * (j + 1) + hf, (j + 1) & 1);
      mask(snext, (int64_t)(2 * (j + 1) + hf) * FA_KB);
      scur = snext;
    } else if (j < nloc) {
      h8 pf[2];
      float alpha;
      bool move;
      softmax(scur, pf, alpha, move);
      update(pf, alpha, move, j & 1);
    }
    __syncthreads();
  }
  // merge of the two halves' softmax states: half 1 leaves its running
  // maximum, sum and O^T in LDS (staging memory, free after the last
  // barrier), half 0 rescales both to the common maximum
  float* mo = (float*)lds + (wave * 64 + lane) * FA_MERGE_STRIDE;
  if (hf == 1) {
#pragma unroll
    for (int db = 0; db < HEAD_DIM / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        *(float4*)(mo + 16 * db + r) = make_float4(o[db][r], o[db][r + 1], o[db][r + 2], o[db][r + 3]);
    mo[HEAD_DIM / 2] = mrun;
    mo[HEAD_DIM / 2 + 1] = lrun;
  }
  __syncthreads();
  if (hf == 1) return;
  {
    const float m1 = mo[HEAD_DIM / 2], l1 = mo[HEAD_DIM / 2 + 1];
    const float mx = fmaxf(mrun, m1);
    // a half without keys for this query has m = -inf and contributes nothing
    const float f0 = mrun == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mrun - mx);
    const float f1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
    lrun = lrun * f0 + l1 * f1;
#pragma unroll
    for (int db = 0; db < HEAD_DIM / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float4 w = *(const float4*)(mo + 16 * db + r);
        o[db][r] = o[db][r] * f0 + w.x * f1;
        o[db][r + 1] = o[db][r + 1] * f0 + w.y * f1;
        o[db][r + 2] = o[db][r + 2] * f0 + w.z * f1;
        o[db][r + 3] = o[db][r + 3] * f0 + w.w * f1;
      }
  }
  // O = O^T / sum: lane holds query qw + li, dims 32 db + 8 (r/4) + 4 g + r % 4
  if (qw + li < M) {
    const float inv = 1.0f / lrun;
    half_t* orow = a.out + ((int64_t)(qw + li) * a.hq + h) * HEAD_DIM;
#pragma unroll
    for (int db = 0; db < HEAD_DIM / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const h2 x01 = {(half_t)(o[db][4 * q4] * inv), (half_t)(o[db][4 * q4 + 1] * inv)};
        const h2 x23 = {(half_t)(o[db][4 * q4 + 2] * inv), (half_t)(o[db][4 * q4 + 3] * inv)};
        *(uint2*)(orow + 32 * db + 8 * q4 + 4 * g) = make_uint2(as_u32(x01), as_u32(x23));
      }
  }
}

// Scratch for callers that cannot allocate (dmq_attention_gqa_noalloc): the
// partial softmax states of the decode path in a fixed array of every GPU's
// code object, allocated when the library is loaded on that GPU and held
// until the process ends.  Every record the merge kernel reads is written by
// the piece kernel of the same call, so nothing needs clearing; calls that
// overlap on one GPU share it and race.
constexpr size_t NOALLOC_SCRATCH_BYTES = DMQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_BYTES / sizeof(float)];

hipError_t noalloc_scratch(float** ptr, size_t* bytes) {
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // host code never uses `scratch` itself: its host-side name is not the
    // device address, which differs per GPU
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = (float*)p;
  }
  *ptr = addr[dev];
  *bytes = NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

// Whether M queries from position pos0 take the split (decode) path.
static bool split_path(int64_t M, int64_t pos0) {
  return M <= ATT_SPLIT_MAX_M && (pos0 + M + SPLIT_S - 1) / SPLIT_S <= MERGE_MAX_PIECES;
}

size_t attention_scratch_bytes(int64_t M, int64_t pos0, int hq) {
  if (!split_path(M, pos0)) return 0;
  const int64_t nsplit = (pos0 + M + SPLIT_S - 1) / SPLIT_S;
  return (size_t)M * hq * nsplit * SPLIT_REC * sizeof(float);
}

// The split path: the pieces' kernel (with ROPE, the fused RoPE variant at
// M = 1), then the merge.  ws_given: a buffer for the partial states, or NULL
// for the stream's workspace.
template <bool ROPE>
static hipError_t launch_split(const AttnArgs& a, const RopeIn& r, int64_t M, int64_t pos0, hipStream_t s,
                               float* ws_given) {
  const int nsplit = (int)((pos0 + M + SPLIT_S - 1) / SPLIT_S);
  // sized for the whole cache when that is at most 64 MiB (every position a
  // later call on this stream can reach), so a decode loop over one cache
  // does not grow it
  const size_t rec_bytes = (size_t)M * a.hq * SPLIT_REC * sizeof(float);
  const int64_t cap = std::min<int64_t>((a.cache_len + SPLIT_S - 1) / SPLIT_S, MERGE_MAX_PIECES);
  size_t want = rec_bytes * (size_t)nsplit;
  if (cap > nsplit && rec_bytes * (size_t)cap <= (size_t(64) << 20)) want = rec_bytes * (size_t)cap;
  void* wp = ws_given;
  hipError_t e = ws_given ? hipSuccess : stream_workspace(WorkspaceUse::AttentionPieces, s, want, &wp);
  if (e != hipSuccess) return e;
  float* ws = (float*)wp;
  const dim3 grid((unsigned)nsplit, (unsigned)a.hkv, (unsigned)M);
  switch (a.hq / a.hkv) {
    case 1: hipLaunchKernelGGL((attention_split_kernel<1, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    case 2: hipLaunchKernelGGL((attention_split_kernel<2, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    case 3: hipLaunchKernelGGL((attention_split_kernel<3, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    case 4: hipLaunchKernelGGL((attention_split_kernel<4, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    case 5: hipLaunchKernelGGL((attention_split_kernel<5, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    case 6: hipLaunchKernelGGL((attention_split_kernel<6, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    case 7: hipLaunchKernelGGL((attention_split_kernel<7, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
    default: hipLaunchKernelGGL((attention_split_kernel<8, ROPE>), grid, dim3(256), 0, s, a, r, ws, nsplit); break;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(attention_merge_kernel, dim3((unsigned)a.hq, (unsigned)M), dim3(HEAD_DIM), 0, s, a, ws, nsplit);
  return hipGetLastError();
}

hipError_t launch_attention(const void* q, const void* k_cache, const void* v_cache, void* out, int64_t cache_len,
                            int64_t M, int64_t pos0, int hq, int hkv, hipStream_t s, float* ws_given) {
  AttnArgs a{(const half_t*)q, (const half_t*)k_cache, (const half_t*)v_cache, (half_t*)out, cache_len,
             (int32_t)pos0, hq, hkv};
  if (split_path(M, pos0)) return launch_split<false>(a, RopeIn{}, M, pos0, s, ws_given);
  if (M > ATT_SPLIT_MAX_M) {
    const int nqb = (int)((M + FA_QB - 1) / FA_QB);
    const int per = (nqb * hq + 7) / 8;   // work items per XCD
    hipLaunchKernelGGL(attention_mfma_kernel, dim3(8u * (unsigned)per), dim3(512), 0, s, a, (int)M, nqb);
    return hipGetLastError();
  }
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

hipError_t launch_rope_attention(const float* q, const float* k, const float* v, const float* ff, void* q_out,
                                 void* k_cache, void* v_cache, void* out, double theta, int64_t cache_len, int64_t M,
                                 int64_t pos0, int hq, int hkv, hipStream_t s) {
  if (M == 1 && split_path(M, pos0)) {
    const AttnArgs a{(const half_t*)q_out, (const half_t*)k_cache, (const half_t*)v_cache, (half_t*)out, cache_len,
                     (int32_t)pos0, hq, hkv};
    const RopeIn r{q, k, v, ff, (half_t*)q_out, (half_t*)k_cache, (half_t*)v_cache, theta};
    return launch_split<true>(a, r, M, pos0, s, nullptr);
  }
  hipError_t e = launch_rope_kv(q, k, v, ff, q_out, k_cache, v_cache, theta, cache_len, M, pos0, hq, hkv, s);
  if (e != hipSuccess) return e;
  return launch_attention(q_out, k_cache, v_cache, out, cache_len, M, pos0, hq, hkv, s);
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
