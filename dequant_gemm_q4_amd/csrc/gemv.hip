// Decode (M = 1) kernel: y[n] = sum_k x[k] * W[n][k] with W in Q4_K or Q6_K.
//
// Decode handles a single token per step and is bound by streaming the weights
// from memory (overview page, "[01] the thesis" and "[04] one decode step";
// article "Building DAMASCUS", "Prefill and decode need different performance
// questions").  The kernel is therefore built around the HBM stream:
//
//  * every byte of W is read exactly once, with 16-byte loads; the 4 lanes
//    that share a super-block read 144 (Q4_K) / 210 (Q6_K) contiguous bytes;
//  * x (K fp16 values) is staged once per workgroup in LDS, so the per-weight
//    x traffic hits LDS, not the vector cache;
//  * each weight is dequantised exactly in fp32 (q*d*sc - dmin*m is one FMA of
//    exact operands, v_fma_mix), rounded to fp16 and multiplied with x by
//    v_dot2_f32_f16 with fp32 accumulation.  Factoring the sub-block scale
//    and min out of the sum would be cheaper, but when d*sc*q and dmin*m
//    nearly cancel its fp32 rounding error is not bounded by sum |x*w|.  Q6_K
//    has no min, so there the scale is factored out of each 16-weight dot;
//  * partial sums are reduced across the wave with cross-lane shuffles.
//
// Lane mapping: 4 lanes per super-block ("part" p = lane & 3).  Q4_K part p
// owns quant bytes 32p..32p+31, i.e. sub-blocks 2p (low nibbles) and 2p+1
// (high nibbles).  Q6_K part p owns half h = p >> 1 and weights with
// l in [16(p&1), 16(p&1)+16) of its four 32-weight quarters.
// A wave runs 16 super-blocks per step over R consecutive rows; R is chosen
// so that R * blocks_per_row is a multiple of 16 and no lane idles.
#include "dmq_common.h"

namespace dmq {

constexpr int GEMV_MAX_GROUP = 8;
constexpr int GEMV_MAX_K = 32768;      // x staged in LDS: 64 KiB

struct GemvDesc {
  const half_t* x;
  const uint8_t* wq;
  void* out;
  int32_t fmt, swiglu, N, K;
  int32_t wg_begin;   // first workgroup of this problem
  int32_t rows_log2;  // log2(R)
};

struct GemvArgs {
  GemvDesc d[GEMV_MAX_GROUP];
  int32_t count;
};

__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Dot product of one Q4_K part (64 weights) with x (LDS), exact fp32 dequant.
__device__ __forceinline__ float q4k_part_dot(const uint8_t* blk, int p, const half_t* xs) {
  uint4 hdr = *(const uint4*)blk;
  uint4 q0 = *(const uint4*)(blk + 16 + 32 * p);
  uint4 q1 = *(const uint4*)(blk + 32 + 32 * p);
  Q4kScales s = unpack_q4k_scales(hdr.y, hdr.z, hdr.w);
  uint32_t scw = p < 2 ? s.sc_lo : s.sc_hi;
  uint32_t mw = p < 2 ? s.m_lo : s.m_hi;
  uint32_t sh = (uint32_t)(p & 1) * 16u;
  float d = half_bits_to_float(hdr.x);
  float dmin = half_bits_to_float(hdr.x >> 16);
  float dsc0 = d * (float)((scw >> sh) & 0xffu);
  float dsc1 = d * (float)((scw >> (sh + 8)) & 0xffu) * 0.0625f;  // high nibble read as 16q
  float ndm0 = -(dmin * (float)((mw >> sh) & 0xffu));
  float ndm1 = -(dmin * (float)((mw >> (sh + 8)) & 0xffu));
  const h2 k1024 = {(half_t)1024.0f, (half_t)1024.0f};
  uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  const uint4* xv = (const uint4*)xs;
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    // x for weights l = 4i .. 4i+7 of sub-block 2p (at 0) and 2p+1 (at 32)
    uint4 xa = xv[i >> 1];
    uint4 xb = xv[4 + (i >> 1)];
    uint32_t xa_w[4] = {xa.x, xa.y, xa.z, xa.w};
    uint32_t xb_w[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t v = qw[i + u];
      uint32_t lo = v & 0x0f0f0f0fu;
      uint32_t hi = v & 0xf0f0f0f0u;
      h2 ql01 = as_h2(magic_pair_lo(lo)) - k1024;
      h2 ql23 = as_h2(magic_pair_hi(lo)) - k1024;
      h2 qh01 = as_h2(magic_pair_lo(hi)) - k1024;
      h2 qh23 = as_h2(magic_pair_hi(hi)) - k1024;
      h2 wl01 = {(half_t)__builtin_fmaf((float)ql01.x, dsc0, ndm0), (half_t)__builtin_fmaf((float)ql01.y, dsc0, ndm0)};
      h2 wl23 = {(half_t)__builtin_fmaf((float)ql23.x, dsc0, ndm0), (half_t)__builtin_fmaf((float)ql23.y, dsc0, ndm0)};
      h2 wh01 = {(half_t)__builtin_fmaf((float)qh01.x, dsc1, ndm1), (half_t)__builtin_fmaf((float)qh01.y, dsc1, ndm1)};
      h2 wh23 = {(half_t)__builtin_fmaf((float)qh23.x, dsc1, ndm1), (half_t)__builtin_fmaf((float)qh23.y, dsc1, ndm1)};
      acc0 = __builtin_amdgcn_fdot2(wl01, as_h2(xa_w[2 * u]), acc0, false);
      acc0 = __builtin_amdgcn_fdot2(wl23, as_h2(xa_w[2 * u + 1]), acc0, false);
      acc1 = __builtin_amdgcn_fdot2(wh01, as_h2(xb_w[2 * u]), acc1, false);
      acc1 = __builtin_amdgcn_fdot2(wh23, as_h2(xb_w[2 * u + 1]), acc1, false);
    }
  }
  return acc0 + acc1;
}

// Dot product of one Q6_K part (64 weights) with x (LDS).
__device__ __forceinline__ float q6k_part_dot(const uint8_t* blk, int p, const half_t* xs) {
  const int h = p >> 1, lh = p & 1;
  // quant fields: 16 B each at 2-aligned addresses; load_u128_a2 reads at
  // most 2 bytes before / 4 after, all inside the block (the last field read
  // ends by byte 176 + 20 = 196 < 210).
  uint4 qa = load_u128_a2(blk + 64 * h + 16 * lh);        // quarters t = 0 (lo), 2 (hi)
  uint4 qb = load_u128_a2(blk + 64 * h + 32 + 16 * lh);   // quarters t = 1 (lo), 3 (hi)
  uint4 qh = load_u128_a2(blk + 128 + 32 * h + 16 * lh);
  // scales (16 B at 192) and d (2 B at 208): read the aligned dwords that
  // cover bytes 192..209 without touching anything past byte 209.
  uintptr_t a = (uintptr_t)(blk + 192);
  const uint32_t* sp = (const uint32_t*)(a & ~(uintptr_t)3);
  uint32_t shb = (uint32_t)(a & 3);
  uint4 sv = *(const uint4*)sp;
  uint32_t s4 = shb ? sp[4] : (uint32_t)(*(const uint16_t*)(blk + 208));
  uint32_t sw[4] = {__builtin_amdgcn_alignbyte(sv.y, sv.x, shb), __builtin_amdgcn_alignbyte(sv.z, sv.y, shb),
                    __builtin_amdgcn_alignbyte(sv.w, sv.z, shb), __builtin_amdgcn_alignbyte(s4, sv.w, shb)};
  float d = half_bits_to_float(shb ? (s4 >> 16) : s4);
  const h2 k1056 = {(half_t)1056.0f, (half_t)1056.0f};
  uint32_t qaw[4] = {qa.x, qa.y, qa.z, qa.w};
  uint32_t qbw[4] = {qb.x, qb.y, qb.z, qb.w};
  uint32_t qhw[4] = {qh.x, qh.y, qh.z, qh.w};
  const uint4* xv = (const uint4*)xs;
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // scale index 8h + 2t + lh -> byte (2t + lh) of the h-th 8-byte group
    uint32_t sidx = 8 * h + 2 * t + lh;
    int sc = (int)(int8_t)((sw[sidx >> 2] >> (8 * (sidx & 3))) & 0xffu);
    float dsc = d * (float)sc;
    const uint32_t* ql = (t & 1) ? qbw : qaw;
    uint32_t nsh = (t >= 2) ? 4u : 0u;
    uint4 x0 = xv[4 * t];          // x[32t + 0 .. 8) relative to this part's base
    uint4 x1 = xv[4 * t + 1];
    uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float dt = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t q = ((ql[i] >> nsh) & 0x0f0f0f0fu) | (((qhw[i] >> (2 * t)) & 0x03030303u) << 4);
      h2 q01 = as_h2(magic_pair_lo(q)) - k1056;   // q - 32, exact
      h2 q23 = as_h2(magic_pair_hi(q)) - k1056;
      dt = __builtin_amdgcn_fdot2(q01, as_h2(xw[2 * i]), dt, false);
      dt = __builtin_amdgcn_fdot2(q23, as_h2(xw[2 * i + 1]), dt, false);
    }
    acc = __builtin_fmaf(dsc, dt, acc);
  }
  return acc;
}

template <int R, bool PAIR>
__device__ __forceinline__ void gemv_rows(const GemvDesc& P, int wg_local, const half_t* xs) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = P.K / QK;
  const int part = lane & 3;
  const int row0 = (wg_local * 4 + wave) * R;          // first row of this wave
  const int nrows_out = PAIR ? P.N / 2 : P.N;
  const int64_t row_bytes = (int64_t)nb * (P.fmt == 0 ? Q4K_BYTES : Q6K_BYTES);
  const int items = R * nb;                            // (row, block) pairs
  float acc[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { acc[r] = 0.0f; accu[r] = 0.0f; }
  for (int it = lane >> 2; it < items; it += 16) {
    const int rl = it / nb;
    const int b = it - rl * nb;
    int row = row0 + rl;
    row = row < nrows_out ? row : nrows_out - 1;        // ragged tail: clamp, result dropped
    const half_t* xp;
    float v, vu = 0.0f;
    if (P.fmt == 0) {
      xp = xs + b * QK + 64 * part;
      v = q4k_part_dot(P.wq + row * row_bytes + (int64_t)b * Q4K_BYTES, part, xp);
      if (PAIR) vu = q4k_part_dot(P.wq + (row + nrows_out) * row_bytes + (int64_t)b * Q4K_BYTES, part, xp);
    } else {
      xp = xs + b * QK + 128 * (part >> 1) + 16 * (part & 1);
      v = q6k_part_dot(P.wq + row * row_bytes + (int64_t)b * Q6K_BYTES, part, xp);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] += (rl == r) ? v : 0.0f;
      if (PAIR) accu[r] += (rl == r) ? vu : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float g = wave_sum(acc[r]);
    float u = PAIR ? wave_sum(accu[r]) : 0.0f;
    const int row = row0 + r;
    if (lane == 0 && row < nrows_out) {
      if (PAIR) {
        ((half_t*)P.out)[row] = (half_t)(silu_f32(g) * u);
      } else {
        ((float*)P.out)[row] = g;
      }
    }
  }
}

__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs args) {
  extern __shared__ __attribute__((aligned(16))) half_t xs[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMV_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].wg_begin) pi = i;
  const GemvDesc& P = args.d[pi];
  const int wg_local = (int)blockIdx.x - P.wg_begin;
  // stage x into LDS (16 B per thread per pass)
  for (int i = threadIdx.x; i < P.K / 8; i += blockDim.x)
    ((uint4*)xs)[i] = ((const uint4*)P.x)[i];
  __syncthreads();
  switch (P.rows_log2 * 2 + P.swiglu) {
    case 0: gemv_rows<1, false>(P, wg_local, xs); break;
    case 1: gemv_rows<1, true>(P, wg_local, xs); break;
    case 2: gemv_rows<2, false>(P, wg_local, xs); break;
    case 3: gemv_rows<2, true>(P, wg_local, xs); break;
    case 4: gemv_rows<4, false>(P, wg_local, xs); break;
    case 5: gemv_rows<4, true>(P, wg_local, xs); break;
    case 6: gemv_rows<8, false>(P, wg_local, xs); break;
    case 7: gemv_rows<8, true>(P, wg_local, xs); break;
    case 8: gemv_rows<16, false>(P, wg_local, xs); break;
    default: gemv_rows<16, true>(P, wg_local, xs); break;
  }
}

static int rows_log2_for(int nb) {
  // smallest R (power of 2, <= 16) with R * nb a multiple of 16
  for (int lg = 0; lg <= 4; ++lg)
    if (((nb << lg) & 15) == 0) return lg;
  return 4;
}

hipError_t launch_gemv(const GemmProblem* probs, int count, hipStream_t s) {
  for (int base = 0; base < count; base += GEMV_MAX_GROUP) {
    GemvArgs a{};
    int n = count - base < GEMV_MAX_GROUP ? count - base : GEMV_MAX_GROUP;
    int wgs = 0, kmax = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = probs[base + i];
      GemvDesc& d = a.d[i];
      d.x = (const half_t*)p.x;
      d.wq = p.wq;
      d.out = p.out;
      d.fmt = p.fmt;
      d.swiglu = p.swiglu;
      d.N = p.N;
      d.K = p.K;
      d.rows_log2 = rows_log2_for(p.K / QK);
      d.wg_begin = wgs;
      int rows = p.swiglu ? p.N / 2 : p.N;
      int rows_per_wg = 4 << d.rows_log2;
      wgs += (rows + rows_per_wg - 1) / rows_per_wg;
      kmax = p.K > kmax ? p.K : kmax;
    }
    a.count = n;
    hipLaunchKernelGGL(gemv_kernel, dim3(wgs), dim3(256), (size_t)kmax * sizeof(half_t), s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dmq
