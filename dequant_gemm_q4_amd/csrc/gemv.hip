// Decode (M = 1) kernel: y[n] = sum_k x[k] * W[n][k] with W in Q4_K or Q6_K.
//
// Decode handles a single token per step and is bound by streaming the weights
// from memory (overview page, "[01] the thesis" and "[04] one decode step";
// article "Building DAMASCUS", "Prefill and decode need different performance
// questions").  The kernel is built around the HBM stream:
//
//  * a workgroup owns 16 consecutive rows; lane l of each wave works on row
//    l/4 and on part l%4 of every super-block of it, so each lane adds into
//    one row only and a wave reads 16 rows' blocks side by side;
//  * the 4 waves split the row's super-blocks into 4 contiguous slices: a
//    wave stages only its slice of x in LDS, streams its blocks with the
//    next block's loads in flight, and the 4 partial sums per row are added
//    through LDS in wave order (no atomics, the same result every run);
//  * every byte of W is read exactly once; Q6_K blocks (210 bytes, so a
//    field may start 2 mod 4) are read with 2-byte-aligned 16-byte loads;
//  * the sub-block scale and min are factored out of the dot products, so
//    four weights cost one byte permute, two masks, two packed fp16
//    subtracts and two v_dot2_f32_f16.  Q4_K: per 32-weight sub-block with
//    a = d*sc and b = dmin*m,
//    sum x (a q - b) = a * sum x (q - c) - (b - a c) * sum x,
//    where c is the integer in [0, 15] nearest b / a.  q - c is exact in
//    fp16, and centring on c keeps every term's size within a small multiple
//    of |a q - b| (|b - a c| <= a / 2 unless c is clamped, and then no
//    weight changes sign), so the fp32 rounding error stays a few units of
//    2^-24 times sum |x*w| even where the weights cancel to exact zeros.
//    The sums of x per sub-block are formed once, as x is staged.  Q6_K has
//    no min: its scale is factored out of each 16-weight dot, with the
//    quants as fp16 magic numbers minus 1056 (exact);
//  * SwiGLU pairs (gate row r and up row r + N/2 in the same lane) live in
//    their own kernel instance: they need twice the registers.
//
// Lane parts: Q4_K part p owns quant bytes 32p..32p+31, i.e. sub-blocks 2p
// (low nibbles) and 2p+1 (high nibbles).  Q6_K part p owns half h = p >> 1
// and weights with l in [16(p&1), 16(p&1)+16) of its four 32-weight quarters.
#include "dmq_common.h"
#include "gemv.h"

#include <utility>

namespace dmq {

constexpr int GEMV_MAX_GROUP = 8;

// Activation rows of one launch: 1, or 2 with both rows' x staged (at most
// 96 KB of LDS, so K up to 20480 at two rows).
bool gemv_rows_fit(int64_t m, int64_t kmax) {
  return m >= 1 && m <= GEMV_MAX_ROWS && m * ((kmax / 64) * 144 + (kmax / 32) * 4) <= 96 * 1024;
}

struct GemvDesc {
  const half_t* x;
  const uint8_t* wq;
  void* out;
  const float* g;     // RMSNorm weights (K floats), or NULL: x is used as it is
  float eps;
  half_t* xn;         // with g: workgroup 0 writes the normalized x here (if set)
  const float* hin;   // residual mode (with g): x = h_in + hadd in fp32, x is unused ...
  const float* hadd;
  float* hout;        // ... and workgroup 0 writes that sum here (if set)
  int32_t fmt, swiglu, N, K;
  int32_t m;          // activation rows (the few-rows kernel; 1 otherwise)
  int32_t wg_begin;   // first workgroup of this problem
};

struct GemvArgs {
  GemvDesc d[GEMV_MAX_GROUP];
  int32_t count;
  int32_t sx_offset;   // byte offset of the sums of x per 32 values in dynamic LDS
};

// x in LDS: each group of 64 values (128 bytes) is followed by 16 bytes of
// padding.  A wave's lanes read the x of the four parts of one block at a
// time; Q4_K parts are one group apart, which unpadded would put parts 0 and
// 2 (and 1 and 3) on the same banks, and padded puts all four on distinct
// ones.  (Q6_K parts 1 and 2 still share banks; a layout without that
// conflict measured no faster.)  After the whole row's x come the fp32 sums
// of x over each run of 32 values (Q4_K sub-blocks), K / 32 floats.
constexpr int X_GROUP_BYTES = 144;

typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// fp32 pair -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ h2 pack_h2(float a, float b) {
  const f2 v = {a, b};
  return __builtin_convertvector(v, h2);
}

// Raw bytes of one lane's part of one block, loaded before any is used.
struct PartQ4 {
  uint4 hdr, q0, q1;
};
struct PartQ6 {
  uint4 qa, qb, qh;    // low nibbles (quarters 0/2, 1/3) and high bits
  uint2 sc;            // the 8 scales of half h
  uint32_t s206;       // halfwords 206 and 208: d in the high half
};
template <int FMT> struct PartOf { typedef PartQ4 T; };
template <> struct PartOf<1> { typedef PartQ6 T; };

typedef uint32_t u32_a2 __attribute__((aligned(2)));

__device__ __forceinline__ void load_part(const uint8_t* blk, int p, PartQ4& r) {
  r.hdr = *(const uint4*)blk;
  r.q0 = *(const uint4*)(blk + 16 + 32 * p);
  r.q1 = *(const uint4*)(blk + 32 + 32 * p);
}
// Q6_K blocks are 210 bytes, so a block (and every field in it) may start
// 2 mod 4; the loads below are 2-byte aligned, which the global memory path
// serves like aligned ones.
typedef uint4 u4_a2 __attribute__((aligned(2)));
typedef uint2 u2_a2 __attribute__((aligned(2)));
__device__ __forceinline__ void load_part(const uint8_t* blk, int p, PartQ6& r) {
  const int h = p >> 1, lh = p & 1;
  r.qa = *(const u4_a2*)(blk + 64 * h + 16 * lh);
  r.qb = *(const u4_a2*)(blk + 64 * h + 32 + 16 * lh);
  r.qh = *(const u4_a2*)(blk + 128 + 32 * h + 16 * lh);
  r.sc = *(const u2_a2*)(blk + 192 + 8 * h);
  r.s206 = *(const u32_a2*)(blk + 206);
}

// Dot product of one Q4_K part (64 weights) with x (LDS; xs = x of this part:
// xs[0..31] for sub-block 2p, xs[32..63] for sub-block 2p+1; sx = the sums of
// those two runs of x), factored per sub-block around c = round(b / a).
__device__ __forceinline__ float part_dot(const PartQ4& r, int p, const half_t* xs, const float* sx) {
  Q4kScales s = unpack_q4k_scales(r.hdr.y, r.hdr.z, r.hdr.w);
  const uint32_t scw = p < 2 ? s.sc_lo : s.sc_hi;
  const uint32_t mw = p < 2 ? s.m_lo : s.m_hi;
  const uint32_t sh = (uint32_t)(p & 1) * 16u;
  const float d = half_bits_to_float(r.hdr.x);
  const float dmin = half_bits_to_float(r.hdr.x >> 16);
  // a = d*sc and b = dmin*m are exact in fp32 (11-bit times 6-bit)
  const float a0 = d * (float)((scw >> sh) & 0xffu);
  const float a1 = d * (float)((scw >> (sh + 8)) & 0xffu);
  const float b0 = dmin * (float)((mw >> sh) & 0xffu);
  const float b1 = dmin * (float)((mw >> (sh + 8)) & 0xffu);
  // c in [0, 15]; a = 0 gives b * inf (or NaN when b = 0 too), which the
  // clamp turns into 15 (or 0): any c is correct, it only sizes the terms
  const float c0 = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(b0 * __builtin_amdgcn_rcpf(a0)), 0.0f), 15.0f);
  const float c1 = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(b1 * __builtin_amdgcn_rcpf(a1)), 0.0f), 15.0f);
  const float e0 = __builtin_fmaf(-a0, c0, b0);   // b - a c (exact where it matters)
  const float e1 = __builtin_fmaf(-a1, c1, b1);
  // a quant byte B goes to fp16 as [0x64, B]: masked to the low nibble that
  // is 1024 + q, to the high nibble 1024 + 16 q; subtracting 1024 + c (or
  // 1024 + 16 c) leaves q - c (or 16 (q - c)) exactly
  const half_t n0 = (half_t)(-1024.0f - c0), n1 = (half_t)(-1024.0f - 16.0f * c1);
  const h2 bias0 = {n0, n0}, bias1 = {n1, n1};
  const uint32_t qw[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
  const uint4* xv = (const uint4*)xs;
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    // x for weights l = 4i .. 4i+7 of sub-block 2p (at 0) and 2p+1 (at 32)
    const uint4 xa = xv[i >> 1];
    const uint4 xb = xv[4 + (i >> 1)];
    const uint32_t xa_w[4] = {xa.x, xa.y, xa.z, xa.w};
    const uint32_t xb_w[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // bytes [0x64, B1, 0x64, B0] and [0x64, B3, 0x64, B2] of the quant word
      const uint32_t p01 = __builtin_amdgcn_perm(0x64646464u, qw[i + u], 0x04010400u);
      const uint32_t p23 = __builtin_amdgcn_perm(0x64646464u, qw[i + u], 0x04030402u);
      const h2 l01 = as_h2(p01 & 0xff0fff0fu) + bias0;
      const h2 l23 = as_h2(p23 & 0xff0fff0fu) + bias0;
      const h2 h01 = as_h2(p01 & 0xfff0fff0u) + bias1;
      const h2 h23 = as_h2(p23 & 0xfff0fff0u) + bias1;
      acc0 = __builtin_amdgcn_fdot2(l01, as_h2(xa_w[2 * u]), acc0, false);
      acc0 = __builtin_amdgcn_fdot2(l23, as_h2(xa_w[2 * u + 1]), acc0, false);
      acc1 = __builtin_amdgcn_fdot2(h01, as_h2(xb_w[2 * u]), acc1, false);
      acc1 = __builtin_amdgcn_fdot2(h23, as_h2(xb_w[2 * u + 1]), acc1, false);
    }
  }
  const float2 sxp = *(const float2*)sx;
  float y = a0 * acc0;
  y = __builtin_fmaf(-e0, sxp.x, y);
  y = __builtin_fmaf(a1 * 0.0625f, acc1, y);
  return __builtin_fmaf(-e1, sxp.y, y);
}

// Dot product of one Q6_K part (64 weights) with x (LDS, padded layout; xs =
// x of weight 128h + 16lh of the block: quarter t's 16 values start
// X_GROUP_BYTES * (t / 2) + 64 * (t % 2) bytes further).
__device__ __forceinline__ float part_dot(const PartQ6& r, int p, const half_t* xs) {
  const int lh = p & 1;
  const uint4 qa = r.qa, qb = r.qb, qh = r.qh;
  const float d = half_bits_to_float(r.s206 >> 16);
  const h2 k1056 = {(half_t)1056.0f, (half_t)1056.0f};
  const uint32_t qaw[4] = {qa.x, qa.y, qa.z, qa.w};
  const uint32_t qbw[4] = {qb.x, qb.y, qb.z, qb.w};
  const uint32_t qhw[4] = {qh.x, qh.y, qh.z, qh.w};
  const uint4* xv = (const uint4*)xs;
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // scale index 8h + 2t + lh -> byte (2t + lh) of the h-th 8-byte group
    const uint32_t sb = 2 * t + lh;
    const int sc = (int)(int8_t)((((sb >> 2) ? r.sc.y : r.sc.x) >> (8 * (sb & 3))) & 0xffu);
    const float dsc = d * (float)sc;
    const uint32_t* ql = (t & 1) ? qbw : qaw;
    const uint32_t nsh = (t >= 2) ? 4u : 0u;
    const uint4* xq = (const uint4*)((const uint8_t*)xv + X_GROUP_BYTES * (t >> 1) + 64 * (t & 1));
    const uint4 x0 = xq[0];              // x[32t + 0 .. 8) relative to this part's base
    const uint4 x1 = xq[1];
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float dt = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t q = ((ql[i] >> nsh) & 0x0f0f0f0fu) | (((qhw[i] >> (2 * t)) & 0x03030303u) << 4);
      const h2 q01 = as_h2(magic_pair_lo(q)) - k1056;   // q - 32, exact
      const h2 q23 = as_h2(magic_pair_hi(q)) - k1056;
      dt = __builtin_amdgcn_fdot2(q01, as_h2(xw[2 * i]), dt, false);
      dt = __builtin_amdgcn_fdot2(q23, as_h2(xw[2 * i + 1]), dt, false);
    }
    acc = __builtin_fmaf(dsc, dt, acc);
  }
  return acc;
}

// The same dot products for NR activation rows at once: the quants are
// converted once and meet each row's x (row r's staged x at xs + r * xrb
// bytes, its sums of x at sx + r * srb floats).  Each row's arithmetic is
// the single-row part_dot's, in the same order; the part's value is added
// to tot[r].
template <int NR>
__device__ __forceinline__ void part_dot_nr(const PartQ4& r_, int p, const uint8_t* xs, int xrb, const float* sx, int srb,
                                            float (&tot)[NR]) {
  Q4kScales s = unpack_q4k_scales(r_.hdr.y, r_.hdr.z, r_.hdr.w);
  const uint32_t scw = p < 2 ? s.sc_lo : s.sc_hi;
  const uint32_t mw = p < 2 ? s.m_lo : s.m_hi;
  const uint32_t sh = (uint32_t)(p & 1) * 16u;
  const float d = half_bits_to_float(r_.hdr.x);
  const float dmin = half_bits_to_float(r_.hdr.x >> 16);
  const float a0 = d * (float)((scw >> sh) & 0xffu);
  const float a1 = d * (float)((scw >> (sh + 8)) & 0xffu);
  const float b0 = dmin * (float)((mw >> sh) & 0xffu);
  const float b1 = dmin * (float)((mw >> (sh + 8)) & 0xffu);
  const float c0 = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(b0 * __builtin_amdgcn_rcpf(a0)), 0.0f), 15.0f);
  const float c1 = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(b1 * __builtin_amdgcn_rcpf(a1)), 0.0f), 15.0f);
  const float e0 = __builtin_fmaf(-a0, c0, b0);
  const float e1 = __builtin_fmaf(-a1, c1, b1);
  const half_t n0 = (half_t)(-1024.0f - c0), n1 = (half_t)(-1024.0f - 16.0f * c1);
  const h2 bias0 = {n0, n0}, bias1 = {n1, n1};
  const uint32_t qw[8] = {r_.q0.x, r_.q0.y, r_.q0.z, r_.q0.w, r_.q1.x, r_.q1.y, r_.q1.z, r_.q1.w};
  float acc0[NR], acc1[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc0[r] = acc1[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t p01 = __builtin_amdgcn_perm(0x64646464u, qw[i + u], 0x04010400u);
      const uint32_t p23 = __builtin_amdgcn_perm(0x64646464u, qw[i + u], 0x04030402u);
      const h2 l01 = as_h2(p01 & 0xff0fff0fu) + bias0;
      const h2 l23 = as_h2(p23 & 0xff0fff0fu) + bias0;
      const h2 h01 = as_h2(p01 & 0xfff0fff0u) + bias1;
      const h2 h23 = as_h2(p23 & 0xfff0fff0u) + bias1;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint4* xv = (const uint4*)(xs + r * xrb);
        const uint4 xa = xv[i >> 1];
        const uint4 xb = xv[4 + (i >> 1)];
        const uint32_t xa_w[4] = {xa.x, xa.y, xa.z, xa.w};
        const uint32_t xb_w[4] = {xb.x, xb.y, xb.z, xb.w};
        acc0[r] = __builtin_amdgcn_fdot2(l01, as_h2(xa_w[2 * u]), acc0[r], false);
        acc0[r] = __builtin_amdgcn_fdot2(l23, as_h2(xa_w[2 * u + 1]), acc0[r], false);
        acc1[r] = __builtin_amdgcn_fdot2(h01, as_h2(xb_w[2 * u]), acc1[r], false);
        acc1[r] = __builtin_amdgcn_fdot2(h23, as_h2(xb_w[2 * u + 1]), acc1[r], false);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float2 sxp = *(const float2*)(sx + r * srb);
    float y = a0 * acc0[r];
    y = __builtin_fmaf(-e0, sxp.x, y);
    y = __builtin_fmaf(a1 * 0.0625f, acc1[r], y);
    tot[r] += __builtin_fmaf(-e1, sxp.y, y);
  }
}

template <int NR>
__device__ __forceinline__ void part_dot_nr(const PartQ6& r_, int p, const uint8_t* xs, int xrb, const float*, int,
                                            float (&tot)[NR]) {
  const int lh = p & 1;
  const uint4 qa = r_.qa, qb = r_.qb, qh = r_.qh;
  const float d = half_bits_to_float(r_.s206 >> 16);
  const h2 k1056 = {(half_t)1056.0f, (half_t)1056.0f};
  const uint32_t qaw[4] = {qa.x, qa.y, qa.z, qa.w};
  const uint32_t qbw[4] = {qb.x, qb.y, qb.z, qb.w};
  const uint32_t qhw[4] = {qh.x, qh.y, qh.z, qh.w};
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t sb = 2 * t + lh;
    const int sc = (int)(int8_t)((((sb >> 2) ? r_.sc.y : r_.sc.x) >> (8 * (sb & 3))) & 0xffu);
    const float dsc = d * (float)sc;
    const uint32_t* ql = (t & 1) ? qbw : qaw;
    const uint32_t nsh = (t >= 2) ? 4u : 0u;
    const int xo = X_GROUP_BYTES * (t >> 1) + 64 * (t & 1);
    float dt[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) dt[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t q = ((ql[i] >> nsh) & 0x0f0f0f0fu) | (((qhw[i] >> (2 * t)) & 0x03030303u) << 4);
      const h2 q01 = as_h2(magic_pair_lo(q)) - k1056;
      const h2 q23 = as_h2(magic_pair_hi(q)) - k1056;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint4 xq = *(const uint4*)(xs + r * xrb + xo + 16 * (i >> 1));
        const uint32_t xw0 = (i & 1) ? xq.z : xq.x, xw1 = (i & 1) ? xq.w : xq.y;
        dt[r] = __builtin_amdgcn_fdot2(q01, as_h2(xw0), dt[r], false);
        dt[r] = __builtin_amdgcn_fdot2(q23, as_h2(xw1), dt[r], false);
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = __builtin_fmaf(dsc, dt[r], acc[r]);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) tot[r] += acc[r];
}

// byte offset of the x of a lane's part of block b
template <int FMT>
__device__ __forceinline__ int part_x_offset(int b, int part) {
  return FMT == 0 ? X_GROUP_BYTES * (4 * b + part) : X_GROUP_BYTES * (4 * b + 2 * (part >> 1)) + 32 * (part & 1);
}

// A wave covers 16 rows x 4 parts; the 4 waves of a workgroup split the
// super-blocks of the same 16 rows.
constexpr int GEMV_ROWS = 16;

// Sum of x over 32 values (chunk i holds values 8i .. 8i+7 as staged): each
// lane adds its chunk's 8 values in a fixed order, the 4 lanes of a quad
// (chunks 4j .. 4j+3, which every caller keeps active together) add theirs,
// and the quad's first lane stores the sum of run j.
__device__ __forceinline__ void put_xsum(float* sxs, int i, uint4 v) {
  const h2 v0 = as_h2(v.x), v1 = as_h2(v.y), v2 = as_h2(v.z), v3 = as_h2(v.w);
  float t = (((float)v0.x + (float)v0.y) + ((float)v1.x + (float)v1.y)) +
            (((float)v2.x + (float)v2.y) + ((float)v3.x + (float)v3.y));
  t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0xb1, 0xf, 0xf, false));
  t += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, t), 0x4e, 0xf, 0xf, false));
  if ((threadIdx.x & 3) == 0) sxs[i >> 2] = t;
}

// 1 / sqrt(mean((a + b)^2) + eps) over a row of K fp32 values: the sum a + b
// rounded to fp32 first, as the residual connection stores it.
__device__ __forceinline__ float rms_inv_sum(const float* a, const float* b, int K, float eps, float* red4) {
  float ss = 0.0f;
  for (int i = (int)threadIdx.x; i < K / 4; i += 256) {
    const float4 x = ((const float4*)a)[i], y = ((const float4*)b)[i];
    const float4 h = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    ss += (h.x * h.x + h.y * h.y) + (h.z * h.z + h.w * h.w);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float t = (red4[0] + red4[1]) + (red4[2] + red4[3]);
  return 1.0f / __builtin_sqrtf(t / (float)K + eps);
}

template <int FMT, bool PAIR>
__device__ __forceinline__ void gemv_tile(const GemvDesc& P, int wg_local, half_t* xs, float* sxs, float* red,
                                          float* red4) {
  typedef typename PartOf<FMT>::T Part;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = lane & 3, rq = lane >> 2;
  const int nb = P.K / QK;
  const int rows_out = PAIR ? P.N / 2 : P.N;
  const int64_t row_bytes = (int64_t)nb * BLOCK_BYTES;
  const int row = wg_local * GEMV_ROWS + rq;
  const int rowc = row < rows_out ? row : rows_out - 1;   // ragged tail: clamp, result dropped
  const int b0 = wave * nb / 4, b1 = (wave + 1) * nb / 4;  // this wave's super-blocks
  const uint8_t* wg_ = P.wq + (int64_t)rowc * row_bytes;
  const uint8_t* wu_ = P.wq + (int64_t)(rowc + rows_out) * row_bytes;

  // x of this wave's slice: global loads first, so the weight loads issued
  // next stay in flight while the slice is written to LDS
  const int xchunks = (b1 - b0) * 32;                     // 16-byte chunks
  const bool res = P.hin != nullptr;                      // residual mode: no fp16 x
  const uint4* xg = (const uint4*)P.x + b0 * 32;
  const bool xa = !res && lane < xchunks, xb = !res && lane + 64 < xchunks;
  uint4 xra = {0, 0, 0, 0}, xrb = {0, 0, 0, 0};
  if (xa) xra = xg[lane];
  if (xb) xrb = xg[lane + 64];

  Part g0, u0p, g1, u1p;
  if (b0 < b1) {
    load_part(wg_ + (int64_t)b0 * BLOCK_BYTES, part, g0);
    if (PAIR) load_part(wu_ + (int64_t)b0 * BLOCK_BYTES, part, u0p);
  }
  // RMSNorm (when P.g is set): the workgroup's sum of squares over the
  // whole row, then each wave scales its slice as it stages it
  // residual mode with slices of at most 4 blocks (K <= 4096, the same test in
  // every wave): one pass, each lane keeps the sums of its own (at most two)
  // chunks in registers while the row's sum of squares is reduced
  const bool res1 = res && nb <= 16;
  float4 hk[2][2];
  float ss1 = 0.0f;
  if (res1) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = b0 * 32 + lane + 64 * j;
      if (lane + 64 * j < xchunks) {
        const float4 a0 = ((const float4*)P.hin)[2 * i], a1 = ((const float4*)P.hin)[2 * i + 1];
        const float4 c0 = ((const float4*)P.hadd)[2 * i], c1 = ((const float4*)P.hadd)[2 * i + 1];
        hk[j][0] = make_float4(a0.x + c0.x, a0.y + c0.y, a0.z + c0.z, a0.w + c0.w);
        hk[j][1] = make_float4(a1.x + c1.x, a1.y + c1.y, a1.z + c1.z, a1.w + c1.w);
        ss1 += ((hk[j][0].x * hk[j][0].x + hk[j][0].y * hk[j][0].y) +
                (hk[j][0].z * hk[j][0].z + hk[j][0].w * hk[j][0].w)) +
               ((hk[j][1].x * hk[j][1].x + hk[j][1].y * hk[j][1].y) +
                (hk[j][1].z * hk[j][1].z + hk[j][1].w * hk[j][1].w));
      }
    }
    ss1 = wave_sum(ss1);
    if (lane == 0) red4[wave] = ss1;
    __syncthreads();
  }
  const float rn = !P.g ? 1.0f
                 : res1 ? 1.0f / __builtin_sqrtf(((red4[0] + red4[1]) + (red4[2] + red4[3])) / (float)P.K + P.eps)
                 : res  ? rms_inv_sum(P.hin, P.hadd, P.K, P.eps, red4)
                        : rms_inv(P.x, P.K, P.eps, red4);
  auto xput = [&](int i, uint4 v) {
    if (P.g) {
      v = norm8(v, P.g + 8 * i, rn);
      if (P.xn && wg_local == 0) ((uint4*)P.xn)[i] = v;
    }
    *(uint4*)((uint8_t*)xs + X_GROUP_BYTES * (i >> 3) + 16 * (i & 7)) = v;
    if (FMT == 0) put_xsum(sxs, i, v);
  };
  if (!res) {
    if (xa) xput(b0 * 32 + lane, xra);
    if (xb) xput(b0 * 32 + lane + 64, xrb);
    for (int i = b0 * 32 + lane + 128; i < b1 * 32; i += 64)   // slices of more than 4 blocks
      xput(i, ((const uint4*)P.x)[i]);
  } else {
    // residual mode: h = h_in + hadd (fp32, the residual stream; workgroup 0
    // stores it), staged as fp16(h * g * r) like the residual kernel's xn
    for (int i = b0 * 32 + lane, j = 0; i < b1 * 32; i += 64, ++j) {
      float4 h0, h1;
      if (res1) {   // j < 2 here: the slice has at most 128 chunks
        h0 = j == 0 ? hk[0][0] : hk[1][0];
        h1 = j == 0 ? hk[0][1] : hk[1][1];
      } else {
        const float4 a0 = ((const float4*)P.hin)[2 * i], a1 = ((const float4*)P.hin)[2 * i + 1];
        const float4 c0 = ((const float4*)P.hadd)[2 * i], c1 = ((const float4*)P.hadd)[2 * i + 1];
        h0 = make_float4(a0.x + c0.x, a0.y + c0.y, a0.z + c0.z, a0.w + c0.w);
        h1 = make_float4(a1.x + c1.x, a1.y + c1.y, a1.z + c1.z, a1.w + c1.w);
      }
      if (P.hout && wg_local == 0) {
        ((float4*)P.hout)[2 * i] = h0;
        ((float4*)P.hout)[2 * i + 1] = h1;
      }
      const float4 g0 = ((const float4*)P.g)[2 * i], g1 = ((const float4*)P.g)[2 * i + 1];
      const h2 p0 = {(half_t)((h0.x * g0.x) * rn), (half_t)((h0.y * g0.y) * rn)};
      const h2 p1 = {(half_t)((h0.z * g0.z) * rn), (half_t)((h0.w * g0.w) * rn)};
      const h2 p2 = {(half_t)((h1.x * g1.x) * rn), (half_t)((h1.y * g1.y) * rn)};
      const h2 p3 = {(half_t)((h1.z * g1.z) * rn), (half_t)((h1.w * g1.w) * rn)};
      const uint4 v = make_uint4(as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3));
      if (P.xn && wg_local == 0) ((uint4*)P.xn)[i] = v;
      *(uint4*)((uint8_t*)xs + X_GROUP_BYTES * (i >> 3) + 16 * (i & 7)) = v;
      if (FMT == 0) put_xsum(sxs, i, v);
    }
  }
  // only this wave reads its slice: wait for its own LDS writes, no barrier
  // (the asm is also a compiler barrier for the LDS accesses around it)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  float acc = 0.0f, accu = 0.0f;
  auto step = [&](int b, const Part& g, const Part& up) {
    const half_t* xp = (const half_t*)((const uint8_t*)xs + part_x_offset<FMT>(b, part));
    if constexpr (FMT == 0) {
      const float* sp = sxs + 8 * b + 2 * part;   // sub-blocks 2p, 2p+1 of block b
      acc += part_dot(g, part, xp, sp);
      if (PAIR) accu += part_dot(up, part, xp, sp);
    } else {
      acc += part_dot(g, part, xp);
    }
  };
  // the next block's loads go out at raised wave priority, so that the other
  // waves' dequant on this SIMD does not hold back the memory requests
  for (int b = b0; b < b1; b += 2) {
    if (b + 1 < b1) {
      __builtin_amdgcn_s_setprio(2);
      load_part(wg_ + (int64_t)(b + 1) * BLOCK_BYTES, part, g1);
      if (PAIR) load_part(wu_ + (int64_t)(b + 1) * BLOCK_BYTES, part, u1p);
      __builtin_amdgcn_s_setprio(0);
    }
    step(b, g0, u0p);
    if (b + 1 < b1) {
      if (b + 2 < b1) {
        __builtin_amdgcn_s_setprio(2);
        load_part(wg_ + (int64_t)(b + 2) * BLOCK_BYTES, part, g0);
        if (PAIR) load_part(wu_ + (int64_t)(b + 2) * BLOCK_BYTES, part, u0p);
        __builtin_amdgcn_s_setprio(0);
      }
      step(b + 1, g1, u1p);
    }
  }

  auto quad_sum = [](float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
    return v;
  };
  acc = quad_sum(acc);
  if (PAIR) accu = quad_sum(accu);
  if (part == 0) {
    red[wave * 2 * GEMV_ROWS + rq] = acc;
    if (PAIR) red[wave * 2 * GEMV_ROWS + GEMV_ROWS + rq] = accu;
  }
  __syncthreads();
  if (threadIdx.x < GEMV_ROWS) {
    const int r = threadIdx.x;
    const int orow = wg_local * GEMV_ROWS + r;
    float gs = red[r], us = red[GEMV_ROWS + r];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      gs += red[w * 2 * GEMV_ROWS + r];
      if (PAIR) us += red[w * 2 * GEMV_ROWS + GEMV_ROWS + r];
    }
    if (orow < rows_out) {
      if (PAIR)
        ((half_t*)P.out)[orow] = (half_t)(silu_f32(gs) * us);
      else
        ((float*)P.out)[orow] = gs;
    }
  }
}

template <bool PAIRS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs args) {
  extern __shared__ __attribute__((aligned(16))) half_t xs[];
  __shared__ float red[4 * 2 * GEMV_ROWS];
  __shared__ float red4[4];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMV_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].wg_begin) pi = i;
  const GemvDesc& P = args.d[pi];
  const int wg_local = (int)blockIdx.x - P.wg_begin;
  float* sxs = (float*)((uint8_t*)xs + args.sx_offset);
  if (P.fmt == 0) {
    if (PAIRS && P.swiglu)
      gemv_tile<0, PAIRS>(P, wg_local, xs, sxs, red, red4);
    else
      gemv_tile<0, false>(P, wg_local, xs, sxs, red, red4);
  } else {
    gemv_tile<1, false>(P, wg_local, xs, sxs, red, red4);
  }
}

// Decode kernel for NR activation rows (M <= NR; launched with NR = 2 for
// M = 2): the single-row kernel's shape and arithmetic, with the x of every
// row staged (rows past M as zeros) and each part's quants converted once
// for all rows.  Row r's result has the same bits as a single-row call on
// row r.  No RMSNorm or residual modes.  LDS: NR rows of x (xrb bytes
// each), then NR rows of sums (srb floats each).  A four-row form ran
// slower than the small-M MFMA kernel at M = 3 and 4 (its SwiGLU pair
// holds 230 VGPRs), so it is not built.
template <int FMT, bool PAIR, int NR>
__device__ __forceinline__ void gemv_tile_nr(const GemvDesc& P, int wg_local, int M, uint8_t* xl, int xrb, int srb,
                                             float* red) {
  typedef typename PartOf<FMT>::T Part;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = lane & 3, rq = lane >> 2;
  const int nb = P.K / QK;
  const int rows_out = PAIR ? P.N / 2 : P.N;
  const int64_t row_bytes = (int64_t)nb * BLOCK_BYTES;
  const int row = wg_local * GEMV_ROWS + rq;
  const int rowc = row < rows_out ? row : rows_out - 1;   // ragged tail: clamp, result dropped
  const int b0 = wave * nb / 4, b1 = (wave + 1) * nb / 4;
  const uint8_t* wg_ = P.wq + (int64_t)rowc * row_bytes;
  const uint8_t* wu_ = P.wq + (int64_t)(rowc + rows_out) * row_bytes;
  float* const sxl = (float*)(xl + NR * xrb);

  Part g0, u0p, g1, u1p;
  if (b0 < b1) {
    load_part(wg_ + (int64_t)b0 * BLOCK_BYTES, part, g0);
    if (PAIR) load_part(wu_ + (int64_t)b0 * BLOCK_BYTES, part, u0p);
  }
  // this wave's slice of every row's x (each row's sums as in the
  // single-row kernel); only this wave reads it
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    for (int i = b0 * 32 + lane; i < b1 * 32; i += 64) {
      const uint4 v = r < M ? ((const uint4*)P.x)[(int64_t)r * (P.K / 8) + i] : make_uint4(0, 0, 0, 0);
      *(uint4*)(xl + r * xrb + X_GROUP_BYTES * (i >> 3) + 16 * (i & 7)) = v;
      if (FMT == 0) put_xsum(sxl + r * srb, i, v);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  float acc[NR], accu[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = accu[r] = 0.0f;
  auto step = [&](int b, const Part& g, const Part& up) {
    const uint8_t* xp = xl + part_x_offset<FMT>(b, part);
    const float* sp = sxl + 8 * b + 2 * part;
    part_dot_nr<NR>(g, part, xp, xrb, sp, srb, acc);
    if (PAIR) part_dot_nr<NR>(up, part, xp, xrb, sp, srb, accu);
  };
  for (int b = b0; b < b1; b += 2) {
    if (b + 1 < b1) {
      __builtin_amdgcn_s_setprio(2);
      load_part(wg_ + (int64_t)(b + 1) * BLOCK_BYTES, part, g1);
      if (PAIR) load_part(wu_ + (int64_t)(b + 1) * BLOCK_BYTES, part, u1p);
      __builtin_amdgcn_s_setprio(0);
    }
    step(b, g0, u0p);
    if (b + 1 < b1) {
      if (b + 2 < b1) {
        __builtin_amdgcn_s_setprio(2);
        load_part(wg_ + (int64_t)(b + 2) * BLOCK_BYTES, part, g0);
        if (PAIR) load_part(wu_ + (int64_t)(b + 2) * BLOCK_BYTES, part, u0p);
        __builtin_amdgcn_s_setprio(0);
      }
      step(b + 1, g1, u1p);
    }
  }

  auto quad_sum = [](float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
    return v;
  };
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    acc[r] = quad_sum(acc[r]);
    if (PAIR) accu[r] = quad_sum(accu[r]);
    if (part == 0) {
      red[(wave * NR + r) * 2 * GEMV_ROWS + rq] = acc[r];
      if (PAIR) red[(wave * NR + r) * 2 * GEMV_ROWS + GEMV_ROWS + rq] = accu[r];
    }
  }
  __syncthreads();
  if (threadIdx.x < GEMV_ROWS * NR) {
    const int r = threadIdx.x / GEMV_ROWS, q = threadIdx.x % GEMV_ROWS;
    const int orow = wg_local * GEMV_ROWS + q;
    float gs = red[r * 2 * GEMV_ROWS + q], us = red[r * 2 * GEMV_ROWS + GEMV_ROWS + q];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      gs += red[(w * NR + r) * 2 * GEMV_ROWS + q];
      if (PAIR) us += red[(w * NR + r) * 2 * GEMV_ROWS + GEMV_ROWS + q];
    }
    if (r < M && orow < rows_out) {
      if (PAIR)
        ((half_t*)P.out)[(int64_t)r * rows_out + orow] = (half_t)(silu_f32(gs) * us);
      else
        ((float*)P.out)[(int64_t)r * P.N + orow] = gs;
    }
  }
}

template <bool PAIRS, int NR>
__global__ __launch_bounds__(256) void gemv_kernel_nr(GemvArgs args, int xrb, int srb) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
  __shared__ float red[4 * NR * 2 * GEMV_ROWS];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMV_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].wg_begin) pi = i;
  const GemvDesc& P = args.d[pi];
  const int wg_local = (int)blockIdx.x - P.wg_begin;
  const int M = P.m;
  if (P.fmt == 0) {
    if (PAIRS && P.swiglu)
      gemv_tile_nr<0, PAIRS, NR>(P, wg_local, M, xl, xrb, srb, red);
    else
      gemv_tile_nr<0, false, NR>(P, wg_local, M, xl, xrb, srb, red);
  } else {
    gemv_tile_nr<1, false, NR>(P, wg_local, M, xl, xrb, srb, red);
  }
}

// One workgroup per 16 rows; problems with the most bytes per workgroup
// (the deepest K) are dispatched first so they do not trail.
static hipError_t launch_gemv_impl(const GemmProblem* probs, int count, const float* h_in, const float* h_add,
                                   float* h_out, hipStream_t s) {
  for (int base = 0; base < count; base += GEMV_MAX_GROUP) {
    const int n = count - base < GEMV_MAX_GROUP ? count - base : GEMV_MAX_GROUP;
    int order[GEMV_MAX_GROUP];
    for (int i = 0; i < n; ++i) order[i] = base + i;
    auto wg_bytes = [&](int i) {
      return (int64_t)(probs[i].K / QK) * (probs[i].fmt == 0 ? Q4K_BYTES : Q6K_BYTES) * (probs[i].swiglu ? 2 : 1);
    };
    for (int i = 1; i < n; ++i)   // insertion sort, stable, by bytes per workgroup (descending)
      for (int j = i; j > 0 && wg_bytes(order[j]) > wg_bytes(order[j - 1]); --j) std::swap(order[j], order[j - 1]);
    GemvArgs a{};
    int wgs = 0, kmax = 0, pairs = 0, mmax = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = probs[order[i]];
      GemvDesc& d = a.d[i];
      d.x = (const half_t*)p.x;
      d.wq = p.wq;
      d.out = p.out;
      d.g = p.g;
      d.eps = p.eps;
      d.xn = (half_t*)p.xn;
      d.hin = h_in;
      d.hadd = h_add;
      d.hout = order[i] == 0 ? h_out : nullptr;   // one writer of the residual stream
      d.fmt = p.fmt;
      d.swiglu = p.swiglu;
      d.N = p.N;
      d.K = p.K;
      d.m = p.M;
      mmax = p.M > mmax ? p.M : mmax;
      const int rows = p.swiglu ? p.N / 2 : p.N;
      d.wg_begin = wgs;
      wgs += (rows + GEMV_ROWS - 1) / GEMV_ROWS;
      pairs |= p.swiglu;
      kmax = p.K > kmax ? p.K : kmax;
    }
    a.count = n;
    a.sx_offset = (kmax / 64) * X_GROUP_BYTES;   // a multiple of 16
    if (mmax > 1) {   // a few rows: no residual or RMSNorm modes
      if (mmax > GEMV_MAX_ROWS || h_in || !gemv_rows_fit(mmax, kmax)) return hipErrorInvalidValue;
      const int xrb = a.sx_offset, srb = kmax / 32;
      const size_t lds = 2 * ((size_t)xrb + (size_t)srb * sizeof(float));
      if (pairs)
        hipLaunchKernelGGL((gemv_kernel_nr<true, 2>), dim3(wgs), dim3(256), lds, s, a, xrb, srb);
      else
        hipLaunchKernelGGL((gemv_kernel_nr<false, 2>), dim3(wgs), dim3(256), lds, s, a, xrb, srb);
    } else {
      const size_t xbytes = (size_t)a.sx_offset + (size_t)(kmax / 32) * sizeof(float);
      if (pairs)
        hipLaunchKernelGGL(gemv_kernel<true>, dim3(wgs), dim3(256), xbytes, s, a);
      else
        hipLaunchKernelGGL(gemv_kernel<false>, dim3(wgs), dim3(256), xbytes, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemv(const GemmProblem* probs, int count, hipStream_t s) {
  return launch_gemv_impl(probs, count, nullptr, nullptr, nullptr, s);
}

hipError_t launch_gemv_residual(const GemmProblem* probs, int count, const float* h_in, const float* h_add,
                                float* h_out, hipStream_t s) {
  return launch_gemv_impl(probs, count, h_in, h_add, h_out, s);
}

}  // namespace dmq
