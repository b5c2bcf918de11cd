// Decode (M = 1) kernel: y[n] = sum_k x[k] * W[n][k] with W in Q4_K or Q6_K.
//
// Decode handles a single token per step and is bound by streaming the weights
// from memory (overview page, "[01] the thesis" and "[04] one decode step";
// article "Building DAMASCUS", "Prefill and decode need different performance
// questions").  The kernel is built around the HBM stream:
//
//  * every byte of W is read exactly once, with 16-byte loads; the 4 lanes
//    that share a super-block read 144 (Q4_K) / 210 (Q6_K) contiguous bytes;
//  * each problem gets workgroups in proportion to its bytes; a wave owns a
//    contiguous range of units (R whole rows) and streams its steps (16
//    super-blocks each) with the next step's loads in flight while it
//    computes the current one; the first loads are issued before x staging;
//  * x (K fp16 values) is staged once per workgroup in LDS, so the per-weight
//    x traffic hits LDS, not the vector cache;
//  * each weight is dequantised exactly: the quant byte goes to fp32
//    (v_cvt_f32_ubyte), one fp32 FMA of exact operands gives q*d*sc - dmin*m
//    rounded once to fp32, and v_cvt_pk_f16_f32 rounds pairs to fp16; the
//    fp16 pairs meet x in v_dot2_f32_f16 with fp32 accumulation.  These are
//    full-rate VALU instructions on gfx950.  Factoring the sub-block scale
//    and min out of the sum would be cheaper, but when d*sc*q and dmin*m
//    nearly cancel its fp32 rounding error is not bounded by sum |x*w|.  Q6_K
//    has no min, so there the scale is factored out of each 16-weight dot;
//  * partial sums are reduced across the wave with DPP moves (no LDS).
//
// Lane mapping: 4 lanes per super-block ("part" p = lane & 3).  Q4_K part p
// owns quant bytes 32p..32p+31, i.e. sub-blocks 2p (low nibbles) and 2p+1
// (high nibbles).  Q6_K part p owns half h = p >> 1 and weights with
// l in [16(p&1), 16(p&1)+16) of its four 32-weight quarters.
// A step covers 16 super-blocks of a unit of R consecutive rows; R is chosen
// so that R * blocks_per_row is a multiple of 16 (no lane idles) and a unit
// has at least 4 steps when the row is short (R <= 8).
#include "dmq_common.h"

namespace dmq {

constexpr int GEMV_MAX_GROUP = 8;
constexpr int GEMV_MAX_K = 32768;      // x staged in LDS: 72 KiB with padding

struct GemvDesc {
  const half_t* x;
  const uint8_t* wq;
  void* out;
  int32_t fmt, swiglu, N, K;
  int32_t wg_begin;   // first workgroup of this problem
  int32_t wg_count;   // workgroups of this problem
  int32_t rows_log2;  // log2(R): rows per unit
};

struct GemvArgs {
  GemvDesc d[GEMV_MAX_GROUP];
  int32_t count;
};

// x in LDS: each group of 64 values (128 bytes) is followed by 16 bytes of
// padding, so the x reads of the 16 blocks of a step (512 bytes apart
// unpadded, i.e. the same banks) spread over all 64 banks.
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

// 20-byte window starting at an aligned address (Q6_K fields may start 2 mod 4)
struct Win5 {
  uint4 w;
  uint32_t w4;
};
__device__ __forceinline__ void load_win5(const uint8_t* aligned, Win5& r) {
  r.w = *(const uint4*)aligned;
  r.w4 = *((const uint32_t*)aligned + 4);
}
__device__ __forceinline__ uint4 realign5(const Win5& r, uint32_t sh) {
  return make_uint4(__builtin_amdgcn_alignbyte(r.w.y, r.w.x, sh), __builtin_amdgcn_alignbyte(r.w.z, r.w.y, sh),
                    __builtin_amdgcn_alignbyte(r.w.w, r.w.z, sh), __builtin_amdgcn_alignbyte(r.w4, r.w.w, sh));
}

// Raw bytes of one lane's part of one block, loaded before any is used.
struct PartQ4 {
  uint4 hdr, q0, q1;
};
struct PartQ6 {
  Win5 qa, qb, qh;     // low nibbles (quarters 0/2, 1/3) and high bits
  uint4 sw;            // scales: 16 bytes from byte 192 - sh
  uint32_t s206;       // dword at byte 206 (2-byte aligned): scale tail and d
  uint32_t sh;         // block address mod 4 (0 or 2)
};
template <int FMT> struct PartOf { typedef PartQ4 T; };
template <> struct PartOf<1> { typedef PartQ6 T; };

typedef uint32_t u32_a2 __attribute__((aligned(2)));

__device__ __forceinline__ void load_part(const uint8_t* blk, int p, PartQ4& r) {
  r.hdr = *(const uint4*)blk;
  r.q0 = *(const uint4*)(blk + 16 + 32 * p);
  r.q1 = *(const uint4*)(blk + 32 + 32 * p);
}
__device__ __forceinline__ void load_part(const uint8_t* blk, int p, PartQ6& r) {
  const int h = p >> 1, lh = p & 1;
  r.sh = (uint32_t)((uintptr_t)blk & 3);
  const uint8_t* a = blk - r.sh;   // the block's fields at offsets 0 mod 4 of `a` (+ sh)
  // quant fields: 16 bytes each; the window reads at most 2 bytes before and
  // 4 after, all inside the block (the last field ends by byte 176 + 16)
  load_win5(a + 64 * h + 16 * lh, r.qa);
  load_win5(a + 64 * h + 32 + 16 * lh, r.qb);
  load_win5(a + 128 + 32 * h + 16 * lh, r.qh);
  r.sw = *(const uint4*)(a + 192);
  r.s206 = *(const u32_a2*)(blk + 206);
}

// Dot product of one Q4_K part (64 weights) with x (LDS; xs = x of this part:
// xs[0..31] for sub-block 2p, xs[32..63] for sub-block 2p+1).
__device__ __forceinline__ float part_dot(const PartQ4& r, int p, const half_t* xs) {
  Q4kScales s = unpack_q4k_scales(r.hdr.y, r.hdr.z, r.hdr.w);
  const uint32_t scw = p < 2 ? s.sc_lo : s.sc_hi;
  const uint32_t mw = p < 2 ? s.m_lo : s.m_hi;
  const uint32_t sh = (uint32_t)(p & 1) * 16u;
  const float d = half_bits_to_float(r.hdr.x);
  const float dmin = half_bits_to_float(r.hdr.x >> 16);
  const float dsc0 = d * (float)((scw >> sh) & 0xffu);
  const float dsc1 = d * (float)((scw >> (sh + 8)) & 0xffu) * 0.0625f;  // high nibble read as 16q
  const float ndm0 = -(dmin * (float)((mw >> sh) & 0xffu));
  const float ndm1 = -(dmin * (float)((mw >> (sh + 8)) & 0xffu));
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
      uint32_t lo = qw[i + u] & 0x0f0f0f0fu;
      uint32_t hi = qw[i + u] & 0xf0f0f0f0u;
      // hide the masks from the optimiser: with them known it extracts each
      // nibble with v_bfe and converts byte 0, instead of one v_cvt_f32_ubyteN
      asm("" : "+v"(lo));
      asm("" : "+v"(hi));
      const h2 wl01 = pack_h2(__builtin_fmaf((float)(lo & 0xffu), dsc0, ndm0),
                              __builtin_fmaf((float)((lo >> 8) & 0xffu), dsc0, ndm0));
      const h2 wl23 = pack_h2(__builtin_fmaf((float)((lo >> 16) & 0xffu), dsc0, ndm0),
                              __builtin_fmaf((float)(lo >> 24), dsc0, ndm0));
      const h2 wh01 = pack_h2(__builtin_fmaf((float)(hi & 0xffu), dsc1, ndm1),
                              __builtin_fmaf((float)((hi >> 8) & 0xffu), dsc1, ndm1));
      const h2 wh23 = pack_h2(__builtin_fmaf((float)((hi >> 16) & 0xffu), dsc1, ndm1),
                              __builtin_fmaf((float)(hi >> 24), dsc1, ndm1));
      acc0 = __builtin_amdgcn_fdot2(wl01, as_h2(xa_w[2 * u]), acc0, false);
      acc0 = __builtin_amdgcn_fdot2(wl23, as_h2(xa_w[2 * u + 1]), acc0, false);
      acc1 = __builtin_amdgcn_fdot2(wh01, as_h2(xb_w[2 * u]), acc1, false);
      acc1 = __builtin_amdgcn_fdot2(wh23, as_h2(xb_w[2 * u + 1]), acc1, false);
    }
  }
  return acc0 + acc1;
}

// Dot product of one Q6_K part (64 weights) with x (LDS, padded layout; xs =
// x of weight 128h + 16lh of the block: quarter t's 16 values start
// X_GROUP_BYTES * (t / 2) + 64 * (t % 2) bytes further).
__device__ __forceinline__ float part_dot(const PartQ6& r, int p, const half_t* xs) {
  const int h = p >> 1, lh = p & 1;
  const uint4 qa = realign5(r.qa, r.sh);   // quarters t = 0 (low nibble), 2 (high nibble)
  const uint4 qb = realign5(r.qb, r.sh);   // quarters t = 1, 3
  const uint4 qh = realign5(r.qh, r.sh);
  // scales at byte 192: for sh = 2 the 20-byte window is sw and s206
  const uint32_t sw[4] = {__builtin_amdgcn_alignbyte(r.sw.y, r.sw.x, r.sh), __builtin_amdgcn_alignbyte(r.sw.z, r.sw.y, r.sh),
                          __builtin_amdgcn_alignbyte(r.sw.w, r.sw.z, r.sh), __builtin_amdgcn_alignbyte(r.s206, r.sw.w, r.sh)};
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
    const uint32_t sidx = 8 * h + 2 * t + lh;
    const int sc = (int)(int8_t)((sw[sidx >> 2] >> (8 * (sidx & 3))) & 0xffu);
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

// byte offset of the x of a lane's part of block b
template <int FMT>
__device__ __forceinline__ int part_x_offset(int b, int part) {
  return FMT == 0 ? X_GROUP_BYTES * (4 * b + part) : X_GROUP_BYTES * (4 * b + 2 * (part >> 1)) + 32 * (part & 1);
}

// Sum over the 64 lanes with DPP moves (no LDS round trips); the total ends
// up in lane 63.  Quad butterflies, then half-row and row mirrors give every
// lane its 16-lane row sum; row_bcast15 / row_bcast31 fold rows 0..3 into
// row 3.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));  // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));  // row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));  // row_bcast15 -> rows 1, 3
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));  // row_bcast31 -> rows 2, 3
  return v;
}

// Work split of one problem: its units (R consecutive rows = spu steps of 16
// super-blocks) are divided into contiguous ranges, one per wave of the
// problem's workgroups.  Each wave streams its steps with the next step's
// loads in flight while it computes the current one.
template <int FMT, int R, bool PAIR>
__device__ __forceinline__ void gemv_rows(const GemvDesc& P, int wg_local, half_t* xs) {
  typedef typename PartOf<FMT>::T Part;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = P.K / QK;
  const int part = lane & 3;
  const int nrows_out = PAIR ? P.N / 2 : P.N;
  const int64_t row_bytes = (int64_t)nb * BLOCK_BYTES;
  const int spu = (R * nb) >> 4;                       // steps per unit (R * nb is a multiple of 16)
  const int units = (nrows_out + R - 1) / R;
  const int64_t nwaves = 4 * (int64_t)P.wg_count;
  const int64_t wv = 4 * (int64_t)wg_local + wave;
  const int u_begin = (int)(units * wv / nwaves);
  const int u_end = (int)(units * (wv + 1) / nwaves);
  const int s_end = (u_end - u_begin) * spu;           // steps of this wave

  // The lane's item of local step ls is it = lane/4 + 16 ls, i.e. row
  // it / nb of the unit and block it % nb; (rl, b) advance by (16 / nb,
  // 16 % nb) per step, with one carry.
  const int q16 = 16 / nb, r16 = 16 - q16 * nb;
  auto advance = [&](int& rl, int& b) {
    rl += q16;
    b += r16;
    if (b >= nb) { b -= nb; ++rl; }
  };
  const int rl0 = (lane >> 2) / nb, b0 = (lane >> 2) - rl0 * nb;   // local step 0
  auto load_step = [&](int u, int rl, int b, Part& g, Part& up) {
    int row = u * R + rl;
    row = row < nrows_out ? row : nrows_out - 1;        // ragged tail: clamp, result dropped
    load_part(P.wq + row * row_bytes + (int64_t)b * BLOCK_BYTES, part, g);
    if (PAIR) load_part(P.wq + (row + nrows_out) * row_bytes + (int64_t)b * BLOCK_BYTES, part, up);
  };

  float acc[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { acc[r] = 0.0f; accu[r] = 0.0f; }

  auto compute_step = [&](int rl, int b, const Part& g, const Part& up) {
    const half_t* xp = (const half_t*)((const uint8_t*)xs + part_x_offset<FMT>(b, part));
    const float v = part_dot(g, part, xp);
    const float vu = PAIR ? part_dot(up, part, xp) : 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] += (rl == r) ? v : 0.0f;
      if (PAIR) accu[r] += (rl == r) ? vu : 0.0f;
    }
  };
  auto finish_unit = [&](int u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float gs = wave_sum_dpp(acc[r]);
      const float us = PAIR ? wave_sum_dpp(accu[r]) : 0.0f;
      const int row = u * R + r;
      if (lane == 63 && row < nrows_out) {
        if (PAIR)
          ((half_t*)P.out)[row] = (half_t)(silu_f32(gs) * us);
        else
          ((float*)P.out)[row] = gs;
      }
      acc[r] = 0.0f;
      accu[r] = 0.0f;
    }
  };

  Part g0, u0p, g1, u1p;
  // first loads before x staging: their latency overlaps the staging
  if (s_end > 0) load_step(u_begin, rl0, b0, g0, u0p);
  for (int i = threadIdx.x; i < P.K / 8; i += blockDim.x)
    *(uint4*)((uint8_t*)xs + X_GROUP_BYTES * (i >> 3) + 16 * (i & 7)) = ((const uint4*)P.x)[i];
  __syncthreads();

  // position of the step being computed (u, ls, rl, b) and of the next one
  int u = u_begin, ls = 0, rl = rl0, b = b0;
  auto next_pos = [&](int& un, int& lsn, int& rln, int& bn) {
    if (ls + 1 == spu) {
      un = u + 1; lsn = 0; rln = rl0; bn = b0;
    } else {
      un = u; lsn = ls + 1; rln = rl; bn = b;
      advance(rln, bn);
    }
  };
  for (int s = 0; s < s_end; s += 2) {
    int un, lsn, rln, bn;
    // step s (buffers 0), with step s+1 loading into buffers 1
    next_pos(un, lsn, rln, bn);
    if (s + 1 < s_end) load_step(un, rln, bn, g1, u1p);
    compute_step(rl, b, g0, u0p);
    if (ls + 1 == spu) finish_unit(u);
    u = un; ls = lsn; rl = rln; b = bn;
    if (s + 1 < s_end) {
      // step s+1 (buffers 1), with step s+2 loading into buffers 0
      next_pos(un, lsn, rln, bn);
      if (s + 2 < s_end) load_step(un, rln, bn, g0, u0p);
      compute_step(rl, b, g1, u1p);
      if (ls + 1 == spu) finish_unit(u);
      u = un; ls = lsn; rl = rln; b = bn;
    }
  }
}

// FULL: the kernel also carries the R = 16 paths (odd blocks-per-row, i.e.
// K an odd multiple of 256) and the SwiGLU pairs (Q4_K only); they need more
// registers, so they live in their own kernel and do not lower the occupancy
// of the common shapes.
template <int FMT, bool FULL>
__device__ __forceinline__ void gemv_dispatch(const GemvDesc& P, int wg_local, half_t* xs) {
  constexpr bool PAIRS = FULL && FMT == 0;
  switch (P.rows_log2 * 2 + P.swiglu) {
    case 0: gemv_rows<FMT, 1, false>(P, wg_local, xs); break;
    case 1: if constexpr (PAIRS) gemv_rows<FMT, 1, true>(P, wg_local, xs); break;
    case 2: gemv_rows<FMT, 2, false>(P, wg_local, xs); break;
    case 3: if constexpr (PAIRS) gemv_rows<FMT, 2, true>(P, wg_local, xs); break;
    case 4: gemv_rows<FMT, 4, false>(P, wg_local, xs); break;
    case 5: if constexpr (PAIRS) gemv_rows<FMT, 4, true>(P, wg_local, xs); break;
    case 6: gemv_rows<FMT, 8, false>(P, wg_local, xs); break;
    case 7: if constexpr (PAIRS) gemv_rows<FMT, 8, true>(P, wg_local, xs); break;
    case 8: if constexpr (FULL) gemv_rows<FMT, 16, false>(P, wg_local, xs); break;
    default: if constexpr (PAIRS) gemv_rows<FMT, 16, true>(P, wg_local, xs); break;
  }
}

template <bool FULL>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs args) {
  extern __shared__ __attribute__((aligned(16))) half_t xs[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMV_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].wg_begin) pi = i;
  const GemvDesc& P = args.d[pi];
  const int wg_local = (int)blockIdx.x - P.wg_begin;
  if (P.fmt == 0)
    gemv_dispatch<0, FULL>(P, wg_local, xs);
  else
    gemv_dispatch<1, FULL>(P, wg_local, xs);
}

// Rows per unit: the smallest power of two R with R * nb a multiple of 16
// (R <= 16 always suffices), doubled (up to 8) while a unit has fewer than 4
// steps.
static int rows_log2_for(int nb) {
  int lg = 0;
  while (lg < 4 && ((nb << lg) & 15) != 0) ++lg;
  while (lg < 3 && ((nb << lg) >> 4) < 4) ++lg;
  return lg;
}

// Workgroups of one launch: about GEMV_WG_PER_CU per compute unit, shared
// among the problems in proportion to their weight bytes (each at least one,
// and no more than its units / 4 so every wave has work).
constexpr int GEMV_WG_PER_CU = 4;

hipError_t launch_gemv(const GemmProblem* probs, int count, hipStream_t s) {
  const int64_t budget = (int64_t)device_cu_count() * GEMV_WG_PER_CU;
  for (int base = 0; base < count; base += GEMV_MAX_GROUP) {
    GemvArgs a{};
    int n = count - base < GEMV_MAX_GROUP ? count - base : GEMV_MAX_GROUP;
    int64_t bytes[GEMV_MAX_GROUP], total = 0;
    int kmax = 0, lgmax = 0, pairs = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = probs[base + i];
      bytes[i] = (int64_t)p.N * (p.K / QK) * (p.fmt == 0 ? Q4K_BYTES : Q6K_BYTES);
      total += bytes[i];
    }
    int wgs = 0;
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
      lgmax = d.rows_log2 > lgmax ? d.rows_log2 : lgmax;
      pairs |= p.swiglu;
      const int rows = p.swiglu ? p.N / 2 : p.N;
      const int64_t units = (rows + (1 << d.rows_log2) - 1) >> d.rows_log2;
      int64_t w = (budget * bytes[i] + total / 2) / total;
      const int64_t wmax = (units + 3) / 4;
      w = w < 1 ? 1 : (w > wmax ? wmax : w);
      d.wg_begin = wgs;
      d.wg_count = (int32_t)w;
      wgs += (int)w;
      kmax = p.K > kmax ? p.K : kmax;
    }
    a.count = n;
    const size_t xbytes = (size_t)(kmax / 64) * X_GROUP_BYTES;
    if (lgmax > 3 || pairs)
      hipLaunchKernelGGL(gemv_kernel<true>, dim3(wgs), dim3(256), xbytes, s, a);
    else
      hipLaunchKernelGGL(gemv_kernel<false>, dim3(wgs), dim3(256), xbytes, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dmq
