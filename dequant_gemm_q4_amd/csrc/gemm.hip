// Prefill kernel (M >= 2): y = x * W^T with the Q4_K / Q6_K dequant fused into
// an MFMA fp16 x fp16 -> fp32 contraction.  Prefill is matrix-matrix work
// where each weight is reused across all prompt rows (overview page, "[01]
// the thesis": prefill is dense, compute-bound GEMM; article "Building
// DAMASCUS", "Prefill and decode need different performance questions"), and
// the fused dequant never writes fp16 weights to memory (overview page, same
// section, and compartment 09 "fused dequant -> ... prefill").
//
// Work decomposition (one workgroup = 4 waves = one BM x BN output tile):
//  * Each wave owns 16*IB weight rows and all BM = 16*JB activation rows.  It
//    decodes its raw blocks straight into MFMA A-operand registers, so every
//    weight is dequantised once per workgroup and no dequantised tile touches
//    LDS or HBM.
//  * x is staged in LDS per 64-wide K chunk (double-buffered) and read as the
//    MFMA B operand by all 4 waves.
//  * Sub-block scales / mins are decoded once per super-block and row into an
//    LDS table (double-buffered), so the per-lane work per weight is: build
//    the fp16 integer q (bit tricks), one fp32 FMA of exact operands
//    (q*d*sc - dmin*m, v_fma_mix) and one rounding to fp16.
//  * v_mfma_f32_16x16x32_f16: A = 16 weight rows x 32 k, B = 32 k x 16
//    activation rows; lane l holds row/col l%16 and k = 8*(l/16) .. +7, and
//    the accumulator lane holds D[4*(l/16) + r][l%16], r = 0..3.  One
//    sub-block (32 weights) is exactly one MFMA K step.
//  * Optional SwiGLU epilogue: a wave's first IB/2 i-blocks are gate rows and
//    the last IB/2 the matching up rows, so g and u of one output sit in the
//    same lane and h = silu(g) * u is formed in registers.
#include "dmq_common.h"

namespace dmq {

constexpr int GEMM_MAX_GROUP = 8;

struct GemmDesc {
  const half_t* x;
  const uint8_t* wq;
  void* out;
  int32_t fmt, swiglu, M, N, K;
  int32_t tile_begin, mt, nt;
};

struct GemmArgs {
  GemmDesc d[GEMM_MAX_GROUP];
  int32_t count;
};

template <int JB, int IB>
struct TileCfg {
  static constexpr int BM = 16 * JB;           // activation rows per tile
  static constexpr int BN = 64 * IB;           // weight rows per tile (4 waves)
  static constexpr int XSTRIDE = 72;           // halves per LDS x row: 64 + 8 pad
  static constexpr int XTILE = BM * XSTRIDE;   // halves per x buffer
  static constexpr int TSTRIDE = 20;           // floats per table row: 16 + 4 pad
  static constexpr int TAB = BN * TSTRIDE;     // floats per table buffer
  static constexpr int XLOADS = BM * 8;        // 16-byte x loads per chunk
  static constexpr int XR = (XLOADS + 255) / 256;
  static constexpr size_t LDS_BYTES = 2 * XTILE * sizeof(half_t) + 2 * TAB * sizeof(float);
};

__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// 8 fp16 weights (4 dwords) of the A operand from 8 nibbles-in-bytes.
// `nib` words hold 4 quants each in the low (mask 0x0f) or, read as 16q, the
// high (mask 0xf0) half of every byte; w = q * dsc + ndm, exact in fp32,
// then one rounding to fp16.
__device__ __forceinline__ h8 q4k_frag(uint32_t w0, uint32_t w1, uint32_t mask, float dsc, float ndm) {
  const h2 k1024 = {(half_t)1024.0f, (half_t)1024.0f};
  uint32_t a = w0 & mask, b = w1 & mask;
  h2 q[4] = {as_h2(magic_pair_lo(a)) - k1024, as_h2(magic_pair_hi(a)) - k1024,
             as_h2(magic_pair_lo(b)) - k1024, as_h2(magic_pair_hi(b)) - k1024};
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (half_t)__builtin_fmaf((float)q[i].x, dsc, ndm);
    r[2 * i + 1] = (half_t)__builtin_fmaf((float)q[i].y, dsc, ndm);
  }
  return r;
}

// 8 fp16 weights of a Q6_K quarter t: q = low nibble (shifted by nsh) | two
// high bits << 4, w = (q - 32) * dsc (exact in fp32, one rounding).
__device__ __forceinline__ h8 q6k_frag(uint2 ql, uint2 qh, uint32_t nsh, uint32_t hsh, float dsc) {
  const h2 k1056 = {(half_t)1056.0f, (half_t)1056.0f};
  uint32_t a = ((ql.x >> nsh) & 0x0f0f0f0fu) | (((qh.x >> hsh) & 0x03030303u) << 4);
  uint32_t b = ((ql.y >> nsh) & 0x0f0f0f0fu) | (((qh.y >> hsh) & 0x03030303u) << 4);
  h2 q[4] = {as_h2(magic_pair_lo(a)) - k1056, as_h2(magic_pair_hi(a)) - k1056,
             as_h2(magic_pair_lo(b)) - k1056, as_h2(magic_pair_hi(b)) - k1056};
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (half_t)((float)q[i].x * dsc);
    r[2 * i + 1] = (half_t)((float)q[i].y * dsc);
  }
  return r;
}

// Load / store helpers of the K-chunk pipeline.  Arrays are passed by
// reference into force-inlined functions with compile-time trip counts so
// that they stay in registers.
template <int JB, int IB, int XR>
__device__ __forceinline__ void x_load(u32x4 (&xr)[XR], const half_t* x, int m0, int M, int K, int ck, int tid) {
  typedef TileCfg<JB, IB> C;
#pragma unroll
  for (int i = 0; i < C::XR; ++i) {
    int e = tid + 256 * i;
    if (e < C::XLOADS) {
      int r = e >> 3;
      int m = m0 + r < M ? m0 + r : M - 1;      // ragged M: repeat the last row
      xr[i] = *(const u32x4*)(x + (int64_t)m * K + 64 * ck + 8 * (e & 7));
    }
  }
}

template <int JB, int IB, int XR>
__device__ __forceinline__ void x_store(const u32x4 (&xr)[XR], half_t* xs, int tid) {
  typedef TileCfg<JB, IB> C;
#pragma unroll
  for (int i = 0; i < C::XR; ++i) {
    int e = tid + 256 * i;
    if (e < C::XLOADS) *(u32x4*)(xs + (e >> 3) * C::XSTRIDE + 8 * (e & 7)) = xr[i];
  }
}

// Scale-table header of one block: Q4_K bytes 0..15 (d, dmin, 12 scale
// bytes); Q6_K bytes 192..209 (16 scales, d) read through the enclosing
// aligned dwords without touching anything past byte 209.
template <int FMT>
__device__ __forceinline__ void hdr_load(const uint8_t* blk, uint4& hdr, uint32_t& hdr4) {
  if constexpr (FMT == 0) {
    hdr = *(const uint4*)blk;
  } else {
    uintptr_t a = (uintptr_t)(blk + 192);
    const uint32_t* sp = (const uint32_t*)(a & ~(uintptr_t)3);
    hdr = *(const uint4*)sp;
    hdr4 = (a & 3) ? sp[4] : (uint32_t)(*(const uint16_t*)(blk + 208)) << 16;
  }
}

// Decode one row's header into 16 floats of the LDS table.
// Q4_K: (d*sc_j [/16 for odd j, whose quant is read as 16q], -dmin*m_j) pairs.
// Q6_K: d*sc_s for the 16 sub-blocks.
template <int FMT>
__device__ __forceinline__ void tab_store(float* t, const uint4& hdr, uint32_t hdr4, uint32_t sh) {
  float v[16];
  if constexpr (FMT == 0) {
    Q4kScales s = unpack_q4k_scales(hdr.y, hdr.z, hdr.w);
    float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float dsc = d * (float)q4k_sc(s, j);
      v[2 * j] = (j & 1) ? dsc * 0.0625f : dsc;
      v[2 * j + 1] = -(dmin * (float)q4k_m(s, j));
    }
  } else {
    // sh = block address mod 4 (0 or 2); with sh == 0 d sits in hdr4's high half
    uint32_t w[4] = {__builtin_amdgcn_alignbyte(hdr.y, hdr.x, sh), __builtin_amdgcn_alignbyte(hdr.z, hdr.y, sh),
                     __builtin_amdgcn_alignbyte(hdr.w, hdr.z, sh), __builtin_amdgcn_alignbyte(hdr4, hdr.w, sh)};
    float d = half_bits_to_float(hdr4 >> 16);
#pragma unroll
    for (int s = 0; s < 16; ++s) v[s] = d * (float)(int)(int8_t)((w[s >> 2] >> (8 * (s & 3))) & 0xffu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) ((float4*)t)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// Raw quant bytes of one 64-wide K chunk for one lane and i-block.
// Q4_K: 8 quant bytes (k = 8g .. 8g+7 of both sub-blocks of the chunk).
// Q6_K: low-nibble bytes of quarters t and t+1 and the high-bit bytes; all
// 8-byte fields at 2-aligned addresses, read by load_u64_a2 inside the block
// (last byte read <= 196 < 210).
template <int FMT>
__device__ __forceinline__ void raw_load(const uint8_t* wrow, int ck, int g, uint2& a, uint2& b, uint2& c) {
  const int blk_i = ck >> 2, cc = ck & 3;
  if constexpr (FMT == 0) {
    a = *(const uint2*)(wrow + (int64_t)blk_i * Q4K_BYTES + 16 + 32 * cc + 8 * g);
  } else {
    const uint8_t* blk = wrow + (int64_t)blk_i * Q6K_BYTES;
    const int h = cc >> 1;
    a = load_u64_a2(blk + 64 * h + 8 * g);
    b = load_u64_a2(blk + 64 * h + 32 + 8 * g);
    c = load_u64_a2(blk + 128 + 32 * h + 8 * g);
  }
}

template <int FMT, int JB, int IB, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const GemmDesc& P, int m_tile, int n_tile, uint8_t* smem) {
  typedef TileCfg<JB, IB> C;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  half_t* xs = (half_t*)smem;
  float* tab = (float*)(smem + 2 * C::XTILE * sizeof(half_t));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int M = P.M, N = P.N, K = P.K;
  const int nck = K / 64;
  const int64_t row_bytes = (int64_t)(K / QK) * BLOCK_BYTES;
  const int m0 = m_tile * C::BM;
  const int F = N / 2;                       // SwiGLU: gate rows [0,F), up rows [F,2F)
  const int hb = n_tile * (C::BN / 2);       // SwiGLU: first h column of the tile
  const int n0 = n_tile * C::BN;

  // weight row of local row lr (0..BN), clamped for a ragged N
  const uint8_t* wrow[IB];
#pragma unroll
  for (int c = 0; c < IB; ++c) {
    int r;
    if (SWIGLU) {
      int base = hb + (8 * IB) * wave + li;
      r = c < IB / 2 ? base + 16 * c : F + base + 16 * (c - IB / 2);
    } else {
      r = n0 + 16 * IB * wave + 16 * c + li;
    }
    r = r < N ? r : N - 1;
    wrow[c] = P.wq + (int64_t)r * row_bytes;
  }
  // the table row this thread decodes (threads 0..BN-1, local row = tid)
  const uint8_t* trow;
  {
    int lr = tid < C::BN ? tid : 0, r;
    if (SWIGLU) {
      int w = lr / (16 * IB), c = (lr / 16) % IB, i = lr & 15;
      int base = hb + (8 * IB) * w + i;
      r = c < IB / 2 ? base + 16 * c : F + base + 16 * (c - IB / 2);
    } else {
      r = n0 + lr;
    }
    r = r < N ? r : N - 1;
    trow = P.wq + (int64_t)r * row_bytes;
  }
  float* my_tab = tab + tid * C::TSTRIDE;

  f4 acc[JB][IB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int c = 0; c < IB; ++c) acc[jb][c] = (f4){0.0f, 0.0f, 0.0f, 0.0f};

  u32x4 xr[C::XR];
  uint4 hdr = make_uint4(0, 0, 0, 0);
  uint32_t hdr4 = 0;
  uint2 ra[IB], rb[IB], rc[IB];       // raw quant bytes of the current chunk
  uint2 na[IB], nb[IB], nc[IB];       // ... and of the next one

  x_load<JB, IB>(xr, P.x, m0, M, K, 0, tid);
  if (tid < C::BN) hdr_load<FMT>(trow, hdr, hdr4);
#pragma unroll
  for (int c = 0; c < IB; ++c) raw_load<FMT>(wrow[c], 0, g, ra[c], rb[c], rc[c]);
  x_store<JB, IB>(xr, xs, tid);
  if (tid < C::BN) tab_store<FMT>(my_tab, hdr, hdr4, (uint32_t)((uintptr_t)(trow + 192) & 3));
  __syncthreads();

  for (int ck = 0; ck < nck; ++ck) {
    const bool has_next = ck + 1 < nck;
    const bool next_block = has_next && ((ck + 1) & 3) == 0;
    if (has_next) {
      x_load<JB, IB>(xr, P.x, m0, M, K, ck + 1, tid);
#pragma unroll
      for (int c = 0; c < IB; ++c) raw_load<FMT>(wrow[c], ck + 1, g, na[c], nb[c], nc[c]);
      if (next_block && tid < C::BN) hdr_load<FMT>(trow + (int64_t)((ck + 1) >> 2) * BLOCK_BYTES, hdr, hdr4);
    }
    const int tbuf = (ck >> 2) & 1, cc = ck & 3;
    const half_t* xb = xs + (ck & 1) * C::XTILE + li * C::XSTRIDE + 8 * g;
    // scale values of this lane's rows for this chunk
    float sv[IB][4];
#pragma unroll
    for (int c = 0; c < IB; ++c) {
      const float* t = tab + tbuf * C::TAB + (16 * IB * wave + 16 * c + li) * C::TSTRIDE;
      if constexpr (FMT == 0) {
        float4 v = *(const float4*)(t + 4 * cc);     // sub-blocks 2cc, 2cc+1
        sv[c][0] = v.x; sv[c][1] = v.y; sv[c][2] = v.z; sv[c][3] = v.w;
      } else {
        const int h = cc >> 1, t0 = 2 * (cc & 1);
        sv[c][0] = t[8 * h + 2 * t0 + (g >> 1)];
        sv[c][1] = t[8 * h + 2 * (t0 + 1) + (g >> 1)];
        sv[c][2] = 0.0f;
        sv[c][3] = 0.0f;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      h8 af[IB];
#pragma unroll
      for (int c = 0; c < IB; ++c) {
        if constexpr (FMT == 0) {
          af[c] = ks == 0 ? q4k_frag(ra[c].x, ra[c].y, 0x0f0f0f0fu, sv[c][0], sv[c][1])
                          : q4k_frag(ra[c].x, ra[c].y, 0xf0f0f0f0u, sv[c][2], sv[c][3]);
        } else {
          const int t = 2 * (cc & 1) + ks;
          af[c] = q6k_frag(ks ? rb[c] : ra[c], rc[c], (cc & 1) ? 4u : 0u, 2u * (uint32_t)t, sv[c][ks]);
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        h8 bf = *(const h8*)(xb + jb * 16 * C::XSTRIDE + 32 * ks);
#pragma unroll
        for (int c = 0; c < IB; ++c)
          acc[jb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[c], bf, acc[jb][c], 0, 0, 0);
      }
    }
    if (has_next) {
      x_store<JB, IB>(xr, xs + ((ck + 1) & 1) * C::XTILE, tid);
      if (next_block && tid < C::BN)
        tab_store<FMT>(my_tab + (((ck + 1) >> 2) & 1) * C::TAB, hdr, hdr4,
                       (uint32_t)((uintptr_t)(trow + (int64_t)((ck + 1) >> 2) * BLOCK_BYTES + 192) & 3));
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < IB; ++c) {
      ra[c] = na[c];
      rb[c] = nb[c];
      rc[c] = nc[c];
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const int m = m0 + 16 * jb + li;
    if (m >= M) continue;
    if (SWIGLU) {
      half_t* h = (half_t*)P.out;
#pragma unroll
      for (int c = 0; c < IB / 2; ++c) {
        const int col = hb + (8 * IB) * wave + 16 * c + 4 * g;
        f4 gv = acc[jb][c], uv = acc[jb][c + IB / 2];
        h2 h01 = {(half_t)(silu_fast(gv[0]) * uv[0]), (half_t)(silu_fast(gv[1]) * uv[1])};
        h2 h23 = {(half_t)(silu_fast(gv[2]) * uv[2]), (half_t)(silu_fast(gv[3]) * uv[3])};
        *(uint2*)(h + (int64_t)m * F + col) = make_uint2(as_u32(h01), as_u32(h23));
      }
    } else {
      float* y = (float*)P.out;
#pragma unroll
      for (int c = 0; c < IB; ++c) {
        const int n = n0 + 16 * IB * wave + 16 * c + 4 * g;
        float* yp = y + (int64_t)m * N + n;
        f4 v = acc[jb][c];
        if ((N & 3) == 0 && n + 3 < N) {
          *(float4*)yp = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) yp[r] = v[r];
        }
      }
    }
  }
}

template <int JB, int IB, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs args) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMM_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].tile_begin) pi = i;
  const GemmDesc& P = args.d[pi];
  // Tile order within a problem: groups of 8 N-tiles x all M-tiles, with the
  // N-tile fastest, so workgroups bid, bid+8, bid+16, ... (which the
  // dispatcher places on the same XCD) share one weight panel in that XCD's
  // L2 while the 8 XCDs work on 8 different panels.
  const int o = (int)blockIdx.x - P.tile_begin;
  const int mt = P.mt, nt = P.nt;
  const int grp = o / (8 * mt);
  const int u = o - grp * 8 * mt;
  const int nrem = nt - 8 * grp < 8 ? nt - 8 * grp : 8;
  const int m_tile = u / nrem;
  const int n_tile = 8 * grp + (u - m_tile * nrem);
  if (P.fmt == 0)
    gemm_tile<0, JB, IB, SWIGLU>(P, m_tile, n_tile, smem);
  else
    gemm_tile<1, JB, IB, SWIGLU>(P, m_tile, n_tile, smem);
}

template <int JB, int IB, bool SWIGLU>
static hipError_t launch_cfg(const GemmProblem* probs, int count, hipStream_t s) {
  typedef TileCfg<JB, IB> C;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<JB, IB, SWIGLU>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  for (int base = 0; base < count; base += GEMM_MAX_GROUP) {
    GemmArgs a{};
    int n = count - base < GEMM_MAX_GROUP ? count - base : GEMM_MAX_GROUP;
    int tiles = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = probs[base + i];
      GemmDesc& d = a.d[i];
      d.x = (const half_t*)p.x;
      d.wq = p.wq;
      d.out = p.out;
      d.fmt = p.fmt;
      d.swiglu = p.swiglu;
      d.M = p.M;
      d.N = p.N;
      d.K = p.K;
      d.mt = (p.M + C::BM - 1) / C::BM;
      d.nt = SWIGLU ? (p.N / 2 + C::BN / 2 - 1) / (C::BN / 2) : (p.N + C::BN - 1) / C::BN;
      d.tile_begin = tiles;
      tiles += d.mt * d.nt;
    }
    a.count = n;
    hipLaunchKernelGGL((gemm_kernel<JB, IB, SWIGLU>), dim3(tiles), dim3(256), C::LDS_BYTES, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// All problems of one call share the tile shape, picked from the largest M.
hipError_t launch_gemm(const GemmProblem* probs, int count, hipStream_t s) {
  int mmax = 0;
  bool swiglu = probs[0].swiglu != 0;
  for (int i = 0; i < count; ++i) mmax = probs[i].M > mmax ? probs[i].M : mmax;
  if (swiglu) {
    if (mmax > 64) return launch_cfg<16, 4, true>(probs, count, s);
    if (mmax > 16) return launch_cfg<4, 2, true>(probs, count, s);
    return launch_cfg<1, 2, true>(probs, count, s);
  }
  if (mmax > 64) return launch_cfg<16, 4, false>(probs, count, s);
  if (mmax > 16) return launch_cfg<4, 1, false>(probs, count, s);
  return launch_cfg<1, 1, false>(probs, count, s);
}

}  // namespace dmq
