// Prefill kernel (M >= 2): y = x * W^T with the Q4_K / Q6_K dequant fused into
// an MFMA fp16 x fp16 -> fp32 contraction.  Prefill is matrix-matrix work in
// which every weight is reused across all prompt rows (overview page, "[01]
// the thesis": prefill is dense, compute-bound GEMM; article "Building
// DAMASCUS", "Prefill and decode need different performance questions"), and
// the fused dequant never writes fp16 weights to memory (overview page, same
// section, and compartment 09 of "[02] the pipeline").
//
// One workgroup = 4 waves = one BM x BN output tile, BM = 32*JB activation
// rows, BN = 4 * 32*IB weight rows.
//  * Each wave owns 32*IB weight rows and all BM activation rows.  It decodes
//    its raw blocks straight into MFMA A-operand registers: every weight is
//    dequantised once per workgroup and no dequantised tile touches LDS or
//    HBM.
//  * x is staged in LDS per 64-wide K chunk by direct global->LDS loads
//    (global_load_lds_dwordx4, no VGPR staging), double-buffered, with the
//    16-byte chunks of each 128-byte row XOR-swizzled by (row & 7) so that
//    eight consecutive rows read the same column without bank conflicts.
//  * Sub-block scales / mins are decoded once per super-block and weight row
//    into an LDS table (double-buffered).  Per weight the lanes then do: mask
//    and byte-permute the quant into an fp16 integer (1024 + q), subtract
//    1024 (exact), and one fp32 FMA of exact operands (q*d*sc - dmin*m) with a
//    single rounding to fp16 (v_fma_mix).
//  * v_mfma_f32_32x32x16_f16: lane l holds operand row l%32 and k-slots
//    8*(l/32) .. +7; the accumulator lane holds D[8*(r/4) + 4*(l/32) + r%4]
//    [l%32], r = 0..15.  The K order inside a 64-wide chunk is permuted (the
//    same way for both operands) so that each lane's 8 weights of a step come
//    from 8 consecutive quant bytes: step s, lane half g, slot e covers
//    k = 32*(s/2) + 16*g + 8*(s%2) + e.
//  * Dequant of the next K step is issued between the MFMAs of the current
//    one, so VALU work overlaps the matrix core.
//  * Optional SwiGLU epilogue: a wave's first i-block holds gate rows, its
//    second the matching up rows, so g and u of one output sit in the same
//    lane and h = silu(g) * u is formed in registers.
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

typedef float f16x __attribute__((ext_vector_type(16)));

template <int JB, int IB>
struct TileCfg {
  static constexpr int BM = 32 * JB;                 // activation rows per tile
  static constexpr int BN = 128 * IB;                // weight rows per tile
  static constexpr int XBUF = BM * 128;              // bytes per x buffer (64 fp16 per row)
  static constexpr int TSTRIDE = 20;                 // floats per table row (16 + 4 pad)
  static constexpr int TBUF = BN * TSTRIDE * 4;      // bytes per table buffer
  static constexpr size_t LDS_BYTES = 2 * XBUF + 2 * TBUF;
};

__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// fp16 pair (q0, q1) -> (fp16(q0*s + c), fp16(q1*s + c)): one fp32 FMA per
// element with a single rounding to fp16.  Written as one h2 of two fmaf so
// that the compiler selects v_fma_mixlo/hi_f16 (fp16 inputs, fp32 FMA).
__device__ __forceinline__ uint32_t fma_mix_pair(uint32_t q, float s, float c) {
  const h2 v = as_h2(q);
  const h2 r = {(half_t)__builtin_fmaf((float)v.x, s, c), (half_t)__builtin_fmaf((float)v.y, s, c)};
  return as_u32(r);
}

__device__ __forceinline__ uint32_t pk_sub(uint32_t a, uint32_t k) {
  return as_u32(as_h2(a) - as_h2(k));
}

// Four quant bytes (each < 64) -> two fp16 pairs of (q - off).
__device__ __forceinline__ void bytes_to_pairs(uint32_t b, uint32_t koff, uint32_t& p0, uint32_t& p1) {
  p0 = pk_sub(magic_pair_lo(b), koff);
  p1 = pk_sub(magic_pair_hi(b), koff);
}

constexpr uint32_t K1024 = 0x64006400u;   // fp16 pair (1024, 1024)
constexpr uint32_t K1056 = 0x64206420u;   // fp16 pair (1056, 1056): 1024 + 32

// 8 Q4_K weights (one A fragment) from two quant dwords.
__device__ __forceinline__ h8 q4k_frag(uint32_t w0, uint32_t w1, uint32_t mask, float dsc, float ndm) {
  uint32_t a0, a1, b0, b1;
  bytes_to_pairs(w0 & mask, K1024, a0, a1);
  bytes_to_pairs(w1 & mask, K1024, b0, b1);
  u32x4 r = {fma_mix_pair(a0, dsc, ndm), fma_mix_pair(a1, dsc, ndm), fma_mix_pair(b0, dsc, ndm),
             fma_mix_pair(b1, dsc, ndm)};
  return __builtin_bit_cast(h8, r);
}

// 8 Q6_K weights: low nibbles (shifted by nsh) | two high bits (at hsh) << 4.
__device__ __forceinline__ h8 q6k_frag(uint32_t l0, uint32_t l1, uint32_t h0, uint32_t h1, uint32_t nsh,
                                       uint32_t hsh, float dsc) {
  uint32_t q0 = ((l0 >> nsh) & 0x0f0f0f0fu) | (((h0 >> hsh) << 4) & 0x30303030u);
  uint32_t q1 = ((l1 >> nsh) & 0x0f0f0f0fu) | (((h1 >> hsh) << 4) & 0x30303030u);
  uint32_t a0, a1, b0, b1;
  bytes_to_pairs(q0, K1056, a0, a1);
  bytes_to_pairs(q1, K1056, b0, b1);
  u32x4 r = {fma_mix_pair(a0, dsc, 0.0f), fma_mix_pair(a1, dsc, 0.0f), fma_mix_pair(b0, dsc, 0.0f),
             fma_mix_pair(b1, dsc, 0.0f)};
  return __builtin_bit_cast(h8, r);
}

// Block header for the scale table.  Q4_K: bytes 0..15 (d, dmin, 12 scale
// bytes).  Q6_K: bytes 192..209 (16 int8 scales, fp16 d), read through the
// enclosing aligned dwords without touching anything past byte 209.
template <int FMT>
__device__ __forceinline__ void hdr_load(const uint8_t* blk, u32x4& hdr, uint32_t& hdr4) {
  if constexpr (FMT == 0) {
    hdr = *(const u32x4*)blk;
  } else {
    const uint8_t* p = blk + 192;
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
    const uint32_t* sp = (const uint32_t*)(p - sh);
    hdr = (u32x4){sp[0], sp[1], sp[2], sp[3]};
    hdr4 = sh ? sp[4] : (uint32_t)(*(const uint16_t*)(blk + 208)) << 16;
  }
}

// Decode one header into 16 floats of the table row.
//  Q4_K: pairs (d*sc_j, -dmin*m_j), with d*sc_j / 16 for odd j (their quant
//        is read from the high nibble as 16q).
//  Q6_K: d*sc_s for the 16 sub-blocks.
template <int FMT>
__device__ __forceinline__ void tab_store(float* t, const u32x4& hdr, uint32_t hdr4, uint32_t sh) {
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
    // sh = block address mod 4; with sh == 0 the d field sits in hdr4's high half
    uint32_t w[4] = {__builtin_amdgcn_alignbyte(hdr.y, hdr.x, sh), __builtin_amdgcn_alignbyte(hdr.z, hdr.y, sh),
                     __builtin_amdgcn_alignbyte(hdr.w, hdr.z, sh), __builtin_amdgcn_alignbyte(hdr4, hdr.w, sh)};
    float d = half_bits_to_float(hdr4 >> 16);
#pragma unroll
    for (int s = 0; s < 16; ++s) v[s] = d * (float)(int)(int8_t)((w[s >> 2] >> (8 * (s & 3))) & 0xffu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) ((float4*)t)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// Buffer resource (base, byte size) for the raw buffer loads: a 32-bit
// per-lane offset plus a scalar per-chunk offset, so no 64-bit address math
// per load, and loads past the end of the described range return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(uint32_t)n, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Raw quant bytes of one lane and i-block.
//  Q4_K, per 64-wide chunk: quant bytes 32p + 16g .. +16 (p = chunk in block).
//  Q6_K, per 128-weight half h (two chunks): low-nibble bytes 64h + 16g and
//  64h + 32 + 16g, high-bit bytes 128 + 32h + 16g.  Blocks are 210 bytes, so
//  a field may start 2 mod 4: it is read as the 5 enclosing aligned dwords
//  (at most 2 bytes before and 4 after the field; the last byte read is at
//  most 176 + 20 = 196 < 210) and shifted into place.
struct RawQ4 { u32x4 q; };
struct RawQ6 { u32x4 la, lb, hb; };
template <int FMT> struct RawOf { typedef RawQ4 T; };
template <> struct RawOf<1> { typedef RawQ6 T; };

__device__ __forceinline__ u32x4 load16_a2(rsrc_t r, uint32_t lane_off, uint32_t uni_off) {
  const uint32_t off = lane_off + uni_off;
  const uint32_t sh = off & 3u;
  const uint32_t v = off - sh;                   // aligned down; >= 0 since off >= sh
  const u32x4 w = buf_load16(r, v, 0);
  const uint32_t w4 = buf_load4(r, v + 16, 0);
  return (u32x4){__builtin_amdgcn_alignbyte(w.y, w.x, sh), __builtin_amdgcn_alignbyte(w.z, w.y, sh),
                 __builtin_amdgcn_alignbyte(w.w, w.z, sh), __builtin_amdgcn_alignbyte(w4, w.w, sh)};
}

// wr: this i-block's 32 weight rows; roff: li * row_bytes (+ 16 g for Q4_K)
template <int FMT>
__device__ __forceinline__ void raw_load(rsrc_t wr, uint32_t roff, int ck, int g, typename RawOf<FMT>::T& r) {
  const int bi = ck >> 2, cc = ck & 3;
  if constexpr (FMT == 0) {
    r.q = buf_load16(wr, roff, (uint32_t)(bi * Q4K_BYTES + 16 + 32 * cc));
  } else {
    const uint32_t blk = (uint32_t)(bi * Q6K_BYTES), h = (uint32_t)(cc >> 1);
    const uint32_t lo = roff + 16u * (uint32_t)g;
    r.la = load16_a2(wr, lo, blk + 64 * h);
    r.lb = load16_a2(wr, lo, blk + 64 * h + 32);
    r.hb = load16_a2(wr, lo, blk + 128 + 32 * h);
  }
}

// A fragment of K step s (0..3) of chunk cc from the raw bytes.
template <int FMT>
__device__ __forceinline__ h8 a_frag(const typename RawOf<FMT>::T& r, int s, int cc, const float (&sv)[4]) {
  if constexpr (FMT == 0) {
    const uint32_t w0 = (s & 1) ? r.q.z : r.q.x;
    const uint32_t w1 = (s & 1) ? r.q.w : r.q.y;
    return s < 2 ? q4k_frag(w0, w1, 0x0f0f0f0fu, sv[0], sv[1]) : q4k_frag(w0, w1, 0xf0f0f0f0u, sv[2], sv[3]);
  } else {
    const u32x4& l = (s >> 1) ? r.lb : r.la;
    const uint32_t l0 = (s & 1) ? l.z : l.x, l1 = (s & 1) ? l.w : l.y;
    const uint32_t h0 = (s & 1) ? r.hb.z : r.hb.x, h1 = (s & 1) ? r.hb.w : r.hb.y;
    const uint32_t nsh = (cc & 1) ? 4u : 0u;
    const uint32_t hsh = 4u * (uint32_t)(cc & 1) + 2u * (uint32_t)(s >> 1);
    return q6k_frag(l0, l1, h0, h1, nsh, hsh, sv[s >> 1]);
  }
}

// First global weight row of i-block c of wave w.
// SwiGLU (IB == 2): i-block 0 holds gate rows, i-block 1 the matching up rows.
template <int IB, bool SWIGLU>
__device__ __forceinline__ int iblock_row0(int w, int c, int n0, int hb, int F) {
  return SWIGLU ? (c == 0 ? 0 : F) + hb + 32 * w : n0 + 32 * IB * w + 32 * c;
}

// x0 / x1 (BM rows x 128 B each) and tab (2 x BN x TSTRIDE floats) are
// distinct LDS objects: the compiler's wait-count tracking then knows that
// reading one x buffer does not depend on the direct loads into the other.
// x rows are stored with their 16-byte chunks XOR-swizzled by (row >> 1) & 7:
// a ds_read_b128 of one column by 16 consecutive rows then covers all 64
// banks once (two rows share one 256-byte bank line).
template <int FMT, int JB, int IB, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const GemmDesc& P, int m_tile, int n_tile, uint8_t* x0, uint8_t* x1,
                                          float* tab) {
  typedef TileCfg<JB, IB> C;
  typedef typename RawOf<FMT>::T Raw;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  constexpr int XQ = (C::BM / 8 + 3) / 4;            // x load instructions per wave per chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int M = P.M, N = P.N, K = P.K;
  const int nck = K / 64;
  const int64_t row_bytes = (int64_t)(K / QK) * BLOCK_BYTES;
  const int m0 = m_tile * C::BM;
  const int F = N / 2;                               // SwiGLU: gate rows [0,F), up rows [F,2F)
  const int hb = n_tile * (C::BN / 2);               // SwiGLU: first h column of the tile
  const int n0 = n_tile * C::BN;

  // weight rows: one buffer per 32-row i-block; rows past N read as zero
  rsrc_t wr[IB];
#pragma unroll
  for (int c = 0; c < IB; ++c) {
    const int r0 = iblock_row0<IB, SWIGLU>(wave, c, n0, hb, F);
    const int nrows = N - r0 < 32 ? N - r0 : 32;
    wr[c] = make_rsrc(P.wq + (int64_t)r0 * row_bytes, (int64_t)nrows * row_bytes);
  }
  const uint32_t roff = (uint32_t)(li * row_bytes) + (FMT == 0 ? 16u * (uint32_t)g : 0u);
  // table thread tt decodes local row tt = 32*IB*w + 32*c + i (clamped to a valid row)
  const bool tab_thread = tid < C::BN;
  const int tt = tab_thread ? tid : 0;
  int trow_i = iblock_row0<IB, SWIGLU>(tt / (32 * IB), (tt / 32) % IB, n0, hb, F) + (tt & 31);
  trow_i = trow_i < N ? trow_i : N - 1;
  const uint8_t* trow = P.wq + (int64_t)trow_i * row_bytes;
  float* my_tab = tab + tt * C::TSTRIDE;

  // x: one buffer over this tile's rows (rows past M read as zero).  Wave
  // instruction q (of BM/8) fills LDS rows 8q .. 8q+7; lane t writes row
  // r = 8q + t/8, slot t%8, which holds 16-byte chunk (t%8) ^ ((r>>1)&7).
  const rsrc_t xr = make_rsrc(P.x + (int64_t)m0 * K, (int64_t)(M - m0) * K * 2);
  uint32_t xoff[XQ];
#pragma unroll
  for (int i = 0; i < XQ; ++i) {
    const int r = 8 * (4 * i + wave) + (lane >> 3);
    xoff[i] = (uint32_t)r * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  auto load_x = [&](int ck, uint8_t* xd) {
#pragma unroll
    for (int i = 0; i < XQ; ++i) {
      const int q = 4 * i + wave;
      if (q < C::BM / 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xd + q * 1024), 16,
                                                 xoff[i], (uint32_t)(128 * ck), 0, 0);
    }
  };

  f16x acc[JB][IB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int c = 0; c < IB; ++c) acc[jb][c] = (f16x){};

  u32x4 hdr = {0, 0, 0, 0};
  uint32_t hdr4 = 0;
  Raw ra[IB], rn[IB];

  // prologue: chunk 0 of x, table of block 0, raw bytes of chunk 0
  load_x(0, x0);
  if (tab_thread) hdr_load<FMT>(trow, hdr, hdr4);
#pragma unroll
  for (int c = 0; c < IB; ++c) raw_load<FMT>(wr[c], roff, 0, g, ra[c]);
  if (tab_thread) tab_store<FMT>(my_tab, hdr, hdr4, (uint32_t)((uintptr_t)(trow + 192) & 3));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // B-fragment LDS addresses of row li of j-block 0 for the 4 K steps and the
  // two buffers: 16-byte chunk 4*(s/2) + 2*g + (s%2), swizzled by the row
  // (rows of other j-blocks differ by multiples of 32: same swizzle).
  const uint8_t* bp[2][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int off = li * 128 + 16 * ((4 * (s >> 1) + 2 * g + (s & 1)) ^ ((li >> 1) & 7));
    bp[0][s] = x0 + off;
    bp[1][s] = x1 + off;
  }

  // chunks in pairs (nck is a multiple of 4): the even chunk reads x0 while
  // the next chunk streams into x1, the odd chunk the other way round
  for (int ck2 = 0; ck2 < nck; ck2 += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ck = ck2 + half;
      uint8_t* const xnext = half ? x0 : x1;
      const bool has_next = ck + 1 < nck;
      const bool next_block = has_next && ((ck + 1) & 3) == 0;
      const bool next_raw = has_next && (FMT == 0 || ((ck + 1) & 1) == 0);
      if (has_next) load_x(ck + 1, xnext);
      if (next_raw) {
#pragma unroll
        for (int c = 0; c < IB; ++c) raw_load<FMT>(wr[c], roff, ck + 1, g, rn[c]);
      }
      if (next_block && tab_thread) hdr_load<FMT>(trow + (int64_t)((ck + 1) >> 2) * BLOCK_BYTES, hdr, hdr4);

      const int cc = ck & 3;
      const float* tb = tab + ((ck >> 2) & 1) * (C::TBUF / 4);
      float sv[IB][4];
#pragma unroll
      for (int c = 0; c < IB; ++c) {
        const float* t = tb + (32 * IB * wave + 32 * c + li) * C::TSTRIDE;
        if constexpr (FMT == 0) {
          float4 v = *(const float4*)(t + 4 * cc);   // sub-blocks 2cc, 2cc+1
          sv[c][0] = v.x; sv[c][1] = v.y; sv[c][2] = v.z; sv[c][3] = v.w;
        } else {
          const int base = 8 * (cc >> 1) + 4 * (cc & 1) + g;   // scale index 8h + 2t + g
          sv[c][0] = t[base];
          sv[c][1] = t[base + 2];
          sv[c][2] = 0.0f;
          sv[c][3] = 0.0f;
        }
      }
      h8 af[IB], bf[JB];
#pragma unroll
      for (int c = 0; c < IB; ++c) af[c] = a_frag<FMT>(ra[c], 0, cc, sv[c]);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) bf[jb] = *(const h8*)(bp[half][0] + jb * 32 * 128);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        h8 afn[IB], bfn[JB];
        if (s < 3) {
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) bfn[jb] = *(const h8*)(bp[half][s + 1] + jb * 32 * 128);
#pragma unroll
          for (int c = 0; c < IB; ++c) afn[c] = a_frag<FMT>(ra[c], s + 1, cc, sv[c]);
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int c = 0; c < IB; ++c)
            acc[jb][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c], bf[jb], acc[jb][c], 0, 0, 0);
        if (s < 3) {
#pragma unroll
          for (int c = 0; c < IB; ++c) af[c] = afn[c];
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) bf[jb] = bfn[jb];
        }
      }
      if (next_block && tab_thread)
        tab_store<FMT>(my_tab + (((ck + 1) >> 2) & 1) * (C::TBUF / 4), hdr, hdr4,
                       (uint32_t)((uintptr_t)(trow + (int64_t)((ck + 1) >> 2) * BLOCK_BYTES + 192) & 3));
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (next_raw) {
#pragma unroll
        for (int c = 0; c < IB; ++c) ra[c] = rn[c];
      }
    }
  }

  // ---- epilogue: the lane holds rows 8q + 4g + e (q, e = 0..3) of each i-block ----
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const int m = m0 + 32 * jb + li;
    if (m >= M) continue;
    if (SWIGLU) {
      half_t* h = (half_t*)P.out + (int64_t)m * F;
      const f16x& gv = acc[jb][0];
      const f16x& uv = acc[jb][1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = hb + 32 * wave + 8 * q + 4 * g;
        h2 h01 = {(half_t)(silu_fast(gv[4 * q]) * uv[4 * q]), (half_t)(silu_fast(gv[4 * q + 1]) * uv[4 * q + 1])};
        h2 h23 = {(half_t)(silu_fast(gv[4 * q + 2]) * uv[4 * q + 2]),
                  (half_t)(silu_fast(gv[4 * q + 3]) * uv[4 * q + 3])};
        *(uint2*)(h + col) = make_uint2(as_u32(h01), as_u32(h23));
      }
    } else {
      float* yrow = (float*)P.out + (int64_t)m * N;
#pragma unroll
      for (int c = 0; c < IB; ++c) {
        const f16x& v = acc[jb][c];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + 32 * IB * wave + 32 * c + 8 * q + 4 * g;
          if ((N & 3) == 0 && n + 3 < N) {
            *(float4*)(yrow + n) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) yrow[n + e] = v[4 * q + e];
          }
        }
      }
    }
  }
}

// Workgroup -> (problem, tile).  Within a problem, tiles go in groups of 8
// N-tiles x all M-tiles with the N-tile fastest, so workgroups bid, bid+8,
// bid+16, ... (placed on the same XCD by the dispatcher) share one weight
// panel in that XCD's L2 while the 8 XCDs work on 8 different panels.
__device__ __forceinline__ const GemmDesc& tile_of(const GemmArgs& args, int& m_tile, int& n_tile) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMM_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].tile_begin) pi = i;
  const GemmDesc& P = args.d[pi];
  const int o = (int)blockIdx.x - P.tile_begin;
  const int mt = P.mt, nt = P.nt;
  const int grp = o / (8 * mt);
  const int u = o - grp * 8 * mt;
  const int nrem = nt - 8 * grp < 8 ? nt - 8 * grp : 8;
  m_tile = u / nrem;
  n_tile = 8 * grp + (u - m_tile * nrem);
  return P;
}

template <int FMT, int JB, int IB, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs args) {
  typedef TileCfg<JB, IB> C;
  __shared__ __attribute__((aligned(16))) uint8_t x0[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x1[C::XBUF];
  __shared__ __attribute__((aligned(16))) float tab[2 * C::TBUF / 4];
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
  int m_tile, n_tile;
  const GemmDesc& P = tile_of(args, m_tile, n_tile);
  gemm_tile<FMT, JB, IB, SWIGLU>(P, m_tile, n_tile, x0, x1, tab);
#endif
}

// Mixed Q4_K / Q6_K groups: one kernel per format would serialise on the
// stream, so this kernel branches per workgroup (uniformly) on the format.
// Q6_K problems run with JB6 <= JB j-blocks per tile: in a layer the Q6_K
// down projection has the longest reduction (K = 8192), and shorter tiles
// spread it over more CUs so it does not set the end of the launch.
template <int JB, int IB, int JB6>
__global__ __launch_bounds__(256, 1) void gemm_kernel_mixed(GemmArgs args) {
  typedef TileCfg<JB, IB> C;
  __shared__ __attribute__((aligned(16))) uint8_t x0[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x1[C::XBUF];
  __shared__ __attribute__((aligned(16))) float tab[2 * C::TBUF / 4];
#if defined(__HIP_DEVICE_COMPILE__)
  int m_tile, n_tile;
  const GemmDesc& P = tile_of(args, m_tile, n_tile);
  if (P.fmt == 0)
    gemm_tile<0, JB, IB, false>(P, m_tile, n_tile, x0, x1, tab);
  else
    gemm_tile<1, JB6, IB, false>(P, m_tile, n_tile, x0, x1, tab);
#endif
}

template <typename Kern>
static hipError_t launch_one(Kern k, int tiles, const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k, dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Tile counts of one problem for BM = 32*jb rows and BN = 128*ib weight rows.
static void set_tiles(GemmDesc& d, const GemmProblem& p, int jb, int ib, bool swiglu) {
  const int bm = 32 * jb, bn = 128 * ib;
  d.x = (const half_t*)p.x;
  d.wq = p.wq;
  d.out = p.out;
  d.fmt = p.fmt;
  d.swiglu = p.swiglu;
  d.M = p.M;
  d.N = p.N;
  d.K = p.K;
  d.mt = (p.M + bm - 1) / bm;
  d.nt = swiglu ? (p.N / 2 + bn / 2 - 1) / (bn / 2) : (p.N + bn - 1) / bn;
}

// JB: j-blocks per tile for Q4_K (and single-format) problems; JB6 for Q6_K
// problems of a mixed group.
template <int JB, int IB, bool SWIGLU, int JB6 = JB>
static hipError_t launch_cfg(const GemmProblem* probs, int count, hipStream_t s) {
  for (int base = 0; base < count; base += GEMM_MAX_GROUP) {
    GemmArgs a{};
    int n = count - base < GEMM_MAX_GROUP ? count - base : GEMM_MAX_GROUP;
    int fmt_mask = 0;
    for (int i = 0; i < n; ++i) fmt_mask |= 1 << probs[base + i].fmt;
    const bool mixed = !SWIGLU && fmt_mask == 3;
    int tiles = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = probs[base + i];
      GemmDesc& d = a.d[i];
      set_tiles(d, p, (mixed && p.fmt == 1) ? JB6 : JB, IB, SWIGLU);
      d.tile_begin = tiles;
      tiles += d.mt * d.nt;
    }
    a.count = n;
    hipError_t e;
    if constexpr (SWIGLU) {
      e = launch_one(gemm_kernel<0, JB, IB, true>, tiles, a, s);
    } else {
      if (fmt_mask == 1)
        e = launch_one(gemm_kernel<0, JB, IB, false>, tiles, a, s);
      else if (fmt_mask == 2)
        e = launch_one(gemm_kernel<1, JB, IB, false>, tiles, a, s);
      else
        e = launch_one(gemm_kernel_mixed<JB, IB, JB6>, tiles, a, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Relative time of a launch with tiles of jb j-blocks (32 activation rows
// each) and ib i-blocks per wave (32 weight rows each).  Workgroups run in
// rounds of one tile per CU; per K chunk a tile costs the dequant of its
// weight panel (~ 2 MFMA j-blocks per i-block) plus jb * ib MFMA j-blocks.
static double launch_cost(const GemmProblem* probs, int count, int jb, int ib, bool swiglu, int ncu) {
  int64_t tiles = 0, kmax = 0;
  double work = 0.0;
  for (int i = 0; i < count; ++i) {
    GemmDesc d;
    set_tiles(d, probs[i], jb, ib, swiglu);
    tiles += (int64_t)d.mt * d.nt;
    work += (double)d.mt * d.nt * probs[i].K;
    kmax = probs[i].K > kmax ? probs[i].K : kmax;
  }
  const double per_chunk = ib * (2.0 + 0.5 * jb);
  const double rounds = (double)((tiles + ncu - 1) / ncu);
  // full rounds of the mean tile, but never less than the longest tile
  double t = rounds * (work / (double)tiles);
  if (t < (double)kmax) t = (double)kmax;
  return t * per_chunk;
}

hipError_t launch_gemm(const GemmProblem* probs, int count, hipStream_t s) {
  int mmax = 0, fmt_mask = 0;
  const bool swiglu = probs[0].swiglu != 0;
  for (int i = 0; i < count; ++i) {
    mmax = probs[i].M > mmax ? probs[i].M : mmax;
    fmt_mask |= 1 << probs[i].fmt;
  }
  const int ncu = device_cu_count();
  // candidate tile shapes (jb, ib); SwiGLU needs ib == 2 (gate + up)
  static const int cand[6][2] = {{8, 2}, {4, 2}, {2, 2}, {1, 2}, {2, 1}, {1, 1}};
  int best_jb = 1, best_ib = 2;
  double best = 0.0;
  for (const auto& c : cand) {
    const int jb = c[0], ib = c[1];
    if (swiglu && ib != 2) continue;
    if (jb > 1 && 32 * (jb / 2) >= mmax) continue;          // taller than needed
    const double t = launch_cost(probs, count, jb, ib, swiglu, ncu);
    if (best == 0.0 || t < best * 0.97) {
      best = t;
      best_jb = jb;
      best_ib = ib;
    }
  }
  if (swiglu) {
    switch (best_jb) {
      case 8: return launch_cfg<8, 2, true>(probs, count, s);
      case 4: return launch_cfg<4, 2, true>(probs, count, s);
      case 2: return launch_cfg<2, 2, true>(probs, count, s);
      default: return launch_cfg<1, 2, true>(probs, count, s);
    }
  }
  const bool mixed = fmt_mask == 3;
  if (best_ib == 1) return best_jb == 2 ? launch_cfg<2, 1, false>(probs, count, s) : launch_cfg<1, 1, false>(probs, count, s);
  switch (best_jb) {
    case 8: return mixed ? launch_cfg<8, 2, false, 4>(probs, count, s) : launch_cfg<8, 2, false>(probs, count, s);
    case 4: return mixed ? launch_cfg<4, 2, false, 2>(probs, count, s) : launch_cfg<4, 2, false>(probs, count, s);
    case 2: return launch_cfg<2, 2, false>(probs, count, s);
    default: return launch_cfg<1, 2, false>(probs, count, s);
  }
}

}  // namespace dmq
