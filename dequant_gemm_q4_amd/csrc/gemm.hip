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
//    (buffer_load ... lds, no VGPR staging) into four buffers, three chunks
//    ahead, with the 16-byte chunks of each 128-byte row XOR-swizzled by the
//    row so that B-fragment reads are free of bank conflicts.
//  * Sub-block scales / mins are decoded once per super-block and weight row
//    into an LDS table.  Per weight the lanes then do: mask the nibble in
//    place, convert the byte to fp32 (v_cvt_f32_ubyteN, exact), one fp32 FMA
//    of exact operands (q*d*sc - dmin*m) and a round-to-nearest-even pack of
//    two results to fp16 (v_cvt_pk_f16_f32).
//  * v_mfma_f32_32x32x16_f16: lane l holds operand row l%32 and k-slots
//    8*(l/32) .. +7; the accumulator lane holds D[8*(r/4) + 4*(l/32) + r%4]
//    [l%32], r = 0..15.  The K order inside a 64-wide chunk is permuted (the
//    same way for both operands) so that each lane's 8 weights of a step come
//    from 8 consecutive quant bytes: step s, lane half g, slot e covers
//    k = 32*(s/2) + 16*g + 8*(s%2) + e.
//  * Dequant of the next K step is issued between the MFMAs of the current
//    one.
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
  static constexpr int TBUF = BN * TSTRIDE * 4;      // bytes of the scale table
  static constexpr size_t LDS_BYTES = 4 * XBUF + TBUF;
};

__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

typedef float f2 __attribute__((ext_vector_type(2)));

// Four quant bytes b0..b3 -> the fp16 pairs (w0, w1), (w2, w3) with
// w_i = fp16(b_i * s + c): v_cvt_f32_ubyteN (exact), one fp32 FMA of exact
// operands, and v_cvt_pk_f16_f32 (round to nearest even).  All three are
// full-rate VALU instructions on gfx950, where v_fma_mix runs at about half
// rate.  The empty asm hides the masks applied by the caller, so that the
// compiler converts byte N directly instead of extracting it first.
__device__ __forceinline__ void bytes_fma_pairs(uint32_t b, float s, float c, uint32_t& p0, uint32_t& p1) {
  asm("" : "+v"(b));
  const f2 v0 = {__builtin_fmaf((float)(b & 0xffu), s, c), __builtin_fmaf((float)((b >> 8) & 0xffu), s, c)};
  const f2 v1 = {__builtin_fmaf((float)((b >> 16) & 0xffu), s, c), __builtin_fmaf((float)(b >> 24), s, c)};
  p0 = as_u32(__builtin_convertvector(v0, h2));
  p1 = as_u32(__builtin_convertvector(v1, h2));
}

// 8 Q4_K weights (one A fragment) from two quant dwords.  The nibbles are
// masked in place (low: q, high: 16 q); the table scale s is d*sc (d*sc/16
// for high nibbles, exact), so b*s is exactly q*d*sc and the FMA with
// -dmin*m rounds once.
__device__ __forceinline__ h8 q4k_frag(uint32_t w0, uint32_t w1, uint32_t mask, float dsc, float ndm) {
  uint32_t r0, r1, r2, r3;
  bytes_fma_pairs(w0 & mask, dsc, ndm, r0, r1);
  bytes_fma_pairs(w1 & mask, dsc, ndm, r2, r3);
  const u32x4 r = {r0, r1, r2, r3};
  return __builtin_bit_cast(h8, r);
}

// 8 Q6_K weights: q = low nibbles (shifted by nsh) | two high bits (at hsh)
// << 4; w = q*dsc - 32*dsc with dsc = d*sc.
__device__ __forceinline__ h8 q6k_frag(uint32_t l0, uint32_t l1, uint32_t h0, uint32_t h1, uint32_t nsh,
                                       uint32_t hsh, float dsc) {
  const uint32_t q0 = ((l0 >> nsh) & 0x0f0f0f0fu) | (((h0 >> hsh) << 4) & 0x30303030u);
  const uint32_t q1 = ((l1 >> nsh) & 0x0f0f0f0fu) | (((h1 >> hsh) << 4) & 0x30303030u);
  const float off = dsc * -32.0f;
  uint32_t r0, r1, r2, r3;
  bytes_fma_pairs(q0, dsc, off, r0, r1);
  bytes_fma_pairs(q1, dsc, off, r2, r3);
  const u32x4 r = {r0, r1, r2, r3};
  return __builtin_bit_cast(h8, r);
}

// Block header for the scale table.  Q4_K: bytes 0..15 (d, dmin, 12 scale
// bytes).  Q6_K: bytes 192..209 (16 int8 scales, fp16 d), read through the
// enclosing aligned dwords without touching anything past byte 209.
// The dword at byte 206 of a Q6_K block (halfwords 206 and 208; 2-byte
// aligned, which the hardware's unaligned global loads handle).
typedef uint32_t u32_a2 __attribute__((aligned(2)));

template <int FMT>
__device__ __forceinline__ void hdr_load(const uint8_t* blk, u32x4& hdr, uint32_t& hdr4) {
  if constexpr (FMT == 0) {
    hdr = *(const u32x4*)blk;
  } else {
    // Q6_K: the aligned dwords from byte 192 (or 190) and the dword at 206,
    // all inside the block.  Nothing here combines the values: that waits
    // until the decode, so the loads' latency stays hidden.
    const uint8_t* p = blk + 192;
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
    const uint32_t* sp = (const uint32_t*)(p - sh);
    hdr = (u32x4){sp[0], sp[1], sp[2], sp[3]};
    hdr4 = *(const u32_a2*)(blk + 206);
  }
}

// Decode one header into 16 floats of the table row.
//  Q4_K: pairs (d*sc_j, -dmin*m_j), with d*sc_j/16 for odd j (their quant
//        is read from the high nibble as 16q).
//  Q6_K: d*sc_s for the 16 sub-blocks, even s first (s = 0, 2, .., 14
//        in floats 0..7), then odd s (floats 8..15): a lane only needs the
//        sub-blocks of one parity.
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
    // sh = (block address + 192) mod 4: the 20 bytes from byte 192 - sh are
    // hdr and, for sh = 2, hdr4 (the dword at 206); d is hdr4's high half
    uint32_t w[4] = {__builtin_amdgcn_alignbyte(hdr.y, hdr.x, sh), __builtin_amdgcn_alignbyte(hdr.z, hdr.y, sh),
                     __builtin_amdgcn_alignbyte(hdr.w, hdr.z, sh), __builtin_amdgcn_alignbyte(hdr4, hdr.w, sh)};
    float d = half_bits_to_float(hdr4 >> 16);
#pragma unroll
    for (int s = 0; s < 16; ++s)
      v[(s >> 1) + 8 * (s & 1)] = d * (float)(int)(int8_t)((w[s >> 2] >> (8 * (s & 3))) & 0xffu);
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
//  a field may start 2 mod 4: it is loaded as the 5 enclosing aligned dwords
//  (at most 2 bytes before and 4 after the field; the last byte read is at
//  most 176 + 20 = 196 < 210) and shifted into place only when first used,
//  so that the load's latency is not exposed where it is issued.
struct RawQ4 { u32x4 q; };
struct Win { u32x4 w; uint32_t w4; };                  // 20-byte aligned window
struct RawQ6 { Win la, lb, hb; uint32_t sh; };         // sh: field start mod 4
struct Q6Fields { u32x4 la, lb, hb; };                 // realigned 16-byte fields
template <int FMT> struct RawOf { typedef RawQ4 T; };
template <> struct RawOf<1> { typedef RawQ6 T; };

__device__ __forceinline__ void load_win(rsrc_t r, uint32_t aligned_off, Win& w) {
  w.w = buf_load16(r, aligned_off, 0);
  w.w4 = buf_load4(r, aligned_off + 16, 0);
}
__device__ __forceinline__ u32x4 realign(const Win& w, uint32_t sh) {
  return (u32x4){__builtin_amdgcn_alignbyte(w.w.y, w.w.x, sh), __builtin_amdgcn_alignbyte(w.w.z, w.w.y, sh),
                 __builtin_amdgcn_alignbyte(w.w.w, w.w.z, sh), __builtin_amdgcn_alignbyte(w.w4, w.w.w, sh)};
}

// Q4_K raw bytes of chunk ck (wr: this i-block's 32 rows; roff: li * row_bytes + 16 g)
__device__ __forceinline__ void raw_load_q4(rsrc_t wr, uint32_t roff, int ck, RawQ4& r) {
  r.q = buf_load16(wr, roff, (uint32_t)((ck >> 2) * Q4K_BYTES + 16 + 32 * (ck & 3)));
}
// Q6_K raw bytes of half h of block bi (roff: li * row_bytes)
__device__ __forceinline__ void raw_load_q6(rsrc_t wr, uint32_t roff, int bi, int h, int g, RawQ6& r) {
  const uint32_t lo = roff + (uint32_t)(bi * Q6K_BYTES) + 16u * (uint32_t)g;   // lane's field offset, before h
  r.sh = lo & 3u;                                      // same for the three fields (offsets differ by 32/64)
  const uint32_t base = lo - r.sh;
  load_win(wr, base + 64u * (uint32_t)h, r.la);
  load_win(wr, base + 64u * (uint32_t)h + 32u, r.lb);
  load_win(wr, base + 128u + 32u * (uint32_t)h, r.hb);
}
__device__ __forceinline__ Q6Fields q6_fields(const RawQ6& r) {
  return Q6Fields{realign(r.la, r.sh), realign(r.lb, r.sh), realign(r.hb, r.sh)};
}

// A fragment of K step s (0..3) of chunk cc (0..3 within the block).
// sv: Q4_K (d*sc and -dmin*m of the chunk's even and odd sub-block, d*sc/16
// for the odd one); Q6_K (d*sc of the lane's two sub-blocks of the chunk).
__device__ __forceinline__ h8 a_frag_q4(const RawQ4& r, int s, const float (&sv)[4]) {
  const uint32_t w0 = (s & 1) ? r.q.z : r.q.x;
  const uint32_t w1 = (s & 1) ? r.q.w : r.q.y;
  return s < 2 ? q4k_frag(w0, w1, 0x0f0f0f0fu, sv[0], sv[1]) : q4k_frag(w0, w1, 0xf0f0f0f0u, sv[2], sv[3]);
}
__device__ __forceinline__ h8 a_frag_q6(const Q6Fields& f, int s, int cc, const float (&sv)[4]) {
  const u32x4& l = (s >> 1) ? f.lb : f.la;
  const uint32_t l0 = (s & 1) ? l.z : l.x, l1 = (s & 1) ? l.w : l.y;
  const uint32_t h0 = (s & 1) ? f.hb.z : f.hb.x, h1 = (s & 1) ? f.hb.w : f.hb.y;
  const uint32_t nsh = (cc & 1) ? 4u : 0u;
  const uint32_t hsh = 4u * (uint32_t)(cc & 1) + 2u * (uint32_t)(s >> 1);
  return q6k_frag(l0, l1, h0, h1, nsh, hsh, sv[s >> 1]);
}

// First global weight row of i-block c of wave w.
// SwiGLU (IB == 2): i-block 0 holds gate rows, i-block 1 the matching up rows.
template <int IB, bool SWIGLU>
__device__ __forceinline__ int iblock_row0(int w, int c, int n0, int hb, int F) {
  return SWIGLU ? (c == 0 ? 0 : F) + hb + 32 * w : n0 + 32 * IB * w + 32 * c;
}

// s_waitcnt vmcnt(n) lgkmcnt(0) followed by a workgroup barrier, as one asm
// statement with a memory clobber: the compiler neither moves memory
// accesses across it nor adds a full vmcnt(0) drain (as a fence would).
template <int n>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

// One BM x BN output tile.  The reduction runs over 64-wide K chunks, four per
// super-block, as a software pipeline:
//  * x chunk ck is staged by direct global->LDS loads into buffer ck % 4,
//    issued three chunks ahead (x0..x3 are distinct LDS objects, so the
//    compiler's wait-count tracking knows that reading one buffer does not
//    depend on the direct loads into another);
//  * raw quant bytes go to registers, issued three chunks ahead (Q4_K, four
//    register sets) or half a block ahead (Q6_K, two sets);
//  * every chunk has one barrier, before its last K step, after which the
//    next chunk's x buffer and (at a block boundary) the next scale table are
//    visible; the last step's MFMAs then overlap the next chunk's first
//    dequant and B-fragment reads, so no chunk starts with an exposed
//    prologue;
//  * within a step, the B fragments of the next step are requested first and
//    the next step's dequant (VALU) is interleaved with this step's MFMAs.
// The scale table holds one super-block: per weight row, decoded by one
// thread, from a header loaded a block ahead; each lane copies its rows'
// entries to registers once per block.
// x rows are stored with their 16-byte chunks XOR-swizzled by (row >> 1) & 7:
// a ds_read_b128 of one column by 16 consecutive rows then covers all 64
// banks once (two rows share one 256-byte bank line).
template <int FMT, int JB, int IB, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const GemmDesc& P, int m_tile, int n_tile, uint8_t* x0, uint8_t* x1,
                                          uint8_t* x2, uint8_t* x3, float* tab) {
  typedef TileCfg<JB, IB> C;
  typedef typename RawOf<FMT>::T Raw;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  constexpr int XQ = JB;                             // x load instructions per wave per chunk (BM/8 row groups / 4 waves)
  constexpr int NRAW = FMT == 0 ? IB : 6 * IB;       // VMEM instructions of one raw load round
  constexpr int NSC = FMT == 0 ? 16 : 8;             // scale floats per row a lane keeps
  uint8_t* const xb[4] = {x0, x1, x2, x3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int M = P.M, N = P.N, K = P.K;
  const int nb = K / QK;
  const int64_t row_bytes = (int64_t)nb * BLOCK_BYTES;
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
    for (int i = 0; i < XQ; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xd + (4 * i + wave) * 1024),
                                               16, xoff[i], (uint32_t)(128 * ck), 0, 0);
  };
  // B-fragment offsets of row li (j-block 0) in an x buffer for the 4 K
  // steps: 16-byte chunk 4*(s/2) + 2*g + (s%2), swizzled by the row (rows of
  // other j-blocks differ by multiples of 32: same swizzle).
  uint32_t boff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) boff[s] = (uint32_t)(li * 128 + 16 * ((4 * (s >> 1) + 2 * g + (s & 1)) ^ ((li >> 1) & 7)));

  f16x acc[JB][IB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int c = 0; c < IB; ++c) acc[jb][c] = (f16x){};

  u32x4 hdr = {0, 0, 0, 0};
  uint32_t hdr4 = 0;
  constexpr int NSET = FMT == 0 ? 4 : 2;
  Raw rs[NSET][IB];          // raw quant sets: Q4_K chunk mod 4, Q6_K block half
  float scl[IB][NSC];        // this block's scale-table entries of the lane's rows
  float sv[IB][4];           // scales of the current chunk
  h8 af[IB], bf[JB];

  auto read_scales = [&]() {
#pragma unroll
    for (int c = 0; c < IB; ++c) {
      const float* t = tab + (32 * IB * wave + 32 * c + li) * C::TSTRIDE + (FMT == 0 ? 0 : 8 * g);
#pragma unroll
      for (int i = 0; i < NSC / 4; ++i) {
        const float4 v = ((const float4*)t)[i];
        scl[c][4 * i] = v.x; scl[c][4 * i + 1] = v.y; scl[c][4 * i + 2] = v.z; scl[c][4 * i + 3] = v.w;
      }
    }
  };
  // chunk cc's scales (Q6_K: scale index 8h + 2t + g, t = 2(cc&1) + s/2, is
  // entry 4(cc>>1) + 2(cc&1) + s/2 of the lane's parity list)
  auto chunk_scales = [&](int cc, float (&o)[IB][4]) {
#pragma unroll
    for (int c = 0; c < IB; ++c) {
      if constexpr (FMT == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[c][e] = scl[c][4 * cc + e];
      } else {
        const int e0 = 4 * (cc >> 1) + 2 * (cc & 1);
        o[c][0] = scl[c][e0];
        o[c][1] = scl[c][e0 + 1];
        o[c][2] = 0.0f;
        o[c][3] = 0.0f;
      }
    }
  };
  auto frag = [&](const Raw& r, int s, int cc, const float (&v)[4]) -> h8 {
    if constexpr (FMT == 0) {
      return a_frag_q4(r, s, v);
    } else {
      return a_frag_q6(q6_fields(r), s, cc, v);
    }
  };
  auto mfma_step = [&](const h8 (&a)[IB], const h8 (&bm)[JB]) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int c = 0; c < IB; ++c)
        acc[jb][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c], bm[jb], acc[jb][c], 0, 0, 0);
  };
  auto interleave = [&]() {
    // spread the VALU work of the next fragment between this step's MFMAs
#pragma unroll
    for (int i = 0; i < JB * IB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  };

  // ---- prologue: block 0's table, x and raw bytes of the first chunks
  if (tab_thread) hdr_load<FMT>(trow, hdr, hdr4);
#pragma unroll
  for (int c = 0; c < IB; ++c) {
    if constexpr (FMT == 0) {
#pragma unroll
      for (int k = 0; k < 3; ++k) raw_load_q4(wr[c], roff, k, rs[k][c]);
    } else {
      raw_load_q6(wr[c], roff, 0, 0, g, rs[0][c]);
      raw_load_q6(wr[c], roff, 0, 1, g, rs[1][c]);
    }
  }
  load_x(0, x0);
  load_x(1, x1);
  load_x(2, x2);
  if (tab_thread) tab_store<FMT>(my_tab, hdr, hdr4, (uint32_t)((uintptr_t)(trow + 192) & 3));
  wait_vm_barrier<0>();
  read_scales();
  chunk_scales(0, sv);
#pragma unroll
  for (int c = 0; c < IB; ++c) af[c] = frag(rs[0][c], 0, 0, sv[c]);
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) bf[jb] = *(const h8*)(x0 + boff[0] + jb * 32 * 128);

  for (int b = 0; b < nb; ++b) {
    const bool more = b + 1 < nb;
    // header of the next block (decoded into the table during chunk 3).
    // Loads are issued unconditionally (past the end they re-read the last
    // block or chunk into buffers nobody reads), so every iteration issues
    // the same VMEM instructions and the wait counts below are exact.
    const int bnext = more ? b + 1 : b;
    if (tab_thread) hdr_load<FMT>(trow + (int64_t)bnext * BLOCK_BYTES, hdr, hdr4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ck = 4 * b + j;
      const uint8_t* const xc = xb[j];
      const uint8_t* const xn = xb[(j + 1) & 3];
      const bool pf1 = j < 3 || more;     // chunk ck + 1 exists
      const int cur = FMT == 0 ? j : (j >> 1);                    // raw set of chunk ck
      const int nxt = FMT == 0 ? ((j + 1) & 3) : (((j + 1) & 3) >> 1);
      // x (and Q4_K raw bytes) of chunk ck+3, into the buffers chunk ck-1 used
      const int ck3 = ck + 3 < 4 * nb ? ck + 3 : 4 * nb - 1;
      load_x(ck3, xb[(j + 3) & 3]);
      if constexpr (FMT == 0) {
#pragma unroll
        for (int c = 0; c < IB; ++c) raw_load_q4(wr[c], roff, ck3, rs[(j + 3) & 3][c]);
      }

      // K steps 0..2
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        h8 afn[IB], bfn[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) bfn[jb] = *(const h8*)(xc + boff[s + 1] + jb * 32 * 128);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < IB; ++c) afn[c] = frag(rs[cur][c], s + 1, j, sv[c]);
        if (j == 3 && s == 0 && more && tab_thread)
          tab_store<FMT>(my_tab, hdr, hdr4, (uint32_t)((uintptr_t)(trow + (int64_t)(b + 1) * BLOCK_BYTES + 192) & 3));
        mfma_step(af, bf);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < IB; ++c) af[c] = afn[c];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) bf[jb] = bfn[jb];
      }

      // K step 3: wait for chunk ck+1's x and raw bytes and, at a block
      // boundary, the new table; the loads of later chunks stay in flight
      // (counts: VMEM instructions issued after the last one needed here)
      if constexpr (FMT == 0) {
        wait_vm_barrier<2 * (XQ + NRAW)>();
      } else {
        if (j == 0 || j == 2) wait_vm_barrier<2 * XQ + NRAW>();
        else wait_vm_barrier<2 * XQ>();
      }
      h8 afn[IB], bfn[JB];
      float svn[IB][4];
      if (pf1) {
        if (j == 3) read_scales();
        chunk_scales((j + 1) & 3, svn);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) bfn[jb] = *(const h8*)(xn + boff[0] + jb * 32 * 128);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (pf1) {
#pragma unroll
        for (int c = 0; c < IB; ++c) afn[c] = frag(rs[nxt][c], 0, (j + 1) & 3, svn[c]);
      }
      mfma_step(af, bf);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      if (pf1) {
#pragma unroll
        for (int c = 0; c < IB; ++c) {
          af[c] = afn[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[c][e] = svn[c][e];
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) bf[jb] = bfn[jb];
      }
      // Q6_K raw bytes ahead: the next block's half j/2 once this block's
      // half is used up
      if constexpr (FMT == 1) {
        if (j & 1) {
#pragma unroll
          for (int c = 0; c < IB; ++c) raw_load_q6(wr[c], roff, bnext, j >> 1, g, rs[j >> 1][c]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // no direct-to-LDS load may still be in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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

// Workgroup -> (problem, tile).  Within a problem the M-tile runs fastest:
// the dispatcher places workgroup bid on XCD bid % 8, so with mt dividing 8
// each XCD keeps seeing the same one or two activation panels (they stay in
// that XCD's L2) while its compute units stream different weight panels,
// each once per M-tile.  (N-tile-fastest order would instead stream every
// activation panel through every XCD once per N-tile.)
__device__ __forceinline__ const GemmDesc& tile_of(const GemmArgs& args, int& m_tile, int& n_tile) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMM_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].tile_begin) pi = i;
  const GemmDesc& P = args.d[pi];
  const int o = (int)blockIdx.x - P.tile_begin;
  n_tile = o / P.mt;
  m_tile = o - n_tile * P.mt;
  return P;
}

template <int FMT, int JB, int IB, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs args) {
  typedef TileCfg<JB, IB> C;
  __shared__ __attribute__((aligned(16))) uint8_t x0[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x1[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x2[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x3[C::XBUF];
  __shared__ __attribute__((aligned(16))) float tab[C::TBUF / 4];
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
  int m_tile, n_tile;
  const GemmDesc& P = tile_of(args, m_tile, n_tile);
  gemm_tile<FMT, JB, IB, SWIGLU>(P, m_tile, n_tile, x0, x1, x2, x3, tab);
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
  __shared__ __attribute__((aligned(16))) uint8_t x2[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x3[C::XBUF];
  __shared__ __attribute__((aligned(16))) float tab[C::TBUF / 4];
#if defined(__HIP_DEVICE_COMPILE__)
  int m_tile, n_tile;
  const GemmDesc& P = tile_of(args, m_tile, n_tile);
  if (P.fmt == 0)
    gemm_tile<0, JB, IB, false>(P, m_tile, n_tile, x0, x1, x2, x3, tab);
  else
    gemm_tile<1, JB6, IB, false>(P, m_tile, n_tile, x0, x1, x2, x3, tab);
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
