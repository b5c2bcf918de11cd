// Prefill kernel (M >= 2): y = x * W^T with the Q4_K / Q6_K dequant fused into
// an MFMA fp16 x fp16 -> fp32 contraction.  Prefill is matrix-matrix work in
// which every weight is reused across all prompt rows (overview page, "[01]
// the thesis": prefill is dense, compute-bound GEMM; article "Building
// DAMASCUS", "Prefill and decode need different performance questions"), and
// the fused dequant never writes fp16 weights to memory (overview page, same
// section, and compartment 09 of "[02] the pipeline").
//
// One workgroup = NW waves = one BM x BN output tile, BM = 32*JB activation
// rows, BN = NW * 32*IB = 256 weight rows: 4 waves of two 32-row i-blocks, or
// (tiles of at least 64 activation rows, no SwiGLU) 8 waves of one, two per
// SIMD, so that one wave's dequantisation runs beside the other's MFMAs.
//  * Each wave owns 32*IB weight rows and all BM activation rows.  It decodes
//    its raw blocks straight into the registers of the MFMA's B operand (the
//    weights; x fragments read from LDS are the A operand, so an accumulator
//    lane holds one output column): every weight is dequantised once per
//    workgroup and no dequantised tile touches LDS or HBM.  (In the code,
//    `wf` names the weight fragments and `xf` the x fragments.)
//  * x is staged in LDS per 64-wide K chunk by direct global->LDS loads
//    (buffer_load ... lds, no VGPR staging) into four buffers, three chunks
//    ahead, with the 16-byte chunks of each 128-byte row XOR-swizzled by the
//    row so that the x-fragment reads are free of bank conflicts.
//  * Sub-block scales / mins are decoded once per super-block and weight row
//    into an LDS table.  Per weight the lanes then do: isolate the quant in
//    a byte, convert it to fp32 exactly (Q4_K: the nibble read as an fp8
//    E4M3 pattern is q * 2^-9, two per v_cvt_pk_f32_fp8, with 2^9 folded
//    into the scale; Q6_K: v_cvt_f32_ubyteN), one fp32 FMA of exact operands
//    (q*d*sc - dmin*m) and a round-to-nearest-even pack of two results to
//    fp16 (v_cvt_pk_f16_f32).
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
#include "plan.h"

#include <algorithm>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

namespace dmq {


// One segment of a launch: the tiles of n-tiles [n_begin, n_begin + nt) of
// one problem, all of one tile height (alt = 0: the kernel's tall height,
// 1: its short one), workgroups tile_begin .. tile_begin + ks*mt*nt - 1.
// With ks > 1 the reduction is split: piece s covers K blocks [s*kbs,
// (s+1)*kbs) and writes its fp32 partial sums to out + s*out_stride floats
// (a workspace that a second kernel sums in piece order).
struct GemmDesc {
  const half_t* x;
  const uint8_t* wq;
  void* out;
  int64_t out_stride;
  int32_t fmt, swiglu, M, N, K;
  int32_t tile_begin, mt, nt, n_begin, alt, ks, kbs;
};

struct GemmArgs {
  GemmDesc d[GEMM_MAX_SEG];
  int32_t count;
};

typedef float f16x __attribute__((ext_vector_type(16)));

template <int JB, int IB, int NW = 4>
struct TileCfg {
  static constexpr int BM = 32 * JB;                 // activation rows per tile
  static constexpr int BN = 32 * IB * NW;            // weight rows per tile (NW waves of 32*IB rows)
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

// Four nibbles (one per byte, 0..15) -> the fp16 pairs (w0, w1), (w2, w3)
// with w_i = fp16(q_i * d*sc + c).  v_cvt_pk_f32_fp8 reads byte patterns
// 0..15 as the fp8 E4M3 values q * 2^-9 exactly, two per instruction, so the
// scale s512 carries 2^9: the product is exactly q*d*sc and the FMA rounds
// once, as with an integer q.
__device__ __forceinline__ void nibbles_fma_pairs(uint32_t b, float s512, float c, uint32_t& p0, uint32_t& p1) {
  const f2 q01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
  const f2 q23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, true);
  const f2 v0 = {__builtin_fmaf(q01.x, s512, c), __builtin_fmaf(q01.y, s512, c)};
  const f2 v1 = {__builtin_fmaf(q23.x, s512, c), __builtin_fmaf(q23.y, s512, c)};
  p0 = as_u32(__builtin_convertvector(v0, h2));
  p1 = as_u32(__builtin_convertvector(v1, h2));
}

// 8 Q4_K weights (one weight fragment) from two quant dwords: their low (hi =
// false) or high nibbles; dsc512 = d*sc*2^9, ndm = -dmin*m.
__device__ __forceinline__ h8 q4k_frag(uint32_t w0, uint32_t w1, bool hi, float dsc512, float ndm) {
  const uint32_t b0 = (hi ? w0 >> 4 : w0) & 0x0f0f0f0fu;
  const uint32_t b1 = (hi ? w1 >> 4 : w1) & 0x0f0f0f0fu;
  uint32_t r0, r1, r2, r3;
  nibbles_fma_pairs(b0, dsc512, ndm, r0, r1);
  nibbles_fma_pairs(b1, dsc512, ndm, r2, r3);
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

typedef u32x4 u32x4_a2 __attribute__((aligned(2)));

template <int FMT>
__device__ __forceinline__ void hdr_load(const uint8_t* blk, u32x4& hdr, uint32_t& hdr4) {
  if constexpr (FMT == 0) {
    hdr = *(const u32x4*)blk;
  } else {
    // Q6_K: the 16 scale bytes (192..207) and the dword at 206 (d in its
    // high half), both 2-byte aligned, both inside the block
    hdr = *(const u32x4_a2*)(blk + 192);
    hdr4 = *(const u32_a2*)(blk + 206);
  }
}

// Decode one header into 16 floats of the table row.
//  Q4_K: pairs (d*sc_j * 2^9, -dmin*m_j); the nibbles reach fp32 as
//        q * 2^-9.
//  Q6_K: d*sc_s for the 16 sub-blocks, even s first (s = 0, 2, .., 14
//        in floats 0..7), then odd s (floats 8..15): a lane only needs the
//        sub-blocks of one parity.
template <int FMT>
__device__ __forceinline__ void tab_store(float* t, const u32x4& hdr, uint32_t hdr4) {
  float v[16];
  if constexpr (FMT == 0) {
    Q4kScales s = unpack_q4k_scales(hdr.y, hdr.z, hdr.w);
    float d = half_bits_to_float(hdr.x), dmin = half_bits_to_float(hdr.x >> 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float dsc = d * (float)q4k_sc(s, j);
      v[2 * j] = dsc * 512.0f;
      v[2 * j + 1] = -(dmin * (float)q4k_m(s, j));
    }
  } else {
    const uint32_t w[4] = {hdr.x, hdr.y, hdr.z, hdr.w};
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
//  a field may start 2 mod 4; the 16-byte buffer loads take such 2-byte
//  aligned offsets as they are (the memory path splits them), which costs
//  less than loading the enclosing aligned dwords and shifting.
struct RawQ4 { u32x4 q; };
struct RawQ6 { u32x4 la, lb, hb; };
typedef RawQ6 Q6Fields;
template <int FMT> struct RawOf { typedef RawQ4 T; };
template <> struct RawOf<1> { typedef RawQ6 T; };

// Q4_K raw bytes of chunk ck (wr: this i-block's 32 rows; roff: li * row_bytes + 16 g)
__device__ __forceinline__ void raw_load_q4(rsrc_t wr, uint32_t roff, int ck, RawQ4& r) {
  r.q = buf_load16(wr, roff, (uint32_t)((ck >> 2) * Q4K_BYTES + 16 + 32 * (ck & 3)));
}
// One of the three loads of the Q6_K raw bytes of half h of block bi (part
// 0: la, 1: lb, 2: hb; roff: li * row_bytes).
__device__ __forceinline__ void raw_load_q6_part(rsrc_t wr, uint32_t roff, int bi, int h, int g, int part, RawQ6& r) {
  const uint32_t lo = roff + (uint32_t)(bi * Q6K_BYTES) + 16u * (uint32_t)g;   // lane's field offset, before h
  const uint32_t off = part == 0 ? lo + 64u * (uint32_t)h : part == 1 ? lo + 64u * (uint32_t)h + 32u
                                                                      : lo + 128u + 32u * (uint32_t)h;
  u32x4& w = part == 0 ? r.la : part == 1 ? r.lb : r.hb;
  w = buf_load16(wr, off, 0);
}
__device__ __forceinline__ void raw_load_q6(rsrc_t wr, uint32_t roff, int bi, int h, int g, RawQ6& r) {
#pragma unroll
  for (int part = 0; part < 3; ++part) raw_load_q6_part(wr, roff, bi, h, g, part, r);
}
__device__ __forceinline__ const Q6Fields& q6_fields(const RawQ6& r) { return r; }

// Weight fragment of K step s (0..3) of chunk cc (0..3 within the block).
// sv: Q4_K (d*sc*2^9 and -dmin*m of the chunk's even and odd sub-block);
// Q6_K (d*sc of the lane's two sub-blocks of the chunk).
__device__ __forceinline__ h8 a_frag_q4(const RawQ4& r, int s, const float (&sv)[4]) {
  const uint32_t w0 = (s & 1) ? r.q.z : r.q.x;
  const uint32_t w1 = (s & 1) ? r.q.w : r.q.y;
  return s < 2 ? q4k_frag(w0, w1, false, sv[0], sv[1]) : q4k_frag(w0, w1, true, sv[2], sv[3]);
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
//    register sets) or about half a block ahead (Q6_K, two sets);
//  * a chunk's loads are spread over its first three K steps, between the
//    MFMAs: issued as one burst they fill the texture-address FIFO, and the
//    wave's MFMA issue stalls behind them;
//  * every chunk has one barrier, before its last K step, after which the
//    next chunk's x buffer and (at a block boundary) the next scale table are
//    visible; the last step's MFMAs then overlap the next chunk's first
//    dequant and x-fragment reads, so no chunk starts with an exposed
//    prologue;
//  * within a step, the x fragments of the next step are requested first and
//    the next step's dequant (VALU) is interleaved with this step's MFMAs.
// The scale table holds one super-block: per weight row, decoded by one
// thread, from a header loaded a block ahead; each lane copies its rows'
// entries to registers once per block.
// x rows are stored with their 16-byte chunks XOR-swizzled by (row >> 1) & 7:
// a ds_read_b128 of one column by 16 consecutive rows then covers all 64
// banks once (two rows share one 256-byte bank line).
// The x fragment is the MFMA's A operand and the weight fragment its B
// operand, so an accumulator lane holds one output column n (its lane % 32)
// and 16 rows m: for a fixed accumulator register the 64 lanes hold 32
// consecutive columns of two rows, and the epilogue's dword stores write
// whole 128-byte lines of y straight from the accumulators.
template <int FMT, int JB, int IB, int NW, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const GemmDesc& P, int m_tile, int n_tile, int kb0, int nbk, void* out,
                                          uint8_t* x0, uint8_t* x1, uint8_t* x2, uint8_t* x3, float* tab) {
  typedef TileCfg<JB, IB, NW> C;
  typedef typename RawOf<FMT>::T Raw;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  constexpr int XQ = 4 * JB / NW;                    // x load instructions per wave per chunk (BM/8 row groups / NW waves)
  static_assert(XQ * NW == 4 * JB, "the tile's 8-row groups must split evenly over the waves");
  constexpr int NRAW = FMT == 0 ? IB : 3 * IB;       // VMEM instructions of one raw load round
  constexpr int NSC = FMT == 0 ? 16 : 8;             // scale floats per row a lane keeps
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int M = P.M, N = P.N, K = P.K;
  const int nb = nbk;                                // K blocks of this piece, from block kb0
  const int64_t row_bytes = (int64_t)(K / QK) * BLOCK_BYTES;
  const int64_t kb_bytes = (int64_t)kb0 * BLOCK_BYTES;
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
    wr[c] = make_rsrc(P.wq + (int64_t)r0 * row_bytes + kb_bytes, (int64_t)nrows * row_bytes - kb_bytes);
  }
  const uint32_t roff = (uint32_t)(li * row_bytes) + (FMT == 0 ? 16u * (uint32_t)g : 0u);
  // table thread tt decodes local row tt = 32*IB*w + 32*c + i (clamped to a valid row)
  const bool tab_thread = tid < C::BN;
  // the same test per wave (BN is a multiple of 64): a scalar branch, so
  // waves without table rows skip the decode instead of issuing it masked
  static_assert(C::BN % 64 == 0 && 64 * NW >= C::BN, "table rows fill whole waves");
  const bool tab_wave = wave < C::BN / 64;
  const int tt = tab_thread ? tid : 0;
  int trow_i = iblock_row0<IB, SWIGLU>(tt / (32 * IB), (tt / 32) % IB, n0, hb, F) + (tt & 31);
  trow_i = trow_i < N ? trow_i : N - 1;
  const uint8_t* trow = P.wq + (int64_t)trow_i * row_bytes + kb_bytes;
  float* my_tab = tab + tt * C::TSTRIDE;

  // x: one buffer over this tile's rows (rows past M read as zero).  Wave
  // instruction q (of BM/8) fills LDS rows 8q .. 8q+7; lane t writes row
  // r = 8q + t/8, slot t%8, which holds 16-byte chunk (t%8) ^ ((r>>1)&7).
  const rsrc_t xr = make_rsrc(P.x + (int64_t)m0 * K + kb0 * QK, (int64_t)(M - m0) * K * 2 - kb0 * QK * 2);
  uint32_t xoff[XQ];
#pragma unroll
  for (int i = 0; i < XQ; ++i) {
    const int r = 8 * (NW * i + wave) + (lane >> 3);
    xoff[i] = (uint32_t)r * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  uint8_t* const xb[4] = {x0, x1, x2, x3};
  auto load_x = [&](int ck, uint8_t* xd) {
#pragma unroll
    for (int i = 0; i < XQ; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xd + (NW * i + wave) * 1024),
                                               16, xoff[i], (uint32_t)(128 * ck), 0, 0);
  };
  // x-fragment offsets of row li (j-block 0) in an x buffer for the 4 K
  // steps: 16-byte chunk 4*(s/2) + 2*g + (s%2), swizzled by the row (rows of
  // other j-blocks differ by multiples of 32: same swizzle).
  uint32_t boff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) boff[s] = (uint32_t)(li * 128 + 16 * ((4 * (s >> 1) + 2 * g + (s & 1)) ^ ((li >> 1) & 7)));
  // The same offsets plus 64 KiB, opaque to the compiler: buffers x2 and x3
  // lie above 64 KiB of LDS, beyond a ds_read's 16-bit immediate offset, and
  // from boff the compiler re-forms their addresses with one v_or per read.
  // Addressed as x2/x3 + (boffh - 64 KiB), they take these registers plus an
  // immediate offset, and the pointer still derives from the buffer (the
  // compiler's LDS-DMA alias tracking sees which buffer a read touches).
  uint32_t boffh[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    boffh[s] = boff[s] + 65536u;
    asm volatile("" : "+v"(boffh[s]));
  }
  // x fragment of K step s, j-block jb, from x buffer j
  auto bread = [&](int j, int s, int jb) -> h8 {
    const uint8_t* const p = j >= 2 ? xb[j] + (boffh[s] - 65536u) : xb[j] + boff[s];
    return *(const h8*)(p + jb * 32 * 128);
  };

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
  h8 wf[IB], xf[JB];

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
        acc[jb][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bm[jb], a[c], acc[jb][c], 0, 0, 0);
  };
  // spread the VALU work of the next fragment (va instructions per MFMA),
  // and nv VMEM loads, between this step's MFMAs
  auto interleave = [&](int nv, int va) {
#pragma unroll
    for (int i = 0; i < JB * IB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int v = (i + 1) * nv / (JB * IB) - i * nv / (JB * IB);
#pragma unroll
      for (int k = 0; k < v; ++k) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
      for (int k = 0; k < va; ++k) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
  };
  // NW = 8 (one i-block per wave): each x fragment feeds exactly one MFMA, so
  // its next-step read follows that MFMA into the same registers (no second
  // set of fragments); the order per MFMA: the MFMA, its fragment's read,
  // the step's share of VMEM loads, va VALU instructions.
  auto interleave_rd = [&](int nv, int va) {
#pragma unroll
    for (int i = 0; i < JB * IB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      const int v = (i + 1) * nv / (JB * IB) - i * nv / (JB * IB);
#pragma unroll
      for (int k = 0; k < v; ++k) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
      for (int k = 0; k < va; ++k) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
  };
  // The VMEM loads chunk j of a block issues for later chunks, spread over its
  // K steps 0..2 (a burst of them at the chunk start would fill the
  // texture-address FIFO and stall the wave's MFMA issue behind it):
  //  Q4_K: x of chunk ck+3 (XQ loads), then its raw quant bytes (IB loads);
  //  Q6_K: at j = 0 the raw bytes of half 1 of this block, at j = 2 those
  //  of half 0 of the next block (3*IB loads, issued first), then x of
  //  chunk ck+3.  Returns the number of loads issued in step s.
  auto issue_loads = [&](int j, int s, int ck3, int b, int bnext) -> int {
    constexpr int NR6 = 3 * IB;
    const int nr = FMT == 0 ? 0 : ((j & 1) ? 0 : NR6);    // raw loads before the x loads
    const int total = nr + XQ + (FMT == 0 ? IB : 0);
    const int lo = s * total / 3, hi = (s + 1) * total / 3;
#pragma unroll
    for (int t = lo; t < hi; ++t) {
      if (t < nr) {
        if constexpr (FMT == 1) {
          if (j == 0) raw_load_q6_part(wr[t / 3], roff, b, 1, g, t % 3, rs[1][t / 3]);
          else raw_load_q6_part(wr[t / 3], roff, bnext, 0, g, t % 3, rs[0][t / 3]);
        }
      } else if (t < nr + XQ) {
        const int i = t - nr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xb[(j + 3) & 3] + (NW * i + wave) * 1024),
                                                 16, xoff[i], (uint32_t)(128 * ck3), 0, 0);
      } else if constexpr (FMT == 0) {
        raw_load_q4(wr[t - nr - XQ], roff, ck3, rs[(j + 3) & 3][t - nr - XQ]);
      }
    }
    return hi - lo;
  };

  // ---- prologue: block 0's table, x and raw bytes of the first chunks,
  // issued chunk by chunk; only chunk 0's have to land before the first
  // step (Q6_K: half 1 of block 0 is loaded by chunk 0 of the loop)
  if (tab_thread) hdr_load<FMT>(trow, hdr, hdr4);
  if constexpr (FMT == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      load_x(k, xb[k]);
#pragma unroll
      for (int c = 0; c < IB; ++c) raw_load_q4(wr[c], roff, k, rs[k][c]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < IB; ++c) raw_load_q6(wr[c], roff, 0, 0, g, rs[0][c]);
    load_x(0, x0);
    load_x(1, x1);
    load_x(2, x2);
  }
  if (tab_thread) tab_store<FMT>(my_tab, hdr, hdr4);
  if constexpr (FMT == 0) wait_vm_barrier<2 * (XQ + NRAW)>();
  else wait_vm_barrier<2 * XQ>();
  read_scales();
  chunk_scales(0, sv);
#pragma unroll
  for (int c = 0; c < IB; ++c) wf[c] = frag(rs[0][c], 0, 0, sv[c]);
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) xf[jb] = bread(0, 0, jb);

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
      const int cur = FMT == 0 ? j : (j >> 1);                    // raw set of chunk ck
      const int nxt = FMT == 0 ? ((j + 1) & 3) : (((j + 1) & 3) >> 1);
      // x (and raw bytes) of chunk ck+3 go into the buffers chunk ck-1 used
      const int ck3 = ck + 3 < 4 * nb ? ck + 3 : 4 * nb - 1;

      if constexpr (NW == 8) {
        // K steps 0..2
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          h8 wfn[IB];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < IB; ++c) wfn[c] = frag(rs[cur][c], s + 1, j, sv[c]);
          if (j == 3 && s == 0 && more && tab_wave)
            tab_store<FMT>(my_tab, hdr, hdr4);
          const int nv = issue_loads(j, s, ck3, b, bnext);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
            for (int c = 0; c < IB; ++c)
              acc[jb][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[jb], wf[c], acc[jb][c], 0, 0, 0);
            xf[jb] = bread(j, s + 1, jb);
          }
          interleave_rd(nv, j == 3 && s == 0 ? 6 : 3);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < IB; ++c) wf[c] = wfn[c];
        }
        // K step 3: as below; the next chunk's fragments are read from its
        // buffer after the barrier, each after the MFMA that frees it
        if constexpr (FMT == 0) {
          wait_vm_barrier<2 * (XQ + NRAW)>();
        } else {
          if (j == 0 || j == 2) wait_vm_barrier<2 * XQ + NRAW>();
          else wait_vm_barrier<2 * XQ>();
        }
        h8 wfn[IB];
        float svn[IB][4];
        if (j == 3) read_scales();
        chunk_scales((j + 1) & 3, svn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < IB; ++c) wfn[c] = frag(rs[nxt][c], 0, (j + 1) & 3, svn[c]);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
          for (int c = 0; c < IB; ++c)
            acc[jb][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[jb], wf[c], acc[jb][c], 0, 0, 0);
          xf[jb] = bread((j + 1) & 3, 0, jb);
        }
        interleave_rd(0, 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < IB; ++c) {
          wf[c] = wfn[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[c][e] = svn[c][e];
        }
        continue;
      }

      // K steps 0..2
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        h8 wfn[IB], xfn[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) xfn[jb] = bread(j, s + 1, jb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < IB; ++c) wfn[c] = frag(rs[cur][c], s + 1, j, sv[c]);
        if (j == 3 && s == 0 && more && tab_wave)
          tab_store<FMT>(my_tab, hdr, hdr4);
        const int nv = issue_loads(j, s, ck3, b, bnext);
        mfma_step(wf, xf);
        // the step that also decodes the next block's scale table has more
        // VALU work to place
        interleave(nv, j == 3 && s == 0 ? 6 : 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < IB; ++c) wf[c] = wfn[c];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) xf[jb] = xfn[jb];
      }

      // K step 3: wait for chunk ck+1's x and raw bytes and, at a block
      // boundary, the new table; the loads of later chunks stay in flight
      // (counts: VMEM instructions issued after the last one needed here).
      // After the tile's last chunk there is no chunk ck+1: its fragments
      // are still read and decoded (from LDS and registers the tile owns,
      // results unused), so no step carries a branch that would keep the
      // scheduler from interleaving the decode with the MFMAs.
      if constexpr (FMT == 0) {
        wait_vm_barrier<2 * (XQ + NRAW)>();
      } else {
        if (j == 0 || j == 2) wait_vm_barrier<2 * XQ + NRAW>();
        else wait_vm_barrier<2 * XQ>();
      }
      h8 wfn[IB], xfn[JB];
      float svn[IB][4];
      if (j == 3) read_scales();
      chunk_scales((j + 1) & 3, svn);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) xfn[jb] = bread((j + 1) & 3, 0, jb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < IB; ++c) wfn[c] = frag(rs[nxt][c], 0, (j + 1) & 3, svn[c]);
      mfma_step(wf, xf);
      interleave(0, 3);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < IB; ++c) {
        wf[c] = wfn[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[c][e] = svn[c][e];
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) xf[jb] = xfn[jb];
    }
  }
  // no direct-to-LDS load may still be in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: register r of acc[jb][c] holds y[m][n], n = the lane's
  // column of i-block c, m = m0 + 32 jb + 8 (r / 4) + 4 g + r % 4 ----
  if constexpr (SWIGLU) {
    // h[m][j] = silu(g) * u, j = hb + 32 w + li: gate in i-block 0, up in 1
    const int j = hb + 32 * wave + li;
    if (j < F) {
      half_t* const hc = (half_t*)out + j;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m < M) hc[(int64_t)m * F] = (half_t)(silu_fast(acc[jb][0][r]) * acc[jb][1][r]);
        }
    }
  } else {
    // Whole tile inside M and y below 4 GB: buffer stores, a scalar row
    // offset plus the lane's fixed byte offset, no guard and no per-store
    // address arithmetic in the lanes.
    const bool fast = m0 + C::BM <= M && (int64_t)M * N < ((int64_t)1 << 30);
    const rsrc_t yr = make_rsrc(out, 4 * (int64_t)M * N);
#pragma unroll
    for (int c = 0; c < IB; ++c) {
      const int n = n0 + 32 * IB * wave + 32 * c + li;
      if (n >= N) continue;
      if (fast) {
        const uint32_t lo = 4u * (uint32_t)(4 * g * N + n);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t so = 4u * (uint32_t)(m0 + 32 * jb + 8 * (r >> 2) + (r & 3)) * (uint32_t)N;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[jb][c][r]), yr, lo, so, 0);
          }
      } else {
        float* const yc = (float*)out + n;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (m < M) yc[(int64_t)m * N] = acc[jb][c][r];
          }
      }
    }
  }
}

// Workgroup -> (segment, tile).  Within a segment the M-tile runs fastest:
// the dispatcher places workgroup bid on XCD bid % 8, so with mt dividing 8
// each XCD keeps seeing the same one or two activation panels (they stay in
// that XCD's L2) while its compute units stream different weight panels,
// each once per M-tile.  (N-tile-fastest order would instead stream every
// activation panel through every XCD once per N-tile.)
// Split pieces run slowest: all tiles of piece 0, then of piece 1, ...
__device__ __forceinline__ const GemmDesc& tile_of(const GemmArgs& args, int& m_tile, int& n_tile, int& piece) {
  int pi = 0;
#pragma unroll
  for (int i = 1; i < GEMM_MAX_SEG; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].tile_begin) pi = i;
  const GemmDesc& P = args.d[pi];
  const int per = P.mt * P.nt;
  const int o = (int)blockIdx.x - P.tile_begin;
  piece = o / per;
  const int r = o - piece * per;
  const int nl = r / P.mt;
  m_tile = r - nl * P.mt;
  n_tile = P.n_begin + nl;
  return P;
}

template <int FMT, int JBA, int JBB, bool SWIGLU, int NW>
__device__ __forceinline__ void run_tile(const GemmDesc& P, int m_tile, int n_tile, int piece, uint8_t* x0,
                                         uint8_t* x1, uint8_t* x2, uint8_t* x3, float* tab) {
  constexpr int IB = 8 / NW;   // weight i-blocks per wave: 256 weight rows per tile
  const int kb0 = piece * P.kbs;
  const int left = P.K / QK - kb0;
  const int nbk = left < P.kbs ? left : P.kbs;
  void* out = SWIGLU ? P.out : (void*)((float*)P.out + piece * P.out_stride);
  if constexpr (JBA == JBB) {
    gemm_tile<FMT, JBA, IB, NW, SWIGLU>(P, m_tile, n_tile, kb0, nbk, out, x0, x1, x2, x3, tab);
  } else {
    if (P.alt)
      gemm_tile<FMT, JBB, IB, NW, SWIGLU>(P, m_tile, n_tile, kb0, nbk, out, x0, x1, x2, x3, tab);
    else
      gemm_tile<FMT, JBA, IB, NW, SWIGLU>(P, m_tile, n_tile, kb0, nbk, out, x0, x1, x2, x3, tab);
  }
}

// One workgroup = one tile of 32*JBA or 32*JBB activation rows (per
// segment) by 256 weight rows.  FMT_MASK: bit 0 Q4_K, bit 1 Q6_K; with both,
// the kernel branches per workgroup (uniformly) on the segment's format, so
// a group of mixed-format problems is one launch rather than one per format
// serialised on the stream.
template <int FMT_MASK, int JBA, int JBB, bool SWIGLU, int NW = 4>
__global__ __launch_bounds__(64 * NW, 1) void gemm_kernel(GemmArgs args) {
  static_assert(!SWIGLU || NW == 4, "the SwiGLU epilogue pairs a wave's two i-blocks");
  typedef TileCfg<JBA, 8 / NW, NW> C;   // LDS sized for the taller tile
  __shared__ __attribute__((aligned(16))) uint8_t x0[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x1[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x2[C::XBUF];
  __shared__ __attribute__((aligned(16))) uint8_t x3[C::XBUF];
  __shared__ __attribute__((aligned(16))) float tab[C::TBUF / 4];
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
  int m_tile, n_tile, piece;
  const GemmDesc& P = tile_of(args, m_tile, n_tile, piece);
  if constexpr (FMT_MASK == 1) {
    run_tile<0, JBA, JBB, SWIGLU, NW>(P, m_tile, n_tile, piece, x0, x1, x2, x3, tab);
  } else if constexpr (FMT_MASK == 2) {
    run_tile<1, JBA, JBB, SWIGLU, NW>(P, m_tile, n_tile, piece, x0, x1, x2, x3, tab);
  } else {
    if (P.fmt == 0)
      run_tile<0, JBA, JBB, SWIGLU, NW>(P, m_tile, n_tile, piece, x0, x1, x2, x3, tab);
    else
      run_tile<1, JBA, JBB, SWIGLU, NW>(P, m_tile, n_tile, piece, x0, x1, x2, x3, tab);
  }
#else
  (void)args, (void)x0, (void)x1, (void)x2, (void)x3, (void)tab;
#endif
}

// Split-K combine: y = sum over pieces s = 0 .. ks-1 of part[s], added in
// piece order, so a result does not depend on which piece finished first.
struct ReduceDesc {
  const float* part;   // ks slices of n floats, stride floats apart
  float* y;            // n floats
  int64_t n, stride;   // n = M * N; stride = n rounded up to a multiple of 4
  int32_t ks;
};
struct ReduceArgs {
  ReduceDesc d[GEMM_MAX_GROUP];
  int64_t begin[GEMM_MAX_GROUP + 1];   // float4 index where each problem starts
  int32_t count;
};

__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceArgs a) {
  const int64_t total = a.begin[a.count];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    int pi = 0;
    for (int k = 1; k < a.count; ++k)
      if (i >= a.begin[k]) pi = k;
    const ReduceDesc& d = a.d[pi];
    const int64_t e = 4 * (i - a.begin[pi]);   // first float of this thread's group of 4
    if (e + 4 <= d.n) {
      float4 acc = *(const float4*)(d.part + e);
      for (int s = 1; s < d.ks; ++s) {
        const float4 v = *(const float4*)(d.part + s * d.stride + e);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      *(float4*)(d.y + e) = acc;
    } else {
      for (int64_t f = e; f < d.n; ++f) {
        float acc = d.part[f];
        for (int s = 1; s < d.ks; ++s) acc += d.part[s * d.stride + f];
        d.y[f] = acc;
      }
    }
  }
}

template <int FMT_MASK, int JBA, int JBB, bool SWIGLU, int NW>
static hipError_t launch_k(int tiles, const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<FMT_MASK, JBA, JBB, SWIGLU, NW>), dim3(tiles), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// nw: waves per workgroup, 4 (two i-blocks each) or 8 (one each, two waves
// per SIMD); 8 needs tiles of at least 64 rows and no SwiGLU epilogue.
template <int JBA, int JBB>
static hipError_t launch_pair(const Plan& pl, int tiles, const GemmArgs& a, hipStream_t s, int nw) {
  if (pl.swiglu) return launch_k<1, JBA, JBB, true, 4>(tiles, a, s);
  if constexpr (JBB >= 2) {
    if (nw == 8) {
      switch (pl.fmt_mask) {
        case 1: return launch_k<1, JBA, JBB, false, 8>(tiles, a, s);
        case 2: return launch_k<2, JBA, JBB, false, 8>(tiles, a, s);
        default: return launch_k<3, JBA, JBB, false, 8>(tiles, a, s);
      }
    }
  }
  switch (pl.fmt_mask) {
    case 1: return launch_k<1, JBA, JBB, false, 4>(tiles, a, s);
    case 2: return launch_k<2, JBA, JBB, false, 4>(tiles, a, s);
    default: return launch_k<3, JBA, JBB, false, 4>(tiles, a, s);
  }
}

// Waves per workgroup for a plan: 8 where the kernel has them (tiles of at
// least 64 rows, no SwiGLU epilogue), else 4.
static int plan_waves(const Plan& pl) { return !pl.swiglu && pl.jbb >= 2 ? 8 : 4; }

static hipError_t launch_chunk_nw(const GemmProblem* probs, int count, hipStream_t s, int nw);

static hipError_t launch_chunk(const GemmProblem* probs, int count, hipStream_t s) {
  return launch_chunk_nw(probs, count, s, plan_waves(get_plan(probs, count)));
}

static hipError_t launch_chunk_nw(const GemmProblem* probs, int count, hipStream_t s, int nw) {
  const Plan pl = get_plan(probs, count);
  // workspace slices of the split problems (slice stride rounded to 4 floats)
  int64_t ws_floats = 0;
  int64_t ws_at[GEMM_MAX_SEG];
  for (int i = 0; i < pl.nseg; ++i) {
    const Seg& sg = pl.seg[i];
    ws_at[i] = ws_floats;
    if (sg.ks > 1) ws_floats += sg.ks * ((((int64_t)probs[sg.prob].M * probs[sg.prob].N) + 3) & ~(int64_t)3);
  }
  float* ws = nullptr;
  if (ws_floats > 0) {
    void* p = nullptr;
    const hipError_t e = stream_workspace(WorkspaceUse::SplitK, s, (size_t)ws_floats * 4, &p);
    if (e != hipSuccess) return e;
    ws = (float*)p;
  }
  GemmArgs a{};
  ReduceArgs r{};
  int tiles = 0;
  for (int i = 0; i < pl.nseg; ++i) {
    const Seg& sg = pl.seg[i];
    const GemmProblem& p = probs[sg.prob];
    GemmDesc& d = a.d[i];
    d.x = (const half_t*)p.x;
    d.wq = p.wq;
    d.fmt = p.fmt;
    d.swiglu = p.swiglu;
    d.M = p.M;
    d.N = p.N;
    d.K = p.K;
    d.mt = m_tiles(p, sg.alt ? pl.jbb : pl.jba);
    d.nt = sg.nt;
    d.n_begin = sg.n_begin;
    d.alt = sg.alt;
    d.ks = sg.ks;
    d.kbs = sg.kbs;
    d.tile_begin = tiles;
    if (sg.ks > 1) {
      const int64_t n = (int64_t)p.M * p.N;
      d.out = ws + ws_at[i];
      d.out_stride = (n + 3) & ~(int64_t)3;
      ReduceDesc& rd = r.d[r.count];
      rd.part = ws + ws_at[i];
      rd.y = (float*)p.out;
      rd.n = n;
      rd.stride = d.out_stride;
      rd.ks = sg.ks;
      r.begin[r.count + 1] = r.begin[r.count] + (n + 3) / 4;
      ++r.count;
    } else {
      d.out = p.out;
      d.out_stride = 0;
    }
    tiles += d.ks * d.mt * d.nt;
  }
  a.count = pl.nseg;
  hipError_t e;
  switch (pl.jba) {
    case 8: e = pl.jbb == 2 ? launch_pair<8, 2>(pl, tiles, a, s, nw) : launch_pair<8, 4>(pl, tiles, a, s, nw); break;
    case 4: e = launch_pair<4, 2>(pl, tiles, a, s, nw); break;
    case 2: e = launch_pair<2, 1>(pl, tiles, a, s, nw); break;
    default: e = launch_pair<1, 1>(pl, tiles, a, s, nw); break;
  }
  if (e != hipSuccess || r.count == 0) return e;
  const int64_t groups = r.begin[r.count];
  const int64_t blocks = (groups + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, s, r);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmProblem* probs, int count, hipStream_t s) {
  // A SwiGLU problem runs alone (its epilogue is the kernel's).
  for (int base = 0; base < count; base += GEMM_MAX_GROUP) {
    const int n = count - base < GEMM_MAX_GROUP ? count - base : GEMM_MAX_GROUP;
    const hipError_t e = launch_chunk(probs + base, n, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dmq
