// Small-M kernel (2 <= M <= 32): y = x * W^T for a few activation rows.
//
// With a handful of rows the work is still a stream of the weights (each
// weight is used M times, far below the MFMA ridge), so this kernel keeps
// the decode kernel's shape and hands the per-weight multiply-adds of all
// M rows to the matrix cores (article "Building DAMASCUS", "Prefill and
// decode need different performance questions": prefill reuses each weight
// across the prompt rows; overview page, compartment 09 of "[02] the
// pipeline": the dequant is fused and fp16 weights are never written):
//
//  * a workgroup owns 16 consecutive weight rows; its waves split the row's
//    super-blocks into contiguous slices, and a lane works on row l%16 and
//    part l/16 of every super-block of its wave's slice.  A single
//    projection takes one wave per super-block (up to 16), so every load of
//    the workgroup is issued before the first multiply and the matrix
//    streams in about one memory round trip instead of one per block; a
//    grid of at least two workgroups per CU (several projections in one
//    launch) takes 4-wave workgroups, four per CU; deeper rows of a single
//    projection take 16 waves.  Each wave walks its slice a block at a time;
//  * x goes through LDS: a wave copies a block's x, 16 rows x 512 bytes,
//    with 8 direct-to-LDS loads that each cover two whole rows, i.e. full
//    128-byte lines.  Loaded straight into the B operand, each load would
//    instead touch half of 16 lines (16 rows x 64 bytes), and the x loads
//    would cost the L1 twice the lookups;
//  * v_mfma_f32_16x16x32_f16 (A: lane l holds row l%16 and k-slots
//    8*(l/16) .. +7; B: column l%16, the same k-slots; D: column l%16, rows
//    4*(l/16) .. +3) takes 8 dequantised weights per lane as the A operand
//    and the matching 8 x values of activation row l%16 as B (zeros for
//    rows past M), so every weight is dequantised once and used by all M
//    rows;
//  * the K order inside an MFMA is free (A and B use the same one): part p
//    of a Q4_K block is quant bytes 32p..32p+31 (sub-blocks 2p and 2p+1),
//    and MFMA step s takes the low (s < 4) or high nibbles of its bytes
//    8(s%4) .. +7; Q6_K part p is half p/2, 16-weight column p%2 of each
//    32-weight quarter, and step s covers quarter s/2, weights 8(s%2) .. +7;
//  * the waves' partial sums are added in wave order through LDS (the same
//    result every run);
//  * SwiGLU gate|up pairs: a workgroup takes 8 gate rows and the matching 8
//    up rows, and forms h = fp16(silu(g) * u) from the two sums;
//  * 17 <= M <= 32: two 16-row groups of activation rows, each dequantised
//    weight fragment feeding two MFMAs (16 KB x slots, at most 8 waves).
//
// Dequant is exact as in the other kernels: Q4_K nibbles reach fp32 as fp8
// E4M3 patterns (q * 2^-9, scale carrying 2^9), Q6_K quants through
// v_cvt_f32_ubyte; one fp32 FMA of exact operands; fp16 pairs by RNE.
#include "dmq_common.h"

#include <utility>

namespace dmq {

constexpr int SKINNY_MAX_GROUP = 8;

// Buffer resource over [base, base + bytes): loads past the end read zeros.
typedef __amdgpu_buffer_rsrc_t sk_rsrc_t;
__device__ __forceinline__ sk_rsrc_t sk_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(uint32_t)n, 0x00020000);
}
constexpr int SKINNY_ROWS = 16;
constexpr int SKINNY_MAX_WAVES = 16;

struct SkinnyDesc {
  const half_t* x;
  const uint8_t* wq;
  void* out;             // y [M, N] fp32, or h [M, N/2] fp16 in SwiGLU mode
  int32_t fmt, swiglu, M, N, K;
  int32_t wg_begin;
};

struct SkinnyArgs {
  SkinnyDesc d[SKINNY_MAX_GROUP];
  int32_t count;
};

typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32_a2 __attribute__((aligned(2)));
typedef uint4 u4_a2 __attribute__((aligned(2)));
typedef uint2 u2_a2 __attribute__((aligned(2)));

// One lane's bytes of one super-block.  MFMA step s covers the 32 weights
// k = 32s .. 32s+31 of the block, and part p (= lane / 16) the 8 weights
// 32s + 8p .. +7, so the 4 parts of a step read one 64-byte piece of each
// activation row.
//  Q4_K: sub-block s; its quant bytes 32(s/2) + 8p .. +7, low nibbles for
//        even s, high for odd s.  A lane loads the 8 bytes 32c + 8p (c =
//        0..3) and the 16-byte header.
//  Q6_K: half h = s/4, quarter t = s%4, weights l = 8p .. 8p+7 of the
//        quarter: low bits in ql byte 64h + 32(t%2) + l (low nibble for
//        t < 2), high bits 2t..2t+1 of qh byte 32h + l, scale 8h + 2t +
//        (p >= 2).  A lane loads 8 bytes at 64h + 32u + 8p (h, u = 0..1), 8
//        bytes at 128 + 32h + 8p, the 16 scales and d.
struct SkQ4 {
  uint4 hdr;
  uint2 q[4];          // quant bytes 32c + 8p .. +7, c = 0..3
};
struct SkQ6 {
  uint2 ql[4];         // index 2h + u
  uint2 qh[2];         // index h
  uint4 sc;            // 16 int8 scales
  uint32_t s206;       // halfwords 206, 208: d in the high half
};
template <int FMT> struct SkPart { typedef SkQ4 T; };
template <> struct SkPart<1> { typedef SkQ6 T; };

__device__ __forceinline__ void sk_load(const uint8_t* blk, int p, SkQ4& r) {
  r.hdr = *(const uint4*)blk;
#pragma unroll
  for (int c = 0; c < 4; ++c) r.q[c] = *(const uint2*)(blk + 16 + 32 * c + 8 * p);
}
// Q6_K blocks are 210 bytes, so a field may start 2 mod 4: 2-byte-aligned
// loads, which the global memory path serves like aligned ones.
__device__ __forceinline__ void sk_load(const uint8_t* blk, int p, SkQ6& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.ql[i] = *(const u2_a2*)(blk + 64 * (i >> 1) + 32 * (i & 1) + 8 * p);
#pragma unroll
  for (int h = 0; h < 2; ++h) r.qh[h] = *(const u2_a2*)(blk + 128 + 32 * h + 8 * p);
  r.sc = *(const u4_a2*)(blk + 192);
  r.s206 = *(const u32_a2*)(blk + 206);
}

// k offset inside the super-block of the 8 weights of part p, MFMA step s
__device__ __forceinline__ int sk_kofs(int p, int s) { return 32 * s + 8 * p; }

__device__ __forceinline__ h2 sk_pack(float a, float b) {
  const f2 v = {a, b};
  return __builtin_convertvector(v, h2);
}

// Per-block scale fields of a lane, decoded once per block; the two scale
// values of an MFMA step come from them on the fly (few live registers).
//  Q4_K: the unpacked 6-bit scales and mins, d * 2^9 and dmin; step s is
//        sub-block s: d*sc_s*2^9 and -dmin*m_s.
//  Q6_K: d; step s uses int8 scale byte 2s + (p >= 2) of the 16 scales.
struct SkScales {
  Q4kScales q4;
  float d, dmin;
};
__device__ __forceinline__ SkScales sk_scales(const SkQ4& r, int p) {
  (void)p;
  SkScales o;
  o.q4 = unpack_q4k_scales(r.hdr.y, r.hdr.z, r.hdr.w);
  o.d = half_bits_to_float(r.hdr.x) * 512.0f;
  o.dmin = half_bits_to_float(r.hdr.x >> 16);
  return o;
}
__device__ __forceinline__ SkScales sk_scales(const SkQ6& r, int p) {
  (void)p;
  SkScales o;
  o.q4 = Q4kScales{0, 0, 0, 0};
  o.d = half_bits_to_float(r.s206 >> 16);
  o.dmin = 0.0f;
  return o;
}

// The 8 fp16 weights of MFMA step s (exact dequant, one rounding to fp32,
// RNE to fp16).
__device__ __forceinline__ h8 sk_frag(const SkQ4& r, const SkScales& sc, int s, int p) {
  (void)p;
  const uint2 qv = r.q[s >> 1];
  const bool hi = s & 1;
  const float m = sc.d * (float)q4k_sc(sc.q4, s), c = -(sc.dmin * (float)q4k_m(sc.q4, s));
  const int b0 = (int)((hi ? qv.x >> 4 : qv.x) & 0x0f0f0f0fu);
  const int b1 = (int)((hi ? qv.y >> 4 : qv.y) & 0x0f0f0f0fu);
  const f2 q0 = __builtin_amdgcn_cvt_pk_f32_fp8(b0, false), q1 = __builtin_amdgcn_cvt_pk_f32_fp8(b0, true);
  const f2 q2 = __builtin_amdgcn_cvt_pk_f32_fp8(b1, false), q3 = __builtin_amdgcn_cvt_pk_f32_fp8(b1, true);
  const h2 w01 = sk_pack(__builtin_fmaf(q0.x, m, c), __builtin_fmaf(q0.y, m, c));
  const h2 w23 = sk_pack(__builtin_fmaf(q1.x, m, c), __builtin_fmaf(q1.y, m, c));
  const h2 w45 = sk_pack(__builtin_fmaf(q2.x, m, c), __builtin_fmaf(q2.y, m, c));
  const h2 w67 = sk_pack(__builtin_fmaf(q3.x, m, c), __builtin_fmaf(q3.y, m, c));
  return (h8){w01.x, w01.y, w23.x, w23.y, w45.x, w45.y, w67.x, w67.y};
}
__device__ __forceinline__ h8 sk_frag(const SkQ6& r, const SkScales& sc, int s, int p) {
  const int h = s >> 2, t = s & 3;
  const uint2 l = r.ql[2 * h + (t & 1)];
  const uint2 hb = r.qh[h];
  const uint32_t nsh = t >= 2 ? 4u : 0u;
  // scale index 8h + 2t + (p >= 2) = byte 2s + (p >= 2) of the 16 scales
  const uint32_t sw = s < 2 ? r.sc.x : s < 4 ? r.sc.y : s < 6 ? r.sc.z : r.sc.w;
  const int scb = (int)(int8_t)((sw >> (16 * (s & 1) + (p >= 2 ? 8 : 0))) & 0xffu);
  const float dsc = sc.d * (float)scb, off = dsc * -32.0f;
  uint32_t q0 = ((l.x >> nsh) & 0x0f0f0f0fu) | (((hb.x >> (2 * t)) & 0x03030303u) << 4);
  uint32_t q1 = ((l.y >> nsh) & 0x0f0f0f0fu) | (((hb.y >> (2 * t)) & 0x03030303u) << 4);
  asm("" : "+v"(q0));   // keep v_cvt_f32_ubyteN on the packed bytes
  asm("" : "+v"(q1));
  const h2 w01 = sk_pack(__builtin_fmaf((float)(q0 & 0xffu), dsc, off), __builtin_fmaf((float)((q0 >> 8) & 0xffu), dsc, off));
  const h2 w23 = sk_pack(__builtin_fmaf((float)((q0 >> 16) & 0xffu), dsc, off), __builtin_fmaf((float)(q0 >> 24), dsc, off));
  const h2 w45 = sk_pack(__builtin_fmaf((float)(q1 & 0xffu), dsc, off), __builtin_fmaf((float)((q1 >> 8) & 0xffu), dsc, off));
  const h2 w67 = sk_pack(__builtin_fmaf((float)((q1 >> 16) & 0xffu), dsc, off), __builtin_fmaf((float)(q1 >> 24), dsc, off));
  return (h8){w01.x, w01.y, w23.x, w23.y, w45.x, w45.y, w67.x, w67.y};
}

__device__ __forceinline__ float sk_silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// One workgroup: 16 weight rows of one problem (SwiGLU: 8 gate rows and the
// matching 8 up rows); wave w takes super-blocks [w nb / nw, (w+1) nb / nw)
// of them, a block at a time.
// NT: 16-row groups of activation rows (M <= 16 NT).
template <int FMT, int NT>
__device__ __forceinline__ void skinny_tile(const SkinnyDesc& P, int wg_local, float* red) {
  typedef typename SkPart<FMT>::T Part;
  constexpr int BLOCK_BYTES = FMT == 0 ? Q4K_BYTES : Q6K_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rl = lane & 15, p = lane >> 4;
  const int M = P.M, N = P.N, K = P.K;
  const int nb = K / QK;
  const int64_t row_bytes = (int64_t)nb * BLOCK_BYTES;
  // local row rl: row n0 + rl; SwiGLU: gate row n0 + rl%8 for rl < 8, the
  // up row F + n0 + rl%8 after it (ragged tails clamped, results dropped)
  const int F = N / 2;
  const int n0 = wg_local * (P.swiglu ? SKINNY_ROWS / 2 : SKINNY_ROWS);
  const int row = P.swiglu ? (n0 + (rl & 7) < F ? n0 + (rl & 7) : F - 1) + (rl >> 3) * F
                           : (n0 + rl < N ? n0 + rl : N - 1);
  const int nw = (int)(blockDim.x >> 6);                 // waves of the workgroup
  const int b0 = wave * nb / nw, b1 = (wave + 1) * nb / nw;
  const uint8_t* wrow = P.wq + (int64_t)row * row_bytes;

  f4 acc[NT];
#pragma unroll
  for (int g = 0; g < NT; ++g) acc[g] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
  // 8 MFMA steps of one block: the lane's dequantised weights (A) against
  // the 8 x values of activation row rl + 16 g at the step's k-slots (B)
  auto compute = [&](const Part& w, const uint4 (&xf)[NT][8]) {
    const SkScales sc = sk_scales(w, p);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const h8 a = sk_frag(w, sc, s, p);
#pragma unroll
      for (int g = 0; g < NT; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(h8, xf[g][s]), acc[g], 0, 0, 0);
    }
  };

  // block by block: the block's quant bytes into registers and its x (16 NT
  // rows x 512 bytes) into the wave's LDS slot with 8 NT direct-to-LDS
  // loads of 2 whole rows each; row r's 16-byte chunk c lands at slot
  // c ^ r, so the 8 lanes of one fragment read (rows r .. r+7 of one group,
  // one chunk) hit distinct banks.  Rows past M read as zero (the buffer's
  // range).
  uint8_t* const xsl = (uint8_t*)red + nw * NT * 1024 + wave * NT * 8192;
  const sk_rsrc_t xrs = sk_rsrc(P.x, (int64_t)M * K * 2);
  for (int b = b0; b < b1; ++b) {
    Part w;
    asm volatile("" ::: "memory");   // the slot's previous reads stay above
    sk_load(wrow + (int64_t)b * BLOCK_BYTES, p, w);
#pragma unroll
    for (int i = 0; i < 8 * NT; ++i) {
      const int r = 2 * i + (lane >> 5), j = lane & 31;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void*)(xsl + i * 1024), 16,
                                               (uint32_t)(r * K * 2 + b * 512 + 16 * (j ^ r)), 0, 0, 0);
    }
    // only this wave reads its slot: its own loads landing is enough
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint4 xf[NT][8];
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const int r = rl + 16 * g;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        xf[g][s] = *(const uint4*)(xsl + (r >> 1) * 1024 + (r & 1) * 512 + 16 * ((sk_kofs(p, s) / 8) ^ r));
    }
    compute(w, xf);
  }

  // D: lane l holds activation row l%16 and weight rows 4(l/16) .. +3 of
  // the tile.  LDS: red[wave][activation row m][weight row n], the four
  // 4-float chunks of row m permuted by chunk ^ red_swz(m) so that the
  // lanes' 16-byte stores (16 rows, one chunk each) and the 4-byte loads of
  // 64 consecutive outputs both hit distinct banks.
  const auto red_swz = [](int m) { return ((m >> 1) ^ (m >> 3)) & 3; };
#pragma unroll
  for (int g = 0; g < NT; ++g) ((f4*)red)[((wave * NT + g) * 16 + rl) * 4 + (p ^ red_swz(rl))] = acc[g];
  __syncthreads();
  // the waves' sums of local row nl for activation row m, in wave order
  auto total = [&](int m, int nl) {
    const int g = m >> 4, ml = m & 15;
    const int col = ((((nl >> 2) ^ red_swz(ml)) << 2) | (nl & 3));
    float v = red[(g * 16 + ml) * 16 + col];
    for (int w = 1; w < nw; ++w) v += red[((w * NT + g) * 16 + ml) * 16 + col];
    return v;
  };
  // output t = (activation row m, weight row n) of the 16 x 16 tile:
  // consecutive t write consecutive n.  A workgroup may have fewer than 256
  // threads (one wave per block).  SwiGLU: h[m][n0 + j] = silu(g) * u from
  // local rows j and j + 8, rounded once to fp16.
  if (P.swiglu) {
    for (int t = (int)threadIdx.x; t < 128 * NT; t += (int)blockDim.x) {
      const int m = t >> 3, j = t & 7;
      if (m < M && n0 + j < F)
        ((half_t*)P.out)[(int64_t)m * F + n0 + j] = (half_t)(sk_silu(total(m, j)) * total(m, j + 8));
    }
  } else {
    for (int t = (int)threadIdx.x; t < 256 * NT; t += (int)blockDim.x) {
      const int m = t >> 4, nl = t & 15, n = n0 + nl;
      if (m < M && n < N) ((float*)P.out)[(int64_t)m * N + n] = total(m, nl);
    }
  }
}

// Up to 16 waves; the dynamic LDS holds, per wave, NT 16 x 16 partial sums
// (NT KB) and then an 8 NT KB x slot.
template <int NT>
__global__ __launch_bounds__(1024) void skinny_kernel(SkinnyArgs args) {
  extern __shared__ __align__(16) float red[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < SKINNY_MAX_GROUP; ++i)
    if (i < args.count && (int)blockIdx.x >= args.d[i].wg_begin) pi = i;
  const SkinnyDesc& P = args.d[pi];
  const int wg_local = (int)blockIdx.x - P.wg_begin;
  if (P.fmt == 0)
    skinny_tile<0, NT>(P, wg_local, red);
  else
    skinny_tile<1, NT>(P, wg_local, red);
}

// One workgroup per 16 weight rows, one wave per super-block of the deepest
// row (at most 16); problems with the most bytes per workgroup (the deepest
// K) are dispatched first so they do not trail.
hipError_t launch_skinny(const GemmProblem* probs, int count, hipStream_t s) {
  for (int base = 0; base < count; base += SKINNY_MAX_GROUP) {
    const int n = count - base < SKINNY_MAX_GROUP ? count - base : SKINNY_MAX_GROUP;
    int order[SKINNY_MAX_GROUP];
    int mmax = 0, nbmax = 0;
    for (int i = 0; i < n; ++i) {
      order[i] = base + i;
      mmax = probs[base + i].M > mmax ? probs[base + i].M : mmax;
      nbmax = probs[base + i].K / QK > nbmax ? probs[base + i].K / QK : nbmax;
    }
    auto wg_bytes = [&](int i) { return (int64_t)(probs[i].K / QK) * (probs[i].fmt == 0 ? Q4K_BYTES : Q6K_BYTES); };
    for (int i = 1; i < n; ++i)
      for (int j = i; j > 0 && wg_bytes(order[j]) > wg_bytes(order[j - 1]); --j) std::swap(order[j], order[j - 1]);
    SkinnyArgs a{};
    int wgs = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = probs[order[i]];
      SkinnyDesc& d = a.d[i];
      d.x = (const half_t*)p.x;
      d.wq = p.wq;
      d.out = p.out;
      d.fmt = p.fmt;
      d.swiglu = p.swiglu;
      d.M = p.M;
      d.N = p.N;
      d.K = p.K;
      d.wg_begin = wgs;
      wgs += p.swiglu ? (p.N / 2 + SKINNY_ROWS / 2 - 1) / (SKINNY_ROWS / 2) : (p.N + SKINNY_ROWS - 1) / SKINNY_ROWS;
    }
    a.count = n;
    if (mmax > 32) return hipErrorInvalidValue;   // the caller routes larger M to the tiled kernel
    // A grid of at least two workgroups per CU keeps every CU busy with
    // several small workgroups (4 waves, 36 KB of LDS: four per CU).  A
    // smaller grid (one projection) takes one wave per block up to 16, so
    // that all its loads are issued before the first multiply; deeper rows
    // 16 waves, each walking its slice (up to 144 KB of LDS).
    const int nt = mmax > 16 ? 2 : 1;   // 16-row groups of activation rows
    const size_t wave_lds = (size_t)nt * (256 * sizeof(float) + 8192);   // partial sums + x slot
    const int wmax = SKINNY_MAX_WAVES / nt;                            // at most 144 KB
    const int waves = wgs >= 2 * device_cu_count() ? 4 : (nbmax < wmax ? nbmax : wmax);
    if (nt == 1)
      hipLaunchKernelGGL(skinny_kernel<1>, dim3(wgs), dim3(64 * waves), waves * wave_lds, s, a);
    else
      hipLaunchKernelGGL(skinny_kernel<2>, dim3(wgs), dim3(64 * waves), waves * wave_lds, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dmq
