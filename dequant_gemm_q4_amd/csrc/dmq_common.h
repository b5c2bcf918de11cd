// Internal device helpers and launcher declarations of libdmq.so (gfx950).
//
// Block formats (GGUF k-quants; the DAMASCUS pages name Q4_K and Q6_K -- article
// "Building DAMASCUS", "Read the model, then reproduce its operations" -- but
// do not print their bytes):
//   Q4_K, 144 B / 256 weights: fp16 d @0, fp16 dmin @2, 12 B packed 6-bit
//         scales and mins @4, 128 B of 4-bit quants @16.  Sub-block j of 32
//         weights: w = d*sc_j*q - dmin*m_j; quant of weight 32j+l is the low
//         (j even) or high (j odd) nibble of quant byte 32*(j/2)+l.
//   Q6_K, 210 B / 256 weights: 128 B low nibbles @0, 64 B high 2-bit pairs
//         @128, 16 int8 scales @192, fp16 d @208.  Weight 128h+32t+l:
//         low 4 bits from byte 64h+32(t%2)+l (low nibble t<2, high t>=2),
//         high 2 bits = bits 2t..2t+1 of byte 128+32h+l, w = d*sc[i/16]*(q-32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmq {

constexpr int QK = 256;
constexpr int Q4K_BYTES = 144;
constexpr int Q6K_BYTES = 210;

typedef _Float16 half_t;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp16 constant 0x6400 = 1024.0: OR-ing an integer v < 1024 into the low
// mantissa bits gives the fp16 value 1024 + v exactly.
constexpr uint32_t MAGIC_PAIR = 0x64006400u;
constexpr uint32_t MAGIC_BYTES = 0x64646464u;

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)(bits & 0xffffu));
}

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Bytes b0, b1 of `bytes` (each < 64) -> fp16 pair (1024 + b0, 1024 + b1).
// sel picks bytes {lo byte of half 0, lo byte of half 1}; the high byte of
// each half comes from MAGIC_BYTES.  v_perm_b32 byte selectors: 0..3 pick
// from the second operand, 4..7 from the first.
__device__ __forceinline__ uint32_t magic_pair_lo(uint32_t bytes) {
  // result bytes: [bytes.b0, 0x64, bytes.b1, 0x64]
  return __builtin_amdgcn_perm(MAGIC_BYTES, bytes, 0x04010400u);
}
__device__ __forceinline__ uint32_t magic_pair_hi(uint32_t bytes) {
  // result bytes: [bytes.b2, 0x64, bytes.b3, 0x64]
  return __builtin_amdgcn_perm(MAGIC_BYTES, bytes, 0x04030402u);
}

// Unpack the 12 packed scale bytes of a Q4_K block (as dwords s0 = bytes
// 4..7, s1 = 8..11, s2 = 12..15 of the block) into four dwords of 6-bit
// values, one per byte: sc[0..3], m[0..3], sc[4..7], m[4..7].
struct Q4kScales {
  uint32_t sc_lo, m_lo, sc_hi, m_hi;
};
__device__ __forceinline__ Q4kScales unpack_q4k_scales(uint32_t s0, uint32_t s1, uint32_t s2) {
  Q4kScales r;
  r.sc_lo = s0 & 0x3f3f3f3fu;
  r.m_lo = s1 & 0x3f3f3f3fu;
  r.sc_hi = (s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u);
  r.m_hi = ((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u);
  return r;
}

// Byte j (0..7) of the unpacked scales / mins.
__device__ __forceinline__ uint32_t q4k_sc(const Q4kScales& s, int j) {
  uint32_t w = j < 4 ? s.sc_lo : s.sc_hi;
  return (w >> (8 * (j & 3))) & 0xffu;
}
__device__ __forceinline__ uint32_t q4k_m(const Q4kScales& s, int j) {
  uint32_t w = j < 4 ? s.m_lo : s.m_hi;
  return (w >> (8 * (j & 3))) & 0xffu;
}

// Little-endian dword loads from a 2-byte aligned address (Q6_K blocks are
// 210 bytes, so every other block starts 2 mod 4).  Reads the enclosing
// aligned dwords and shifts; the caller guarantees those dwords lie inside
// the block (the field plus up to 2 bytes on each side).
__device__ __forceinline__ uint2 load_u64_a2(const uint8_t* p) {
  uintptr_t a = (uintptr_t)p;
  const uint32_t* q = (const uint32_t*)(a & ~(uintptr_t)3);
  uint32_t sh = (uint32_t)(a & 3);
  uint32_t w0 = q[0], w1 = q[1], w2 = q[2];
  return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh));
}

__device__ __forceinline__ uint4 load_u128_a2(const uint8_t* p) {
  uintptr_t a = (uintptr_t)p;
  const uint32_t* q = (const uint32_t*)(a & ~(uintptr_t)3);
  uint32_t sh = (uint32_t)(a & 3);
  uint4 lo = *(const uint4*)q;
  uint32_t w4 = q[4];
  return make_uint4(__builtin_amdgcn_alignbyte(lo.y, lo.x, sh), __builtin_amdgcn_alignbyte(lo.z, lo.y, sh),
                    __builtin_amdgcn_alignbyte(lo.w, lo.z, sh), __builtin_amdgcn_alignbyte(w4, lo.w, sh));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------- RMSNorm ---
// RMSNorm (the layer description on the article page: one before the QKV
// projections, one before the feed-forward network): x * g / sqrt(mean(x^2)
// + eps) per row, in fp32, the result rounded once to fp16 for the MFMA / dot
// operands.

// Sum of squares of 8 fp16 values (one 16-byte chunk), pairwise.
__device__ __forceinline__ float sumsq8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 h = as_h2(w[i]);
    const float a = (float)h.x, b = (float)h.y;
    p[i] = a * a + b * b;
  }
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// 1 / sqrt(mean(x^2) + eps) of one row of K fp16 values, computed by a whole
// 256-thread workgroup (chunk i = thread + 256 j); red4 is 4 floats of LDS.
// Every thread of the workgroup must call it (it has a barrier); all get the
// same value.
__device__ __forceinline__ float rms_inv(const half_t* row, int K, float eps, float* red4) {
  const uint4* xr = (const uint4*)row;
  float ss = 0.0f;
  for (int i = (int)threadIdx.x; i < K / 8; i += 256) ss += sumsq8(xr[i]);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float t = (red4[0] + red4[1]) + (red4[2] + red4[3]);
  return 1.0f / __builtin_sqrtf(t / (float)K + eps);
}

// 8 fp16 values -> fp16(x * g * r), g: the 8 matching weights.
__device__ __forceinline__ uint4 norm8(uint4 v, const float* g, float r) {
  const float4 g0 = ((const float4*)g)[0], g1 = ((const float4*)g)[1];
  const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 h = as_h2(w[i]);
    const h2 o = {(half_t)(((float)h.x * gv[2 * i]) * r), (half_t)(((float)h.y * gv[2 * i + 1]) * r)};
    w[i] = as_u32(o);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------ launchers ---
// All launchers assume arguments were validated on the host (dmq_api.cpp).

hipError_t launch_dequant_q4k(const void* wq, void* w, int64_t rows, int64_t k, hipStream_t s);
hipError_t launch_dequant_q6k(const void* wq, void* w, int64_t rows, int64_t k, hipStream_t s);
// xn[m] = fp16(x[m] * g / sqrt(mean(x[m]^2) + eps)) for each of the M rows.
hipError_t launch_rmsnorm(const void* x, const float* g, float eps, void* xn, int64_t M, int64_t K, hipStream_t s);

// One GEMM problem as the kernels see it.
struct GemmProblem {
  const void* x;      // [M, K] fp16
  const uint8_t* wq;  // N rows of K/256 blocks
  void* out;          // y [M, N] fp32, or h [M, N/2] fp16 in SwiGLU mode
  int32_t fmt;        // 0 = Q4_K, 1 = Q6_K
  int32_t swiglu;     // 1: rows [0,N/2) are gate, [N/2,N) up; out = h
  int32_t M, N, K;
  const float* g;     // decode kernel only: RMSNorm x with weights g (K floats) ...
  float eps;          // ... and this eps while staging it; NULL g: no norm
  void* xn;           // decode kernel, with g: if set, the normalized x (K fp16) is written here
};

// Decode kernel: y[m][n] = sum_k x[m][k] w[n][k] for every problem, M = 1,
// or M = 2 where gemv_rows_fit (then without the RMSNorm and residual
// modes).
constexpr int GEMV_MAX_ROWS = 2;
bool gemv_rows_fit(int64_t m, int64_t kmax);
hipError_t launch_gemv(const GemmProblem* probs, int count, hipStream_t s);
// MFMA kernel (M >= 2).
hipError_t launch_gemm(const GemmProblem* probs, int count, hipStream_t s);
// Small-M MFMA kernel (M <= 32): the decode kernel's work split with the
// rows' multiply-adds on v_mfma_f32_16x16x32_f16.
hipError_t launch_skinny(const GemmProblem* probs, int count, hipStream_t s);

int device_cu_count();

// Device workspace of one use, per (device, stream), kept by the library
// (workspace.cpp): grown with stream-ordered allocations, never freed.
enum class WorkspaceUse { SplitK = 0, AttentionPieces = 1 };
hipError_t stream_workspace(WorkspaceUse use, hipStream_t s, size_t bytes, void** out);

}  // namespace dmq
