// Stand-alone dequantisation kernels: Q4_K / Q6_K blocks -> fp16, bit-exact
// to the exact value rounded once (the dequantizers of article "Building
// DAMASCUS", section "Read the model, then reproduce its operations";
// compartment 09 of the overview page's pipeline).
//
// HBM-bound: each block is read once (144 / 210 B) and written once (512 B).
// 32 lanes per block, 8 weights per lane, one 16-byte store per lane, so a
// wave writes two whole blocks (1 KiB) with fully coalesced stores.
#include "dmq_common.h"

namespace dmq {

// RNE-to-fp16 of (a - b) for fp32 a, b that are exact products, with a
// single rounding.  s = fl32(a - b) alone would round twice (to fp32, then
// to fp16), which differs from one rounding when s lands on an fp16 tie.
// The exact error e of the fp32 subtraction comes from TwoSum (Knuth); s is
// then replaced by its round-to-odd version (truncate toward zero, set the
// last bit when inexact).  Rounding a round-to-odd value with >= 2 extra bits
// to a narrower format equals rounding the exact value directly (Boldo &
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", IEEE Trans. Computers 57(4), 2008).  fp32 has 24
// bits, fp16 11, so the condition holds.  Adding +0 maps an exact -0 to +0.
__device__ __forceinline__ half_t round_once_sub(float a, float b) {
  float c = -b;
  float s = a + c;
  float bb = s - a;
  float e = (a - (s - bb)) + (c - bb);
  uint32_t u = __float_as_uint(s);
  bool fix = (e != 0.0f) && (__builtin_isfinite(s));
  bool toward_zero = (__float_as_uint(e) ^ u) >> 31;  // e and s differ in sign
  uint32_t uo = (u - (toward_zero ? 1u : 0u)) | 1u;
  float r = __uint_as_float(fix ? uo : u);
  return (half_t)(r + 0.0f);
}

__device__ __forceinline__ uint32_t pack_h2(half_t a, half_t b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__global__ __launch_bounds__(256) void dequant_q4k_kernel(const uint8_t* __restrict__ wq,
                                                          half_t* __restrict__ out, int64_t nblocks) {
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 5);
  const int t = (int)(threadIdx.x & 31);   // this lane's weights: 8t .. 8t+7
  const int j = t >> 2;                    // sub-block
  const int l0 = (t & 3) * 8;              // first weight within the sub-block
  const uint32_t shift = (j & 1) ? 4u : 0u;
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 5) + (threadIdx.x >> 5); b < nblocks; b += stride) {
    const uint8_t* blk = wq + b * Q4K_BYTES;
    uint4 hdr = *(const uint4*)blk;        // d | dmin, scale bytes 0..3, 4..7, 8..11
    uint2 qv = *(const uint2*)(blk + 16 + 32 * (j >> 1) + l0);
    Q4kScales sc = unpack_q4k_scales(hdr.y, hdr.z, hdr.w);
    float d = half_bits_to_float(hdr.x);
    float dmin = half_bits_to_float(hdr.x >> 16);
    float dsc = d * (float)q4k_sc(sc, j);  // exact: 11 + 6 bits
    float dmm = dmin * (float)q4k_m(sc, j);
    half_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t word = i < 4 ? qv.x : qv.y;
      uint32_t q = (word >> (8 * (i & 3) + shift)) & 15u;
      float a = (float)q * dsc;            // exact: <= 21 bits
      w[i] = round_once_sub(a, dmm);
    }
    *(uint4*)(out + b * QK + 8 * t) =
        make_uint4(pack_h2(w[0], w[1]), pack_h2(w[2], w[3]), pack_h2(w[4], w[5]), pack_h2(w[6], w[7]));
  }
}

__global__ __launch_bounds__(256) void dequant_q6k_kernel(const uint8_t* __restrict__ wq,
                                                          half_t* __restrict__ out, int64_t nblocks) {
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 5);
  const int t = (int)(threadIdx.x & 31);   // weights i = 8t .. 8t+7
  const int h = t >> 4;                    // 128-weight half
  const int tq = (t >> 2) & 3;             // 32-weight quarter within the half
  const int l0 = (t & 3) * 8;
  const uint32_t lshift = tq < 2 ? 0u : 4u;
  const uint32_t hshift = 2u * (uint32_t)tq;
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 5) + (threadIdx.x >> 5); b < nblocks; b += stride) {
    const uint8_t* blk = wq + b * Q6K_BYTES;
    // Field offsets are multiples of 8 but the block may start 2 mod 4;
    // load_u64_a2 reads the enclosing dwords, at most 2 bytes before and 4
    // after each 8-byte field: ql fields end by byte 128, qh fields by 192,
    // so every read stays inside the block.
    uint2 lo = load_u64_a2(blk + 64 * h + 32 * (tq & 1) + l0);
    uint2 hi = load_u64_a2(blk + 128 + 32 * h + l0);
    int sc = (int)(int8_t)blk[192 + (t >> 1)];
    float d = half_bits_to_float(*(const uint16_t*)(blk + 208));
    float dsc = d * (float)sc;             // exact: 11 + 8 bits
    half_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t lw = i < 4 ? lo.x : lo.y;
      uint32_t hw = i < 4 ? hi.x : hi.y;
      uint32_t low = (lw >> (8 * (i & 3) + lshift)) & 15u;
      uint32_t high = (hw >> (8 * (i & 3) + hshift)) & 3u;
      int q = (int)(low | (high << 4)) - 32;
      float v = dsc * (float)q;            // exact: <= 23 bits
      w[i] = (half_t)(v + 0.0f);           // one rounding; -0 -> +0
    }
    *(uint4*)(out + b * QK + 8 * t) =
        make_uint4(pack_h2(w[0], w[1]), pack_h2(w[2], w[3]), pack_h2(w[4], w[5]), pack_h2(w[6], w[7]));
  }
}

hipError_t launch_dequant_q4k(const void* wq, void* w, int64_t rows, int64_t k, hipStream_t s) {
  int64_t nblocks = rows * (k / QK);
  int64_t wgs = (nblocks + 7) / 8;               // 8 blocks per 256-thread group
  dim3 grid((unsigned)(wgs < (1 << 20) ? wgs : (1 << 20)));
  hipLaunchKernelGGL(dequant_q4k_kernel, grid, dim3(256), 0, s, (const uint8_t*)wq, (half_t*)w, nblocks);
  return hipGetLastError();
}

hipError_t launch_dequant_q6k(const void* wq, void* w, int64_t rows, int64_t k, hipStream_t s) {
  int64_t nblocks = rows * (k / QK);
  int64_t wgs = (nblocks + 7) / 8;               // 8 blocks per 256-thread group
  dim3 grid((unsigned)(wgs < (1 << 20) ? wgs : (1 << 20)));
  hipLaunchKernelGGL(dequant_q6k_kernel, grid, dim3(256), 0, s, (const uint8_t*)wq, (half_t*)w, nblocks);
  return hipGetLastError();
}

}  // namespace dmq
