// C ABI of libdmq.so: host-side argument checks, dispatch by M, status text.
// Declarations and the contract of every call are in include/dmq.h.
//
// All checks run before the first HIP call, so a rejected call touches no
// device state (and the checks can be exercised on a machine without a GPU).
#include "../../include/dmq.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <string_view>

#include "attention.h"
#include "gemv.h"
#include "dmq_common.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Reduction length limit of the GEMM kernels: their buffer loads use 32-bit
// offsets within one tile (256 rows of x, 32 rows of blocks).
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int kMaxGroup = 64;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dim_ok(int64_t v) { return v >= 1 && v <= kMaxDim; }

// [p, p + pn) and [q, q + qn) share a byte
bool overlap(const void* p, int64_t pn, const void* q, int64_t qn) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qn && b < a + (uintptr_t)pn;
}

// A byte range a launch reads or writes (NULL: none).
struct Range {
  const void* p;
  int64_t n;
};

// True when one of the written ranges shares a byte with another written
// range or with a range the same launches read: kernels would race on it.
bool races(const Range* out, int nout, const Range* in, int nin) {
  for (int i = 0; i < nout; ++i) {
    if (!out[i].p) continue;
    for (int j = i + 1; j < nout; ++j)
      if (out[j].p && overlap(out[i].p, out[i].n, out[j].p, out[j].n)) return true;
    for (int j = 0; j < nin; ++j)
      if (in[j].p && overlap(out[i].p, out[i].n, in[j].p, in[j].n)) return true;
  }
  return false;
}

int64_t weight_bytes(int fmt, int64_t n, int64_t k) { return n * (k / 256) * (fmt == DMQ_FMT_Q4K ? 144 : 210); }

int check_quant_k(int64_t k) { return (dim_ok(k) && k % 256 == 0) ? DMQ_OK : DMQ_ERR_INVALID_ARG; }

int check_weights(int fmt, const void* wq) {
  if (!wq) return DMQ_ERR_INVALID_ARG;
  if (fmt == DMQ_FMT_Q4K) return aligned(wq, 16) ? DMQ_OK : DMQ_ERR_ALIGNMENT;
  if (fmt == DMQ_FMT_Q6K) return aligned(wq, 2) ? DMQ_OK : DMQ_ERR_ALIGNMENT;
  return DMQ_ERR_INVALID_ARG;
}

// Byte size of N rows of K-wide quantised weights (for overflow checks).
bool weight_bytes_ok(int fmt, int64_t n, int64_t k) {
  int64_t per_block = fmt == DMQ_FMT_Q4K ? 144 : 210;
  int64_t blocks = n * (k / 256);                 // n, k < 2^31: no overflow in int64
  return blocks <= (int64_t(1) << 40) / per_block;
}

int check_gemm(int fmt, const void* x, const void* wq, const void* y, int64_t M, int64_t N, int64_t K) {
  if (!x || !y) return DMQ_ERR_INVALID_ARG;
  if (!dim_ok(M) || !dim_ok(N)) return DMQ_ERR_INVALID_ARG;
  if (check_quant_k(K) != DMQ_OK || K > kMaxK) return DMQ_ERR_INVALID_ARG;
  int w = check_weights(fmt, wq);
  if (w != DMQ_OK) return w;
  if (!weight_bytes_ok(fmt, N, K)) return DMQ_ERR_INVALID_ARG;
  if (M * K > (int64_t(1) << 40) || M * N > (int64_t(1) << 40)) return DMQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16)) return DMQ_ERR_ALIGNMENT;
  return DMQ_OK;
}

// Device check: the kernels are built for gfx950 only.  Cached per device,
// together with the compute-unit count used to size launches.
std::mutex g_dev_mu;
int g_dev_status[64];
int g_dev_cus[64];
bool g_dev_init = false;

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DMQ_ERR_UNSUPPORTED;
  if (dev < 0 || dev >= 64) return DMQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_dev_init) {
    for (int& c : g_dev_status) c = 1;   // 1 = not queried yet
    g_dev_init = true;
  }
  if (g_dev_status[dev] == 1) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DMQ_ERR_UNSUPPORTED;
    g_dev_status[dev] = (prop.gcnArchName[0] && std::string_view(prop.gcnArchName).substr(0, 6) == "gfx950")
                            ? DMQ_OK : DMQ_ERR_UNSUPPORTED;
    g_dev_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  }
  return g_dev_status[dev];
}

int hip_status(hipError_t e) { return e == hipSuccess ? DMQ_OK : DMQ_ERR_HIP; }

// The decode kernel stages x in LDS; it takes K up to this size.
constexpr int64_t kGemvMaxK = 32768;

// The small-M kernel takes M <= 16 always (one 16-row MFMA column group).
// At M = 17 .. 32 (two groups) it takes launches with a SwiGLU gate|up pair
// and launches of fewer than two of its workgroups per CU: the FFN 3072 ->
// 8192 -> 3072 runs in 36 us there against 49-50 us on the tiled kernel,
// while one layer's seven projections (1,728 workgroups) run faster tiled
// (37.5-38.3 against 40.9-41.4 us).
constexpr int kSkinnyMaxM = 16;
constexpr int kSkinnyWideMaxM = 32;

int run_gemm(const dmq::GemmProblem* probs, int count, bool decode, hipStream_t s) {
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  if (decode) return hip_status(dmq::launch_gemv(probs, count, s));
  int64_t mmax = 0, wgs = 0;   // wgs: the small-M kernel's workgroups (16 weight rows each)
  bool swiglu = false;
  for (int i = 0; i < count; ++i) {
    mmax = probs[i].M > mmax ? probs[i].M : mmax;
    swiglu = swiglu || probs[i].swiglu;
    wgs += (probs[i].N + 15) / 16;
  }
  // 2 rows: the decode kernel with both rows' x staged (it shares each
  // weight's conversion between the rows), where that x fits in LDS; one
  // layer's seven projections take 19.5 us there against 26.0 on the
  // small-M kernel, the FFN 3072 -> 8192 -> 3072 23.0 against 25.0
  int64_t kmax = 0;
  for (int i = 0; i < count; ++i) kmax = probs[i].K > kmax ? probs[i].K : kmax;
  if (mmax >= 2 && mmax <= dmq::GEMV_MAX_ROWS && dmq::gemv_rows_fit(mmax, kmax))
    return hip_status(dmq::launch_gemv(probs, count, s));
  const bool skinny = mmax <= kSkinnyMaxM ||
                      (mmax <= kSkinnyWideMaxM && (swiglu || wgs < 2 * (int64_t)dmq::device_cu_count()));
  return hip_status(skinny ? dmq::launch_skinny(probs, count, s) : dmq::launch_gemm(probs, count, s));
}

dmq::GemmProblem make_problem(int fmt, const void* x, const void* wq, void* out, int64_t M, int64_t N, int64_t K,
                              int swiglu) {
  dmq::GemmProblem p;
  p.x = x;
  p.wq = (const uint8_t*)wq;
  p.out = out;
  p.fmt = fmt;
  p.swiglu = swiglu;
  p.M = (int32_t)M;
  p.N = (int32_t)N;
  p.K = (int32_t)K;
  p.g = nullptr;
  p.eps = 0.0f;
  p.xn = nullptr;
  return p;
}

int gemm_one(int fmt, const void* x, const void* wq, float* y, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_gemm(fmt, x, wq, y, M, N, K);
  if (st != DMQ_OK) return st;
  const Range out[1] = {{y, M * N * 4}}, in[2] = {{x, M * K * 2}, {wq, weight_bytes(fmt, N, K)}};
  if (races(out, 1, in, 2)) return DMQ_ERR_INVALID_ARG;
  dmq::GemmProblem p = make_problem(fmt, x, wq, y, M, N, K, 0);
  bool decode = (M == 1 && K <= kGemvMaxK);
  return run_gemm(&p, 1, decode, (hipStream_t)stream);
}

}  // namespace

namespace dmq {
// Compute units of the current device (valid after check_device succeeded).
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  return g_dev_init && g_dev_cus[dev] > 0 ? g_dev_cus[dev] : 256;
}
}  // namespace dmq

extern "C" {

int dmq_version(void) { return 1; }

const char* dmq_status_string(int status) {
  switch (status) {
    case DMQ_OK: return "ok";
    case DMQ_ERR_INVALID_ARG: return "invalid argument (null pointer, size out of range, K not a multiple of 256, or bad format)";
    case DMQ_ERR_ALIGNMENT: return "misaligned pointer (x, y, h, w_f16 and Q4_K weights need 16 bytes, Q6_K weights 2)";
    case DMQ_ERR_UNSUPPORTED: return "unsupported device (needs a gfx950 GPU)";
    case DMQ_ERR_HIP: return "HIP runtime error on launch";
    case DMQ_ERR_SCRATCH: return "the call needs more than the fixed no-allocation scratch (DMQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int dmq_dequant_q4k(const void* wq, void* w_f16, int64_t rows, int64_t k, void* stream) {
  if (!w_f16 || !dim_ok(rows) || check_quant_k(k) != DMQ_OK) return DMQ_ERR_INVALID_ARG;
  int w = check_weights(DMQ_FMT_Q4K, wq);
  if (w != DMQ_OK) return w;
  if (!weight_bytes_ok(DMQ_FMT_Q4K, rows, k)) return DMQ_ERR_INVALID_ARG;
  if (!aligned(w_f16, 16)) return DMQ_ERR_ALIGNMENT;
  if (overlap(w_f16, rows * k * 2, wq, weight_bytes(DMQ_FMT_Q4K, rows, k))) return DMQ_ERR_INVALID_ARG;
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  return hip_status(dmq::launch_dequant_q4k(wq, w_f16, rows, k, (hipStream_t)stream));
}

int dmq_dequant_q6k(const void* wq, void* w_f16, int64_t rows, int64_t k, void* stream) {
  if (!w_f16 || !dim_ok(rows) || check_quant_k(k) != DMQ_OK) return DMQ_ERR_INVALID_ARG;
  int w = check_weights(DMQ_FMT_Q6K, wq);
  if (w != DMQ_OK) return w;
  if (!weight_bytes_ok(DMQ_FMT_Q6K, rows, k)) return DMQ_ERR_INVALID_ARG;
  if (!aligned(w_f16, 16)) return DMQ_ERR_ALIGNMENT;
  if (overlap(w_f16, rows * k * 2, wq, weight_bytes(DMQ_FMT_Q6K, rows, k))) return DMQ_ERR_INVALID_ARG;
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  return hip_status(dmq::launch_dequant_q6k(wq, w_f16, rows, k, (hipStream_t)stream));
}

int dmq_gemm_q4k(const void* x_f16, const void* wq, float* y, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_one(DMQ_FMT_Q4K, x_f16, wq, y, M, N, K, stream);
}

int dmq_gemm_q6k(const void* x_f16, const void* wq, float* y, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_one(DMQ_FMT_Q6K, x_f16, wq, y, M, N, K, stream);
}

int dmq_ffn_swiglu_q4k(const void* x_f16, const void* w_gate_up_q4k, const void* w_down_q6k, void* h_f16, float* y,
                       int64_t M, int64_t D, int64_t F, void* stream) {
  if (!h_f16 || !dim_ok(F) || F > kMaxDim / 2) return DMQ_ERR_INVALID_ARG;
  int st = check_gemm(DMQ_FMT_Q4K, x_f16, w_gate_up_q4k, h_f16, M, 2 * F, D);
  if (st != DMQ_OK) return st;
  st = check_gemm(DMQ_FMT_Q6K, h_f16, w_down_q6k, y, M, D, F);
  if (st != DMQ_OK) return st;
  const Range out[2] = {{h_f16, M * F * 2}, {y, M * D * 4}};
  const Range in[3] = {{x_f16, M * D * 2}, {w_gate_up_q4k, weight_bytes(DMQ_FMT_Q4K, 2 * F, D)},
                       {w_down_q6k, weight_bytes(DMQ_FMT_Q6K, D, F)}};
  if (races(out, 2, in, 3)) return DMQ_ERR_INVALID_ARG;
  bool decode = (M == 1 && D <= kGemvMaxK && F <= kGemvMaxK);
  dmq::GemmProblem up = make_problem(DMQ_FMT_Q4K, x_f16, w_gate_up_q4k, h_f16, M, 2 * F, D, 1);
  st = run_gemm(&up, 1, decode, (hipStream_t)stream);
  if (st != DMQ_OK) return st;
  dmq::GemmProblem down = make_problem(DMQ_FMT_Q6K, h_f16, w_down_q6k, y, M, D, F, 0);
  return run_gemm(&down, 1, decode, (hipStream_t)stream);
}

int dmq_gemm_group(const dmq_gemm_desc* descs, int32_t count, void* stream) {
  if (!descs || count < 1 || count > kMaxGroup) return DMQ_ERR_INVALID_ARG;
  dmq::GemmProblem probs[kMaxGroup];
  int n_decode = 0;
  for (int i = 0; i < count; ++i) {
    const dmq_gemm_desc& d = descs[i];
    if (d.reserved != 0 || (d.format != DMQ_FMT_Q4K && d.format != DMQ_FMT_Q6K)) return DMQ_ERR_INVALID_ARG;
    int st = check_gemm(d.format, d.x_f16, d.wq, d.y, d.M, d.N, d.K);
    if (st != DMQ_OK) return st;
    if (d.M == 1 && d.K <= kGemvMaxK) ++n_decode;
    probs[i] = make_problem(d.format, d.x_f16, d.wq, d.y, d.M, d.N, d.K, 0);
  }
  if (n_decode != 0 && n_decode != count) return DMQ_ERR_INVALID_ARG;   // one kernel kind per call
  {
    Range out[kMaxGroup], in[2 * kMaxGroup];
    for (int i = 0; i < count; ++i) {
      const dmq_gemm_desc& d = descs[i];
      out[i] = Range{d.y, d.M * d.N * 4};
      in[2 * i] = Range{d.x_f16, d.M * d.K * 2};
      in[2 * i + 1] = Range{d.wq, weight_bytes(d.format, d.N, d.K)};
    }
    if (races(out, count, in, 2 * count)) return DMQ_ERR_INVALID_ARG;
  }
  // Longest reduction first: tiles of the deepest K are dispatched first so
  // they do not trail at the end of the launch.
  std::stable_sort(probs, probs + count,
                   [](const dmq::GemmProblem& a, const dmq::GemmProblem& b) { return a.K > b.K; });
  return run_gemm(probs, count, n_decode == count, (hipStream_t)stream);
}

namespace {

// The projections of dmq_rmsnorm_gemm / dmq_residual_rmsnorm_gemm as problems
// with activations x; with DMQ_PROJ_SWIGLU a Q4_K gate|up pair (N/2 a
// multiple of 256) whose output is h = silu(gate) * up in fp16 [M, N/2].
// No output may overlap another output or any of the `busy` ranges: in one
// launch some workgroups write an output while others still read its inputs.
int proj_problems(const dmq_proj_desc* projs, int32_t count, const void* x, int64_t M, int64_t K,
                  const Range* busy, int nbusy, dmq::GemmProblem* probs) {
  if (!projs || count < 1 || count > kMaxGroup) return DMQ_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    const dmq_proj_desc& d = projs[i];
    if ((d.flags & ~DMQ_PROJ_SWIGLU) != 0 || (d.format != DMQ_FMT_Q4K && d.format != DMQ_FMT_Q6K))
      return DMQ_ERR_INVALID_ARG;
    const int swiglu = (d.flags & DMQ_PROJ_SWIGLU) ? 1 : 0;
    if (swiglu && (d.format != DMQ_FMT_Q4K || d.N % 512 != 0)) return DMQ_ERR_INVALID_ARG;
    int st = check_gemm(d.format, x, d.wq, d.y, M, d.N, K);
    if (st != DMQ_OK) return st;
    probs[i] = make_problem(d.format, x, d.wq, d.y, M, d.N, K, swiglu);
  }
  auto out_bytes = [&](int i) { return projs[i].flags & DMQ_PROJ_SWIGLU ? M * (projs[i].N / 2) * 2 : M * projs[i].N * 4; };
  for (int i = 0; i < count; ++i) {
    for (int b = 0; b < nbusy; ++b)
      if (busy[b].p && overlap(projs[i].y, out_bytes(i), busy[b].p, busy[b].n)) return DMQ_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlap(projs[i].y, out_bytes(i), projs[j].y, out_bytes(j))) return DMQ_ERR_INVALID_ARG;
  }
  return DMQ_OK;
}

// Projections of one activation matrix: the decode kernel takes a mixed
// group; the MFMA kernels take SwiGLU pairs one per launch (the epilogue is
// the launch's), the plain projections together.
int run_projs(const dmq::GemmProblem* probs, int count, bool decode, hipStream_t s) {
  if (decode) return run_gemm(probs, count, true, s);
  dmq::GemmProblem plain[kMaxGroup];
  int np = 0;
  for (int i = 0; i < count; ++i)
    if (!probs[i].swiglu) plain[np++] = probs[i];
  if (np > 0) {
    int st = run_gemm(plain, np, false, s);
    if (st != DMQ_OK) return st;
  }
  for (int i = 0; i < count; ++i)
    if (probs[i].swiglu) {
      int st = run_gemm(&probs[i], 1, false, s);
      if (st != DMQ_OK) return st;
    }
  return DMQ_OK;
}

}  // namespace

int dmq_rmsnorm_gemm(const void* x_f16, const float* g, float eps, void* xn_f16, int64_t M, int64_t K,
                     const dmq_proj_desc* projs, int32_t count, void* stream) {
  if (!x_f16 || !g || !(eps >= 0.0f) || eps > 3.0e38f) return DMQ_ERR_INVALID_ARG;   // rejects NaN too
  if (!dim_ok(M) || check_quant_k(K) != DMQ_OK || K > kMaxK) return DMQ_ERR_INVALID_ARG;
  if (!aligned(x_f16, 16) || !aligned(g, 16)) return DMQ_ERR_ALIGNMENT;
  const bool decode = (M == 1 && K <= kGemvMaxK);
  if (!decode && !xn_f16) return DMQ_ERR_INVALID_ARG;
  if (xn_f16) {
    if (xn_f16 == x_f16) return DMQ_ERR_INVALID_ARG;
    if (!aligned(xn_f16, 16)) return DMQ_ERR_ALIGNMENT;
  }
  dmq::GemmProblem probs[kMaxGroup];
  const Range busy[3] = {{x_f16, M * K * 2}, {g, K * 4}, {xn_f16, M * K * 2}};
  int st = proj_problems(projs, count, decode ? x_f16 : xn_f16, M, K, busy, 3, probs);
  if (st != DMQ_OK) return st;
  if (decode) {
    for (int i = 0; i < count; ++i) {
      probs[i].g = g;
      probs[i].eps = eps;
      probs[i].xn = i == 0 ? xn_f16 : nullptr;
    }
  }
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  if (!decode) {
    st = hip_status(dmq::launch_rmsnorm(x_f16, g, eps, xn_f16, M, K, (hipStream_t)stream));
    if (st != DMQ_OK) return st;
  }
  return run_projs(probs, count, decode, (hipStream_t)stream);
}

int dmq_residual_rmsnorm_gemm(const float* h_in, const float* y_add, const float* g, float eps, float* h_out,
                              void* xn_f16, int64_t M, int64_t K, const dmq_proj_desc* projs, int32_t count,
                              void* stream) {
  if (!h_in || !y_add || !g || !h_out || !(eps >= 0.0f) || eps > 3.0e38f) return DMQ_ERR_INVALID_ARG;
  if (!dim_ok(M) || check_quant_k(K) != DMQ_OK || K > kMaxK || M * K > (int64_t(1) << 40))
    return DMQ_ERR_INVALID_ARG;
  if (!aligned(h_in, 16) || !aligned(y_add, 16) || !aligned(g, 16) || !aligned(h_out, 16)) return DMQ_ERR_ALIGNMENT;
  const int64_t hb = M * K * 4;
  if (overlap(h_out, hb, h_in, hb) || overlap(h_out, hb, y_add, hb) || overlap(h_out, hb, g, K * 4))
    return DMQ_ERR_INVALID_ARG;
  const bool decode = (M == 1 && K <= kGemvMaxK);
  if (!decode && !xn_f16) return DMQ_ERR_INVALID_ARG;
  if (xn_f16) {
    if (!aligned(xn_f16, 16)) return DMQ_ERR_ALIGNMENT;
    const int64_t xb = M * K * 2;
    if (overlap(xn_f16, xb, h_in, hb) || overlap(xn_f16, xb, y_add, hb) || overlap(xn_f16, xb, h_out, hb) ||
        overlap(xn_f16, xb, g, K * 4))
      return DMQ_ERR_INVALID_ARG;
  }
  dmq::GemmProblem probs[kMaxGroup];
  // decode: the kernel reads h_in and y_add, not x; h_in stands in for the
  // validation of the activation pointer
  const Range busy[5] = {{h_in, hb}, {y_add, hb}, {h_out, hb}, {g, K * 4}, {xn_f16, M * K * 2}};
  int st = proj_problems(projs, count, decode ? (const void*)h_in : xn_f16, M, K, busy, 5, probs);
  if (st != DMQ_OK) return st;
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  if (decode) {
    for (int i = 0; i < count; ++i) {
      probs[i].g = g;
      probs[i].eps = eps;
      probs[i].xn = i == 0 ? xn_f16 : nullptr;
    }
    return hip_status(dmq::launch_gemv_residual(probs, count, h_in, y_add, h_out, (hipStream_t)stream));
  }
  st = hip_status(dmq::launch_residual_rmsnorm(h_in, y_add, g, eps, h_out, xn_f16, M, K, (hipStream_t)stream));
  if (st != DMQ_OK) return st;
  return run_projs(probs, count, false, (hipStream_t)stream);
}

static bool heads_ok(int32_t hq, int32_t hkv) {
  return hq >= 1 && hkv >= 1 && hq <= 1024 && hq % hkv == 0 && hq / hkv <= 8;
}

// KV-cache geometry: [hkv, cache_len, 128] fp16, positions pos0 .. pos0+M-1 inside it.
static bool cache_ok(int64_t M, int64_t pos0, int32_t hkv, int64_t cache_len) {
  return dim_ok(M) && pos0 >= 0 && dim_ok(cache_len) && pos0 + M <= cache_len &&
         (int64_t)hkv * cache_len * 128 <= (int64_t(1) << 40) && M * 1024 * 128 <= (int64_t(1) << 40);
}

// The attention output sharing a byte with the queries or the caches it reads.
static bool attention_races(const void* q, const void* kc, const void* vc, const void* out, int64_t M, int32_t hq,
                            int32_t hkv, int64_t cache_len) {
  const int64_t qd = (int64_t)hq * 128, cb = (int64_t)hkv * 128 * cache_len * 2;
  const Range o[1] = {{out, M * qd * 2}}, in[3] = {{q, M * qd * 2}, {kc, cb}, {vc, cb}};
  return races(o, 1, in, 3);
}

int dmq_rope_kv_cache(const float* q, const float* k, const float* v, int64_t M, int64_t pos0, int32_t n_q_heads,
                      int32_t n_kv_heads, double theta, const float* freq_factors, void* q_f16, void* k_cache_f16,
                      void* v_cache_f16, int64_t cache_len, void* stream) {
  if (!q || !k || !v || !q_f16 || !k_cache_f16 || !v_cache_f16) return DMQ_ERR_INVALID_ARG;
  if (!heads_ok(n_q_heads, n_kv_heads) || !cache_ok(M, pos0, n_kv_heads, cache_len)) return DMQ_ERR_INVALID_ARG;
  if (!(theta > 1.0) || theta > 1e30) return DMQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q_f16, 16) || !aligned(k_cache_f16, 16) ||
      !aligned(v_cache_f16, 16) || (freq_factors && !aligned(freq_factors, 4)))
    return DMQ_ERR_ALIGNMENT;
  {
    const int64_t qd = (int64_t)n_q_heads * 128, kd = (int64_t)n_kv_heads * 128, cb = kd * cache_len * 2;
    const Range out[3] = {{q_f16, M * qd * 2}, {k_cache_f16, cb}, {v_cache_f16, cb}};
    const Range in[4] = {{q, M * qd * 4}, {k, M * kd * 4}, {v, M * kd * 4}, {freq_factors, 64 * 4}};
    if (races(out, 3, in, 4)) return DMQ_ERR_INVALID_ARG;
  }
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  return hip_status(dmq::launch_rope_kv(q, k, v, freq_factors, q_f16, k_cache_f16, v_cache_f16, theta, cache_len, M,
                                        pos0, n_q_heads, n_kv_heads, (hipStream_t)stream));
}

int dmq_attention_gqa(const void* q_f16, const void* k_cache_f16, const void* v_cache_f16, void* out_f16, int64_t M,
                      int64_t pos0, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_len, void* stream) {
  if (!q_f16 || !k_cache_f16 || !v_cache_f16 || !out_f16 || out_f16 == q_f16) return DMQ_ERR_INVALID_ARG;
  if (!heads_ok(n_q_heads, n_kv_heads) || !cache_ok(M, pos0, n_kv_heads, cache_len)) return DMQ_ERR_INVALID_ARG;
  if (!aligned(q_f16, 16) || !aligned(k_cache_f16, 16) || !aligned(v_cache_f16, 16) || !aligned(out_f16, 16))
    return DMQ_ERR_ALIGNMENT;
  if (attention_races(q_f16, k_cache_f16, v_cache_f16, out_f16, M, n_q_heads, n_kv_heads, cache_len))
    return DMQ_ERR_INVALID_ARG;
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  return hip_status(dmq::launch_attention(q_f16, k_cache_f16, v_cache_f16, out_f16, cache_len, M, pos0, n_q_heads,
                                          n_kv_heads, (hipStream_t)stream));
}

int dmq_rope_attention_gqa(const float* q, const float* k, const float* v, int64_t M, int64_t pos0,
                           int32_t n_q_heads, int32_t n_kv_heads, double theta, const float* freq_factors,
                           void* q_f16, void* k_cache_f16, void* v_cache_f16, int64_t cache_len, void* out_f16,
                           void* stream) {
  if (!q || !k || !v || !q_f16 || !k_cache_f16 || !v_cache_f16 || !out_f16) return DMQ_ERR_INVALID_ARG;
  if (!heads_ok(n_q_heads, n_kv_heads) || !cache_ok(M, pos0, n_kv_heads, cache_len)) return DMQ_ERR_INVALID_ARG;
  if (!(theta > 1.0) || theta > 1e30) return DMQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q_f16, 16) || !aligned(k_cache_f16, 16) ||
      !aligned(v_cache_f16, 16) || !aligned(out_f16, 16) || (freq_factors && !aligned(freq_factors, 4)))
    return DMQ_ERR_ALIGNMENT;
  {
    // written: the rotated queries, both caches (rows pos0 .. pos0+M-1) and
    // the output; read: the projections, the frequency factors, and (by the
    // attention) the rotated queries and the caches
    const int64_t qd = (int64_t)n_q_heads * 128, kd = (int64_t)n_kv_heads * 128, cb = kd * cache_len * 2;
    const Range out[4] = {{q_f16, M * qd * 2}, {k_cache_f16, cb}, {v_cache_f16, cb}, {out_f16, M * qd * 2}};
    const Range in[4] = {{q, M * qd * 4}, {k, M * kd * 4}, {v, M * kd * 4}, {freq_factors, 64 * 4}};
    if (races(out, 4, in, 4)) return DMQ_ERR_INVALID_ARG;
  }
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  return hip_status(dmq::launch_rope_attention(q, k, v, freq_factors, q_f16, k_cache_f16, v_cache_f16, out_f16, theta,
                                               cache_len, M, pos0, n_q_heads, n_kv_heads, (hipStream_t)stream));
}

int dmq_attention_gqa_noalloc(const void* q_f16, const void* k_cache_f16, const void* v_cache_f16, void* out_f16,
                              int64_t M, int64_t pos0, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_len,
                              void* stream) {
  if (!q_f16 || !k_cache_f16 || !v_cache_f16 || !out_f16 || out_f16 == q_f16) return DMQ_ERR_INVALID_ARG;
  if (!heads_ok(n_q_heads, n_kv_heads) || !cache_ok(M, pos0, n_kv_heads, cache_len)) return DMQ_ERR_INVALID_ARG;
  if (!aligned(q_f16, 16) || !aligned(k_cache_f16, 16) || !aligned(v_cache_f16, 16) || !aligned(out_f16, 16))
    return DMQ_ERR_ALIGNMENT;
  if (attention_races(q_f16, k_cache_f16, v_cache_f16, out_f16, M, n_q_heads, n_kv_heads, cache_len))
    return DMQ_ERR_INVALID_ARG;
  const size_t need = dmq::attention_scratch_bytes(M, pos0, n_q_heads);
  if (need > DMQ_NOALLOC_SCRATCH_BYTES) return DMQ_ERR_SCRATCH;
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  float* scratch = nullptr;
  size_t have = 0;
  if (need > 0) {
    if (dmq::noalloc_scratch(&scratch, &have) != hipSuccess) return DMQ_ERR_HIP;
    if (need > have) return DMQ_ERR_SCRATCH;
  }
  // the decode path uses the scratch; the other paths take no workspace at all
  return hip_status(dmq::launch_attention(q_f16, k_cache_f16, v_cache_f16, out_f16, cache_len, M, pos0, n_q_heads,
                                          n_kv_heads, (hipStream_t)stream, need > 0 ? scratch : nullptr));
}

int dmq_residual_rmsnorm(const float* h_in, const float* y, const float* g, float eps, float* h_out, void* xn_f16,
                         int64_t M, int64_t K, void* stream) {
  if (!h_in || !y || !h_out || (g && !xn_f16)) return DMQ_ERR_INVALID_ARG;
  if (g && (!(eps >= 0.0f) || eps > 3.0e38f)) return DMQ_ERR_INVALID_ARG;
  if (!dim_ok(M) || check_quant_k(K) != DMQ_OK || K > kMaxK || M * K > (int64_t(1) << 40)) return DMQ_ERR_INVALID_ARG;
  if (!aligned(h_in, 16) || !aligned(y, 16) || !aligned(h_out, 16) || (g && (!aligned(g, 16) || !aligned(xn_f16, 16))))
    return DMQ_ERR_ALIGNMENT;
  {
    // h_out may be h_in or y exactly (each element is read before it is
    // written, by the same thread), but not overlap them otherwise; xn and g
    // overlap nothing written
    const int64_t hb = M * K * 4;
    if ((h_out != h_in && overlap(h_out, hb, h_in, hb)) || (h_out != y && overlap(h_out, hb, y, hb)))
      return DMQ_ERR_INVALID_ARG;
    if (g) {
      const Range out[2] = {{h_out, hb}, {xn_f16, M * K * 2}};
      const Range in[3] = {{h_in, hb}, {y, hb}, {g, K * 4}};
      if (races(out + 1, 1, in, 3) || races(out, 2, in + 2, 1) || overlap(xn_f16, M * K * 2, h_out, hb))
        return DMQ_ERR_INVALID_ARG;
    }
  }
  int dc = check_device();
  if (dc != DMQ_OK) return dc;
  return hip_status(dmq::launch_residual_rmsnorm(h_in, y, g, eps, h_out, g ? xn_f16 : nullptr, M, K,
                                                 (hipStream_t)stream));
}

}  // extern "C"

namespace dmq {
// The requirements of every single call dmq_layer_prefill makes, checked for
// all M rows at once (each chunk's arguments are row ranges of these), and no
// written buffer overlapping another buffer, cache or weight array: run
// before the layer records an event or enqueues a kernel.
int check_layer(const dmq_layer_weights* w, const dmq_layer_buffers* b, int64_t M, int64_t pos0, int32_t D,
                int32_t F, int32_t hq, int32_t hkv, int64_t cache_len, double theta, float eps) {
  if (!w || !b) return DMQ_ERR_INVALID_ARG;
  if (!heads_ok(hq, hkv) || (int64_t)hq * 128 % 256 || !cache_ok(M, pos0, hkv, cache_len)) return DMQ_ERR_INVALID_ARG;
  if (!(theta > 1.0) || theta > 1e30 || !(eps >= 0.0f) || eps > 3.0e38f) return DMQ_ERR_INVALID_ARG;
  if (!dim_ok(D) || !dim_ok(F)) return DMQ_ERR_INVALID_ARG;
  const int64_t QD = (int64_t)hq * 128, KD = (int64_t)hkv * 128;
  int st;
  if ((st = check_gemm(w->fmt_q, b->xn_in, w->wq, b->yq, M, QD, D)) != DMQ_OK) return st;
  if ((st = check_gemm(w->fmt_k, b->xn_in, w->wk, b->yk, M, KD, D)) != DMQ_OK) return st;
  if ((st = check_gemm(w->fmt_v, b->xn_in, w->wv, b->yv, M, KD, D)) != DMQ_OK) return st;
  if ((st = check_gemm(w->fmt_o, b->attn, w->wo, b->yo, M, D, QD)) != DMQ_OK) return st;
  if ((st = check_gemm(DMQ_FMT_Q4K, b->xn_ffn, w->w_gate_up, b->h_ffn, M, 2 * (int64_t)F, D)) != DMQ_OK) return st;
  if ((st = check_gemm(DMQ_FMT_Q6K, b->h_ffn, w->w_down, b->y_down, M, D, F)) != DMQ_OK) return st;
  if (!b->h_in || !b->q_rot || !b->h_mid || !b->h_out || !w->g_ffn || !w->k_cache || !w->v_cache)
    return DMQ_ERR_INVALID_ARG;
  if (w->g_next && !b->xn_out) return DMQ_ERR_INVALID_ARG;
  if (!aligned(w->g_ffn, 16) || (w->g_next && !aligned(w->g_next, 16)) || !aligned(w->k_cache, 16) ||
      !aligned(w->v_cache, 16) || (w->freq_factors && !aligned(w->freq_factors, 4)))
    return DMQ_ERR_ALIGNMENT;
  auto wbytes = weight_bytes;
  const int64_t cache_bytes = (int64_t)hkv * cache_len * 128 * 2;
  const Range written[] = {{b->yq, M * QD * 4}, {b->yk, M * KD * 4}, {b->yv, M * KD * 4},
                           {b->q_rot, M * QD * 2}, {b->attn, M * QD * 2}, {b->yo, M * D * 4},
                           {b->h_mid, M * D * 4}, {b->xn_ffn, M * D * 2}, {b->h_ffn, M * (int64_t)F * 2},
                           {b->y_down, M * D * 4}, {b->h_out, M * D * 4}, {w->g_next ? b->xn_out : nullptr, M * D * 2},
                           {w->k_cache, cache_bytes}, {w->v_cache, cache_bytes}};
  const Range read[] = {{b->h_in, M * D * 4}, {b->xn_in, M * D * 2},
                        {w->wq, wbytes(w->fmt_q, QD, D)}, {w->wk, wbytes(w->fmt_k, KD, D)},
                        {w->wv, wbytes(w->fmt_v, KD, D)}, {w->wo, wbytes(w->fmt_o, D, QD)},
                        {w->w_gate_up, wbytes(DMQ_FMT_Q4K, 2 * (int64_t)F, D)}, {w->w_down, wbytes(DMQ_FMT_Q6K, D, F)},
                        {w->g_ffn, (int64_t)D * 4}, {w->g_next, (int64_t)D * 4}, {w->freq_factors, 64 * 4}};
  const int nw = (int)(sizeof(written) / sizeof(written[0])), nr = (int)(sizeof(read) / sizeof(read[0]));
  return races(written, nw, read, nr) ? DMQ_ERR_INVALID_ARG : DMQ_OK;
}
}  // namespace dmq
