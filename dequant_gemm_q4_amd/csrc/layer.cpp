// One decoder layer's prefill with the attention side and the feed-forward
// side running concurrently on two streams (dmq_layer_prefill).
//
// The overview page's "[03] zero-copy / unified memory" splits a layer's
// work between two engines that share one buffer (attention on the GPU, the
// FFN on the matrix coprocessor).  On one MI355X both sides are kernels of
// this library; what carries over is the overlap: the prompt is cut into
// row chunks, and while one stream runs chunk c+1's attention side (Q|K|V
// projections, RoPE and the cache append, attention, O projection, residual
// add and RMSNorm), a second stream runs chunk c's FFN (gate|up with the
// SwiGLU epilogue, down projection, residual add and the next RMSNorm) on the
// rows the first stream has finished.  Every buffer is shared device memory;
// the streams hand chunks over with events.  Chunk c+1's attention reads the
// cache rows of chunks <= c+1, which the attention stream wrote itself, so the
// only cross-stream dependencies are chunk hand-overs and the final join.
// With one stream for both sides the same kernels run in the same order per
// stream, which gives the same bits.
#include "../../include/dmq.h"
#include "layer.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

namespace {

// Events for stream hand-overs, created once per device and reused: an
// event may be re-recorded as soon as the waits on its earlier recording are
// enqueued (a wait takes the state the event had when it was enqueued).  The
// caller holds g_ev_mu for the whole call, so calls from several host
// threads do not interleave their recordings.
struct EventPool {
  std::vector<hipEvent_t> ev[64];
};
std::mutex g_ev_mu;
EventPool g_pool;

int events(int n, hipEvent_t* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DMQ_ERR_UNSUPPORTED;
  auto& v = g_pool.ev[dev];
  while ((int)v.size() < n) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return DMQ_ERR_HIP;
    v.push_back(e);
  }
  for (int i = 0; i < n; ++i) out[i] = v[i];
  return DMQ_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" int dmq_layer_prefill(const dmq_layer_weights* w, const dmq_layer_buffers* b, int64_t M, int64_t pos0,
                                 int32_t D, int32_t F, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_len,
                                 double theta, float eps, int64_t chunk, void* stream_attn, void* stream_ffn) {
  if (!w || !b || M < 1 || chunk < 1 || D < 256 || F < 256 || D % 256 || F % 256) return DMQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_kv_heads < 1 || (int64_t)n_q_heads * 128 % 256) return DMQ_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return DMQ_ERR_INVALID_ARG;
  if (!w->wq || !w->wk || !w->wv || !w->wo || !w->w_gate_up || !w->w_down || !w->g_ffn) return DMQ_ERR_INVALID_ARG;
  if (!w->k_cache || !w->v_cache) return DMQ_ERR_INVALID_ARG;
  for (int32_t f : {w->fmt_q, w->fmt_k, w->fmt_v, w->fmt_o})
    if (f != DMQ_FMT_Q4K && f != DMQ_FMT_Q6K) return DMQ_ERR_INVALID_ARG;
  if (!b->h_in || !b->xn_in || !b->yq || !b->yk || !b->yv || !b->q_rot || !b->attn || !b->yo || !b->h_mid ||
      !b->xn_ffn || !b->h_ffn || !b->y_down || !b->h_out)
    return DMQ_ERR_INVALID_ARG;
  if (w->g_next && !b->xn_out) return DMQ_ERR_INVALID_ARG;
  // row slices of every buffer stay 16-byte aligned
  const int64_t QD = (int64_t)n_q_heads * 128, KD = (int64_t)n_kv_heads * 128;
  if (!aligned16(b->h_in) || !aligned16(b->xn_in) || !aligned16(b->yq) || !aligned16(b->yk) || !aligned16(b->yv) ||
      !aligned16(b->q_rot) || !aligned16(b->attn) || !aligned16(b->yo) || !aligned16(b->h_mid) ||
      !aligned16(b->xn_ffn) || !aligned16(b->h_ffn) || !aligned16(b->y_down) || !aligned16(b->h_out) ||
      (b->xn_out && !aligned16(b->xn_out)))
    return DMQ_ERR_ALIGNMENT;
  hipStream_t sa = (hipStream_t)stream_attn, sf = (hipStream_t)stream_ffn;
  const bool two = sa != sf;
  const int64_t nchunks = (M + chunk - 1) / chunk;
  if (nchunks > 4096) return DMQ_ERR_INVALID_ARG;
  // everything the single calls below would reject, before any is made
  const int chk = dmq::check_layer(w, b, M, pos0, D, F, n_q_heads, n_kv_heads, cache_len, theta, eps);
  if (chk != DMQ_OK) return chk;
  std::lock_guard<std::mutex> lock(g_ev_mu);
  std::vector<hipEvent_t> ev;
  if (two) {
    ev.resize((size_t)nchunks + 2);
    int st = events((int)ev.size(), ev.data());
    if (st != DMQ_OK) return st;
    // the FFN stream starts after the work already queued on the attention
    // stream (which produced this layer's inputs)
    if (hipEventRecord(ev[0], sa) != hipSuccess || hipStreamWaitEvent(sf, ev[0], 0) != hipSuccess)
      return DMQ_ERR_HIP;
  }
  auto f16 = [](const void* p, int64_t off) { return (void*)((uint16_t*)p + off); };
  auto f32 = [](const float* p, int64_t off) { return (float*)(p + off); };
  // attention side of chunk c, then (on the FFN stream) its feed-forward side
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t r0 = c * chunk, C = M - r0 < chunk ? M - r0 : chunk;
    const dmq_gemm_desc qkv[3] = {
        {w->fmt_q, 0, f16(b->xn_in, r0 * D), w->wq, f32(b->yq, r0 * QD), C, QD, D},
        {w->fmt_k, 0, f16(b->xn_in, r0 * D), w->wk, f32(b->yk, r0 * KD), C, KD, D},
        {w->fmt_v, 0, f16(b->xn_in, r0 * D), w->wv, f32(b->yv, r0 * KD), C, KD, D}};
    int st = dmq_gemm_group(qkv, 3, sa);
    if (st == DMQ_OK)
      st = dmq_rope_kv_cache(f32(b->yq, r0 * QD), f32(b->yk, r0 * KD), f32(b->yv, r0 * KD), C, pos0 + r0, n_q_heads,
                             n_kv_heads, theta, w->freq_factors, f16(b->q_rot, r0 * QD), w->k_cache, w->v_cache,
                             cache_len, sa);
    if (st == DMQ_OK)
      st = dmq_attention_gqa(f16(b->q_rot, r0 * QD), w->k_cache, w->v_cache, f16(b->attn, r0 * QD), C, pos0 + r0,
                             n_q_heads, n_kv_heads, cache_len, sa);
    if (st == DMQ_OK) {
      const dmq_gemm_desc o = {w->fmt_o, 0, f16(b->attn, r0 * QD), w->wo, f32(b->yo, r0 * D), C, D, QD};
      st = dmq_gemm_group(&o, 1, sa);
    }
    if (st == DMQ_OK)
      st = dmq_residual_rmsnorm(f32(b->h_in, r0 * D), f32(b->yo, r0 * D), w->g_ffn, eps, f32(b->h_mid, r0 * D),
                                f16(b->xn_ffn, r0 * D), C, D, sa);
    if (st != DMQ_OK) return st;
    hipStream_t s2 = sa;
    if (two) {
      if (hipEventRecord(ev[1 + c], sa) != hipSuccess || hipStreamWaitEvent(sf, ev[1 + c], 0) != hipSuccess)
        return DMQ_ERR_HIP;
      s2 = sf;
    }
    st = dmq_ffn_swiglu_q4k(f16(b->xn_ffn, r0 * D), w->w_gate_up, w->w_down, f16(b->h_ffn, r0 * F),
                            f32(b->y_down, r0 * D), C, D, F, s2);
    if (st == DMQ_OK)
      st = dmq_residual_rmsnorm(f32(b->h_mid, r0 * D), f32(b->y_down, r0 * D), w->g_next, eps, f32(b->h_out, r0 * D),
                                w->g_next ? f16(b->xn_out, r0 * D) : nullptr, C, D, s2);
    if (st != DMQ_OK) return st;
  }
  if (two) {
    // join: everything is ordered before later work on the attention stream
    if (hipEventRecord(ev[1 + nchunks], sf) != hipSuccess || hipStreamWaitEvent(sa, ev[1 + nchunks], 0) != hipSuccess)
      return DMQ_ERR_HIP;
  }
  return DMQ_OK;
}
