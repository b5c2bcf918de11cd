/*
 * dmq -- fused Q4_K / Q6_K dequant-GEMM for AMD MI355X (gfx950).
 *
 * C ABI of the shared library libdmq.so.  Every entry point takes plain
 * pointers and sizes, returns an int status (dmq_status), never throws, and
 * runs asynchronously on the HIP stream it is given.
 *
 * What the calls compute comes from the DAMASCUS pages:
 *  - Overview page, "[02] the pipeline", compartment 09 (Quantization & AMX),
 *    which lists the Q4_K_M dequantizer, the quantised matmul and a prefill
 *    kernel with fused dequant; and "[01] the thesis": that fused path never
 *    materialises fp16 weights.
 *  - Article "Building DAMASCUS", "Read the model, then reproduce its
 *    operations": the Q4_K and Q6_K dequantizers; and "Prefill and decode
 *    need different performance questions": decode is matrix-vector work
 *    bound by streaming the weights, prefill is matrix-matrix work.
 *  - Same article, layer description: each decoder layer ends with a second
 *    RMSNorm followed by a SwiGLU feed-forward network.
 *
 * Conventions shared by all calls
 *  - Pointers named *_f16 point to IEEE binary16 data, y points to fp32 data.
 *  - Activations x are [M, K] row-major, contiguous.
 *  - A quantised weight matrix W is [N, K]: N rows, each a contiguous run of
 *    K/256 super-blocks in GGUF k-quant byte layout (Q4_K: 144 bytes, Q6_K:
 *    210 bytes per 256 weights); rows follow each other with no padding.
 *  - Products are y = x * W^T, i.e. y[m][n] = sum_k x[m][k] * W[n][k], [M, N]
 *    row-major fp32, accumulated in fp32.
 *  - Every pointer except the stream is DEVICE memory owned by the caller
 *    (for example a torch tensor's data_ptr()).  Passing host memory is
 *    undefined behaviour.  The library keeps cached device properties,
 *    cached launch plans and two kinds of device workspace, one buffer of
 *    each per (device, stream): the partial sums of GEMMs whose plan splits
 *    the reduction (see dmq_gemm_q4k) and the partial softmax states of the
 *    decode attention (see dmq_attention_gqa).  A call that needs a larger
 *    buffer than its stream has allocates one with hipMallocAsync on that
 *    stream (stream-ordered: the call does not wait for queued work and does
 *    not synchronise), at least twice the old size; the old buffer is kept,
 *    never freed, because work queued earlier and HIP graphs captured
 *    earlier on that stream may still use it.  Workspaces live until the
 *    process ends.  Nothing else is allocated.  A call made while its stream
 *    is being captured into a HIP graph must not need a new or larger
 *    workspace (it then returns DMQ_ERR_HIP and enqueues nothing): make the
 *    same call once on that stream before capturing, or use
 *    dmq_attention_gqa_noalloc.
 *  - stream is a hipStream_t passed as void*; NULL means the null stream.  The
 *    call only enqueues work: results are ready once the stream is
 *    synchronised.  The device is the caller's current HIP device.
 *  - Arguments are checked on the host before any HIP call; a rejected call
 *    enqueues nothing.  Checks: non-NULL pointers, sizes >= 1 and < 2^31,
 *    K (and D, F) a multiple of 256 and, for the GEMM calls, at most 2^20,
 *    x / y / h / w_f16 16-byte aligned, Q4_K weights 16-byte aligned, Q6_K
 *    weights 2-byte aligned.
 *  - An output may not share a byte with an input of the same call or with
 *    another output (workgroups would write it while others still read it):
 *    such calls are rejected with DMQ_ERR_INVALID_ARG.  Inputs may share
 *    memory (several projections of one x, one weight array twice).
 */
#ifndef DMQ_H
#define DMQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DMQ_OK = 0,
  DMQ_ERR_INVALID_ARG = -1,   /* NULL pointer, size out of range, bad format */
  DMQ_ERR_ALIGNMENT = -2,     /* a pointer breaks the alignment rule above   */
  DMQ_ERR_UNSUPPORTED = -3,   /* no HIP device / not a gfx950 device         */
  DMQ_ERR_HIP = -4,           /* the HIP runtime reported a launch error     */
  DMQ_ERR_SCRATCH = -5        /* a *_noalloc call needs more than its fixed
                                 scratch (DMQ_NOALLOC_SCRATCH_BYTES)         */
} dmq_status;

/* Weight formats for dmq_gemm_desc.format. */
#define DMQ_FMT_Q4K 0
#define DMQ_FMT_Q6K 1

/*
 * Dequantise a Q4_K matrix to fp16.
 *   wq    : rows x (k/256) Q4_K blocks (rows*k/256*144 bytes), 16-byte aligned.
 *   w_f16 : rows x k fp16, row-major (output).
 * Each weight of sub-block j of a block is w = d*sc_j*q - dmin*m_j (d, dmin the
 * block's fp16 super-scales, sc_j/m_j its 6-bit scale and min, q the 4-bit
 * quant), computed exactly and rounded ONCE to fp16 (round to nearest even,
 * subnormals kept, overflow to inf); an exact zero is +0.  Bit-exact.
 * Non-finite d/dmin propagate as IEEE arithmetic on (d*sc_j)*q - dmin*m_j.
 */
int dmq_dequant_q4k(const void* wq, void* w_f16, int64_t rows, int64_t k, void* stream);

/*
 * Dequantise a Q6_K matrix to fp16.
 *   wq    : rows x (k/256) Q6_K blocks (rows*k/256*210 bytes), 2-byte aligned.
 *   w_f16 : rows x k fp16 (output).
 * w = d * sc[i/16] * (q - 32), q the 6-bit quant (4 low bits + 2 high bits),
 * sc the int8 sub-block scale; exact in fp32, rounded once to fp16; exact zero
 * is +0.  Bit-exact.
 */
int dmq_dequant_q6k(const void* wq, void* w_f16, int64_t rows, int64_t k, void* stream);

/*
 * y = x * W^T with W in Q4_K, dequantised inside the kernel (no fp16 weight
 * matrix is ever written to memory).
 *   x_f16 : [M, K] fp16;  wq : N rows of K/256 Q4_K blocks;  y : [M, N] fp32.
 * M = 1 runs the decode matrix-vector kernel, and so does M = 2 with
 * K <= 20480 (both rows' x staged; each row then gets the bits of an M = 1
 * call on it); other M up to 16 a small-M MFMA kernel (up to M = 32 too for
 * launches with a SwiGLU pair or of a few rows); larger M the tiled MFMA
 * prefill kernel.  When a problem has too
 * few output tiles to fill the GPU, the tiled kernel splits the K blocks
 * into pieces whose fp32 partial sums a second kernel adds in piece order
 * (workspace: see above).  Every path gives the same bits on every run.
 * Per output, |y - y_exact| stays within 1e-3 * sum_k |x[m][k] * w[n][k]|
 * + 1e-5 (w the fp16-rounded weight).  The MFMA kernels multiply by the
 * fp16-rounded weights themselves; the M = 1 kernel factors each 32-weight
 * sub-block's scale and min out of the sum (centred so that cancelling
 * weights stay within the bound), so its y can differ from theirs in the
 * last bits.  With an infinite x the M = 1 result can be NaN where the
 * product with the fp16 weights is +-inf (a zero scale or a zero centred
 * min still multiplies the infinite sum of x).
 */
int dmq_gemm_q4k(const void* x_f16, const void* wq, float* y,
                 int64_t M, int64_t N, int64_t K, void* stream);

/* Same as dmq_gemm_q4k with W in Q6_K (down projection, tied LM head). */
int dmq_gemm_q6k(const void* x_f16, const void* wq, float* y,
                 int64_t M, int64_t N, int64_t K, void* stream);

/*
 * SwiGLU feed-forward block: h = silu(x*Wg^T) * (x*Wu^T), y = h * Wd^T.
 *   x_f16         : [M, D] fp16.
 *   w_gate_up_q4k : 2F rows of D/256 Q4_K blocks; rows 0..F-1 are the gate
 *                   projection, rows F..2F-1 the up projection.
 *   w_down_q6k    : D rows of F/256 Q6_K blocks.
 *   h_f16         : [M, F] fp16 (output, caller-provided): silu(g)*u computed
 *                   in fp32 from the fp32 accumulators and rounded once to fp16
 *                   (IEEE: values beyond the fp16 range become +-inf).
 *                   silu(g) = g / (1 + exp(-g)).
 *   y             : [M, D] fp32 (output) = h * Wd^T.
 * g and u are never written to memory; h is written once and read once.
 */
int dmq_ffn_swiglu_q4k(const void* x_f16, const void* w_gate_up_q4k,
                       const void* w_down_q6k, void* h_f16, float* y,
                       int64_t M, int64_t D, int64_t F, void* stream);

/*
 * One problem of a grouped GEMM launch.  Each entry is an independent
 * y = x * W^T with its own format, pointers and sizes, under the same rules
 * as dmq_gemm_q4k / dmq_gemm_q6k.
 */
typedef struct {
  int32_t format;      /* DMQ_FMT_Q4K or DMQ_FMT_Q6K */
  int32_t reserved;    /* must be 0 */
  const void* x_f16;
  const void* wq;
  float* y;
  int64_t M, N, K;
} dmq_gemm_desc;

/*
 * Run `count` GEMMs (1 <= count <= 64) as one launch per kernel kind instead
 * of one launch per GEMM, so that small projections (e.g. the K and V
 * projections of one layer) share the GPU with the large ones.  descs is a
 * HOST array; it is read before the call returns.  All problems must use the
 * same kernel kind: all M = 1 (decode), or all M > 1.  Results meet the same
 * bound as dmq_gemm_q4k / dmq_gemm_q6k per entry; they are the same bits as
 * those calls except where the group's launch plan splits a problem's K
 * differently (tiled kernel only), which changes the fp32 summation order,
 * or where the group runs another kernel than the single call would: the
 * kernel is chosen from the group's largest M and K, its SwiGLU pairs and
 * its total size (e.g. an M = 2 problem beside an M = 3 one takes the
 * small-M kernel, not the two-row decode kernel).
 */
int dmq_gemm_group(const dmq_gemm_desc* descs, int32_t count, void* stream);

/*
 * One weight matrix of dmq_rmsnorm_gemm / dmq_residual_rmsnorm_gemm:
 * y = RMSNorm(x) * W^T with W in the given format (N rows of K/256 blocks)
 * and y [M, N] fp32.  With flags = DMQ_PROJ_SWIGLU, W is a Q4_K gate|up pair
 * as in dmq_ffn_swiglu_q4k (rows 0..N/2-1 gate, N/2..N-1 up; N/2 a multiple
 * of 256) and y points to the fp16 output h [M, N/2], h = silu(gate) * up
 * (the SwiGLU of the FFN, article "Building DAMASCUS", layer description).
 */
#define DMQ_PROJ_SWIGLU 1
typedef struct {
  int32_t format;      /* DMQ_FMT_Q4K or DMQ_FMT_Q6K */
  int32_t flags;       /* 0 or DMQ_PROJ_SWIGLU */
  const void* wq;
  float* y;            /* fp32 y, or fp16 h with DMQ_PROJ_SWIGLU (16-byte aligned) */
  int64_t N;
} dmq_proj_desc;

/*
 * RMSNorm of the activations followed by the projections that read them, as
 * each decoder layer does before its Q|K|V projections and again before its
 * gate|up projections (article "Building DAMASCUS", layer description;
 * overview page, "[04] one decode step").
 *   x_f16  : [M, K] fp16, 16-byte aligned.
 *   g      : K fp32 RMSNorm weights, 16-byte aligned.
 *   eps    : >= 0 and finite (Llama-3.2 uses 1e-5).
 *   xn_f16 : [M, K] fp16 output, 16-byte aligned, not x: the normalized
 *            activations, xn[m][k] = fp16(x[m][k] * g[k] / sqrt(mean_k x[m][k]^2
 *            + eps)), computed in fp32 (the row's sum of squares included) and
 *            rounded once: within one fp16 step of the exact value.  When
 *            M = 1 (and K <= 32768) the decode kernel normalizes x while it
 *            stages it; xn is then optional (NULL: not written).
 *   projs  : 1..64 projections (host array, read before the call returns), all
 *            with reduction length K.  No projection output may overlap x, g,
 *            xn or another projection's output (DMQ_ERR_INVALID_ARG): within
 *            the launch, workgroups write outputs while others still read.
 * y_i = xn * W_i^T for each projection with xn as the activations, under the
 * rules and the per-output bound of dmq_gemm_q4k / dmq_gemm_q6k (one grouped
 * launch after the normalization).  The fp16 rounding of xn is part of the
 * operation: where the normalized values are fp16 subnormals (a row of tiny
 * values under a large eps) it is coarse, and y follows the rounded values.
 */
int dmq_rmsnorm_gemm(const void* x_f16, const float* g, float eps, void* xn_f16,
                     int64_t M, int64_t K, const dmq_proj_desc* projs, int32_t count,
                     void* stream);

/*
 * The residual connection, the next RMSNorm and the projections that read it,
 * as one call: a decoder layer adds the attention output (then the FFN
 * output) to the residual stream and normalizes the sum before the gate|up
 * (then the next layer's Q|K|V) projections (overview page, "[04] one decode
 * step"; article "Building DAMASCUS", layer description).
 *   h_in, y_add : [M, K] fp32, 16-byte aligned (the residual stream and the
 *                 output added to it).
 *   h_out       : [M, K] fp32, 16-byte aligned: h_out = h_in + y_add (IEEE
 *                 fp32 adds, exact to the bit).  It must not overlap h_in,
 *                 y_add or g (other workgroups still read them): keep two
 *                 residual buffers and alternate.  Overlaps are rejected
 *                 (DMQ_ERR_INVALID_ARG).
 *   g, eps      : as in dmq_rmsnorm_gemm, applied to h_out.
 *   xn_f16      : [M, K] fp16, 16-byte aligned, overlapping none of the
 *                 above: fp16(h_out * g / sqrt(mean(h_out^2) + eps)) within
 *                 one fp16 step of the exact value.  Optional (NULL) when
 *                 M = 1 and K <= 32768: the decode kernel then forms the sum,
 *                 the norm and the staged activations in one launch, every
 *                 workgroup from h_in and y_add, one of them writing h_out.
 *                 Otherwise a residual + RMSNorm kernel runs first.
 *   projs       : as in dmq_rmsnorm_gemm, with xn as the activations; no
 *                 projection output may overlap h_in, y_add, h_out, g, xn or
 *                 another output (DMQ_ERR_INVALID_ARG).
 */
int dmq_residual_rmsnorm_gemm(const float* h_in, const float* y_add, const float* g, float eps,
                              float* h_out, void* xn_f16, int64_t M, int64_t K,
                              const dmq_proj_desc* projs, int32_t count, void* stream);

/*
 * The attention side of a decoder layer (overview page, "[04] one decode step":
 * RMSNorm -> QKV projection -> RoPE -> attention over the KV cache (GQA) ->
 * residual add -> RMSNorm -> SwiGLU FFN -> residual add; model table: 24 query
 * heads, 8 KV heads, head dimension 128, RoPE theta 500000).  The head
 * dimension is 128 in all three calls.  The KV cache of one layer is two
 * caller-owned fp16 arrays [n_kv_heads, cache_len, 128]; position p of KV head
 * h is row h * cache_len + p.
 */

/*
 * RoPE on the Q and K projections of M tokens at positions pos0 .. pos0+M-1,
 * and their K and V rows appended to the cache.
 *   q, k, v      : fp32 [M, n_q_heads*128], [M, n_kv_heads*128] (the projection
 *                  outputs y), 16-byte aligned.
 *   theta        : RoPE base (> 1; 500000 for the pages' model).
 *   freq_factors : NULL, or 64 floats f_i dividing the angle of pair i.
 *   q_f16        : [M, n_q_heads*128] fp16 output, the rotated queries.
 *   k_cache_f16, v_cache_f16 : the layer's cache; rows pos0 .. pos0+M-1 of
 *                  every KV head are written (K rotated, V as is), nothing else.
 * Pair i of a head is (dims 2i, 2i+1), turned by pos * theta^(-2i/128) / f_i:
 * (a, b) -> (a cos - b sin, a sin + b cos).  The angle is formed and reduced in
 * fp64, the rotation done in fp32 and each result rounded once to fp16.
 * Requires pos0 >= 0, pos0 + M <= cache_len, n_q_heads a multiple of n_kv_heads
 * with at most 8 query heads per KV head.
 */
int dmq_rope_kv_cache(const float* q, const float* k, const float* v, int64_t M, int64_t pos0, int32_t n_q_heads,
                      int32_t n_kv_heads, double theta, const float* freq_factors, void* q_f16, void* k_cache_f16,
                      void* v_cache_f16, int64_t cache_len, void* stream);

/*
 * Causal grouped-query attention of M queries (positions pos0 .. pos0+M-1)
 * over the cache: query head h reads KV head h / (n_q_heads / n_kv_heads); the
 * query at position p attends to cache positions 0..p with weights
 * softmax(q . k / sqrt(128)).
 *   q_f16   : [M, n_q_heads*128] fp16 (from dmq_rope_kv_cache).
 *   out_f16 : [M, n_q_heads*128] fp16 output (the O projection's input), not q.
 * The cache rows 0 .. pos0+M-1 must have been written.  Scores, softmax and
 * the weighted sum of V are fp32; the output is rounded once to fp16.
 * With M > 16 (prefill) an MFMA flash-attention kernel takes 128 queries of
 * one head per workgroup over 32-key blocks (online softmax in fp32, P
 * rounded to fp16 for the P V product).
 * With M <= 16 (decode) the positions are split into pieces of 64 over many
 * workgroups whose partial softmax states a second kernel merges in piece
 * order; the states go to a workspace the library keeps per (device, stream)
 * (see the conventions above), sized on its first use for every position of
 * the cache when that takes at most 64 MiB, so that a decode loop over one
 * cache does not grow it.  Every path gives the same bits on every run.
 */
int dmq_attention_gqa(const void* q_f16, const void* k_cache_f16, const void* v_cache_f16, void* out_f16, int64_t M,
                      int64_t pos0, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_len, void* stream);

/*
 * dmq_rope_kv_cache followed by dmq_attention_gqa on the same arguments, in
 * one call: the RoPE and cache-append step of the overview's "[04] one decode
 * step" joined to the attention that reads its results.  Arguments as in
 * those two calls (q, k, v: the projections' fp32 rows; q_f16: receives the
 * rotated queries; k_cache_f16, v_cache_f16: rows pos0 .. pos0+M-1 written;
 * out_f16: the attention output), with the checks of both; additionally
 * out_f16 overlapping any other buffer is rejected.  Every output has the
 * bits the two calls give.  At M = 1 (one decode token) the rotation, the
 * cache append and the attention's per-piece pass run in one kernel, saving
 * the RoPE launch; other M run the two calls' kernels in turn.  Uses the
 * attention's per-stream workspace like dmq_attention_gqa.
 */
int dmq_rope_attention_gqa(const float* q, const float* k, const float* v, int64_t M, int64_t pos0,
                           int32_t n_q_heads, int32_t n_kv_heads, double theta, const float* freq_factors,
                           void* q_f16, void* k_cache_f16, void* v_cache_f16, int64_t cache_len, void* out_f16,
                           void* stream);

/*
 * dmq_attention_gqa for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and bits as dmq_attention_gqa; it
 * calls no hipMalloc, hipFree or other allocating routine.  The decode path
 * (M <= 16) keeps its partial softmax states, M * n_q_heads *
 * ceil((pos0 + M) / 64) records of 520 bytes, in a fixed scratch array of
 * DMQ_NOALLOC_SCRATCH_BYTES that each GPU holds from the first call on it
 * until the process ends; a call that needs more returns DMQ_ERR_SCRATCH and
 * enqueues nothing (e.g. 24 query heads: M = 1 up to 172,032 cached
 * positions, M = 16 up to 10,752).  All calls on one GPU share that array,
 * so calls that can overlap on one GPU (different streams, or graphs
 * replayed concurrently) race: order them on one stream.  Nothing in it has
 * to start at zero.  The prefill path (M > 16) takes no scratch.
 */
#define DMQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int dmq_attention_gqa_noalloc(const void* q_f16, const void* k_cache_f16, const void* v_cache_f16, void* out_f16,
                              int64_t M, int64_t pos0, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_len,
                              void* stream);

/*
 * The residual connection, fused with the RMSNorm that follows it:
 *   h_out = h_in + y (fp32, one rounding per element; h_out may be h_in or y);
 *   with g: xn_f16 = fp16(h_out * g / sqrt(mean(h_out^2) + eps)), computed in
 *   fp32 and rounded once, the input of the next projections.  g == NULL: the
 *   add only (xn_f16 unused).
 *   h_in, y, h_out : fp32 [M, K], K a multiple of 256; g: K floats; all 16-byte
 *   aligned.
 */
int dmq_residual_rmsnorm(const float* h_in, const float* y, const float* g, float eps, float* h_out, void* xn_f16,
                         int64_t M, int64_t K, void* stream);

/*
 * One decoder layer's prefill with its attention side and its feed-forward
 * side running concurrently on two streams over shared device buffers: the
 * one-GPU form of the overview page's "[03] zero-copy / unified memory"
 * split (attention on one engine, the FFN on another, one shared buffer).
 *
 * For M tokens at positions pos0 .. pos0+M-1 (D hidden, F FFN width, head
 * dimension 128):
 *   yq|yk|yv = xn_in * Wq|Wk|Wv^T; RoPE + cache append (dmq_rope_kv_cache);
 *   attn = attention over the cache (dmq_attention_gqa); yo = attn * Wo^T;
 *   h_mid = h_in + yo, xn_ffn = RMSNorm(h_mid; g_ffn);
 *   h_ffn = silu(xn_ffn * Wg^T) * (xn_ffn * Wu^T); y_down = h_ffn * Wd^T;
 *   h_out = h_mid + y_down, xn_out = RMSNorm(h_out; g_next)
 * (the layer description of the article "Building DAMASCUS" and the overview
 * page's "[04] one decode step"), each step exactly as the single calls
 * named.  The rows are cut into chunks of `chunk`: the attention side of
 * chunk c+1 runs on stream_attn while the feed-forward side of chunk c runs
 * on stream_ffn; events hand each chunk over, stream_ffn first waits for the
 * work already queued on stream_attn, and stream_attn finally waits for
 * stream_ffn, so the layer's results are ordered before later work on
 * stream_attn.  stream_ffn == stream_attn runs the same chunked schedule on
 * one stream, with the same bits.  Chunking changes the launch plans of the
 * GEMMs (and so may change fp32 summation orders) against one call for all M
 * rows; a chunk of at least M is one pass.
 *   w : weights (formats of Q, K, V, O: DMQ_FMT_Q4K or DMQ_FMT_Q6K; gate|up
 *       Q4_K, 2F rows, gate first; down Q6_K), the two RMSNorm weight vectors
 *       (g_next may be NULL: then xn_out is not written), optional RoPE
 *       frequency factors, and the layer's KV cache (fp16 [n_kv_heads,
 *       cache_len, 128]; rows pos0 .. pos0+M-1 are written).
 *   b : device buffers of M rows, 16-byte aligned, none overlapping another:
 *       inputs h_in (fp32 [M, D]) and xn_in (fp16 [M, D], this layer's input
 *       RMSNorm of h_in); outputs h_mid, h_out (fp32 [M, D]) and xn_out
 *       (fp16 [M, D]); scratch yq (fp32 [M, n_q_heads*128]), yk, yv (fp32 [M,
 *       n_kv_heads*128]), q_rot, attn (fp16 [M, n_q_heads*128]), yo, y_down
 *       (fp32 [M, D]), xn_ffn (fp16 [M, D]), h_ffn (fp16 [M, F]).
 * Requirements: D, F and n_q_heads*128 multiples of 256, chunk >= 1, at most
 * 4096 chunks, those of the single calls (checked for all M rows), and no
 * written buffer or cache overlapping another buffer, cache, weight array or
 * norm vector.  They are checked on the host before any event is recorded or
 * kernel enqueued: a rejected call enqueues nothing.  The library keeps a
 * pool of HIP events per device (created on first use, kept until the process
 * ends); calls from several host threads are serialised on it.  A HIP error
 * in a later step returns its status with the steps before it enqueued.
 */
typedef struct {
  int32_t fmt_q, fmt_k, fmt_v, fmt_o;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* w_gate_up;
  const void* w_down;
  const float* g_ffn;
  const float* g_next;
  const float* freq_factors;
  void* k_cache;
  void* v_cache;
} dmq_layer_weights;

typedef struct {
  const float* h_in;
  const void* xn_in;
  float* yq;
  float* yk;
  float* yv;
  void* q_rot;
  void* attn;
  float* yo;
  float* h_mid;
  void* xn_ffn;
  void* h_ffn;
  float* y_down;
  float* h_out;
  void* xn_out;
} dmq_layer_buffers;

int dmq_layer_prefill(const dmq_layer_weights* w, const dmq_layer_buffers* b, int64_t M, int64_t pos0, int32_t D,
                      int32_t F, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_len, double theta, float eps,
                      int64_t chunk, void* stream_attn, void* stream_ffn);

/* Human-readable text of a status code (static storage). */
const char* dmq_status_string(int status);

/* Library ABI version (currently 1). */
int dmq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DMQ_H */
