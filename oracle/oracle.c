/*
 * Plain CPU oracle for the Q4_K / Q6_K dequant-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no source with the HIP library (no headers, helpers or tables).
 *
 * What it computes, and where that is defined:
 *
 *  - Dequantisation of the two k-quant super-block formats the DAMASCUS pages
 *    name (project overview page, "[02] the pipeline", compartment 09, which
 *    lists the Q4_K_M dequantizer; article "Building DAMASCUS", section "Read
 *    the model, then reproduce its operations", which checks the Q4_K and
 *    Q6_K dequantizers before their output is used).  The
 *    pages name the formats but do not define their bytes; the byte layout is
 *    the public GGUF k-quant layout (restated in the comments below).  Each
 *    weight is computed exactly in fp64 and then rounded once to fp16 with
 *    round-to-nearest-even; an exact zero is returned as +0.
 *
 *  - The quantised matmul (overview page, compartment 09;
 *    section "[01] the thesis": prefill is dense GEMM, decode is GEMV) as the
 *    plain definition y[m][n] = sum_k x[m][k] * w[n][k] over the fp16 inputs
 *    and the oracle's own fp16 weights, accumulated in fp64 in ascending k,
 *    together with S[m][n] = sum_k |x[m][k] * w[n][k]|, the scale of the
 *    acceptance bound.  Comparing against the same dequantised weights, so
 *    that quantisation error does not mix with implementation error, is the
 *    idea of the article's same-weights oracle section.
 *
 * Loops are plain and sequential per output; OpenMP only spreads independent
 * outputs over host cores.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 256
#define Q4K_BYTES 144
#define Q6K_BYTES 210

/* ---------------------------------------------------------------- fp16 --- */

/* IEEE binary16 bits -> double (exact). */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);                 /* zero or subnormal */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* Round a non-negative double that holds a value < 2^52 to an integer,
 * ties to even. */
static double round_half_even(double s) {
  double fl = floor(s);
  double diff = s - fl;                       /* exact for s < 2^52 */
  if (diff > 0.5) return fl + 1.0;
  if (diff < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* double -> IEEE binary16 bits, round to nearest, ties to even, with gradual
 * underflow and overflow to infinity.  NaN -> 0x7E00 (sign kept). */
uint16_t oracle_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(sign | 0x7e00);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);   /* >= max + half ulp */
  if (a < 0x1p-14) {
    /* subnormal range: quantum 2^-24, integer 0..1024 (1024 = min normal) */
    double r = round_half_even(a * 0x1p24);
    return (uint16_t)(sign | (uint16_t)r);
  }
  int e2;
  frexp(a, &e2);                 /* a = fr * 2^e2, fr in [0.5, 1) */
  int e = e2 - 1;                /* a in [2^e, 2^(e+1)), e in [-14, 15] */
  double r = round_half_even(ldexp(a, 10 - e));   /* in [1024, 2048] */
  if (r == 2048.0) { r = 1024.0; e += 1; }
  if (e > 15) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

void oracle_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_f64_to_f16_array(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(v[i]);
}

/* Exact weight value -> fp16 bits, with an exact zero mapped to +0. */
static uint16_t weight_to_f16(double w) {
  if (w == 0.0) return 0;
  return oracle_f64_to_f16(w);
}

static uint16_t load_le16(const uint8_t* p) {
  return (uint16_t)(p[0] | (p[1] << 8));
}

/* ---------------------------------------------------------------- Q4_K --- */
/*
 * Q4_K super-block, 144 bytes, 256 weights in 8 sub-blocks of 32:
 *   bytes   0..1   d     (fp16)  super-block scale of the sub-block scales
 *   bytes   2..3   dmin  (fp16)  super-block scale of the sub-block mins
 *   bytes   4..15  s[12]         eight 6-bit scales sc_j and eight 6-bit mins m_j
 *   bytes  16..143 qs[128]       256 4-bit quants
 * Sub-block j (0..7) holds weights 32j .. 32j+31.
 *   j < 4 : sc_j = low 6 bits of s[j],    m_j = low 6 bits of s[j+4]
 *   j >= 4: sc_j = low nibble of s[j+4] with the top 2 bits of s[j-4] above it,
 *           m_j  = high nibble of s[j+4] with the top 2 bits of s[j] above it.
 * Weight 32j + l (l = 0..31) takes its quant from byte qs[32*(j/2) + l]: the low
 * nibble when j is even, the high nibble when j is odd.
 * Value: w = d * sc_j * q - dmin * m_j.
 */
void oracle_q4k_fields(const uint8_t* block, double* d, double* dmin,
                       int* sc, int* mn, int* q) {
  const uint8_t* s = block + 4;
  const uint8_t* qs = block + 16;
  *d = oracle_f16_to_f64(load_le16(block));
  *dmin = oracle_f16_to_f64(load_le16(block + 2));
  for (int j = 0; j < 8; ++j) {
    if (j < 4) {
      sc[j] = s[j] & 63;
      mn[j] = s[j + 4] & 63;
    } else {
      sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
      mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
  }
  for (int i = 0; i < QK; ++i) {
    int j = i / 32, l = i % 32;
    uint8_t byte = qs[32 * (j / 2) + l];
    q[i] = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
  }
}

/* wq: rows x (k/256) blocks, row-major.  out: rows x k fp16 bits. */
int oracle_dequant_q4k(const uint8_t* wq, int64_t rows, int64_t k, uint16_t* out) {
  if (k % QK) return -1;
  int64_t nb = rows * (k / QK);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    double d, dmin;
    int sc[8], mn[8], q[QK];
    oracle_q4k_fields(wq + b * Q4K_BYTES, &d, &dmin, sc, mn, q);
    for (int i = 0; i < QK; ++i) {
      int j = i / 32;
      /* both products and their difference are exact in fp64 */
      double w = d * sc[j] * q[i] - dmin * mn[j];
      out[b * QK + i] = weight_to_f16(w);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- Q6_K --- */
/*
 * Q6_K super-block, 210 bytes, 256 weights in 16 sub-blocks of 16:
 *   bytes   0..127 ql[128]   low 4 bits of each quant
 *   bytes 128..191 qh[64]    high 2 bits of each quant
 *   bytes 192..207 sc[16]    int8 sub-block scales
 *   bytes 208..209 d (fp16)  super-block scale
 * Weight i = 128h + 32t + l (h = 0..1, t = 0..3, l = 0..31):
 *   low  = nibble of ql[64h + 32*(t%2) + l]: low nibble for t < 2, high for t >= 2
 *   high = bits 2t, 2t+1 of qh[32h + l]
 *   q = low | high << 4, in 0..63
 * Value: w = d * sc[i/16] * (q - 32).
 */
void oracle_q6k_fields(const uint8_t* block, double* d, int* sc, int* q) {
  const uint8_t* ql = block;
  const uint8_t* qh = block + 128;
  const int8_t* s = (const int8_t*)(block + 192);
  *d = oracle_f16_to_f64(load_le16(block + 208));
  for (int i = 0; i < 16; ++i) sc[i] = s[i];
  for (int i = 0; i < QK; ++i) {
    int h = i / 128, t = (i / 32) % 4, l = i % 32;
    uint8_t lb = ql[64 * h + 32 * (t % 2) + l];
    int low = (t < 2) ? (lb & 15) : (lb >> 4);
    int high = (qh[32 * h + l] >> (2 * t)) & 3;
    q[i] = low | (high << 4);
  }
}

int oracle_dequant_q6k(const uint8_t* wq, int64_t rows, int64_t k, uint16_t* out) {
  if (k % QK) return -1;
  int64_t nb = rows * (k / QK);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    double d;
    int sc[16], q[QK];
    oracle_q6k_fields(wq + b * Q6K_BYTES, &d, sc, q);
    for (int i = 0; i < QK; ++i) {
      double w = d * sc[i / 16] * (q[i] - 32);   /* exact in fp64 */
      out[b * QK + i] = weight_to_f16(w);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- GEMM --- */

static double* f16_matrix_to_f64(const uint16_t* a, int64_t n) {
  double* out = (double*)malloc((size_t)n * sizeof(double));
  if (!out) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(a[i]);
  return out;
}

/*
 * y[m][n] = sum_k x[m][k] * w[n][k]   (x: M x K fp16, w: N x K fp16, y = x W^T)
 * s[m][n] = sum_k |x[m][k] * w[n][k]|
 * fp64, k ascending.  y and s are M x N row-major; s may be NULL.
 */
int oracle_gemm_f16(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                    int64_t K, double* y, double* s) {
  double* xd = f16_matrix_to_f64(x, M * K);
  double* wd = f16_matrix_to_f64(w, N * K);
  if (!xd || !wd) { free(xd); free(wd); return -2; }
#pragma omp parallel for schedule(static)
  for (int64_t mn = 0; mn < M * N; ++mn) {
    int64_t m = mn / N, n = mn % N;
    const double* xr = xd + m * K;
    const double* wr = wd + n * K;
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = xr[k] * wr[k];
      acc += p;
      mag += fabs(p);
    }
    y[mn] = acc;
    if (s) s[mn] = mag;
  }
  free(xd);
  free(wd);
  return 0;
}

/* The same definition evaluated only at the listed (m, n) pairs. */
int oracle_gemm_f16_pairs(const uint16_t* x, const uint16_t* w, int64_t K,
                          const int64_t* ms, const int64_t* ns, int64_t count,
                          double* y, double* s) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    const uint16_t* xr = x + ms[i] * K;
    const uint16_t* wr = w + ns[i] * K;
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = oracle_f16_to_f64(xr[k]) * oracle_f16_to_f64(wr[k]);
      acc += p;
      mag += fabs(p);
    }
    y[i] = acc;
    if (s) s[i] = mag;
  }
  return 0;
}

/* ------------------------------------------------------------- RMSNorm --- */

/*
 * RMSNorm of the rows of x (M x K fp16): out[m][k] = x[m][k] * g[k] / r_m with
 * r_m = sqrt(sum_k x[m][k]^2 / K + eps), in fp64 (k ascending), no rounding to
 * fp16.  The layer description on the article page names the operation
 * (RMSNorm before the QKV projections and before the feed-forward network);
 * the definition is the standard one: divide by the root mean square of the
 * row, offset by eps, and scale by the per-column weight g.
 */
void oracle_rmsnorm(const uint16_t* x, const double* g, double eps, int64_t M, int64_t K, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const uint16_t* xr = x + m * K;
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double v = oracle_f16_to_f64(xr[k]);
      ss += v * v;
    }
    double r = sqrt(ss / (double)K + eps);
    for (int64_t k = 0; k < K; ++k) out[m * K + k] = oracle_f16_to_f64(xr[k]) * g[k] / r;
  }
}

/*
 * y = x W^T and s = sum |x w| with x in fp64 (M x K, e.g. the RMSNorm output
 * above) and W fp16 (N x K), fp64, k ascending.
 */
int oracle_gemm_f64x(const double* x, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                     double* y, double* s) {
  double* wd = f16_matrix_to_f64(w, N * K);
  if (!wd) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t mn = 0; mn < M * N; ++mn) {
    int64_t m = mn / N, n = mn % N;
    const double* xr = x + m * K;
    const double* wr = wd + n * K;
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = xr[k] * wr[k];
      acc += p;
      mag += fabs(p);
    }
    y[mn] = acc;
    if (s) s[mn] = mag;
  }
  free(wd);
  return 0;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
