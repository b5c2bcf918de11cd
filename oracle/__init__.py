"""CPU oracle for the fused Q4_K / Q6_K dequant-GEMM path.

TEST INFRASTRUCTURE ONLY: this package is the checker, not the product.  Only
the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library.

* The heavy loops (block decode, exact dequant + fp16 rounding, the fp64
  triple-loop matmul) are plain C in ``oracle.c``, compiled with gcc into
  ``liboracle.so`` and called through ctypes.
* The SwiGLU check (silu and the acceptance interval) is fp64 numpy here.
* RMSNorm (fp64, no intermediate rounding) and the GEMM on its fp64 output
  are C as well; the fp16 acceptance interval of a normalized activation is
  numpy here.
* RoPE, grouped-query attention over a KV cache and the residual add are
  fp64 numpy in ``attention.py``.

Sources (DAMASCUS pages): the dequantisers and the quantised matmul are the
overview page's compartment 09 ("[02] the pipeline") and the article's
section "Read the model, then reproduce its operations"; the SwiGLU FFN is
compartment 05/06 and the article's layer description (a second RMSNorm and
a SwiGLU feed-forward network end each layer; RMSNorm also precedes the QKV
projections, overview "[04] one decode step"); comparing against the same
dequantised blocks is the article's same-weights oracle idea.  The per-output
acceptance bound |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-5 replaces the
pages' own 1e-3 absolute logit threshold (article, same section).

Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_pins.py``.  The
byte layout itself is not printed on the pages; it is the public GGUF
k-quant layout, so the layout pins check the oracle against that
specification as restated in the tests ("parity unpinned by the pages" for
the layout, see the tests' module docstring).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

QK = 256
Q4K_BYTES = 144
Q6K_BYTES = 210

GEMM_REL_TOL = 1e-3
GEMM_ABS_TOL = 1e-5


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math,
    no FMA contraction, OpenMP over independent outputs)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f16_to_f64_array.argtypes = [P, I64, P]
        L.oracle_f16_to_f64_array.restype = None
        L.oracle_f64_to_f16_array.argtypes = [P, I64, P]
        L.oracle_f64_to_f16_array.restype = None
        L.oracle_q4k_fields.argtypes = [P, P, P, P, P, P]
        L.oracle_q4k_fields.restype = None
        L.oracle_q6k_fields.argtypes = [P, P, P, P]
        L.oracle_q6k_fields.restype = None
        for name in ("oracle_dequant_q4k", "oracle_dequant_q6k"):
            fn = getattr(L, name)
            fn.argtypes = [P, I64, I64, P]
            fn.restype = ctypes.c_int
        L.oracle_gemm_f16.argtypes = [P, P, I64, I64, I64, P, P]
        L.oracle_gemm_f16.restype = ctypes.c_int
        L.oracle_gemm_f16_pairs.argtypes = [P, P, I64, P, P, I64, P, P]
        L.oracle_gemm_f16_pairs.restype = ctypes.c_int
        L.oracle_rmsnorm.argtypes = [P, P, ctypes.c_double, I64, I64, P]
        L.oracle_rmsnorm.restype = None
        L.oracle_gemm_f64x.argtypes = [P, P, I64, I64, I64, P, P]
        L.oracle_gemm_f64x.restype = ctypes.c_int
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return int(lib().oracle_threads())


# ------------------------------------------------------------------ fp16 ---

def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_f16_to_f64_array(_ptr(b), b.size, _ptr(out))
    return out


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_f64_to_f16_array(_ptr(a), a.size, _ptr(out))
    return out


# --------------------------------------------------------------- dequant ---

def q4k_fields(block: np.ndarray):
    """Decoded fields of one Q4_K block: (d, dmin, sc[8], m[8], q[256])."""
    b = _c(block, np.uint8)
    assert b.size == Q4K_BYTES
    d = ctypes.c_double()
    dmin = ctypes.c_double()
    sc = np.zeros(8, np.int32)
    mn = np.zeros(8, np.int32)
    q = np.zeros(QK, np.int32)
    lib().oracle_q4k_fields(_ptr(b), ctypes.addressof(d), ctypes.addressof(dmin),
                            _ptr(sc), _ptr(mn), _ptr(q))
    return d.value, dmin.value, sc, mn, q


def q6k_fields(block: np.ndarray):
    """Decoded fields of one Q6_K block: (d, sc[16], q[256])."""
    b = _c(block, np.uint8)
    assert b.size == Q6K_BYTES
    d = ctypes.c_double()
    sc = np.zeros(16, np.int32)
    q = np.zeros(QK, np.int32)
    lib().oracle_q6k_fields(_ptr(b), ctypes.addressof(d), _ptr(sc), _ptr(q))
    return d.value, sc, q


def dequant_q4k(wq: np.ndarray, rows: int, k: int) -> np.ndarray:
    """Q4_K bytes [rows, k/256*144] -> fp16 bits [rows, k] (exact value, one RNE)."""
    b = _c(wq, np.uint8)
    assert k % QK == 0 and b.size == rows * (k // QK) * Q4K_BYTES
    out = np.empty((rows, k), dtype=np.uint16)
    rc = lib().oracle_dequant_q4k(_ptr(b), rows, k, _ptr(out))
    assert rc == 0
    return out


def dequant_q6k(wq: np.ndarray, rows: int, k: int) -> np.ndarray:
    b = _c(wq, np.uint8)
    assert k % QK == 0 and b.size == rows * (k // QK) * Q6K_BYTES
    out = np.empty((rows, k), dtype=np.uint16)
    rc = lib().oracle_dequant_q6k(_ptr(b), rows, k, _ptr(out))
    assert rc == 0
    return out


def dequant(fmt: str, wq: np.ndarray, rows: int, k: int) -> np.ndarray:
    return dequant_q4k(wq, rows, k) if fmt == "q4k" else dequant_q6k(wq, rows, k)


# ------------------------------------------------------------------ GEMM ---

def gemm_f16(x: np.ndarray, w_bits: np.ndarray):
    """y = x W^T and S = sum |x w| in fp64.  x: fp16 [M,K]; w_bits: fp16 bits [N,K]."""
    xb = _c(np.asarray(x, dtype=np.float16).view(np.uint16), np.uint16)
    wb = _c(w_bits, np.uint16)
    M, K = xb.shape
    N, K2 = wb.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = lib().oracle_gemm_f16(_ptr(xb), _ptr(wb), M, N, K, _ptr(y), _ptr(s))
    assert rc == 0
    return y, s


def gemm_f16_pairs(x: np.ndarray, w_bits: np.ndarray, ms: np.ndarray, ns: np.ndarray):
    """The same definition evaluated only at outputs (ms[i], ns[i])."""
    xb = _c(np.asarray(x, dtype=np.float16).view(np.uint16), np.uint16)
    wb = _c(w_bits, np.uint16)
    K = xb.shape[1]
    assert wb.shape[1] == K
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < xb.shape[0])
    assert ns.size == 0 or (ns.min() >= 0 and ns.max() < wb.shape[0])
    y = np.empty(ms.shape, np.float64)
    s = np.empty(ms.shape, np.float64)
    lib().oracle_gemm_f16_pairs(_ptr(xb), _ptr(wb), K, _ptr(ms), _ptr(ns), ms.size,
                                _ptr(y), _ptr(s))
    return y, s


def gemm_quant(fmt: str, x: np.ndarray, wq: np.ndarray, n: int, k: int):
    """Oracle of the fused path: exact dequant -> fp16, then the fp64 matmul."""
    return gemm_f16(x, dequant(fmt, wq, n, k))


def gemm_tolerance(s: np.ndarray) -> np.ndarray:
    """Per-output acceptance bound 1e-3 * S + 1e-5."""
    return GEMM_REL_TOL * s + GEMM_ABS_TOL


# --------------------------------------------------------------- SwiGLU ---

def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)) in fp64 (overflow-safe)."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = g[~pos] * e / (1.0 + e)
    return out


def _silu_min_point():
    """g* where silu has its only minimum.  silu'(g) = sigmoid(g) (1 + g (1 -
    sigmoid(g))) vanishes where 1 - sigmoid(g) = 1/(1 + e^g) = -1/g, i.e. where
    1 + g + e^g = 0; solved by Newton in fp64.  There sigmoid(g*) = 1 + 1/g*,
    so silu(g*) = g* + 1."""
    g = -1.28
    for _ in range(60):
        f = 1.0 + g + math.exp(g)
        fp = 1.0 + math.exp(g)
        g -= f / fp
    return g


SILU_MIN_G = _silu_min_point()
SILU_MIN_VAL = SILU_MIN_G + 1.0

FP16_MAX = 65504.0
FP16_OVERFLOW = 65520.0        # RNE rounds |v| >= this to infinity


def _fp16_grid_down(v: np.ndarray) -> np.ndarray:
    """Largest value <= v on the fp16 grid extended by +-inf (as float64)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        h = v.astype(np.float16)                           # RNE neighbour
        over = h.astype(np.float64) > v
        h[over] = np.nextafter(h[over], np.float16(-np.inf))
    return h.astype(np.float64)


def _fp16_grid_up(v: np.ndarray) -> np.ndarray:
    return -_fp16_grid_down(-np.asarray(v, np.float64))


def swiglu_interval(g: np.ndarray, u: np.ndarray, eg: np.ndarray, eu: np.ndarray,
                    rel_slack: float = 2.0 ** -20):
    """Acceptance interval [lo16, hi16] (fp16 values, as fp64) for
    h = fp16(silu(g') * u') over the box g' in [g-eg, g+eg], u' in [u-eu, u+eu].

    silu is decreasing below g* and increasing above it, so its range over an
    interval is set by the end points and, when g* is inside, by silu(g*).  The
    product with u' is bilinear, so its extremes are at the corners.  The
    bounds are widened by rel_slack (the GPU's exp and division) and rounded
    outward to the fp16 grid; values past the fp16 range map to +-inf as IEEE
    round-to-nearest does.
    """
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    gl, gh = g - eg, g + eg
    sl, sh = silu(gl), silu(gh)
    smin = np.minimum(sl, sh)
    smax = np.maximum(sl, sh)
    inside = (gl <= SILU_MIN_G) & (SILU_MIN_G <= gh)
    smin = np.where(inside, np.minimum(smin, SILU_MIN_VAL), smin)
    ul, uh = u - eu, u + eu
    corners = np.stack([smin * ul, smin * uh, smax * ul, smax * uh])
    lo = corners.min(axis=0)
    hi = corners.max(axis=0)
    lo = lo - np.abs(lo) * rel_slack
    hi = hi + np.abs(hi) * rel_slack
    lo16 = _fp16_grid_down(lo)
    hi16 = _fp16_grid_up(hi)
    # IEEE overflow: anything that rounds past the range is +-inf
    hi16 = np.where(hi >= FP16_OVERFLOW, np.inf, hi16)
    lo16 = np.where(lo <= -FP16_OVERFLOW, -np.inf, lo16)
    lo16 = np.where(lo >= FP16_OVERFLOW, np.inf, lo16)
    hi16 = np.where(hi <= -FP16_OVERFLOW, -np.inf, hi16)
    return lo16, hi16


def swiglu_accepts(h_gpu: np.ndarray, lo16: np.ndarray, hi16: np.ndarray) -> np.ndarray:
    """Boolean mask: h_gpu (fp16 values) inside [lo16, hi16]; NaN never accepted."""
    h = np.asarray(h_gpu, np.float64)
    return (h >= lo16) & (h <= hi16)


# -------------------------------------------------------------- RMSNorm ---

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of the rows of x (fp16 [M,K]) in fp64: x * g / sqrt(mean(x^2) + eps).
    g is the per-column weight (read exactly, e.g. fp32 values), eps >= 0."""
    xb = _c(np.asarray(x, dtype=np.float16).view(np.uint16), np.uint16)
    M, K = xb.shape
    gd = _c(np.asarray(g, dtype=np.float64).reshape(-1), np.float64)
    assert gd.size == K
    out = np.empty((M, K), np.float64)
    lib().oracle_rmsnorm(_ptr(xb), _ptr(gd), float(eps), M, K, _ptr(out))
    return out


def gemm_f64x(x: np.ndarray, w_bits: np.ndarray):
    """y = x W^T and S = sum |x w| in fp64 with fp64 x [M,K] and fp16 W bits [N,K]."""
    xd = _c(x, np.float64)
    wb = _c(w_bits, np.uint16)
    M, K = xd.shape
    N, K2 = wb.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = lib().oracle_gemm_f64x(_ptr(xd), _ptr(wb), M, N, K, _ptr(y), _ptr(s))
    assert rc == 0
    return y, s


def rmsnorm_gemm_quant(fmt: str, x: np.ndarray, g: np.ndarray, eps: float, wq: np.ndarray, n: int, k: int):
    """Oracle of RMSNorm followed by the quantised GEMM: the exact normalized
    activations (fp64, not rounded) times the exactly dequantised fp16 weights."""
    return gemm_f64x(rmsnorm(x, g, eps), dequant(fmt, wq, n, k))


# fp32 arithmetic on the GPU side of a normalized activation: a sum of squares
# over K terms (per-thread runs of at most K/256 terms, then a tree), a square
# root and a division, two products.  2^-16 relative covers that with margin
# for K up to 2^16 and stays below one fp16 ulp (2^-10 relative).
RMSNORM_REL_SLACK = 2.0 ** -16


def f16_interval(exact: np.ndarray, abs_slack: np.ndarray):
    """Acceptance interval [lo16, hi16] (fp16 values as fp64) for an fp16
    result whose exact value is ``exact`` and whose computation before the
    final rounding may be off by ``abs_slack``: the fp16 grid points around
    [exact - abs_slack, exact + abs_slack], rounded outward."""
    e = np.asarray(exact, np.float64)
    sl = np.asarray(abs_slack, np.float64)
    return _fp16_grid_down(e - sl), _fp16_grid_up(e + sl)


def rmsnorm_f16_interval(xhat: np.ndarray, rel_slack: float = RMSNORM_REL_SLACK):
    """Acceptance interval [lo16, hi16] (fp16 values as fp64) for an fp16
    normalized activation whose exact value is xhat: the fp16 grid points
    around [xhat - |xhat| rel_slack, xhat + |xhat| rel_slack], rounded
    outward."""
    xh = np.asarray(xhat, np.float64)
    lo = xh - np.abs(xh) * rel_slack
    hi = xh + np.abs(xh) * rel_slack
    return _fp16_grid_down(lo), _fp16_grid_up(hi)
