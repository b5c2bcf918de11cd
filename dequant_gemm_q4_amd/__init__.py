"""Python binding of libdmq.so (fused Q4_K / Q6_K dequant-GEMM for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libdmq.so.  PyTorch supplies device memory and the current stream.
The functions carry the names of the C ABI (include/dmq.h) and take torch
tensors; each checks dtypes, devices, contiguity and byte sizes (the C side
cannot see buffer sizes) and raises DmqError on a non-zero status.

Importing this package fails loudly when libdmq.so has not been built:
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdmq.so")

DMQ_OK = 0
DMQ_ERR_INVALID_ARG = -1
DMQ_ERR_ALIGNMENT = -2
DMQ_ERR_UNSUPPORTED = -3
DMQ_ERR_HIP = -4
DMQ_ERR_SCRATCH = -5
DMQ_NOALLOC_SCRATCH_BYTES = 32 << 20
DMQ_FMT_Q4K = 0
DMQ_FMT_Q6K = 1

QK = 256
BLOCK_BYTES = {DMQ_FMT_Q4K: 144, DMQ_FMT_Q6K: 210}
FORMATS = {"q4k": DMQ_FMT_Q4K, "q6k": DMQ_FMT_Q6K}

# Every entry point declared in include/dmq.h.
EXPORTS = ("dmq_dequant_q4k", "dmq_dequant_q6k", "dmq_gemm_q4k", "dmq_gemm_q6k",
           "dmq_ffn_swiglu_q4k", "dmq_gemm_group", "dmq_rmsnorm_gemm", "dmq_rope_kv_cache",
           "dmq_attention_gqa", "dmq_rope_attention_gqa", "dmq_attention_gqa_noalloc", "dmq_residual_rmsnorm",
           "dmq_residual_rmsnorm_gemm", "dmq_layer_prefill", "dmq_status_string", "dmq_version")
HEAD_DIM = 128


class DmqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class GemmDesc(ctypes.Structure):
    """Mirror of dmq_gemm_desc."""
    _fields_ = [("format", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("x_f16", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class ProjDesc(ctypes.Structure):
    """Mirror of dmq_proj_desc."""
    _fields_ = [("format", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("wq", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64)]


class LayerWeights(ctypes.Structure):
    """Mirror of dmq_layer_weights."""
    _fields_ = [("fmt_q", ctypes.c_int32), ("fmt_k", ctypes.c_int32), ("fmt_v", ctypes.c_int32),
                ("fmt_o", ctypes.c_int32), ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p),
                ("wo", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("g_ffn", ctypes.c_void_p), ("g_next", ctypes.c_void_p), ("freq_factors", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


class LayerBuffers(ctypes.Structure):
    """Mirror of dmq_layer_buffers."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("h_in", "xn_in", "yq", "yk", "yv", "q_rot", "attn", "yo", "h_mid",
                                                "xn_ffn", "h_ffn", "y_down", "h_out", "xn_out")]


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime with the same SONAME as /opt/rocm's
    # (libamdhip64.so.7).  Loading torch first makes libdmq.so bind to that
    # already-loaded runtime, so torch's streams and device pointers are valid
    # in our calls; loading libdmq.so first would map a second HIP / HSA
    # runtime into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python dequant_gemm_q4_amd/build.py) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.dmq_dequant_q4k.argtypes = [P, P, I64, I64, P]
    L.dmq_dequant_q6k.argtypes = [P, P, I64, I64, P]
    L.dmq_gemm_q4k.argtypes = [P, P, P, I64, I64, I64, P]
    L.dmq_gemm_q6k.argtypes = [P, P, P, I64, I64, I64, P]
    L.dmq_ffn_swiglu_q4k.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    L.dmq_gemm_group.argtypes = [ctypes.POINTER(GemmDesc), I32, P]
    L.dmq_rmsnorm_gemm.argtypes = [P, P, ctypes.c_float, P, I64, I64, ctypes.POINTER(ProjDesc), I32, P]
    L.dmq_rope_kv_cache.argtypes = [P, P, P, I64, I64, I32, I32, ctypes.c_double, P, P, P, P, I64, P]
    L.dmq_attention_gqa.argtypes = [P, P, P, P, I64, I64, I32, I32, I64, P]
    L.dmq_rope_attention_gqa.argtypes = [P, P, P, I64, I64, I32, I32, ctypes.c_double, P, P, P, P, I64, P, P]
    L.dmq_attention_gqa_noalloc.argtypes = [P, P, P, P, I64, I64, I32, I32, I64, P]
    L.dmq_layer_prefill.argtypes = [ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerBuffers), I64, I64, I32, I32,
                                    I32, I32, I64, ctypes.c_double, ctypes.c_float, I64, P, P]
    L.dmq_residual_rmsnorm.argtypes = [P, P, P, ctypes.c_float, P, P, I64, I64, P]
    L.dmq_residual_rmsnorm_gemm.argtypes = [P, P, P, ctypes.c_float, P, P, I64, I64, ctypes.POINTER(ProjDesc),
                                            I32, P]
    for name in ("dmq_dequant_q4k", "dmq_dequant_q6k", "dmq_gemm_q4k", "dmq_gemm_q6k",
                 "dmq_ffn_swiglu_q4k", "dmq_gemm_group", "dmq_rmsnorm_gemm", "dmq_rope_kv_cache",
                 "dmq_attention_gqa", "dmq_rope_attention_gqa", "dmq_attention_gqa_noalloc",
                 "dmq_residual_rmsnorm", "dmq_residual_rmsnorm_gemm", "dmq_layer_prefill"):
        getattr(L, name).restype = ctypes.c_int
    L.dmq_status_string.argtypes = [ctypes.c_int]
    L.dmq_status_string.restype = ctypes.c_char_p
    L.dmq_version.argtypes = []
    L.dmq_version.restype = ctypes.c_int
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.dmq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != DMQ_OK:
        raise DmqError(status, where)


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev_tensor(t, dtype, name: str, numel: int):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _wq_bytes(fmt: int, rows: int, k: int) -> int:
    if k % QK:
        raise ValueError("K must be a multiple of 256")
    return rows * (k // QK) * BLOCK_BYTES[fmt]


def dmq_dequant_q4k(wq, w_f16, rows: int, k: int, stream=None) -> None:
    """w_f16[rows, k] (float16) <- exact Q4_K dequant of wq (uint8 blocks)."""
    import torch
    pw = _dev_tensor(wq, torch.uint8, "wq", _wq_bytes(DMQ_FMT_Q4K, rows, k))
    po = _dev_tensor(w_f16, torch.float16, "w_f16", rows * k)
    _check(lib.dmq_dequant_q4k(pw, po, rows, k, _stream(stream)), "dmq_dequant_q4k")


def dmq_dequant_q6k(wq, w_f16, rows: int, k: int, stream=None) -> None:
    """w_f16[rows, k] (float16) <- exact Q6_K dequant of wq (uint8 blocks)."""
    import torch
    pw = _dev_tensor(wq, torch.uint8, "wq", _wq_bytes(DMQ_FMT_Q6K, rows, k))
    po = _dev_tensor(w_f16, torch.float16, "w_f16", rows * k)
    _check(lib.dmq_dequant_q6k(pw, po, rows, k, _stream(stream)), "dmq_dequant_q6k")


def _gemm(fmt: int, name: str, x, wq, y, M: int, N: int, K: int, stream) -> None:
    import torch
    px = _dev_tensor(x, torch.float16, "x", M * K)
    pw = _dev_tensor(wq, torch.uint8, "wq", _wq_bytes(fmt, N, K))
    py = _dev_tensor(y, torch.float32, "y", M * N)
    _check(getattr(lib, name)(px, pw, py, M, N, K, _stream(stream)), name)


def dmq_gemm_q4k(x, wq, y, M: int, N: int, K: int, stream=None) -> None:
    """y[M, N] (float32) <- x[M, K] (float16) * W^T, W in Q4_K (N rows of K/256 blocks)."""
    _gemm(DMQ_FMT_Q4K, "dmq_gemm_q4k", x, wq, y, M, N, K, stream)


def dmq_gemm_q6k(x, wq, y, M: int, N: int, K: int, stream=None) -> None:
    """y[M, N] (float32) <- x[M, K] (float16) * W^T, W in Q6_K."""
    _gemm(DMQ_FMT_Q6K, "dmq_gemm_q6k", x, wq, y, M, N, K, stream)


def dmq_ffn_swiglu_q4k(x, w_gate_up_q4k, w_down_q6k, h_f16, y, M: int, D: int, F: int,
                       stream=None) -> None:
    """h = silu(x Wg^T) * (x Wu^T) (float16 [M, F]); y = h Wd^T (float32 [M, D])."""
    import torch
    px = _dev_tensor(x, torch.float16, "x", M * D)
    pgu = _dev_tensor(w_gate_up_q4k, torch.uint8, "w_gate_up_q4k", _wq_bytes(DMQ_FMT_Q4K, 2 * F, D))
    pd = _dev_tensor(w_down_q6k, torch.uint8, "w_down_q6k", _wq_bytes(DMQ_FMT_Q6K, D, F))
    ph = _dev_tensor(h_f16, torch.float16, "h_f16", M * F)
    py = _dev_tensor(y, torch.float32, "y", M * D)
    _check(lib.dmq_ffn_swiglu_q4k(px, pgu, pd, ph, py, M, D, F, _stream(stream)), "dmq_ffn_swiglu_q4k")


def make_group(problems):
    """problems: iterable of (format, x, wq, y, M, N, K) with format 'q4k'/'q6k'
    or DMQ_FMT_*; returns the ctypes dmq_gemm_desc array (sizes checked)."""
    import torch
    problems = list(problems)
    arr = (GemmDesc * len(problems))()
    for i, (fmt, x, wq, y, M, N, K) in enumerate(problems):
        fmt = FORMATS.get(fmt, fmt)
        arr[i].format = fmt
        arr[i].reserved = 0
        arr[i].x_f16 = _dev_tensor(x, torch.float16, f"x[{i}]", M * K)
        arr[i].wq = _dev_tensor(wq, torch.uint8, f"wq[{i}]", _wq_bytes(fmt, N, K))
        arr[i].y = _dev_tensor(y, torch.float32, f"y[{i}]", M * N)
        arr[i].M, arr[i].N, arr[i].K = M, N, K
    return arr


def dmq_gemm_group(problems, stream=None) -> None:
    """Run several independent GEMMs in one launch per kernel kind.

    ``problems`` is a list of (format, x, wq, y, M, N, K) or the array returned
    by make_group (reusing it avoids re-marshalling in timing loops)."""
    arr = problems if isinstance(problems, ctypes.Array) else make_group(problems)
    _check(lib.dmq_gemm_group(arr, len(arr), _stream(stream)), "dmq_gemm_group")


PROJ_SWIGLU = 1


def make_projs(projs, K: int):
    """projs: iterable of (format, wq, y, N) or (format, wq, h, N, "swiglu")
    (a Q4_K gate|up pair whose output is h = silu(gate) * up, float16
    [M, N/2]); returns the ctypes dmq_proj_desc array (sizes checked against
    K and the output's element count / M below)."""
    import torch
    projs = list(projs)
    arr = (ProjDesc * len(projs))()
    for i, pr in enumerate(projs):
        fmt, wq, y, N = pr[:4]
        swiglu = len(pr) > 4 and pr[4] == "swiglu"
        fmt = FORMATS.get(fmt, fmt)
        arr[i].format = fmt
        arr[i].flags = PROJ_SWIGLU if swiglu else 0
        arr[i].wq = _dev_tensor(wq, torch.uint8, f"wq[{i}]", _wq_bytes(fmt, N, K))
        want = torch.float16 if swiglu else torch.float32
        if not isinstance(y, torch.Tensor) or y.dtype != want or not y.is_cuda or not y.is_contiguous():
            raise TypeError(f"y[{i}] must be a contiguous {want} GPU tensor")
        arr[i].y = y.data_ptr()
        arr[i].N = N
    return arr


def _check_proj_outputs(projs, arr, M: int) -> None:
    if isinstance(projs, ctypes.Array):
        return
    for i, pr in enumerate(list(projs)):
        n_out = arr[i].N // 2 if arr[i].flags & PROJ_SWIGLU else arr[i].N
        if pr[2].numel() != M * n_out:
            raise ValueError(f"y[{i}] has {pr[2].numel()} elements, expected {M * n_out}")


def dmq_rmsnorm_gemm(x, g, eps: float, xn, projs, M: int, K: int, stream=None) -> None:
    """y_i[M, N_i] (float32) <- RMSNorm(x; g, eps) * W_i^T for each projection.

    x: float16 [M, K]; g: float32 [K]; xn: float16 [M, K] output (the
    normalized activations), or None when M = 1 and K <= 32768 (the decode
    kernel normalizes while staging x).  ``projs``: list of (format, wq, y, N)
    or the array returned by make_projs."""
    import torch
    px = _dev_tensor(x, torch.float16, "x", M * K)
    pg = _dev_tensor(g, torch.float32, "g", K)
    pn = None if xn is None else _dev_tensor(xn, torch.float16, "xn", M * K)
    arr = projs if isinstance(projs, ctypes.Array) else make_projs(projs, K)
    _check_proj_outputs(projs, arr, M)
    _check(lib.dmq_rmsnorm_gemm(px, pg, float(eps), pn, M, K, arr, len(arr), _stream(stream)),
           "dmq_rmsnorm_gemm")


def dmq_residual_rmsnorm_gemm(h_in, y_add, g, eps: float, h_out, xn, projs, M: int, K: int, stream=None) -> None:
    """h_out <- h_in + y_add (float32 [M, K], h_out a separate buffer), then
    y_i <- RMSNorm(h_out; g, eps) * W_i^T as in dmq_rmsnorm_gemm.  xn: float16
    [M, K] or None when M = 1 and K <= 32768 (one decode launch)."""
    import torch
    ph = _dev_tensor(h_in, torch.float32, "h_in", M * K)
    pa = _dev_tensor(y_add, torch.float32, "y_add", M * K)
    pg = _dev_tensor(g, torch.float32, "g", K)
    po = _dev_tensor(h_out, torch.float32, "h_out", M * K)
    pn = None if xn is None else _dev_tensor(xn, torch.float16, "xn", M * K)
    arr = projs if isinstance(projs, ctypes.Array) else make_projs(projs, K)
    _check_proj_outputs(projs, arr, M)
    _check(lib.dmq_residual_rmsnorm_gemm(ph, pa, pg, float(eps), po, pn, M, K, arr, len(arr), _stream(stream)),
           "dmq_residual_rmsnorm_gemm")


def dmq_rope_kv_cache(q, k, v, M: int, pos0: int, n_q_heads: int, n_kv_heads: int, q_out, k_cache, v_cache,
                      cache_len: int, theta: float = 500000.0, freq_factors=None, stream=None) -> None:
    """RoPE on q [M, Hq*128] and k [M, Hkv*128] (float32, positions pos0..pos0+M-1);
    q_out float16 [M, Hq*128]; rotated k and v written as float16 into rows
    pos0..pos0+M-1 of the caches [Hkv, cache_len, 128]."""
    import torch
    D = HEAD_DIM
    pq = _dev_tensor(q, torch.float32, "q", M * n_q_heads * D)
    pk = _dev_tensor(k, torch.float32, "k", M * n_kv_heads * D)
    pv = _dev_tensor(v, torch.float32, "v", M * n_kv_heads * D)
    pf = None if freq_factors is None else _dev_tensor(freq_factors, torch.float32, "freq_factors", D // 2)
    po = _dev_tensor(q_out, torch.float16, "q_out", M * n_q_heads * D)
    pkc = _dev_tensor(k_cache, torch.float16, "k_cache", n_kv_heads * cache_len * D)
    pvc = _dev_tensor(v_cache, torch.float16, "v_cache", n_kv_heads * cache_len * D)
    _check(lib.dmq_rope_kv_cache(pq, pk, pv, M, pos0, n_q_heads, n_kv_heads, float(theta), pf, po, pkc, pvc,
                                 cache_len, _stream(stream)), "dmq_rope_kv_cache")


def dmq_rope_attention_gqa(q, k, v, M: int, pos0: int, n_q_heads: int, n_kv_heads: int, q_out, k_cache, v_cache,
                           cache_len: int, out, theta: float = 500000.0, freq_factors=None, stream=None) -> None:
    """dmq_rope_kv_cache then dmq_attention_gqa in one call (one kernel fewer at
    M = 1): q_out float16 [M, Hq*128] receives the rotated queries, rows
    pos0..pos0+M-1 of the caches the rotated k and the v, out float16
    [M, Hq*128] the attention output."""
    import torch
    D = HEAD_DIM
    pq = _dev_tensor(q, torch.float32, "q", M * n_q_heads * D)
    pk = _dev_tensor(k, torch.float32, "k", M * n_kv_heads * D)
    pv = _dev_tensor(v, torch.float32, "v", M * n_kv_heads * D)
    pf = None if freq_factors is None else _dev_tensor(freq_factors, torch.float32, "freq_factors", D // 2)
    pqo = _dev_tensor(q_out, torch.float16, "q_out", M * n_q_heads * D)
    pkc = _dev_tensor(k_cache, torch.float16, "k_cache", n_kv_heads * cache_len * D)
    pvc = _dev_tensor(v_cache, torch.float16, "v_cache", n_kv_heads * cache_len * D)
    po = _dev_tensor(out, torch.float16, "out", M * n_q_heads * D)
    _check(lib.dmq_rope_attention_gqa(pq, pk, pv, M, pos0, n_q_heads, n_kv_heads, float(theta), pf, pqo, pkc, pvc,
                                      cache_len, po, _stream(stream)), "dmq_rope_attention_gqa")


def dmq_attention_gqa(q, k_cache, v_cache, out, M: int, pos0: int, n_q_heads: int, n_kv_heads: int,
                      cache_len: int, stream=None) -> None:
    """out float16 [M, Hq*128] <- causal grouped-query attention of q (float16,
    positions pos0..pos0+M-1) over the caches [Hkv, cache_len, 128]."""
    import torch
    D = HEAD_DIM
    pq = _dev_tensor(q, torch.float16, "q", M * n_q_heads * D)
    pkc = _dev_tensor(k_cache, torch.float16, "k_cache", n_kv_heads * cache_len * D)
    pvc = _dev_tensor(v_cache, torch.float16, "v_cache", n_kv_heads * cache_len * D)
    po = _dev_tensor(out, torch.float16, "out", M * n_q_heads * D)
    _check(lib.dmq_attention_gqa(pq, pkc, pvc, po, M, pos0, n_q_heads, n_kv_heads, cache_len, _stream(stream)),
           "dmq_attention_gqa")


def dmq_attention_gqa_noalloc(q, k_cache, v_cache, out, M: int, pos0: int, n_q_heads: int, n_kv_heads: int,
                              cache_len: int, stream=None) -> None:
    """dmq_attention_gqa without any device allocation: the decode path's
    partial states go to the library's fixed per-GPU scratch (calls that
    overlap on one GPU race)."""
    import torch
    D = HEAD_DIM
    pq = _dev_tensor(q, torch.float16, "q", M * n_q_heads * D)
    pkc = _dev_tensor(k_cache, torch.float16, "k_cache", n_kv_heads * cache_len * D)
    pvc = _dev_tensor(v_cache, torch.float16, "v_cache", n_kv_heads * cache_len * D)
    po = _dev_tensor(out, torch.float16, "out", M * n_q_heads * D)
    _check(lib.dmq_attention_gqa_noalloc(pq, pkc, pvc, po, M, pos0, n_q_heads, n_kv_heads, cache_len,
                                         _stream(stream)), "dmq_attention_gqa_noalloc")


def dmq_residual_rmsnorm(h_in, y, g, eps: float, h_out, xn, M: int, K: int, stream=None) -> None:
    """h_out = h_in + y (float32 [M, K]); with g (float32 [K]) also
    xn float16 [M, K] = RMSNorm(h_out; g, eps).  g=None: the add only."""
    import torch
    ph = _dev_tensor(h_in, torch.float32, "h_in", M * K)
    py = _dev_tensor(y, torch.float32, "y", M * K)
    po = _dev_tensor(h_out, torch.float32, "h_out", M * K)
    pg = None if g is None else _dev_tensor(g, torch.float32, "g", K)
    pn = None if g is None else _dev_tensor(xn, torch.float16, "xn", M * K)
    _check(lib.dmq_residual_rmsnorm(ph, py, pg, float(eps), po, pn, M, K, _stream(stream)), "dmq_residual_rmsnorm")


def make_layer(weights: dict, buffers: dict, M: int, D: int, F: int, n_q_heads: int, n_kv_heads: int,
               cache_len: int):
    """(LayerWeights, LayerBuffers) for dmq_layer_prefill from dicts of torch
    tensors, each checked for device, dtype, contiguity and size.  weights:
    q, k, v, o (uint8 blocks; formats fmt_q .. fmt_o, default "q4k"),
    gate_up (Q4_K, 2F rows), down (Q6_K), g_ffn, optional g_next and
    freq_factors (float32), k_cache, v_cache (float16 [Hkv, cache_len, 128]).
    buffers: h_in, xn_in, yq, yk, yv, q_rot, attn, yo, h_mid, xn_ffn, h_ffn,
    y_down, h_out and (with g_next) xn_out.  Keep the tensors alive while the
    structures are in use."""
    import torch
    QD, KD = n_q_heads * HEAD_DIM, n_kv_heads * HEAD_DIM
    fm = {k: FORMATS[weights.get("fmt_" + k, "q4k")] for k in ("q", "k", "v", "o")}
    wt = lambda name, fmt, rows, k: _dev_tensor(weights[name], torch.uint8, name, _wq_bytes(fmt, rows, k))  # noqa: E731
    lw = LayerWeights()
    lw.fmt_q, lw.fmt_k, lw.fmt_v, lw.fmt_o = fm["q"], fm["k"], fm["v"], fm["o"]
    lw.wq = wt("q", fm["q"], QD, D)
    lw.wk = wt("k", fm["k"], KD, D)
    lw.wv = wt("v", fm["v"], KD, D)
    lw.wo = wt("o", fm["o"], D, QD)
    lw.w_gate_up = wt("gate_up", DMQ_FMT_Q4K, 2 * F, D)
    lw.w_down = wt("down", DMQ_FMT_Q6K, D, F)
    lw.g_ffn = _dev_tensor(weights["g_ffn"], torch.float32, "g_ffn", D)
    lw.g_next = None if weights.get("g_next") is None else _dev_tensor(weights["g_next"], torch.float32, "g_next", D)
    ff = weights.get("freq_factors")
    lw.freq_factors = None if ff is None else _dev_tensor(ff, torch.float32, "freq_factors", HEAD_DIM // 2)
    lw.k_cache = _dev_tensor(weights["k_cache"], torch.float16, "k_cache", KD * cache_len)
    lw.v_cache = _dev_tensor(weights["v_cache"], torch.float16, "v_cache", KD * cache_len)
    shapes = {"h_in": (torch.float32, D), "xn_in": (torch.float16, D), "yq": (torch.float32, QD),
              "yk": (torch.float32, KD), "yv": (torch.float32, KD), "q_rot": (torch.float16, QD),
              "attn": (torch.float16, QD), "yo": (torch.float32, D), "h_mid": (torch.float32, D),
              "xn_ffn": (torch.float16, D), "h_ffn": (torch.float16, F), "y_down": (torch.float32, D),
              "h_out": (torch.float32, D), "xn_out": (torch.float16, D)}
    lb = LayerBuffers()
    for name, (dt, width) in shapes.items():
        t = buffers.get(name)
        setattr(lb, name, None if t is None else _dev_tensor(t, dt, name, M * width))
    return lw, lb


def dmq_layer_prefill(layer, M: int, pos0: int, D: int, F: int, n_q_heads: int, n_kv_heads: int, cache_len: int,
                      eps: float, chunk: int, stream_attn=None, stream_ffn=None, theta: float = 500000.0) -> None:
    """One decoder layer's prefill with attention and FFN chunks overlapped
    on two streams (the same stream twice: serial); layer = make_layer(...)."""
    lw, lb = layer
    _check(lib.dmq_layer_prefill(ctypes.byref(lw), ctypes.byref(lb), M, pos0, D, F, n_q_heads, n_kv_heads, cache_len,
                                 float(theta), float(eps), chunk, _stream(stream_attn),
                                 _stream(stream_ffn if stream_ffn is not None else stream_attn)),
           "dmq_layer_prefill")


def dmq_version() -> int:
    return int(lib.dmq_version())
