"""CPU oracle for the attention side of a decoder layer: RoPE, the KV cache and
grouped-query attention, in fp64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
it; it shares no code with the HIP library.

Sources (DAMASCUS pages): the overview page's "[04] one decode step" lists
RMSNorm -> QKV projection -> RoPE -> attention over the KV cache (GQA) ->
residual add; its model table gives 24 attention heads, 8 KV heads, head
dimension 128 and RoPE theta 500000; the article's layer description says
that grouped-query attention reads the KV cache and that the attention
output returns through a residual connection.  The pages do not spell out
the RoPE pairing, the softmax scale or the causal rule; the readings taken
here (adjacent pairs (2i, 2i+1) as in GGUF files, 1/sqrt(head_dim), a query
at position p sees cache positions 0..p) are listed with the others in the
design notes.
"""
from __future__ import annotations

import numpy as np

ROPE_THETA = 500000.0


def rope_angles(pos: np.ndarray, d: int, theta: float = ROPE_THETA, freq_factors=None) -> np.ndarray:
    """Rotation angle of pair i (dims 2i, 2i+1) at each position:
    pos * theta^(-2i/d) / f_i (f_i = 1 without frequency factors).
    Returns [len(pos), d/2] fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / d)
    if freq_factors is not None:
        inv = inv / np.asarray(freq_factors, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(v: np.ndarray, pos: np.ndarray, theta: float = ROPE_THETA, freq_factors=None) -> np.ndarray:
    """Rotate each adjacent pair (v[2i], v[2i+1]) of every head vector by its
    angle: (a cos - b sin, a sin + b cos).  v: [M, H, d] (any float type),
    pos: [M] positions.  Exact arithmetic in fp64, no rounding to fp16."""
    v = np.asarray(v, dtype=np.float64)
    m, h, d = v.shape
    ang = rope_angles(pos, d, theta, freq_factors)          # [M, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = v[..., 0::2]
    b = v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def attention_gqa(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos0: int):
    """Grouped-query causal attention over a KV cache.

    q: [M, Hq, d] (queries at positions pos0 .. pos0+M-1); k_cache, v_cache:
    [Hkv, L, d] with L >= pos0 + M valid positions.  Query head h reads KV
    head h // (Hq / Hkv).  The query at position p attends to cache positions
    0..p with weights softmax_t(q . k_t / sqrt(d)).

    Returns (out [M, Hq, d], mass [M, Hq, d]) in fp64, where mass =
    sum_t p_t |v_t| (the scale of each output, for error bounds)."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    m, hq, d = q.shape
    hkv = kc.shape[0]
    group = hq // hkv
    out = np.zeros((m, hq, d))
    mass = np.zeros((m, hq, d))
    for h in range(hq):
        kv = h // group
        for i in range(m):
            n = pos0 + i + 1                      # visible positions 0..pos0+i
            s = kc[kv, :n, :] @ q[i, h, :] / np.sqrt(d)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[i, h, :] = p @ vc[kv, :n, :]
            mass[i, h, :] = p @ np.abs(vc[kv, :n, :])
    return out, mass


def rmsnorm_f64(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of the rows of x taken as they are (e.g. an fp32 residual
    stream): x * g / sqrt(mean(x^2) + eps), all in fp64."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    return x * g / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def residual_add(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """The residual connection: y + r in fp64."""
    return np.asarray(y, dtype=np.float64) + np.asarray(r, dtype=np.float64)
