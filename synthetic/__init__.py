"""Seeded synthetic inputs for the Q4_K / Q6_K dequant-GEMM path.

This module only draws random numbers and lays them out as raw bytes or fp16
arrays.  It holds none of the method's arithmetic (no decoding, no dequant, no
products): both the CPU oracle's tests and the HIP path's tests and benchmark
draw their inputs from here, and nothing else is shared between the two.

Shapes follow the target model named on the DAMASCUS project overview page,
section "[06] the target": 28 layers, hidden 3072, FFN 8192, 24 heads with
8 KV heads of dim 128, vocabulary 128256, tied embeddings.  The quantised
formats are the GGUF k-quant super-blocks the pages name (the Q4_K_M model
file and its Q4_K and Q6_K dequantizers, article "Building DAMASCUS", section
"Read the model, then reproduce its operations"):

* Q4_K: 144 bytes per 256 weights -- fp16 ``d`` at byte 0, fp16 ``dmin`` at
  byte 2, 12 bytes of packed 6-bit scales/mins at byte 4, 128 bytes of 4-bit
  quants at byte 16.  Every bit of the scale field belongs to exactly one
  6-bit field, so uniform random bytes give uniform scales and mins in 0..63,
  and uniform random quant bytes give uniform nibbles in 0..15.
* Q6_K: 210 bytes per 256 weights -- 128 bytes of low nibbles, 64 bytes of
  high 2-bit pairs, 16 int8 sub-block scales, fp16 ``d`` at byte 208.

The super-scales are drawn from U(1e-3, 2e-2) in fp64 and rounded to fp16
(numpy's round-to-nearest-even); activations are N(0, sigma^2) in fp64,
optionally rescaled per row to unit RMS (post-RMSNorm input), then rounded to
fp16.
"""
from __future__ import annotations

import numpy as np

QK = 256                # weights per super-block
Q4K_BYTES = 144         # bytes per Q4_K super-block
Q6K_BYTES = 210         # bytes per Q6_K super-block

# Llama-3.2-3B shape constants (project overview page, "[06] the target").
N_LAYERS = 28
HIDDEN = 3072
FFN = 8192
N_HEADS = 24
N_KV_HEADS = 8
HEAD_DIM = 128
VOCAB = 128256

# The seven projections of one decoder layer, in the order used for seeds:
# (name, format, N = output features, K = input features).
LAYER_PROJECTIONS = (
    ("q", "q4k", N_HEADS * HEAD_DIM, HIDDEN),
    ("k", "q4k", N_KV_HEADS * HEAD_DIM, HIDDEN),
    ("v", "q4k", N_KV_HEADS * HEAD_DIM, HIDDEN),
    ("o", "q4k", HIDDEN, N_HEADS * HEAD_DIM),
    ("gate", "q4k", FFN, HIDDEN),
    ("up", "q4k", FFN, HIDDEN),
    ("down", "q6k", HIDDEN, FFN),
)
LM_HEAD = ("lm_head", "q6k", VOCAB, HIDDEN)
LM_HEAD_INDEX = 7

ACT_SEED_OFFSET = 500_000_000


def weight_seed(config: int, layer: int, proj_index: int) -> int:
    """Seed of one weight matrix: 1_000_003*config + 1009*layer + proj_index."""
    return 1_000_003 * config + 1009 * layer + proj_index


def act_seed(config: int, layer: int, proj_index: int) -> int:
    return weight_seed(config, layer, proj_index) + ACT_SEED_OFFSET


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _fp16_le_bytes(values: np.ndarray) -> np.ndarray:
    """fp64 values -> fp16 (numpy RNE) -> little-endian byte pairs [n, 2]."""
    h = values.astype(np.float16).astype("<f2")
    return h.view(np.uint8).reshape(-1, 2)


def q4k_blocks(rows: int, k: int, seed: int, d_range=(1e-3, 2e-2),
               dmin_range=(1e-3, 2e-2)) -> np.ndarray:
    """Raw Q4_K bytes of a [rows, k] weight matrix, uint8 [rows, k//256*144].

    Rows are contiguous runs of k/256 super-blocks.  All 6-bit scales, mins and
    4-bit quants are uniform (uniform bytes); d and dmin are U(range) -> fp16.
    """
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = rows * (k // QK)
    rng = _rng(seed)
    blocks = rng.integers(0, 256, size=(nb, Q4K_BYTES), dtype=np.uint8)
    blocks[:, 0:2] = _fp16_le_bytes(rng.uniform(*d_range, size=nb))
    blocks[:, 2:4] = _fp16_le_bytes(rng.uniform(*dmin_range, size=nb))
    return blocks.reshape(rows, (k // QK) * Q4K_BYTES)


def q6k_blocks(rows: int, k: int, seed: int, d_range=(1e-3, 2e-2)) -> np.ndarray:
    """Raw Q6_K bytes of a [rows, k] weight matrix, uint8 [rows, k//256*210].

    ql/qh bytes are uniform (so 6-bit quants are uniform in 0..63), the 16
    sub-scales are uniform int8, and d is U(range) -> fp16.
    """
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = rows * (k // QK)
    rng = _rng(seed)
    blocks = rng.integers(0, 256, size=(nb, Q6K_BYTES), dtype=np.uint8)
    blocks[:, 208:210] = _fp16_le_bytes(rng.uniform(*d_range, size=nb))
    return blocks.reshape(rows, (k // QK) * Q6K_BYTES)


def weight_blocks(fmt: str, rows: int, k: int, seed: int) -> np.ndarray:
    if fmt == "q4k":
        return q4k_blocks(rows, k, seed)
    if fmt == "q6k":
        return q6k_blocks(rows, k, seed)
    raise ValueError(fmt)


def activations(m: int, k: int, seed: int, sigma: float = 1.0,
                unit_rms: bool = False) -> np.ndarray:
    """fp16 [m, k] activations: N(0, sigma^2) in fp64, optionally each row
    divided by sqrt(mean(x^2)) (unit RMS), then rounded to fp16 (RNE)."""
    x = _rng(seed).standard_normal((m, k)) * sigma
    if unit_rms:
        x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    return x.astype(np.float16)


def random_bytes(n: int, seed: int) -> np.ndarray:
    """n uniform random bytes (for adversarial / special-value blocks)."""
    return _rng(seed).integers(0, 256, size=n, dtype=np.uint8)


def layer_weights(config: int, layer: int):
    """The seven projection weights of one layer as (name, fmt, N, K, bytes)."""
    out = []
    for idx, (name, fmt, n, k) in enumerate(LAYER_PROJECTIONS):
        out.append((name, fmt, n, k, weight_blocks(fmt, n, k, weight_seed(config, layer, idx))))
    return out


def lm_head_weights(config: int) -> np.ndarray:
    name, fmt, n, k = LM_HEAD
    return weight_blocks(fmt, n, k, weight_seed(config, 0, LM_HEAD_INDEX))


def row_sample(m: int, count: int, seed: int, tile: int = 256) -> np.ndarray:
    """Sorted sample of row indices in [0, m) that hits every `tile`-row group
    and the last row; used for sampled checks at full size."""
    rng = _rng(seed)
    picks = set([0, m - 1])
    for t0 in range(0, m, tile):
        t1 = min(m, t0 + tile)
        picks.add(int(rng.integers(t0, t1)))
    while len(picks) < min(count, m):
        picks.add(int(rng.integers(0, m)))
    return np.array(sorted(picks), dtype=np.int64)
