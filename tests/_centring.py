"""Q4_K blocks for the decode kernel's factored dot product (test code).

The decode kernel computes, per 32-weight sub-block with a = d*sc and
b = dmin*m, sum x (a q - b) = a * sum x (q - c) - (b - a c) * sum x, where c
is the integer in [0, 15] nearest b / a.  centring_fields() draws sub-blocks
that hit every case sizing those terms: sc = 0 with and without a min, m = 0,
b / a on a half-integer tie, b / a above 15 (c clamped), weights cancelling to
exact zeros, and random fields.  Blocks listed in all_zero_blocks hold only
exact zeros.  pack_fields() turns the fields into GGUF bytes with the
test-side packer.
"""
from __future__ import annotations

import numpy as np

from _packing import f16_bits, pack_q4k


def centring_fields(rng, n_blocks, all_zero_blocks=()):
    """-> d_bits, dmin_bits [n] (fp16 bit patterns), sc, mn [n, 8], q [n, 256]."""
    d_choices = [f16_bits(0.01), f16_bits(0.5), f16_bits(2.0 ** -20), f16_bits(3.0e-3)]
    d_bits = np.zeros(n_blocks, np.int64)
    dmin_bits = np.zeros(n_blocks, np.int64)
    sc = np.zeros((n_blocks, 8), np.int64)
    mn = np.zeros((n_blocks, 8), np.int64)
    q = np.zeros((n_blocks, 256), np.int64)
    for bi in range(n_blocks):
        d = int(rng.choice(d_choices))
        dmin = d if rng.random() < 0.6 else int(rng.choice(d_choices))
        for j in range(8):
            case = (bi * 8 + j) % 9 if bi not in all_zero_blocks else 5
            qj = rng.integers(0, 16, 32)
            if case == 0:      # a = 0, b > 0: every weight is -b
                s, m = 0, int(rng.integers(1, 64))
            elif case == 1:    # a = b = 0
                s, m = 0, 0
            elif case == 2:    # b = 0: c = 0
                s, m = int(rng.integers(1, 64)), 0
            elif case == 3:    # b / a = k + 1/2 when dmin = d (a tie for c)
                s, m = 2, 2 * int(rng.integers(0, 15)) + 1
            elif case == 4:    # b / a > 15: c clamped to 15
                s, m = 1, int(rng.integers(16, 64))
            elif case == 5:    # q = c and b = a c: exact zeros when dmin = d
                q0 = int(rng.integers(0, 16))
                s = int(rng.integers(1, 4))
                m = s * q0
                qj = np.full(32, q0)
            elif case == 6:    # b / a just above 15 (15.25)
                s, m = 4, 61
            elif case == 7:    # half the quants on c, the rest random
                q0 = int(rng.integers(0, 16))
                s = int(rng.integers(1, 4))
                m = s * q0
                qj = np.where(rng.random(32) < 0.5, q0, qj)
            else:              # random fields
                s, m = int(rng.integers(0, 64)), int(rng.integers(0, 64))
            sc[bi, j], mn[bi, j] = s, m
            q[bi, 32 * j:32 * j + 32] = qj
        if bi in all_zero_blocks:
            dmin = d
        d_bits[bi], dmin_bits[bi] = d, dmin
    return d_bits, dmin_bits, sc, mn, q


def pack_fields(d_bits, dmin_bits, sc, mn, q) -> np.ndarray:
    return np.stack([pack_q4k(int(d_bits[i]), int(dmin_bits[i]), sc[i], mn[i], q[i]) for i in range(len(d_bits))])


def centring_blocks(rng, n_blocks, all_zero_blocks=()) -> np.ndarray:
    return pack_fields(*centring_fields(rng, n_blocks, all_zero_blocks))
