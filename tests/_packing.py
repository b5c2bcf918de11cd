"""Test-side block packers: fields -> raw GGUF k-quant bytes.

Written from the public GGUF k-quant byte layout (the pages name the Q4_K /
Q6_K formats -- article "Building DAMASCUS", section "Read the model, then
reproduce its operations" -- but do not print their bytes).  Used to hand-build
blocks with known fields for the oracle pins and the GPU edge cases.  This is
test code: it is not used by the oracle or by the HIP library.

Q4_K (144 B): d fp16 @0, dmin fp16 @2, 12 scale bytes @4, 128 quant bytes @16.
  scale/min j < 4 : low 6 bits of byte j / byte j+4
  scale/min j >= 4: low/high nibble of byte j+4, plus 2 high bits stored in the
                    top 2 bits of byte j-4 (scale) / byte j (min)
  quant of weight 32j + l lives in quant byte 32*(j//2) + l, low nibble for
  even j, high nibble for odd j.
Q6_K (210 B): ql @0 (128 B), qh @128 (64 B), int8 scales @192 (16 B), d @208.
  weight 128h + 32t + l: low 4 bits in ql[64h + 32*(t%2) + l] (low nibble for
  t < 2, high for t >= 2), high 2 bits at bit 2t of qh[32h + l]; scale index
  is weight // 16.
"""
from __future__ import annotations

import numpy as np


def f16_bits(value: float) -> int:
    return int(np.array([value], dtype=np.float16).view(np.uint16)[0])


def pack_q4k(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    q = [int(v) for v in q]
    assert len(sc) == 8 and len(mn) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + mn) and all(0 <= v < 16 for v in q)
    b = np.zeros(144, np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    b[2], b[3] = dmin_bits & 0xFF, dmin_bits >> 8
    s = np.zeros(12, np.int64)
    for j in range(4):
        s[j] |= sc[j]
        s[j + 4] |= mn[j]
    for j in range(4, 8):
        s[j + 4] |= (sc[j] & 15) | ((mn[j] & 15) << 4)
        s[j - 4] |= (sc[j] >> 4) << 6
        s[j] |= (mn[j] >> 4) << 6
    b[4:16] = s.astype(np.uint8)
    qs = np.zeros(128, np.int64)
    for i in range(256):
        j, l = divmod(i, 32)
        idx = 32 * (j // 2) + l
        qs[idx] |= q[i] if j % 2 == 0 else q[i] << 4
    b[16:144] = qs.astype(np.uint8)
    return b


def pack_q6k(d_bits: int, sc, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    q = [int(v) for v in q]
    assert len(sc) == 16 and len(q) == 256
    assert all(-128 <= v < 128 for v in sc) and all(0 <= v < 64 for v in q)
    b = np.zeros(210, np.uint8)
    ql = np.zeros(128, np.int64)
    qh = np.zeros(64, np.int64)
    for i in range(256):
        h, r = divmod(i, 128)
        t, l = divmod(r, 32)
        low, high = q[i] & 15, q[i] >> 4
        li = 64 * h + 32 * (t % 2) + l
        ql[li] |= low if t < 2 else low << 4
        qh[32 * h + l] |= high << (2 * t)
    b[0:128] = ql.astype(np.uint8)
    b[128:192] = qh.astype(np.uint8)
    b[192:208] = np.array(sc, np.int64).astype(np.int8).view(np.uint8)
    b[208], b[209] = d_bits & 0xFF, d_bits >> 8
    return b
