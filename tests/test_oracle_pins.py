"""Pins of the CPU oracle to things other than itself (CPU only).

The pages print no worked dequant values and no GEMM outputs (their results
table is empty, article "Building DAMASCUS", section "What a reproducible
benchmark must record"), so the oracle is pinned by:

* closed-form hand-built blocks (P1, P4, P5, P6) and an exhaustive
  one-field-at-a-time sweep of the 6-bit scale packing and of every quant
  position (P2, P3);
* exact rational arithmetic (``fractions``) plus numpy's own fp64 -> fp16
  rounding for the single-rounding rule, including inputs where rounding
  through fp32 first gives a different fp16 (P7);
* numpy's fp16 conversions, exhaustively (P8);
* the byte count of the model the pages describe against their "1.9 GiB" (P9);
* numpy's fp64 matmul and exact rational sums for the triple loop (P10);
* closed forms of silu and the behaviour of the SwiGLU acceptance interval (P11);
* RMSNorm (P12): rows with a closed-form root mean square, exact scale
  invariance under powers of two, linearity in the weight g, the eps offset
  on a zero row; the fp64-activation GEMM against the fp16 one where the
  activations are fp16 values, and against numpy's matmul;
* RoPE and grouped-query attention (P13): rotations with closed-form angles,
  the identity at position 0, norm keeping, inversion, dependence on the
  distance only; attention with one visible key, with equal keys, the
  causal first query, the query-head-to-KV-head grouping, explicit loops,
  and invariance under a common rotation.

The k-quant byte layout is not on the pages; the blocks here are packed by
``tests/_packing.py`` from the public GGUF layout, so the layout pins check the
oracle against that specification, not against the pages (parity of the layout
is "unpinned by the pages").
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from _packing import f16_bits, pack_q4k, pack_q6k

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def deq4(blocks, rows=None):
    blocks = np.asarray(blocks, np.uint8).reshape(-1, 144)
    rows = rows or blocks.shape[0]
    k = blocks.shape[0] // rows * 256
    return oracle.f16_bits_to_f64(oracle.dequant_q4k(blocks, rows, k))


def deq6(blocks, rows=None):
    blocks = np.asarray(blocks, np.uint8).reshape(-1, 210)
    rows = rows or blocks.shape[0]
    k = blocks.shape[0] // rows * 256
    return oracle.f16_bits_to_f64(oracle.dequant_q6k(blocks, rows, k))


# ------------------------------------------------------------------- P8 ----

def test_p8_f16_to_f64_matches_numpy_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_bits_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_p8_f64_to_f16_rne_matches_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    v = vals[finite]
    # every fp16 value, the midpoints between neighbours, and the midpoints
    # +- one fp64 ulp; plus values beyond the range and deep underflow.
    pos = np.sort(np.unique(np.abs(v)))
    mids = (pos[:-1] + pos[1:]) / 2
    top_mid = 65504.0 + 16.0                      # midpoint to the next binade
    cand = np.concatenate([v, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                           -np.nextafter(mids, 0), -np.nextafter(mids, np.inf),
                           [top_mid, -top_mid, np.nextafter(top_mid, 0), 1e5, -1e5, np.inf,
                            -np.inf, 2.0 ** -25, 2.0 ** -26, -2.0 ** -25, 3 * 2.0 ** -26, 1e-30]])
    ours = oracle.f64_to_f16_bits(cand)
    with np.errstate(over="ignore"):
        ref = cand.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    assert oracle.f64_to_f16_bits(np.array([np.nan]))[0] & 0x7C00 == 0x7C00


def test_p8_random_doubles_match_numpy():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 18, 200000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_f16_bits(x), ref)


# ------------------------------------------------------------------- P1 ----

def test_p1_q4k_closed_form_identity_scale():
    # d = 1, dmin = 0, every scale 1, min 0: w_i is its own quant.  The quant
    # pattern differs between the low- and high-nibble sub-blocks so that a
    # nibble or sub-block mix-up shows.
    q = [(7 * i + i // 32) % 16 for i in range(256)]
    blk = pack_q4k(0x3C00, 0x0000, [1] * 8, [0] * 8, q)
    assert np.array_equal(deq4(blk)[0], np.array(q, np.float64))


def test_p1_q4k_closed_form_small_integers():
    # d = dmin = 1, sc_j = j + 1, m_j = 63 - j: w = (j+1) q - (63 - j), exact.
    q = [(5 * i + 3 * (i // 32)) % 16 for i in range(256)]
    blk = pack_q4k(0x3C00, 0x3C00, [j + 1 for j in range(8)], [63 - j for j in range(8)], q)
    want = [(i // 32 + 1) * q[i] - (63 - i // 32) for i in range(256)]
    assert np.array_equal(deq4(blk)[0], np.array(want, np.float64))


def test_q4k_every_quant_position():
    # For each position alone: q = 15 there, 0 elsewhere, d = 1, dmin = 0:
    # exactly one output equal to 15*sc at that position.
    blocks = []
    for i in range(256):
        q = [0] * 256
        q[i] = 15
        blocks.append(pack_q4k(0x3C00, 0, [2] * 8, [0] * 8, q))
    out = deq4(np.stack(blocks))        # 256 blocks as 256 rows of k=256
    assert np.array_equal(out, np.eye(256) * 30.0)


# ------------------------------------------------------------------- P2 ----

def test_p2_q4k_high_bit_packing():
    # all scales and mins at 63 (every bit of the 12 bytes set)
    blk = pack_q4k(0x3C00, 0x3C00, [63] * 8, [63] * 8, [1] * 256)
    assert np.all(blk[4:16] == 0xFF)
    assert np.all(deq4(blk)[0] == 0.0)       # 63*1 - 63
    # single-field patterns for the upper sub-blocks: only the top 2 bits of
    # each field set (value 48), read back through the dequant
    for j in range(4, 8):
        sc = [0] * 8
        sc[j] = 48
        d, dmin, scd, mnd, _ = oracle.q4k_fields(pack_q4k(0x3C00, 0, sc, [0] * 8, [0] * 256))
        assert list(scd) == sc and list(mnd) == [0] * 8
        mn = [0] * 8
        mn[j] = 48
        d, dmin, scd, mnd, _ = oracle.q4k_fields(pack_q4k(0x3C00, 0, [0] * 8, mn, [0] * 256))
        assert list(mnd) == mn and list(scd) == [0] * 8


# ------------------------------------------------------------------- P3 ----

def test_p3_q4k_scale_min_bijection_exhaustive():
    # every sub-block j and every (sc, m) in 64 x 64, read back through the
    # dequant: with d=1, dmin=0, q=1 the sub-block holds sc; with d=0, dmin=1
    # it holds -m; every other sub-block must stay exactly zero.
    vals = np.arange(64)
    for j in range(8):
        blocks_s, blocks_m, want_s, want_m = [], [], [], []
        for sc in vals:
            for mn in vals:
                scs = [0] * 8
                mns = [0] * 8
                scs[j], mns[j] = int(sc), int(mn)
                blocks_s.append(pack_q4k(0x3C00, 0x0000, scs, mns, [1] * 256))
                blocks_m.append(pack_q4k(0x0000, 0x3C00, scs, mns, [1] * 256))
                row_s = np.zeros(256)
                row_s[32 * j:32 * j + 32] = sc
                row_m = np.zeros(256)
                row_m[32 * j:32 * j + 32] = -mn
                want_s.append(row_s)
                want_m.append(row_m)
        got_s = deq4(np.stack(blocks_s))
        got_m = deq4(np.stack(blocks_m))
        assert np.array_equal(got_s, np.stack(want_s)), j
        assert np.array_equal(got_m, np.stack(want_m)), j


# ------------------------------------------------------------------- P4 ----

def test_p4_zero_quants_give_minus_dmin_m():
    # all q = 0: w = -dmin * m_j per sub-block; dmin = 0.5, m_j = 2j + 1
    blk = pack_q4k(0x3C00, f16_bits(0.5), [37] * 8, [2 * j + 1 for j in range(8)], [0] * 256)
    want = np.repeat([-(j + 0.5) for j in range(8)], 32)
    assert np.array_equal(deq4(blk)[0], want)


# ------------------------------------------------------------------- P5 ----

def test_p5_constant_blocks():
    rng = np.random.default_rng(11)
    for _ in range(50):
        d = f16_bits(rng.uniform(1e-3, 2e-2))
        dmin = f16_bits(rng.uniform(1e-3, 2e-2))
        sc, mn, q = (int(rng.integers(0, 64)), int(rng.integers(0, 64)), int(rng.integers(0, 16)))
        out = deq4(pack_q4k(d, dmin, [sc] * 8, [mn] * 8, [q] * 256))[0]
        exact = (Fraction(oracle.f16_bits_to_f64(np.array([d]))[0]) * sc * q
                 - Fraction(oracle.f16_bits_to_f64(np.array([dmin]))[0]) * mn)
        want = np.array([float(exact)]).astype(np.float16).astype(np.float64)[0]
        if exact == 0:
            want = 0.0
        assert np.all(out == want) and np.all(np.signbit(out) == np.signbit(want))
    # Q6_K constant block
    out6 = deq6(pack_q6k(f16_bits(0.25), [-3] * 16, [40] * 256))[0]
    assert np.all(out6 == 0.25 * -3 * 8)


def test_p5_fields_round_trip_random_blocks():
    rng = np.random.default_rng(12)
    for _ in range(200):
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        d = int(rng.integers(0, 0x7C00))
        dmin = int(rng.integers(0, 0x7C00))
        blk = pack_q4k(d, dmin, sc, mn, q)
        dd, ddm, scd, mnd, qd = oracle.q4k_fields(blk)
        assert list(scd) == list(sc) and list(mnd) == list(mn) and list(qd) == list(q)
        assert dd == np.array([d], np.uint16).view(np.float16).astype(np.float64)[0]
        assert ddm == np.array([dmin], np.uint16).view(np.float16).astype(np.float64)[0]
        sc6 = rng.integers(-128, 128, 16)
        q6 = rng.integers(0, 64, 256)
        d6, scd6, qd6 = oracle.q6k_fields(pack_q6k(d, sc6, q6))
        assert list(scd6) == list(sc6) and list(qd6) == list(q6)


# ------------------------------------------------------------------- P6 ----

def test_p6_q6k_closed_form():
    # d = 1, sc[s] = s - 8 (negative scales included), q_i scrambled so that
    # every quarter of the block differs: w_i = (i//16 - 8) * (q_i - 32).
    q = [(37 * i + 13 * (i // 64)) % 64 for i in range(256)]
    blk = pack_q6k(0x3C00, [s - 8 for s in range(16)], q)
    want = [(i // 16 - 8) * (q[i] - 32) for i in range(256)]
    got = deq6(blk)[0]
    assert np.array_equal(got, np.array(want, np.float64))
    assert not np.any(np.signbit(got[got == 0]))        # exact zeros are +0


def test_p6_q6k_all_q32_is_positive_zero():
    blk = pack_q6k(0x3C00, [-(s + 1) for s in range(16)], [32] * 256)
    bits = oracle.dequant_q6k(blk, 1, 256)
    assert np.all(bits == 0)


def test_q6k_every_quant_position():
    blocks = []
    for i in range(256):
        q = [32] * 256
        q[i] = 63
        blocks.append(pack_q6k(0x3C00, [3] * 16, q))
    out = deq6(np.stack(blocks))
    assert np.array_equal(out, np.eye(256) * 93.0)       # 3 * (63 - 32)


def test_q6k_scale_index_per_16():
    # one scale nonzero at a time: only its 16 weights are nonzero
    blocks = []
    for s in range(16):
        sc = [0] * 16
        sc[s] = -7
        blocks.append(pack_q6k(0x3C00, sc, [33] * 256))
    out = deq6(np.stack(blocks))
    want = np.zeros((16, 256))
    for s in range(16):
        want[s, 16 * s:16 * s + 16] = -7.0
    assert np.array_equal(out, want)


# ------------------------------------------------------------------- P7 ----

ADVERSARIAL = [
    # d bits, sc, q, dmin bits, m  -> expected fp16 bits (exact value, one RNE)
    (0x2458, 63, 15, 0x1423, 11),
    (0x245A, 63, 15, 0x1517, 7),
    (0x245B, 63, 15, 0x14CF, 33),
]


def _exact_q4k(d_bits, sc, q, dmin_bits, m):
    d = Fraction(float(np.array([d_bits], np.uint16).view(np.float16)[0]))
    dm = Fraction(float(np.array([dmin_bits], np.uint16).view(np.float16)[0]))
    return d * sc * q - dm * m


@pytest.mark.parametrize("case", ADVERSARIAL)
def test_p7_adversarial_single_rounding(case):
    d_bits, sc, q, dmin_bits, m = case
    exact = _exact_q4k(*case)
    fv = float(exact)
    assert Fraction(fv) == exact                       # exact in fp64
    want = int(np.array([fv]).astype(np.float16).view(np.uint16)[0])
    via32 = int(np.array([np.float32(fv)]).astype(np.float16).view(np.uint16)[0])
    assert want != via32                               # double rounding differs here
    blk = pack_q4k(d_bits, dmin_bits, [sc] * 8, [m] * 8, [q] * 256)
    got = oracle.dequant_q4k(blk, 1, 256)
    assert np.all(got == want)


def test_p7_random_blocks_against_rationals():
    rng = np.random.default_rng(5)
    blocks = synthetic.q4k_blocks(8, 512, seed=99)
    got = oracle.dequant_q4k(blocks, 8, 512).reshape(-1)
    flat = blocks.reshape(-1, 144)
    idx = rng.integers(0, got.size, 3000)
    for i in idx:
        b, w = divmod(int(i), 256)
        d, dmin, sc, mn, q = oracle.q4k_fields(flat[b])
        j = w // 32
        exact = Fraction(d) * int(sc[j]) * int(q[w]) - Fraction(dmin) * int(mn[j])
        want = int(np.array([float(exact)]).astype(np.float16).view(np.uint16)[0])
        if exact == 0:
            want = 0
        assert Fraction(float(exact)) == exact
        assert int(got[i]) == want


# ------------------------------------------------------------------- P9 ----

def _golden_shapes():
    vals = {}
    with open(os.path.join(GOLDEN, "llama32_3b_shapes.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v) if "." in v else int(v)
    return vals


def test_p9_model_byte_count_matches_pages():
    g = _golden_shapes()
    assert (g["layers"], g["hidden"], g["ffn"]) == (synthetic.N_LAYERS, synthetic.HIDDEN, synthetic.FFN)
    assert (g["heads"], g["kv_heads"], g["head_dim"], g["vocab"]) == (
        synthetic.N_HEADS, synthetic.N_KV_HEADS, synthetic.HEAD_DIM, synthetic.VOCAB)
    size = {"q4k": oracle.Q4K_BYTES, "q6k": oracle.Q6K_BYTES}
    per_layer = sum(n * (k // 256) * size[f] for _, f, n, k in synthetic.LAYER_PROJECTIONS)
    _, f, n, k = synthetic.LM_HEAD
    total = g["layers"] * per_layer + n * (k // 256) * size[f]
    assert per_layer == 63_111_168
    assert total == 2_090_317_824
    gib = total / 2 ** 30
    assert round(gib, 1) == g["file_gib"]              # "1.9 GiB"
    # and the generators emit exactly those sizes
    assert synthetic.q4k_blocks(2, 512, 1).nbytes == 2 * 2 * 144
    assert synthetic.q6k_blocks(2, 512, 1).nbytes == 2 * 2 * 210


# ------------------------------------------------------------------ P10 ----

@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_p10_bruteforce_256_vs_numpy(fmt):
    M, N, K = 256, 256, 256
    x = synthetic.activations(M, K, seed=3)
    wq = synthetic.weight_blocks(fmt, N, K, seed=4)
    w_bits = oracle.dequant(fmt, wq, N, K)
    y, s = oracle.gemm_f16(x, w_bits)
    xd = x.astype(np.float64)
    wd = w_bits.view(np.float16).astype(np.float64)
    ref = xd @ wd.T
    assert np.all(np.abs(y - ref) <= 1e-12 * s)
    assert np.allclose(s, np.abs(xd) @ np.abs(wd).T, rtol=1e-12, atol=0)


def test_p10_nonsquare_orientation():
    M, N, K = 5, 7, 512
    x = synthetic.activations(M, K, seed=21)
    wq = synthetic.q4k_blocks(N, K, seed=22)
    w_bits = oracle.dequant_q4k(wq, N, K)
    y, s = oracle.gemm_f16(x, w_bits)
    ref = x.astype(np.float64) @ w_bits.view(np.float16).astype(np.float64).T
    assert y.shape == (M, N)
    assert np.all(np.abs(y - ref) <= 1e-12 * s)


def test_p10_exact_rational_sample():
    M, N, K = 16, 16, 256
    x = synthetic.activations(M, K, seed=31)
    w_bits = oracle.dequant_q4k(synthetic.q4k_blocks(N, K, seed=32), N, K)
    y, s = oracle.gemm_f16(x, w_bits)
    xf = [[Fraction(float(v)) for v in row] for row in x.astype(np.float64)]
    wf = [[Fraction(float(v)) for v in row] for row in w_bits.view(np.float16).astype(np.float64)]
    rng = np.random.default_rng(1)
    for _ in range(24):
        m, n = int(rng.integers(M)), int(rng.integers(N))
        exact = sum(a * b for a, b in zip(xf[m], wf[n]))
        mag = sum(abs(a * b) for a, b in zip(xf[m], wf[n]))
        assert abs(Fraction(y[m, n]) - exact) <= Fraction(2.0 ** -40) * mag
        assert abs(Fraction(s[m, n]) - mag) <= Fraction(2.0 ** -40) * mag


def test_gemm_pairs_equal_full():
    x = synthetic.activations(9, 768, seed=41)
    w_bits = oracle.dequant_q6k(synthetic.q6k_blocks(11, 768, seed=42), 11, 768)
    y, s = oracle.gemm_f16(x, w_bits)
    ms = np.array([0, 3, 8, 8, 5])
    ns = np.array([10, 0, 7, 10, 4])
    yp, sp = oracle.gemm_f16_pairs(x, w_bits, ms, ns)
    assert np.array_equal(yp, y[ms, ns]) and np.array_equal(sp, s[ms, ns])


# ------------------------------------------------------------------ P11 ----

def test_p11_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    g = oracle.SILU_MIN_G
    assert abs(g - (-1.2784645427610738)) < 1e-12
    assert abs(oracle.silu(np.array([g]))[0] - (g + 1.0)) < 1e-15
    around = oracle.silu(np.array([g - 1e-3, g + 1e-3, g - 0.5, g + 0.5]))
    assert np.all(around > oracle.silu(np.array([g]))[0])
    big = np.array([30.0, 50.0, 700.0])
    assert np.allclose(oracle.silu(big), big, rtol=1e-12)
    assert np.all(np.abs(oracle.silu(-big)) < 1e-11)
    assert oracle.silu(np.array([-800.0]))[0] == 0.0          # no overflow NaN
    # sigmoid symmetry: silu(g) - silu(-g) = g
    z = np.linspace(-20, 20, 101)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-12)


def test_p11_interval_accepts_exact_rejects_two_ulps():
    rng = np.random.default_rng(3)
    g = rng.standard_normal(2000) * 4
    u = rng.standard_normal(2000) * 4
    zero = np.zeros_like(g)
    lo, hi = oracle.swiglu_interval(g, u, zero, zero)
    h = (oracle.silu(g) * u).astype(np.float16)
    assert np.all(oracle.swiglu_accepts(h.astype(np.float64), lo, hi))
    up2 = np.nextafter(np.nextafter(h, np.float16(np.inf)), np.float16(np.inf))
    dn2 = np.nextafter(np.nextafter(h, np.float16(-np.inf)), np.float16(-np.inf))
    assert not np.any(oracle.swiglu_accepts(up2.astype(np.float64), lo, hi))
    assert not np.any(oracle.swiglu_accepts(dn2.astype(np.float64), lo, hi))


def test_p11_interval_overflow_and_minimum():
    # beyond +-65520 the fp16 result must be +-inf
    lo, hi = oracle.swiglu_interval(np.array([400.0, 400.0]), np.array([400.0, -400.0]),
                                    np.zeros(2), np.zeros(2))
    assert lo[0] == np.inf and hi[0] == np.inf
    assert lo[1] == -np.inf and hi[1] == -np.inf
    # a box around g* must reach down to silu(g*) * u
    lo, hi = oracle.swiglu_interval(np.array([-1.0]), np.array([1.0]), np.array([0.5]), np.array([0.0]))
    assert lo[0] <= oracle.SILU_MIN_VAL < hi[0]
    assert lo[0] > oracle.SILU_MIN_VAL - 1e-3


# ------------------------------------------------------------------ P12 ----

def test_p12_rmsnorm_closed_forms():
    K = 256
    # constant row: the root mean square is |c|, so every value is sign(c) * g
    x = np.array([[3.0] * K, [-0.25] * K], dtype=np.float16)
    g = np.ones(K)
    out = oracle.rmsnorm(x, g, 0.0)
    assert np.array_equal(out[0], np.ones(K)) and np.array_equal(out[1], -np.ones(K))
    # +-2 alternating: rms 2, so out = (+-1) * g exactly
    x = np.array([[2.0, -2.0] * (K // 2)], dtype=np.float16)
    g = np.arange(K) / 256.0
    out = oracle.rmsnorm(x, g, 0.0)
    assert np.array_equal(out[0], np.where(np.arange(K) % 2 == 0, 1.0, -1.0) * g)
    # one nonzero value a in K = 256: rms = |a| / 16, so out[0] = 16 sign(a) g[0]
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 0] = -5.0
    out = oracle.rmsnorm(x, np.full(K, 0.5), 0.0)
    assert out[0, 0] == -8.0 and np.all(out[0, 1:] == 0.0)
    # eps: a zero row stays zero; with eps the rms of a +-1 row is sqrt(1 + eps)
    x = np.zeros((1, K), dtype=np.float16)
    assert np.all(oracle.rmsnorm(x, np.ones(K), 1e-5) == 0.0)
    x = np.array([[1.0, -1.0] * (K // 2)], dtype=np.float16)
    out = oracle.rmsnorm(x, np.ones(K), 3.0)
    assert np.allclose(np.abs(out), 0.5, rtol=0, atol=1e-15)


def test_p12_rmsnorm_invariants():
    rng = np.random.default_rng(7)
    K = 768
    # magnitudes in [0.05, 3): scaled by 2^-3 or 2^2 they stay normal fp16
    x = (rng.choice([-1.0, 1.0], (6, K)) * rng.uniform(0.05, 3.0, (6, K))).astype(np.float16)
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    base = oracle.rmsnorm(x, g, 0.0)
    # scaling a row by a power of two (exact in fp16) does not change it
    for j in (-3, 2):
        xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float16)
        assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** j)
        assert np.allclose(oracle.rmsnorm(xs, g, 0.0), base, rtol=1e-14, atol=0)
    # linear in g
    assert np.allclose(oracle.rmsnorm(x, 2.0 * g.astype(np.float64), 0.0), 2.0 * base, rtol=1e-15, atol=0)
    # every row has mean square sum(out^2 / g^2) / K = 1 (eps = 0)
    ms = np.mean((base / g.astype(np.float64)) ** 2, axis=1)
    assert np.allclose(ms, 1.0, rtol=1e-13)
    # eps only shrinks: |out(eps)| < |out(0)| where out(0) != 0
    e = oracle.rmsnorm(x, g, 1e-2)
    nz = base != 0
    assert np.all(np.abs(e[nz]) < np.abs(base[nz]))


def test_p12_gemm_f64x_matches_f16_gemm_and_numpy():
    rng = np.random.default_rng(3)
    wq = synthetic.q4k_blocks(40, 512, seed=31)
    wb = oracle.dequant("q4k", wq, 40, 512)
    # fp16-representable activations: both oracles must agree exactly
    x16 = rng.standard_normal((5, 512)).astype(np.float16)
    y1, s1 = oracle.gemm_f16(x16, wb)
    y2, s2 = oracle.gemm_f64x(x16.astype(np.float64), wb)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    # arbitrary fp64 activations: numpy's matmul in fp64
    xd = rng.standard_normal((5, 512))
    y3, s3 = oracle.gemm_f64x(xd, wb)
    wd = oracle.f16_bits_to_f64(wb)
    mag = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(y3 - xd @ wd.T) <= 1e-12 * mag)
    assert np.allclose(s3, mag, rtol=1e-13)


def test_p12_rmsnorm_interval_accepts_rounded_rejects_two_ulps():
    rng = np.random.default_rng(11)
    xh = rng.standard_normal(4000) * 3.0
    lo, hi = oracle.rmsnorm_f16_interval(xh)
    h = xh.astype(np.float16)
    hv = h.astype(np.float64)
    assert np.all((hv >= lo) & (hv <= hi))
    up2 = np.nextafter(np.nextafter(h, np.float16(np.inf)), np.float16(np.inf)).astype(np.float64)
    dn2 = np.nextafter(np.nextafter(h, np.float16(-np.inf)), np.float16(-np.inf)).astype(np.float64)
    assert not np.any((up2 >= lo) & (up2 <= hi))
    assert not np.any((dn2 >= lo) & (dn2 <= hi))
    # an exact zero only accepts zero
    lo, hi = oracle.rmsnorm_f16_interval(np.zeros(3))
    assert np.all(lo == 0.0) and np.all(hi == 0.0)


# ------------------------------------------------------------------ P13 ----
# RoPE and grouped-query attention (oracle/attention.py).

from oracle import attention as attn  # noqa: E402


def test_p13_rope_closed_forms():
    """Pair 0 has frequency 1: (1, 0) at position p becomes (cos p, sin p);
    pair i at position p turns by p * theta^(-2i/d); position 0 is the
    identity; frequency factors divide the angle."""
    d = 8
    v = np.zeros((4, 1, d))
    v[:, 0, 0] = 1.0
    pos = np.array([0, 1, 2, 3])
    out = attn.rope(v, pos)
    for i, p in enumerate(pos):
        assert out[i, 0, 0] == pytest.approx(np.cos(p), abs=1e-15)
        assert out[i, 0, 1] == pytest.approx(np.sin(p), abs=1e-15)
        assert np.all(out[i, 0, 2:] == 0.0)
    # pair 2 (dims 4, 5): angle p * theta^(-4/8); (0, 1) -> (-sin, cos)
    v = np.zeros((1, 1, d))
    v[0, 0, 5] = 1.0
    a = 7 * 500000.0 ** (-0.5)
    out = attn.rope(v, np.array([7]))
    assert out[0, 0, 4] == pytest.approx(-np.sin(a), abs=1e-15)
    assert out[0, 0, 5] == pytest.approx(np.cos(a), abs=1e-15)
    rng = np.random.default_rng(1)
    w = rng.standard_normal((3, 2, 16))
    assert np.array_equal(attn.rope(w, np.zeros(3)), w)
    f = rng.uniform(1.0, 8.0, 8)
    lhs = attn.rope(w[:1], np.array([5.0]), freq_factors=f)
    # the same rotation without factors, pair by pair, at position 5 / f_i
    for i in range(8):
        ref = attn.rope(w[:1], np.array([5.0 / f[i]]))
        assert np.allclose(lhs[..., 2 * i:2 * i + 2], ref[..., 2 * i:2 * i + 2], atol=1e-13)


def test_p13_rope_invariants():
    """A rotation: pair norms are kept, rotating by -p undoes p, and the dot
    product of a rotated query and key depends only on their distance."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 3, 128))
    k = rng.standard_normal((5, 3, 128))
    pos = np.array([0, 1, 17, 1000, 131071])
    rq = attn.rope(q, pos)
    assert np.allclose(rq[..., 0::2] ** 2 + rq[..., 1::2] ** 2, q[..., 0::2] ** 2 + q[..., 1::2] ** 2, rtol=1e-12)
    assert np.allclose(attn.rope(rq, -pos), q, atol=1e-9)
    for shift in (3, 4096):
        a = np.einsum("mhd,mhd->mh", attn.rope(q, pos), attn.rope(k, pos[::-1]))
        b = np.einsum("mhd,mhd->mh", attn.rope(q, pos + shift), attn.rope(k, pos[::-1] + shift))
        assert np.allclose(a, b, rtol=1e-9, atol=1e-9)


def _attention_loops(q, kc, vc, pos0):
    """Written out with Python loops and math.exp, for the brute-force pin."""
    import math
    m, hq, d = q.shape
    group = hq // kc.shape[0]
    out = np.zeros(q.shape)
    for i in range(m):
        for h in range(hq):
            kv = h // group
            n = pos0 + i + 1
            s = [sum(q[i, h, e] * kc[kv, t, e] for e in range(d)) / math.sqrt(d) for t in range(n)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for e in range(d):
                out[i, h, e] = sum(w[t] * vc[kv, t, e] for t in range(n)) / tot
    return out


def test_p13_attention_closed_forms():
    """One visible key gives its value; equal keys give the mean of the
    values; a prefill's first query sees only position 0; the query heads of
    a group read their own KV head (6 query heads over 2 KV heads)."""
    rng = np.random.default_rng(3)
    d = 16
    q = rng.standard_normal((1, 6, d))
    kc = rng.standard_normal((2, 5, d))
    vc = rng.standard_normal((2, 5, d))
    out, _ = attn.attention_gqa(q, kc, vc, 0)
    for h in range(6):
        assert np.allclose(out[0, h], vc[h // 3, 0], atol=1e-15)
    kc_eq = np.repeat(kc[:, :1, :], 5, axis=1)
    out, _ = attn.attention_gqa(q, kc_eq, vc, 4)
    for h in range(6):
        assert np.allclose(out[0, h], vc[h // 3].mean(axis=0), atol=1e-14)
    qp = rng.standard_normal((5, 6, d))
    out, mass = attn.attention_gqa(qp, kc, vc, 0)
    assert np.allclose(out[0], vc[np.arange(6) // 3, 0], atol=1e-15)
    assert np.all(mass >= np.abs(out) - 1e-12)
    vconst = np.zeros_like(vc)
    vconst[0] = 1.0
    vconst[1] = -2.0
    out, _ = attn.attention_gqa(qp, kc, vconst, 0)
    assert np.allclose(out[:, :3], 1.0) and np.allclose(out[:, 3:], -2.0)


def test_p13_attention_scale():
    """The softmax scale is 1/sqrt(d): a query whose score for key 1
    exceeds that for key 0 by ln 3 after scaling weights them 3 : 1."""
    d = 128
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = np.sqrt(d) * np.log(3.0)
    kc = np.zeros((1, 2, d))
    kc[0, 1, 0] = 1.0
    vc = np.zeros((1, 2, d))
    vc[0, 0, :] = 1.0
    vc[0, 1, :] = 5.0
    out, _ = attn.attention_gqa(q, kc, vc, 1)
    assert np.allclose(out[0, 0], (1.0 + 3 * 5.0) / 4, rtol=1e-14)


def test_p13_rmsnorm_f64_matches_c_oracle_and_closed_forms():
    """The numpy RMSNorm for fp32 rows equals the C oracle's on rows of fp16
    values, and a constant row c gives g * sign(c) up to eps."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 512)).astype(np.float16)
    g = rng.uniform(0.5, 1.5, 512).astype(np.float32)
    assert np.allclose(attn.rmsnorm_f64(x, g, 1e-5), oracle.rmsnorm(x, g, 1e-5), rtol=1e-14, atol=0)
    row = np.full((1, 256), -3.0)
    assert np.allclose(attn.rmsnorm_f64(row, np.ones(256), 0.0), -1.0, rtol=1e-15)


def test_p13_attention_bruteforce_and_shift():
    """Against explicit loops on a small prefill with a cache offset, and
    invariant under a common rotation of queries and keys (RoPE of both by
    the same extra angle keeps every score)."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 4, 8))
    kc = rng.standard_normal((2, 9, 8))
    vc = rng.standard_normal((2, 9, 8))
    out, _ = attn.attention_gqa(q, kc, vc, 5)
    assert np.allclose(out, _attention_loops(q, kc, vc, 5), rtol=1e-12, atol=1e-13)
    s = 11
    q2 = attn.rope(q, np.full(3, s))
    kc2 = attn.rope(kc.reshape(18, 1, 8), np.full(18, s)).reshape(2, 9, 8)
    out2, _ = attn.attention_gqa(q2, kc2, vc, 5)
    assert np.allclose(out, out2, rtol=1e-10, atol=1e-12)


# -------------------------------------------------------- generators -------

def test_generators_deterministic_and_in_range():
    a = synthetic.q4k_blocks(4, 512, seed=123)
    b = synthetic.q4k_blocks(4, 512, seed=123)
    c = synthetic.q4k_blocks(4, 512, seed=124)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    blocks = a.reshape(-1, 144)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64)
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float64)
    assert np.all((d >= 9.9e-4) & (d <= 2.001e-2)) and np.all((dmin >= 9.9e-4) & (dmin <= 2.001e-2))
    b6 = synthetic.q6k_blocks(3, 768, seed=5).reshape(-1, 210)
    d6 = b6[:, 208:210].copy().view("<f2").astype(np.float64)
    assert np.all((d6 >= 9.9e-4) & (d6 <= 2.001e-2))
    x = synthetic.activations(8, 3072, seed=9, unit_rms=True)
    assert x.dtype == np.float16
    rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1))
    assert np.allclose(rms, 1.0, atol=2e-3)
    s = synthetic.row_sample(1024, 40, seed=1)
    assert s[0] == 0 and s[-1] == 1023 and len(set(s // 256)) == 4


# ------------------------------------------------- acceptance intervals -----
# oracle.f16_interval is the acceptance interval of every check whose GPU
# result is one fp16 rounding of a value known within an absolute slack (the
# RoPE outputs).  Pinned here against an exhaustive search of the fp16 grid:
# every finite fp16 value, sorted, extended by -inf and +inf.

def _fp16_grid():
    v = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    v = v[np.isfinite(v)]
    return np.unique(np.concatenate([v, [-np.inf, np.inf]]))     # -0 and +0 merge


def test_f16_interval_closed_forms():
    cases = [
        # (exact, slack, lo, hi)
        (1.0, 0.0, 1.0, 1.0),                                  # on the grid, no slack: degenerate
        (-3.5, 0.0, -3.5, -3.5),
        (0.0, 0.0, 0.0, 0.0),
        (1.0, 1e-6, 1.0 - 2.0 ** -11, 1.0 + 2.0 ** -10),       # binade edge: the step below 1 is half
        (2.0, 1e-6, 2.0 - 2.0 ** -10, 2.0 + 2.0 ** -9),
        (-1.0, 1e-6, -(1.0 + 2.0 ** -10), -(1.0 - 2.0 ** -11)),  # negative: mirrored
        (0.0, 1e-9, -2.0 ** -24, 2.0 ** -24),                  # smallest subnormals
        (1.5 * 2.0 ** -24, 0.0, 2.0 ** -24, 2.0 ** -23),
        (65504.0, 1.0, 65472.0, np.inf),                       # past the largest finite value: inf
        (-65504.0, 1.0, -np.inf, -65472.0),
        (1e6, 0.0, 65504.0, np.inf),                           # RNE(1e6) = inf lies inside
    ]
    ex = np.array([c[0] for c in cases])
    sl = np.array([c[1] for c in cases])
    lo, hi = oracle.f16_interval(ex, sl)
    for i, (e, s, l, h) in enumerate(cases):
        assert lo[i] == l and hi[i] == h, f"f16_interval({e}, {s}) = [{lo[i]}, {hi[i]}], want [{l}, {h}]"


def test_f16_interval_matches_exhaustive_grid_search():
    grid = _fp16_grid()
    rng = np.random.default_rng(21)
    n = 20000
    scale = 2.0 ** rng.integers(-30, 18, n)                       # subnormal range to past overflow
    exact = rng.standard_normal(n) * scale
    exact[:2000] = rng.choice(grid[1:-1], 2000)                   # exact grid points
    slack = np.abs(exact) * rng.choice([0.0, 2.0 ** -30, 2.0 ** -12, 2.0 ** -9, 2.0 ** -6], n)
    slack[2000:2500] = 0.0
    lo, hi = oracle.f16_interval(exact, slack)
    a, b = exact - slack, exact + slack
    lo_ref = grid[np.searchsorted(grid, a, side="right") - 1]     # largest grid value <= a
    hi_ref = grid[np.searchsorted(grid, b, side="left")]          # smallest grid value >= b
    assert np.array_equal(lo, lo_ref) and np.array_equal(hi, hi_ref)


def test_f16_interval_accepts_rne_rejects_two_ulps():
    """With zero slack the interval holds RNE(exact) (and the other grid
    neighbour), and nothing two fp16 steps away."""
    rng = np.random.default_rng(22)
    exact = rng.standard_normal(5000) * 2.0 ** rng.integers(-12, 12, 5000)
    lo, hi = oracle.f16_interval(exact, np.zeros_like(exact))
    h = exact.astype(np.float16)
    assert np.all((h.astype(np.float64) >= lo) & (h.astype(np.float64) <= hi))
    for direction in (np.float16(np.inf), np.float16(-np.inf)):
        far = np.nextafter(np.nextafter(h, direction), direction).astype(np.float64)
        assert not np.any((far >= lo) & (far <= hi))


def test_p13_attention_mass():
    """mass = sum_t p_t |v_t|, the scale of each attention output: one
    visible key gives |v_0|; equal keys give the mean of |v| over the visible
    positions; with nonnegative values it equals the output; against the
    explicit loops (with |v|) on a small prefill."""
    rng = np.random.default_rng(23)
    d = 16
    q = rng.standard_normal((1, 6, d))
    kc = rng.standard_normal((2, 7, d))
    vc = rng.standard_normal((2, 7, d))
    _, mass = attn.attention_gqa(q, kc, vc, 0)
    for h in range(6):
        assert np.array_equal(mass[0, h], np.abs(vc[h // 3, 0]))
    kc_eq = np.repeat(kc[:, :1, :], 7, axis=1)
    _, mass = attn.attention_gqa(q, kc_eq, vc, 4)                 # positions 0..4 visible
    for h in range(6):
        assert np.allclose(mass[0, h], np.abs(vc[h // 3, :5]).mean(axis=0), rtol=1e-14, atol=0)
    qp = rng.standard_normal((3, 6, d))
    out, mass = attn.attention_gqa(qp, kc, np.abs(vc), 2)
    assert np.allclose(mass, out, rtol=1e-14, atol=0)
    _, mass = attn.attention_gqa(qp, kc, vc, 2)
    assert np.allclose(mass, _attention_loops(qp, kc, np.abs(vc), 2), rtol=1e-12, atol=1e-13)
    assert np.all(mass >= np.abs(attn.attention_gqa(qp, kc, vc, 2)[0]) - 1e-12)
