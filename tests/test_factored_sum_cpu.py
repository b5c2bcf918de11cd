"""The decode kernel's factored Q4_K dot product, checked on the CPU.

The M = 1 kernel does not multiply x by dequantised weights.  Per 32-weight
sub-block with a = d*sc and b = dmin*m it forms

    sum_k x_k (a q_k - b) = a * sum_k x_k (q_k - c) - (b - a c) * sum_k x_k,

c the integer in [0, 15] nearest b / a, with q - c exact in fp16 and the sums
in fp32.  Centring on c keeps each term within a small multiple of the weight
it belongs to, so the fp32 rounding stays bounded by sum |x w| even where the
weights cancel.

Here that arithmetic is emulated in numpy float32, in the kernel's order:
  - 16 two-product steps per sub-block, each rounded once to fp32;
  - the sums of x over 8 values, then over the 4 lanes of a quad;
  - the fused multiply-adds of the combine;
  - each lane's blocks, then the 4 parts of a row, then the 4 waves in order.
The result is compared with the oracle's bound (1e-3 * sum |x w| + 1e-5,
against its fp64 product with the fp16-rounded weights).

The same emulation without the centring (c = 0) is shown to break the bound
on a row whose weights are all exact zeros.  That is the case the centring is
for.  This is a test of the method's arithmetic; the GPU parity tests check
the kernel itself.
"""
import numpy as np

import oracle
import synthetic
from _centring import centring_fields, pack_fields
from _packing import f16_bits

f32, f64 = np.float32, np.float64


def _fma(a, b, c):
    """a * b + c rounded once to fp32 (fp64 holds the product of two fp32
    exactly; its rounding of the sum is far below the fp32 step)."""
    return (a.astype(f64) * b.astype(f64) + c.astype(f64)).astype(f32)


def _emulate(d_bits, dmin_bits, sc, mn, q, x, rows, k, centred=True):
    nb = k // 256
    d = d_bits.astype(np.uint16).view(np.float16).astype(f32).reshape(rows, nb, 1)
    dmin = dmin_bits.astype(np.uint16).view(np.float16).astype(f32).reshape(rows, nb, 1)
    a = (d * sc.reshape(rows, nb, 8).astype(f32)).astype(f32)
    b = (dmin * mn.reshape(rows, nb, 8).astype(f32)).astype(f32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = (b * (f32(1) / a)).astype(f32)
    c = np.fmin(np.fmax(np.rint(t), f32(0)), f32(15)).astype(f32) if centred else np.zeros_like(a)
    e = _fma(-a, c, b)                                           # b - a c
    qq = (q.reshape(rows, nb, 8, 32) - c[..., None]).astype(f32)  # exact
    xv = x.reshape(nb, 8, 32).astype(f32)
    # sum x (q - c): 16 steps of two exact products plus the running sum
    dsum = np.zeros((rows, nb, 8), f32)
    for s in range(16):
        dsum = (dsum.astype(f64) + qq[..., 2 * s].astype(f64) * xv[:, :, 2 * s].astype(f64)
                + qq[..., 2 * s + 1].astype(f64) * xv[:, :, 2 * s + 1].astype(f64)).astype(f32)
    # sum x: each lane adds its 8 values as ((v0+v1)+(v2+v3))+((v4+v5)+(v6+v7)),
    # then the quad adds (l0+l1)+(l2+l3)
    v = xv.reshape(nb, 8, 4, 8)
    pair = (v[..., 0::2] + v[..., 1::2]).astype(f32)
    quad = (pair[..., 0::2] + pair[..., 1::2]).astype(f32)
    lane = (quad[..., 0] + quad[..., 1]).astype(f32)
    sx = ((lane[..., 0] + lane[..., 1]).astype(f32) + (lane[..., 2] + lane[..., 3]).astype(f32)).astype(f32)
    sx = np.broadcast_to(sx, (rows, nb, 8))
    # a part p covers sub-blocks 2p (low nibbles) and 2p+1 (high nibbles):
    # y = a0*D0; y = fma(-e0, S0, y); y = fma(a1, D1, y); y = fma(-e1, S1, y)
    lo, hi = slice(0, 8, 2), slice(1, 8, 2)
    y = (a[..., lo] * dsum[..., lo]).astype(f32)
    y = _fma(-e[..., lo], sx[..., lo], y)
    y = _fma(a[..., hi], dsum[..., hi], y)
    part = _fma(-e[..., hi], sx[..., hi], y)                      # [rows, nb, 4]
    # lane = (row, part) of wave w adds its blocks [w nb / 4, (w+1) nb / 4)
    waves = []
    for w in range(4):
        acc = np.zeros((rows, 4), f32)
        for blk in range(w * nb // 4, (w + 1) * nb // 4):
            acc = (acc + part[:, blk]).astype(f32)
        waves.append(((acc[:, 0] + acc[:, 1]).astype(f32) + (acc[:, 2] + acc[:, 3]).astype(f32)).astype(f32))
    out = waves[0]
    for w in range(1, 4):
        out = (out + waves[w]).astype(f32)
    return out


def _check(rows, k, seed, sigma, zero_rows=0, centred=True, spiky_x=False, zero_d=None):
    rng = np.random.default_rng(seed)
    nb = k // 256
    fields = centring_fields(rng, rows * nb, all_zero_blocks=set(range(zero_rows * nb)))
    if zero_d is not None:    # the zero rows' d = dmin (the weights stay exact zeros)
        fields[0][:zero_rows * nb] = zero_d
        fields[1][:zero_rows * nb] = zero_d
    wq = pack_fields(*fields).reshape(-1)
    if spiky_x:               # a value near +-2000 opens every sub-block: the running
        g = np.random.default_rng(seed + 1)     # sums of x q round at that scale
        xs = g.standard_normal(k)
        xs[::32] = np.sign(xs[::32]) * g.uniform(1500, 2000, k // 32)
        x = xs.astype(np.float16).reshape(1, k)
    else:
        x = synthetic.activations(1, k, seed=seed + 1, sigma=sigma)
    y = _emulate(*fields, x.reshape(-1), rows, k, centred=centred)
    ref, s = oracle.gemm_quant("q4k", x, wq, rows, k)
    with np.errstate(invalid="ignore"):
        ratio = np.abs(y.astype(f64) - ref[0]) / oracle.gemm_tolerance(s[0])
    return y, ratio


def test_factored_sum_within_bound_on_centring_cases():
    for seed, sigma, spiky in ((17, 1.0, False), (23, 1.0 / 64, False), (29, 4.0, False), (37, 1.0, True)):
        y, ratio = _check(48, 2048, seed, sigma, zero_rows=1, spiky_x=spiky)
        assert np.isfinite(ratio).all()
        assert ratio.max() <= 0.25, f"seed {seed}: worst err/bound {ratio.max():.3g}"
        assert y[0] == 0.0        # a row of exact zeros sums to exactly 0


def test_factored_sum_within_bound_on_layer_weights():
    # the Q projection's first rows of the decode layer (config 1 seeds)
    name, fmt, n, k, wq = next(iter(synthetic.layer_weights(1, 0)))
    rows = 48
    blocks = wq.reshape(-1)[:rows * (k // 256) * 144].reshape(rows * (k // 256), 144)
    # fields back from the bytes (the layout of tests/_packing.py)
    d_bits = blocks[:, 0].astype(np.int64) | (blocks[:, 1].astype(np.int64) << 8)
    dmin_bits = blocks[:, 2].astype(np.int64) | (blocks[:, 3].astype(np.int64) << 8)
    s = blocks[:, 4:16].astype(np.int64)
    sc = np.concatenate([s[:, 0:4] & 63, (s[:, 8:12] & 15) | ((s[:, 0:4] >> 6) << 4)], axis=1)
    mn = np.concatenate([s[:, 4:8] & 63, (s[:, 8:12] >> 4) | ((s[:, 4:8] >> 6) << 4)], axis=1)
    qs = blocks[:, 16:].astype(np.int64).reshape(-1, 4, 32)
    q = np.stack([qs & 15, qs >> 4], axis=2).reshape(-1, 256)
    assert np.array_equal(pack_fields(d_bits, dmin_bits, sc, mn, q), blocks)   # the read-back is exact
    x = synthetic.activations(1, k, seed=synthetic.act_seed(1, 0, 0))
    y = _emulate(d_bits, dmin_bits, sc, mn, q, x.reshape(-1), rows, k)
    ref, sa = oracle.gemm_quant("q4k", x, blocks.reshape(-1), rows, k)
    ratio = np.abs(y.astype(f64) - ref[0]) / oracle.gemm_tolerance(sa[0])
    assert ratio.max() <= 0.25, f"{name}: worst err/bound {ratio.max():.3g}"


def test_uncentred_sum_breaks_bound_on_exact_zeros():
    # without the centring, the row of exact zeros is a*sum(x q0) - b*sum(x)
    # with b = a q0: two differently rounded sums whose difference, with a
    # large x opening each sub-block, lands far above the row's 1e-5 bound
    d = f16_bits(0.5)
    _, ratio = _check(8, 2048, 31, 1.0, zero_rows=1, centred=False, spiky_x=True, zero_d=d)
    assert ratio[0] > 10.0, f"uncentred zero row within the bound (err/bound {ratio[0]:.3g})"
    _, ratio_c = _check(8, 2048, 31, 1.0, zero_rows=1, centred=True, spiky_x=True, zero_d=d)
    assert ratio_c[0] == 0.0 and ratio_c.max() <= 0.25
