"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (stated per test):
* dequant: bit-exact fp16, NaN matched as NaN;
* GEMM / GEMV: per output |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-5, with
  y_ref and the sum from the oracle's fp64 matmul over its own fp16 weights;
* SwiGLU h: inside the oracle's interval over g, u +- their GEMM bounds,
  widened by 2^-20 and rounded outward to fp16 (IEEE overflow to +-inf);
* FFN down stage: the oracle GEMM applied to the GPU's own h.

Inputs come from `synthetic` (seeded, shaped like the Llama-3.2-3B layer on
the DAMASCUS overview page, "[06] the target").  Sizes the oracle finishes in
seconds are checked on every output; the full benchmark sizes are checked on
sampled rows that hit every 256-row tile, in the grouped launch the benchmark
times.
"""
import numpy as np
import pytest

import oracle
import synthetic
from _centring import centring_blocks
from _packing import f16_bits, pack_q4k, pack_q6k

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dmq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_q4_amd
    return dequant_gemm_q4_amd


DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_dequant(dmq, fmt, wq, rows, k):
    out = torch.empty((rows, k), dtype=torch.float16, device=DEV)
    fn = dmq.dmq_dequant_q4k if fmt == "q4k" else dmq.dmq_dequant_q6k
    fn(dev(wq.reshape(-1)), out, rows, k)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def assert_bits_equal(got, want, what):
    got = got.reshape(-1)
    want = want.reshape(-1)
    nan_w = (want & 0x7C00) == 0x7C00
    nan_w &= (want & 0x03FF) != 0
    nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x03FF) != 0)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN pattern differs"
    diff = (got != want) & ~nan_w
    assert not diff.any(), (f"{what}: {int(diff.sum())} of {got.size} weights differ; first at "
                            f"{int(np.argmax(diff))}: got {got[diff][0]:#06x} want {want[diff][0]:#06x}")


def gpu_gemm(dmq, fmt, x, wq, M, N, K):
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    fn = dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k
    fn(dev(x), dev(wq.reshape(-1)), y, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y, ref, s, what):
    y = y.astype(np.float64)
    tol = oracle.gemm_tolerance(s)
    err = np.abs(y - ref)
    ok = err <= tol
    ratio = float(np.max(np.where(np.isfinite(err), err / tol, np.inf)))
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outputs outside the bound (worst err/bound {ratio:.3g})"
    print(f"{what}: max err/bound = {ratio:.3g}")
    return ratio


# --------------------------------------------------------------- dequant ---

@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("rows,k", [(64, 3072), (3, 768), (1, 256), (5, 8192)])
def test_dequant_random_bitexact(dmq, fmt, rows, k):
    wq = synthetic.weight_blocks(fmt, rows, k, seed=100 + rows + k)
    assert_bits_equal(gpu_dequant(dmq, fmt, wq, rows, k), oracle.dequant(fmt, wq, rows, k), f"{fmt} {rows}x{k}")


def test_dequant_q4k_adversarial_rounding(dmq):
    # the three hand-found vectors, then a sweep of the region where rounding
    # through fp32 first would differ: d near the top of its range, dmin in the
    # lowest binade, large scales and quants
    blocks = [pack_q4k(d, dm, [sc] * 8, [m] * 8, [q] * 256)
              for d, sc, q, dm, m in [(0x2458, 63, 15, 0x1423, 11), (0x245A, 63, 15, 0x1517, 7),
                                      (0x245B, 63, 15, 0x14CF, 33)]]
    rng = np.random.default_rng(2024)
    n = 6000
    sweep = synthetic.random_bytes(n * 144, seed=77).reshape(n, 144).copy()
    d_bits = rng.integers(f16_bits(0.0169), f16_bits(0.02) + 1, n).astype(np.uint16)
    dm_bits = rng.integers(0x1400, 0x1800, n).astype(np.uint16)          # [2^-10, 2^-9)
    sweep[:, 0:2] = d_bits.view(np.uint8).reshape(n, 2)
    sweep[:, 2:4] = dm_bits.view(np.uint8).reshape(n, 2)
    # scales >= 50: low 6 bits of bytes 0..3 (j < 4) and the split fields of j >= 4
    for b in range(n):
        sc = rng.integers(50, 64, 8)
        mn = rng.integers(0, 64, 8)
        q = rng.integers(12, 16, 256)
        sweep[b] = pack_q4k(int(d_bits[b]), int(dm_bits[b]), sc, mn, q)
    wq = np.concatenate([np.stack(blocks), sweep]).reshape(-1)
    rows = len(blocks) + n
    want = oracle.dequant_q4k(wq, rows, 256)
    got = gpu_dequant(dmq, "q4k", wq, rows, 256)
    assert_bits_equal(got, want, "q4k adversarial")
    assert np.all(want[0] == 0x4C01) and np.all(want[1] == 0x4C03) and np.all(want[2] == 0x4C03)
    # the sweep must actually contain double-rounding cases to be a test
    fields = [oracle.q4k_fields(wq[i * 144:(i + 1) * 144]) for i in range(3, 3 + 400)]
    dr = 0
    for (d, dmin, sc, mn, q), row in zip(fields, want[3:403]):
        j = np.arange(256) // 32
        v32 = (np.float32(d) * sc[j].astype(np.float32) * q.astype(np.float32)
               - np.float32(dmin) * mn[j].astype(np.float32))
        dr += int(np.sum(v32.astype(np.float16).view(np.uint16) != row))
    print(f"double-rounding cases in the first 400 sweep blocks: {dr}")
    assert dr > 0


def test_dequant_special_values(dmq):
    cases4 = [
        pack_q4k(0x7C00, 0x3C00, [1] * 8, [1] * 8, [i % 16 for i in range(256)]),   # d = +inf
        pack_q4k(0x3C00, 0x7E00, [1] * 8, [3] * 8, [1] * 256),                      # dmin = NaN
        pack_q4k(0xBC00, 0x0000, [5] * 8, [0] * 8, [i % 16 for i in range(256)]),   # d < 0: -0 -> +0
        pack_q4k(0x0001, 0x0002, [63] * 8, [63] * 8, [i % 16 for i in range(256)]), # subnormal d, dmin
        pack_q4k(0x7BFF, 0x0000, [63] * 8, [0] * 8, [15] * 256),                    # overflow to inf
        pack_q4k(0x3C00, 0x3C00, [7] * 8, [7] * 8, [1] * 256),                      # exact zeros
    ]
    wq = np.stack(cases4).reshape(-1)
    assert_bits_equal(gpu_dequant(dmq, "q4k", wq, len(cases4), 256),
                      oracle.dequant_q4k(wq, len(cases4), 256), "q4k special")
    cases6 = [
        pack_q6k(0x3C00, [-(s + 1) for s in range(16)], [32] * 256),                  # all +0
        pack_q6k(0xFC00, [3] * 16, [(i * 7) % 64 for i in range(256)]),               # d = -inf, q=32 -> NaN
        pack_q6k(0x0003, [-128] * 16, [(i * 5) % 64 for i in range(256)]),            # subnormal d
        pack_q6k(0x7BFF, [127] * 16, [0] * 256),                                      # overflow
    ]
    wq6 = np.stack(cases6).reshape(-1)
    assert_bits_equal(gpu_dequant(dmq, "q6k", wq6, len(cases6), 256),
                      oracle.dequant_q6k(wq6, len(cases6), 256), "q6k special")


# ------------------------------------------------------------------ GEMV ---

def test_gemv_config1_every_output(dmq):
    x = synthetic.activations(1, 3072, seed=synthetic.act_seed(1, 0, 0))
    hx = synthetic.activations(1, 8192, seed=synthetic.act_seed(1, 0, 6))
    for name, fmt, N, K, wq in synthetic.layer_weights(1, 0):
        xin = hx if K == 8192 else x
        y = gpu_gemm(dmq, fmt, xin, wq, 1, N, K)
        ref, s = oracle.gemm_quant(fmt, xin, wq, N, K)
        assert_within(y, ref, s, f"decode {name} {N}x{K}")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("N,K", [(1, 256), (5, 512), (17, 1280), (100, 4096), (33, 2304)])
def test_gemv_ragged(dmq, fmt, N, K):
    x = synthetic.activations(1, K, seed=N + K)
    wq = synthetic.weight_blocks(fmt, N, K, seed=N * 7 + K)
    y = gpu_gemm(dmq, fmt, x, wq, 1, N, K)
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y, ref, s, f"decode {fmt} {N}x{K}")


def test_gemv_group_equals_single_calls(dmq):
    x = dev(synthetic.activations(1, 3072, seed=5))
    hx = dev(synthetic.activations(1, 8192, seed=6))
    probs, singles = [], []
    for name, fmt, N, K, wq in synthetic.layer_weights(1, 3):
        w = dev(wq.reshape(-1))
        xin = hx if K == 8192 else x
        yg = torch.empty((1, N), dtype=torch.float32, device=DEV)
        ys = torch.empty((1, N), dtype=torch.float32, device=DEV)
        probs.append((fmt, xin, w, yg, 1, N, K))
        singles.append((fmt, xin, w, ys, 1, N, K))
    dmq.dmq_gemm_group(probs)
    for fmt, xin, w, ys, M, N, K in singles:
        (dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k)(xin, w, ys, M, N, K)
    torch.cuda.synchronize()
    for (f, _, _, yg, *_), (_, _, _, ys, *_) in zip(probs, singles):
        assert torch.equal(yg, ys)


@pytest.mark.parametrize("M", [2])
def test_gemv_few_rows_equal_single_row_calls(dmq, M):
    """2 activation rows take the decode kernel with both rows' x staged:
    each row's outputs have the bits of an M = 1 call on that row,
    for a decode layer's seven projections in one group (Q4_K and Q6_K,
    K = 3072 and 8192) and for the SwiGLU FFN 3072 -> 8192 -> 3072."""
    x = synthetic.activations(M, 3072, seed=50 + M)
    hx = synthetic.activations(M, 8192, seed=60 + M, sigma=1.0 / 16)
    probs, ws = [], []
    for name, fmt, N, K, wq in synthetic.layer_weights(1, 2):
        w = dev(wq.reshape(-1))
        xin = hx if K == 8192 else x
        probs.append((fmt, dev(xin), w, torch.empty((M, N), dtype=torch.float32, device=DEV), M, N, K))
        ws.append((name, fmt, w, xin, N, K))
    dmq.dmq_gemm_group(probs)
    torch.cuda.synchronize()
    for (name, fmt, w, xin, N, K), (*_, yg, _, _, _) in zip(ws, probs):
        for r in range(M):
            yr = torch.empty((1, N), dtype=torch.float32, device=DEV)
            (dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k)(dev(xin[r:r + 1]), w, yr, 1, N, K)
            torch.cuda.synchronize()
            assert torch.equal(yg[r:r + 1], yr), f"{name} M={M} row {r} differs from the M = 1 call"
    D, F, wgu, wd = _ffn_weights(1)
    xf = synthetic.activations(M, D, seed=70 + M, sigma=1.0 / 16)
    h, y = run_ffn(dmq, xf, wgu, wd, M, D, F)
    for r in range(M):
        h1, y1 = run_ffn(dmq, xf[r:r + 1], wgu, wd, 1, D, F)
        assert np.array_equal(h[r:r + 1].view(np.uint16), h1.view(np.uint16)), f"FFN h, M={M} row {r}"
        assert np.array_equal(y[r:r + 1].view(np.uint32), y1.view(np.uint32)), f"FFN y, M={M} row {r}"
    check_ffn(xf, wgu, wd, h, y, D, F, np.arange(M), f"few-rows FFN M={M}")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("M,N,K", [(2, 37, 10240), (2, 24, 20480), (2, 100, 512), (2, 17, 4864), (2, 9, 20736),
                                   (3, 20, 768)])
def test_gemv_few_rows_every_output(dmq, fmt, M, N, K):
    """The two-row decode kernel against the oracle, every output: ragged N
    and the largest K whose two rows of x fit its LDS (20480); K = 20736
    and M = 3 take the small-M MFMA kernel instead."""
    x = synthetic.activations(M, K, seed=K + M)
    wq = synthetic.weight_blocks(fmt, N, K, seed=K + 7)
    y = gpu_gemm(dmq, fmt, x, wq, M, N, K)
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y, ref, s, f"few-rows gemv {fmt} M={M} N={N} K={K}")


# ------------------------------------------------------------------ GEMM ---

def test_gemm_config0_every_output(dmq):
    M, N, K = 16, 3072, 3072
    x = synthetic.activations(M, K, seed=synthetic.act_seed(0, 0, 0))
    wq = synthetic.q4k_blocks(N, K, seed=synthetic.weight_seed(0, 0, 0))
    y = gpu_gemm(dmq, "q4k", x, wq, M, N, K)
    ref, s = oracle.gemm_quant("q4k", x, wq, N, K)
    assert_within(y, ref, s, "config0 M=16 q4k")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("M,N,K", [(2, 64, 256), (17, 100, 512), (65, 333, 768), (300, 1000, 1024),
                                   (257, 257, 256), (130, 7, 2048), (64, 512, 1536)])
def test_gemm_ragged_every_output(dmq, fmt, M, N, K):
    x = synthetic.activations(M, K, seed=M * 31 + N)
    wq = synthetic.weight_blocks(fmt, N, K, seed=M + N * 3 + K)
    y = gpu_gemm(dmq, fmt, x, wq, M, N, K)
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y, ref, s, f"gemm {fmt} {M}x{N}x{K}")


def test_gemm_adversarial_cancellation(dmq):
    # every weight is d*sc*q - dmin*m with the two terms equal or nearly
    # equal: y_ref ~ 0 and S tiny, so the bound is close to 1e-5 absolute
    rng = np.random.default_rng(9)
    N, K, M = 64, 512, 48
    blocks = []
    for _ in range(N * K // 256):
        sc = rng.integers(1, 64, 8)
        q = rng.integers(1, 16, 256)
        d = f16_bits(0.01)
        # m = sc * q0 for one q0 per sub-block: weights with q == q0 are exact zeros
        q0 = rng.integers(1, 4, 8)
        mn = np.minimum(sc * q0, 63)
        blocks.append(pack_q4k(d, d, sc, mn, q))
    wq = np.stack(blocks).reshape(-1)
    x = synthetic.activations(M, K, seed=10)
    for m_rows in (M, 1):
        y = gpu_gemm(dmq, "q4k", x[:m_rows], wq, m_rows, N, K)
        ref, s = oracle.gemm_quant("q4k", x[:m_rows], wq, N, K)
        assert_within(y, ref, s, f"cancellation M={m_rows}")


def test_gemv_q4k_centring_cases(dmq):
    """The decode kernel's factored Q4_K dot product on the sub-block cases
    that size its terms (tests/_centring.py), at M = 1, every output, and
    as the SwiGLU gate|up pair of a decode FFN.  Row 0 holds only exact
    zeros: its bound is the 1e-5 floor, and the kernel gives exactly 0."""
    rng = np.random.default_rng(17)
    N, K = 96, 2048
    nb = K // 256
    wq = centring_blocks(rng, N * nb, all_zero_blocks=set(range(nb))).reshape(-1)
    spiky = np.random.default_rng(22).standard_normal(K)
    spiky[::32] = np.sign(spiky[::32]) * 1800.0   # a large x opening every sub-block
    xs = [("sigma=1", synthetic.activations(1, K, seed=18, sigma=1.0)),
          ("sigma=1/64", synthetic.activations(1, K, seed=19, sigma=1.0 / 64)),
          ("spiky", spiky.astype(np.float16).reshape(1, K))]
    for what, x in xs:
        y = gpu_gemm(dmq, "q4k", x, wq, 1, N, K)
        ref, s = oracle.gemm_quant("q4k", x, wq, N, K)
        assert_within(y, ref, s, f"centring cases, x {what}")
        assert y[0, 0] == 0.0
    # such blocks as the gate|up pair of a decode FFN (gate row r and up row
    # r + F in one lane), D = K, F = 256, then a random Q6_K down projection
    D, F = K, 256
    wgu = centring_blocks(rng, 2 * F * nb)
    wd = synthetic.q6k_blocks(D, F, seed=21)
    x = synthetic.activations(1, D, seed=20, sigma=1.0 / 16)
    h, y = run_ffn(dmq, x, wgu, wd, 1, D, F)
    check_ffn(x, wgu, wd, h, y, D, F, np.array([0]), "centring cases ffn decode")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_gemv_max_k_every_output(dmq, fmt):
    """M = 1 at K = 32768, the largest K of the decode kernel (its x slice
    fills 73.7 KB of LDS): every output."""
    K, N = 32768, 80
    x = synthetic.activations(1, K, seed=41)
    wq = synthetic.weight_blocks(fmt, N, K, seed=42)
    y = gpu_gemm(dmq, fmt, x, wq, 1, N, K)
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y, ref, s, f"gemv {fmt} K={K}")


def test_ffn_decode_max_k(dmq):
    """The SwiGLU pair decode path (gate and up rows in one lane) at D = K =
    32768, then the Q6_K down projection back to 32768 outputs."""
    D, F = 32768, 256
    wgu = synthetic.q4k_blocks(2 * F, D, seed=43)
    wd = synthetic.q6k_blocks(D, F, seed=44)
    x = synthetic.activations(1, D, seed=45, sigma=1.0 / 16)
    h, y = run_ffn(dmq, x, wgu, wd, 1, D, F)
    check_ffn(x, wgu, wd, h, y, D, F, np.array([0]), f"ffn decode D={D}")


def test_gemm_large_k_m1(dmq):
    # K beyond the decode kernel's LDS staging: M = 1 runs the MFMA kernel
    M, N, K = 1, 24, 33024
    x = synthetic.activations(M, K, seed=1)
    wq = synthetic.q4k_blocks(N, K, seed=2)
    y = gpu_gemm(dmq, "q4k", x, wq, M, N, K)
    ref, s = oracle.gemm_quant("q4k", x, wq, N, K)
    assert_within(y, ref, s, "gemm K=33024 M=1")


def _layer_group(dmq, config, layer, M, unit_rms=True):
    """Inputs and outputs of one layer's 7 projections (O and down get their
    own activations), as the benchmark builds them."""
    items = []
    for idx, (name, fmt, N, K, wq) in enumerate(synthetic.layer_weights(config, layer)):
        x = synthetic.activations(M, K, seed=synthetic.act_seed(config, layer, idx), unit_rms=unit_rms)
        items.append((name, fmt, N, K, wq, x))
    return items


def _run_layer_group(dmq, items, M):
    """One grouped launch of a layer's projections; returns the host copies of y."""
    probs = []
    for name, fmt, N, K, wq, x in items:
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        probs.append((fmt, dev(x), dev(wq.reshape(-1)), y, M, N, K))
    dmq.dmq_gemm_group(probs)
    torch.cuda.synchronize()
    return [p[3].cpu().numpy() for p in probs]


def test_gemm_config2_group_every_output(dmq):
    """The benchmark's step: one layer's seven projections at M = 1024 in one
    grouped launch (Q, K, V, O, gate, up in Q4_K, down in Q6_K; each with its
    own seeded unit-RMS input), every output against the oracle."""
    M = 1024
    items = _layer_group(dmq, 2, 0, M)
    ys = _run_layer_group(dmq, items, M)
    for (name, fmt, N, K, wq, x), y in zip(items, ys):
        ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
        assert_within(y, ref, s, f"config2 {name} M={M} (every output)")


@pytest.mark.parametrize("layer", range(synthetic.N_LAYERS))
def test_gemm_config4_m1024_layer_every_output(dmq, layer):
    """Config 4 at M = 1024: each of the 28 independently seeded layers in
    the grouped launch, every output of all seven projections."""
    M = 1024
    items = _layer_group(dmq, 4, layer, M)
    ys = _run_layer_group(dmq, items, M)
    for (name, fmt, N, K, wq, x), y in zip(items, ys):
        ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
        assert_within(y, ref, s, f"config4 layer {layer} {name} M={M} (every output)")


@pytest.mark.parametrize("M", [2048, 4096])
def test_gemm_config4_large_m_group_sampled(dmq, M):
    """Config 4 at M = 2048 / 4096 in the grouped launch the sweep times: one
    row in every 32-row group (so every M tile of every height the launch
    plan may pick), all columns of all seven projections (every N tile and
    every split-K piece)."""
    items = _layer_group(dmq, 4, 0, M)
    ys = _run_layer_group(dmq, items, M)
    rows = synthetic.row_sample(M, M // 32, seed=M + 1, tile=32)
    assert len(np.unique(rows // 32)) == M // 32
    for (name, fmt, N, K, wq, x), y in zip(items, ys):
        ref, s = oracle.gemm_quant(fmt, x[rows], wq, N, K)
        assert_within(y[rows], ref, s, f"config4 {name} M={M} ({len(rows)} rows, all columns)")


def test_gemm_group_matches_single_calls(dmq):
    """A grouped launch and one call per problem may tile (and split K)
    differently, so their fp32 sums may round differently: both must meet
    the bar, and repeating a call must give the same bits."""
    M = 300
    items = _layer_group(dmq, 2, 1, M)
    probs, singles, host = [], [], []
    for name, fmt, N, K, wq, x in items:
        xd, wd = dev(x), dev(wq.reshape(-1))
        probs.append((fmt, xd, wd, torch.empty((M, N), dtype=torch.float32, device=DEV), M, N, K))
        singles.append((fmt, xd, wd, torch.empty((M, N), dtype=torch.float32, device=DEV), M, N, K))
        host.append((name, fmt, N, K, wq, x))
    dmq.dmq_gemm_group(probs)
    for fmt, xd, wd, ys, M_, N, K in singles:
        (dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k)(xd, wd, ys, M_, N, K)
    torch.cuda.synchronize()
    first = [p[3].clone() for p in probs]
    dmq.dmq_gemm_group(probs)
    torch.cuda.synchronize()
    for p, s_, f, (name, fmt, N, K, wq, x) in zip(probs, singles, first, host):
        assert torch.equal(p[3], f), f"{name}: repeated grouped launch changed bits"
        ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
        assert_within(p[3].cpu().numpy(), ref, s, f"group {name} M={M}")
        assert_within(s_[3].cpu().numpy(), ref, s, f"single {name} M={M}")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("M,N,K", [(40, 37, 8192), (33, 250, 4864), (48, 3072, 768), (1024, 3072, 8192)])
def test_gemm_split_k(dmq, fmt, M, N, K):
    """Too few output tiles to fill the GPU: the launch splits the K blocks
    into pieces whose fp32 partial sums a second kernel adds in piece order
    (M*N not a multiple of 4 takes the combine's scalar tail).  Every output
    is checked (the largest shape, the FFN down projection, on sampled
    rows), and a second call must give the same bits."""
    x = synthetic.activations(M, K, seed=M * 7 + K)
    wq = synthetic.weight_blocks(fmt, N, K, seed=N * 5 + K)
    xd, wd = dev(x), dev(wq.reshape(-1))
    fn = dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k
    y1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    fn(xd, wd, y1, M, N, K)
    fn(xd, wd, y2, M, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "split-K result is not reproducible"
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y1.cpu().numpy(), ref, s, f"split-K {fmt} {M}x{N}x{K} (every output)")


def test_gemm_split_k_interleaved_shapes(dmq):
    """Split launches share a per-stream workspace of partial sums: interleave
    split launches of different piece counts and tile grids on one stream
    (and one launch on a second stream, with its own workspace), repeat
    each, and require the bits of its first call."""
    shapes = [("q6k", 40, 37, 8192), ("q4k", 33, 250, 4864), ("q6k", 1024, 3072, 8192), ("q4k", 48, 3072, 768)]
    runs = []
    for fmt, M, N, K in shapes:
        x = synthetic.activations(M, K, seed=M + 3 * K)
        wq = synthetic.weight_blocks(fmt, N, K, seed=N + 11 * K)
        runs.append((fmt, M, N, K, x, wq, dev(x), dev(wq.reshape(-1))))
    def call(r, stream=None):
        fmt, M, N, K, _, _, xd, wd = r
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        fn = dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k
        fn(xd, wd, y, M, N, K, stream=stream)
        return y
    first = [call(r) for r in runs]
    again = [call(r) for r in reversed(runs)][::-1]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = call(runs[2], stream=side.cuda_stream)
    side.synchronize()
    third = [call(r) for r in runs]
    torch.cuda.synchronize()
    for r, a, b, c in zip(runs, first, again, third):
        assert torch.equal(a, b) and torch.equal(a, c), f"split-K bits changed across launches: {r[:4]}"
    assert torch.equal(first[2], other), "split-K bits differ on a second stream"
    for r, y in zip(runs, first):
        fmt, M, N, K, x, wq = r[:6]
        ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
        assert_within(y.cpu().numpy(), ref, s, f"interleaved split-K {fmt} {M}x{N}x{K}")


def test_concurrent_host_threads_same_bits(dmq):
    """Four host threads call the library at once, each on a stream of its
    own: split-K GEMMs (the plan cache and the per-stream workspaces), a
    decode GEMV, the SwiGLU FFN and RoPE + attention in one call (the
    attention workspace).  Every output has the bits of the same call made
    alone on the default stream."""
    import threading
    rng = np.random.default_rng(77)

    def gemm_case(fmt, M, N, K, seed):
        x = dev(synthetic.activations(M, K, seed=seed))
        wq = dev(synthetic.weight_blocks(fmt, N, K, seed=seed + 1).reshape(-1))
        fn = dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k

        def run(stream):
            y = torch.empty((M, N), dtype=torch.float32, device=DEV)
            fn(x, wq, y, M, N, K, stream=stream)
            return [y]
        return run

    def ffn_case(M, D, F, seed):
        x = dev(synthetic.activations(M, D, seed=seed))
        wgu = dev(synthetic.q4k_blocks(2 * F, D, seed=seed + 1).reshape(-1))
        wd = dev(synthetic.q6k_blocks(D, F, seed=seed + 2).reshape(-1))

        def run(stream):
            h = torch.empty((M, F), dtype=torch.float16, device=DEV)
            y = torch.empty((M, D), dtype=torch.float32, device=DEV)
            dmq.dmq_ffn_swiglu_q4k(x, wgu, wd, h, y, M, D, F, stream=stream)
            return [h, y]
        return run

    def attn_case(pos0, hq, hkv, L):
        q, k, v = (dev(rng.standard_normal((1, n * D_HEAD)).astype(np.float32)) for n in (hq, hkv, hkv))
        base = [rng.standard_normal((hkv, L, D_HEAD)).astype(np.float16) for _ in range(2)]

        def run(stream):
            kc, vc = dev(base[0]), dev(base[1])
            qo = torch.empty((1, hq * D_HEAD), dtype=torch.float16, device=DEV)
            out = torch.empty((1, hq * D_HEAD), dtype=torch.float16, device=DEV)
            # the cache copies above are on the current stream, which is the call's
            dmq.dmq_rope_attention_gqa(q, k, v, 1, pos0, hq, hkv, qo, kc, vc, L, out, stream=stream)
            return [qo, kc, vc, out]
        return run

    jobs = [[gemm_case("q6k", 1024, 3072, 8192, 5), gemm_case("q4k", 1, 3072, 3072, 6)],
            [gemm_case("q4k", 33, 250, 4864, 7), ffn_case(300, 768, 1024, 8)],
            [attn_case(1000, 24, 8, 1024), gemm_case("q6k", 40, 37, 8192, 9)],
            [gemm_case("q4k", 700, 1000, 3072, 10), attn_case(63, 6, 2, 128)]]
    ref = [[[t.clone() for t in run(None)] for run in job] for job in jobs]
    torch.cuda.synchronize()
    got = [None] * len(jobs)
    errors = []

    def worker(j):
        try:
            stream = torch.cuda.Stream()
            res = []
            with torch.cuda.stream(stream):
                for _ in range(5):
                    res.append([run(stream.cuda_stream) for run in jobs[j]])
            stream.synchronize()
            got[j] = res
        except Exception as e:   # reported below, in the main thread
            errors.append(e)
    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    def bits(t):   # NaNs (the FFN's overflowed h feeds inf - inf into y) compare by their bits
        return t.view(torch.int16 if t.dtype == torch.float16 else torch.int32)
    for j, job_ref in enumerate(ref):
        for it, outs in enumerate(got[j]):
            for c, (a, b) in enumerate(zip(job_ref, outs)):
                for ta, tb in zip(a, b):
                    assert torch.equal(bits(ta), bits(tb)), f"thread {j} call {c} round {it}: bits differ from the lone call"


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("M,N,K", [(2, 16, 256), (16, 40, 256), (12, 20, 768), (5, 37, 4864), (9, 33, 512),
                                   (16, 3072, 3072), (16, 48, 8192), (7, 50, 9984), (17, 100, 1280), (32, 257, 768),
                                   (5, 8195, 1280), (3, 8200, 256)])
def test_gemm_small_m_every_output(dmq, fmt, M, N, K):
    """M <= 16 runs the small-M kernel (16 weight rows per workgroup, the
    rows' products on 16x16x32 MFMAs): every output and the same bits on a
    second call.  Shapes: one wave per K block up to 16, workgroups of 1, 2
    and 3 waves with all 16 activation rows live (fewer threads than
    outputs); 16 waves walking several blocks each (uneven slices: 19, 32
    and 39 blocks over 16 waves); grids of at least two
    workgroups per CU (N = 8195, 8200: 4 waves, with rows past M read as
    zero, a ragged last workgroup, and waves without blocks at K = 256).  x
    goes through LDS in every shape.  M = 17 and 32 (single projections,
    fewer than two workgroups per CU) run it with two 16-row groups of
    activation rows."""
    x = synthetic.activations(M, K, seed=M * 11 + N)
    wq = synthetic.weight_blocks(fmt, N, K, seed=N * 13 + K + M)
    xd, wd = dev(x), dev(wq.reshape(-1))
    fn = dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k
    y1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    fn(xd, wd, y1, M, N, K)
    fn(xd, wd, y2, M, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "small-M result is not reproducible"
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y1.cpu().numpy(), ref, s, f"small-M {fmt} {M}x{N}x{K}")


def test_gemm_small_m_layer_group(dmq):
    """The 7 projections of one layer at M = 16 in one grouped launch (mixed
    Q4_K / Q6_K, K = 3072 and 8192) against the oracle on every output."""
    M = 16
    items = _layer_group(dmq, 0, 3, M)
    probs, host = [], []
    for name, fmt, N, K, wq, x in items:
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        probs.append((fmt, dev(x), dev(wq.reshape(-1)), y, M, N, K))
        host.append((name, fmt, N, K, wq, x, y))
    dmq.dmq_gemm_group(probs)
    torch.cuda.synchronize()
    for name, fmt, N, K, wq, x, y in host:
        ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
        assert_within(y.cpu().numpy(), ref, s, f"small-M group {name} M={M}")


def test_lm_head_every_output(dmq):
    """Config 4's tied LM head: Q6_K 3072 -> 128256 on 1024 rows, every
    output (807 GFLOP in the oracle)."""
    name, fmt, N, K = synthetic.LM_HEAD
    M = 1024
    wq = synthetic.lm_head_weights(4)
    x = synthetic.activations(M, K, seed=synthetic.act_seed(4, 0, synthetic.LM_HEAD_INDEX), unit_rms=True)
    y = gpu_gemm(dmq, fmt, x, wq, M, N, K)
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y, ref, s, f"lm_head M={M} (every output)")


def test_lm_head_decode_every_output(dmq):
    """The tied LM head at M = 1 (one decode token): the decode kernel over
    128,256 Q6_K rows in 8,016 workgroups, every output."""
    name, fmt, N, K = synthetic.LM_HEAD
    wq = synthetic.lm_head_weights(4)
    x = synthetic.activations(1, K, seed=synthetic.act_seed(4, 0, synthetic.LM_HEAD_INDEX) + 1, unit_rms=True)
    y = gpu_gemm(dmq, fmt, x, wq, 1, N, K)
    ref, s = oracle.gemm_quant(fmt, x, wq, N, K)
    assert_within(y, ref, s, "lm_head M=1 (every output)")


# ------------------------------------------------------------------- FFN ---

def run_ffn(dmq, x, wgu, wd, M, D, F):
    h = torch.empty((M, F), dtype=torch.float16, device=DEV)
    y = torch.empty((M, D), dtype=torch.float32, device=DEV)
    dmq.dmq_ffn_swiglu_q4k(dev(x), dev(wgu.reshape(-1)), dev(wd.reshape(-1)), h, y, M, D, F)
    torch.cuda.synchronize()
    return h.cpu().numpy(), y.cpu().numpy()


def check_ffn(x, wgu, wd, h, y, D, F, rows, what):
    # stage 1: h against the SwiGLU interval of the oracle's g, u
    gu, s = oracle.gemm_quant("q4k", x[rows], wgu, 2 * F, D)
    eg = oracle.gemm_tolerance(s)
    g, u = gu[:, :F], gu[:, F:]
    lo, hi = oracle.swiglu_interval(g, u, eg[:, :F], eg[:, F:])
    hv = h[rows].astype(np.float64)
    ok = oracle.swiglu_accepts(hv, lo, hi)
    assert ok.all(), f"{what} h: {int((~ok).sum())} of {ok.size} outside the interval"
    overflow = float(np.mean(~np.isfinite(hv)))
    # stage 2: down projection of the GPU's own h
    ref, sd = oracle.gemm_quant("q6k", h[rows], wd, D, F)
    yr = y[rows].astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(yr), np.isnan(ref)), f"{what} y: NaN pattern differs"
    assert np.array_equal(yr[~fin & ~np.isnan(ref)], ref[~fin & ~np.isnan(ref)]), f"{what} y: inf differs"
    if fin.any():
        err = np.abs(yr[fin] - ref[fin])
        tol = oracle.gemm_tolerance(sd[fin])
        assert np.all(err <= tol), f"{what} y: {int((err > tol).sum())} outputs outside the bound"
    print(f"{what}: h overflow fraction {overflow:.4f}")
    return overflow


def _ffn_weights(config):
    D, F = synthetic.HIDDEN, synthetic.FFN
    wgu = synthetic.q4k_blocks(2 * F, D, seed=synthetic.weight_seed(config, 0, 4))
    wd = synthetic.q6k_blocks(D, F, seed=synthetic.weight_seed(config, 0, 6))
    return D, F, wgu, wd


@pytest.mark.parametrize("sigma", [1.0, 1.0 / 16])
def test_ffn_config3_every_output(dmq, sigma):
    """Config 3 at both input scales, every h value and every y output."""
    D, F, wgu, wd = _ffn_weights(3)
    M = 1024
    x = synthetic.activations(M, D, seed=synthetic.act_seed(3, 0, 0), sigma=sigma)
    h, y = run_ffn(dmq, x, wgu, wd, M, D, F)
    ov = check_ffn(x, wgu, wd, h, y, D, F, np.arange(M), f"config3 sigma={sigma} (every output)")
    if sigma < 1:
        assert ov == 0.0


def test_ffn_decode_m1(dmq):
    D, F, wgu, wd = _ffn_weights(3)
    x = synthetic.activations(1, D, seed=12, sigma=1.0 / 16)
    h, y = run_ffn(dmq, x, wgu, wd, 1, D, F)
    check_ffn(x, wgu, wd, h, y, D, F, np.array([0]), "ffn decode M=1")


@pytest.mark.parametrize("M,D,F", [(2, 256, 512), (40, 512, 768), (300, 768, 256), (1, 512, 1024), (16, 3072, 8192),
                                   (7, 1280, 768), (24, 3072, 8192)])
def test_ffn_small_every_output(dmq, M, D, F):
    """The FFN chain on every output.  M = 2, 7 and 16 run the gate|up pair
    in the small-M kernel's SwiGLU mode (8 gate and 8 up rows per
    workgroup): at 3072 -> 2 x 8192 (the Llama-3.2-3B shape) a grid of 1024
    4-wave workgroups, at 1280 -> 2 x 768 one wave per block; the down
    projection then takes 16 waves walking 2 blocks each (K = 8192) or one
    wave per block.  M = 24 runs both stages on the small-M kernel with two
    16-row groups of activation rows (4-wave workgroups for the pair, 8
    waves for the down projection).  M = 1 runs the decode kernel's pairs,
    M = 40 and 300 the tiled kernel."""
    wgu = synthetic.q4k_blocks(2 * F, D, seed=M + D)
    wd = synthetic.q6k_blocks(D, F, seed=M + F)
    x = synthetic.activations(M, D, seed=M * 3, sigma=0.25)
    h, y = run_ffn(dmq, x, wgu, wd, M, D, F)
    check_ffn(x, wgu, wd, h, y, D, F, np.arange(M), f"ffn {M}x{D}x{F}")


def test_single_hip_runtime_and_native_library(dmq):
    """The library runs on the same HIP runtime as torch (one libamdhip64 and
    one libhsa-runtime64 mapped) and is the in-tree build."""
    torch.zeros(1, device=DEV)
    maps = open("/proc/self/maps").read().splitlines()
    paths = {l.split()[-1] for l in maps if len(l.split()) >= 6}
    hip = {p for p in paths if "libamdhip64" in p}
    hsa = {p for p in paths if "libhsa-runtime64" in p}
    assert len(hip) == 1, hip
    assert len(hsa) == 1, hsa
    assert dmq.LIB_PATH in paths


# --------------------------------------------------------------- RMSNorm ---
# dmq_rmsnorm_gemm, checked stage by stage (the reading used for the FFN's h):
# the normalized activations xn must lie within one fp16 step of the oracle's
# exact fp64 RMSNorm (interval rounded outward from +-2^-16 relative: fp32 sum
# of squares, square root, products); y must meet the GEMM bound against the
# oracle's fp64 product of the GPU's own xn with the exactly dequantised
# weights.  At M = 1 the decode kernel writes the xn it staged when asked to.

def _norm_weights(K, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, K).astype(np.float32)


def _rmsnorm_gemm(dmq, x, g, eps, projs, M, K, want_xn=True):
    """projs: list of (fmt, wq, N). Returns (xn or None, [y_i])."""
    xn = torch.empty((M, K), dtype=torch.float16, device=DEV) if want_xn else None
    ys = [torch.empty((M, N), dtype=torch.float32, device=DEV) for _, _, N in projs]
    dmq.dmq_rmsnorm_gemm(dev(x), dev(g), eps, xn,
                         [(fmt, dev(wq.reshape(-1)), y, N) for (fmt, wq, N), y in zip(projs, ys)], M, K)
    torch.cuda.synchronize()
    return (None if xn is None else xn.cpu().numpy()), [y.cpu().numpy() for y in ys]


def _check_rmsnorm_outputs(x, g, eps, projs, K, xn, ys, what, rows=None):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    xhat = oracle.rmsnorm(sel(x), g, eps)
    got = sel(xn)
    lo, hi = oracle.rmsnorm_f16_interval(xhat)
    ok = (got.astype(np.float64) >= lo) & (got.astype(np.float64) <= hi)
    assert ok.all(), f"{what}: xn has {int((~ok).sum())} of {ok.size} values outside the interval"
    for (fmt, wq, N), y in zip(projs, ys):
        ref, s = oracle.gemm_quant(fmt, got, wq, N, K)
        assert_within(sel(y), ref, s, f"{what} {fmt} N={N}")


@pytest.mark.parametrize("M,K", [(2, 256), (5, 768), (16, 3072), (40, 512), (300, 1024), (257, 2304)])
def test_rmsnorm_gemm_every_output(dmq, M, K):
    x = synthetic.activations(M, K, seed=M * 7 + K, sigma=2.0)
    g = _norm_weights(K, seed=K)
    projs = [("q4k", synthetic.q4k_blocks(96, K, seed=M + 1), 96),
             ("q4k", synthetic.q4k_blocks(37, K, seed=M + 2), 37),
             ("q6k", synthetic.q6k_blocks(64, K, seed=M + 3), 64)]
    xn, ys = _rmsnorm_gemm(dmq, x, g, 1e-5, projs, M, K)
    _check_rmsnorm_outputs(x, g, 1e-5, projs, K, xn, ys, f"rmsnorm+gemm M={M} K={K}")


def test_rmsnorm_lm_head_decode_every_output(dmq):
    """The end of a decode step: the final RMSNorm fused into the tied LM
    head (Q6_K 3072 -> 128256) at M = 1, 8,016 workgroups each normalizing
    x while staging it; xn from workgroup 0, every logit."""
    name, fmt, N, K = synthetic.LM_HEAD
    x = synthetic.activations(1, K, seed=77, sigma=3.0)
    g = _norm_weights(K, seed=78)
    projs = [(fmt, synthetic.lm_head_weights(4), N)]
    xn, ys = _rmsnorm_gemm(dmq, x, g, 1e-5, projs, 1, K)
    _check_rmsnorm_outputs(x, g, 1e-5, projs, K, xn, ys, "final rmsnorm + lm_head M=1")


@pytest.mark.parametrize("K", [256, 3072, 8192, 32768])
def test_rmsnorm_gemv_decode_every_output(dmq, K):
    # M = 1: the decode kernel normalizes x while staging it
    x = synthetic.activations(1, K, seed=K + 5, sigma=3.0)
    g = _norm_weights(K, seed=K + 1)
    projs = [("q4k", synthetic.q4k_blocks(200, K, seed=K + 2), 200),
             ("q6k", synthetic.q6k_blocks(33, K, seed=K + 3), 33)]
    xn, ys = _rmsnorm_gemm(dmq, x, g, 1e-5, projs, 1, K)
    _check_rmsnorm_outputs(x, g, 1e-5, projs, K, xn, ys, f"rmsnorm+gemv K={K}")
    # without xn the results are the same bits
    _, ys2 = _rmsnorm_gemm(dmq, x, g, 1e-5, projs, 1, K, want_xn=False)
    for a, b in zip(ys, ys2):
        assert np.array_equal(a, b)


def test_rmsnorm_edge_rows(dmq):
    # a zero row (eps > 0 keeps it zero), a row of one huge value, a row of
    # fp16 subnormals (normalized to subnormals again under a large eps), and
    # a large eps that dominates the mean square
    M, K = 4, 512
    x = np.zeros((M, K), dtype=np.float16)
    x[1, 7] = 60000.0
    x[2, :] = np.float16(3e-7)
    x[3, :] = synthetic.activations(1, K, seed=3)[0]
    g = _norm_weights(K, seed=9)
    projs = [("q4k", synthetic.q4k_blocks(64, K, seed=4), 64), ("q6k", synthetic.q6k_blocks(40, K, seed=5), 40)]
    for eps in (1e-5, 4.0):
        xn, ys = _rmsnorm_gemm(dmq, x, g, eps, projs, M, K)
        assert np.all(xn[0] == 0) and np.all(ys[0][0] == 0) and np.all(ys[1][0] == 0)
        _check_rmsnorm_outputs(x, g, eps, projs, K, xn, ys, f"rmsnorm edge rows eps={eps}")
        # the same rows one at a time through the decode path
        for m in range(M):
            xn1, ys1 = _rmsnorm_gemm(dmq, x[m:m + 1], g, eps, projs, 1, K)
            _check_rmsnorm_outputs(x[m:m + 1], g, eps, projs, K, xn1, ys1, f"rmsnorm edge row {m} decode")


def test_rmsnorm_qkv_layer_shapes_every_output(dmq):
    # the Q|K|V projections of one Llama-3.2-3B-shaped layer behind their
    # RMSNorm, at M = 1024 (tiled kernel, grouped) and M = 1 (decode kernel)
    K = 3072
    g = _norm_weights(K, seed=77)
    projs = [("q4k", synthetic.q4k_blocks(N, K, seed=synthetic.weight_seed(2, 0, i)), N)
             for i, N in enumerate((3072, 1024, 1024))]
    M = 1024
    x = synthetic.activations(M, K, seed=synthetic.act_seed(2, 0, 0), sigma=1.5)
    xn, ys = _rmsnorm_gemm(dmq, x, g, 1e-5, projs, M, K)
    _check_rmsnorm_outputs(x, g, 1e-5, projs, K, xn, ys, "rmsnorm QKV M=1024 (every output)")
    xn1, ys1 = _rmsnorm_gemm(dmq, x[:1], g, 1e-5, projs, 1, K)
    _check_rmsnorm_outputs(x[:1], g, 1e-5, projs, K, xn1, ys1, "rmsnorm QKV M=1")


# -------------------------------------------------------------------------
# The attention side of a decoder layer: RoPE + KV-cache append, grouped-query
# attention over the cache, residual add fused with the next RMSNorm.  Each
# stage is checked against the oracle on the GPU's own inputs to that stage;
# the layer chain at the end adds an end-to-end comparison with the fp64
# oracle layer.

from oracle import attention as attn  # noqa: E402

D_HEAD = 128


def _rope_case(dmq, M, pos0, hq, hkv, cache_len, seed, freq_factors=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((M, hq * D_HEAD)).astype(np.float32)
    k = rng.standard_normal((M, hkv * D_HEAD)).astype(np.float32)
    v = rng.standard_normal((M, hkv * D_HEAD)).astype(np.float32)
    sentinel = np.float16(7.0)
    kc = torch.full((hkv, cache_len, D_HEAD), sentinel, dtype=torch.float16, device=DEV)
    vc = torch.full((hkv, cache_len, D_HEAD), sentinel, dtype=torch.float16, device=DEV)
    qo = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    ff = None if freq_factors is None else dev(freq_factors.astype(np.float32))
    dmq.dmq_rope_kv_cache(dev(q), dev(k), dev(v), M, pos0, hq, hkv, qo, kc, vc, cache_len, freq_factors=ff)
    torch.cuda.synchronize()
    return q, k, v, qo.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy(), sentinel


def _check_rope(q, k, v, qo, kc, vc, sentinel, M, pos0, hq, hkv, what, freq_factors=None):
    pos = np.arange(pos0, pos0 + M)
    for src, got, h in ((q, qo.reshape(M, hq, D_HEAD), hq),
                        (k, kc[:, pos0:pos0 + M, :].transpose(1, 0, 2), hkv)):
        x = src.reshape(M, h, D_HEAD).astype(np.float64)
        exact = attn.rope(x, pos, freq_factors=freq_factors)
        # fp32 cos/sin (one rounding each) and the fp32 rotation: a few units
        # of 2^-24 of the pair's magnitude before the final fp16 rounding
        mag = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
        lo, hi = oracle.f16_interval(exact, mag * 2.0 ** -21)
        g64 = got.astype(np.float64)
        ok = (g64 >= lo) & (g64 <= hi)
        assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} rotated values outside the interval"
    # V rows: fp16 of the fp32 projection, bit for bit
    want_v = v.reshape(M, hkv, D_HEAD).astype(np.float16).transpose(1, 0, 2)
    assert np.array_equal(vc[:, pos0:pos0 + M, :].view(np.uint16), want_v.view(np.uint16)), f"{what}: V rows differ"
    # nothing outside rows pos0 .. pos0+M-1 is touched
    for c in (kc, vc):
        outside = np.concatenate([c[:, :pos0, :].ravel(), c[:, pos0 + M:, :].ravel()])
        assert np.all(outside == sentinel), f"{what}: cache rows outside the written range changed"


@pytest.mark.parametrize("M,pos0,hq,hkv,cache_len", [(1, 0, 24, 8, 8), (1, 1023, 24, 8, 1024), (7, 100, 24, 8, 200),
                                                     (64, 0, 24, 8, 64), (3, 131000, 6, 2, 131072),
                                                     (5, 17, 8, 8, 40), (2, 9, 16, 2, 16)])
def test_rope_kv_cache(dmq, M, pos0, hq, hkv, cache_len):
    q, k, v, qo, kc, vc, sent = _rope_case(dmq, M, pos0, hq, hkv, cache_len, seed=M * 31 + pos0)
    _check_rope(q, k, v, qo, kc, vc, sent, M, pos0, hq, hkv, f"rope M={M} pos0={pos0} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("M,pos0,hq,hkv,cache_len,ff", [(1, 0, 24, 8, 16, False), (1, 63, 24, 8, 128, False),
                                                         (1, 64, 24, 8, 128, True), (1, 1023, 24, 8, 1024, False),
                                                         (1, 4095, 8, 1, 5000, True), (1, 300, 6, 2, 512, False),
                                                         (1, 131071, 24, 8, 131072, False),
                                                         (5, 100, 24, 8, 200, False), (40, 7, 24, 8, 64, True)])
def test_rope_attention_fused_equals_two_calls(dmq, M, pos0, hq, hkv, cache_len, ff):
    """dmq_rope_attention_gqa gives the bits of dmq_rope_kv_cache followed by
    dmq_attention_gqa on every output: the rotated queries, both caches
    whole (the appended rows and every row it must not touch) and the
    attention output.  M = 1 runs the fused decode kernel; M = 5 (split
    path) and M = 40 (MFMA path) run the two launches."""
    rng = np.random.default_rng(M * 7919 + pos0)
    qd, kd = hq * D_HEAD, hkv * D_HEAD
    q = dev(rng.standard_normal((M, qd)).astype(np.float32))
    k = dev(rng.standard_normal((M, kd)).astype(np.float32))
    v = dev(rng.standard_normal((M, kd)).astype(np.float32))
    f = dev(rng.uniform(1.0, 32.0, D_HEAD // 2).astype(np.float32)) if ff else None
    cache0 = [rng.standard_normal((hkv, cache_len, D_HEAD), dtype=np.float32).astype(np.float16) for _ in range(2)]
    outs = []
    for fused in (False, True):
        kc, vc = dev(cache0[0]), dev(cache0[1])
        qo = torch.empty((M, qd), dtype=torch.float16, device=DEV)
        out = torch.empty((M, qd), dtype=torch.float16, device=DEV)
        if fused:
            dmq.dmq_rope_attention_gqa(q, k, v, M, pos0, hq, hkv, qo, kc, vc, cache_len, out, freq_factors=f)
        else:
            dmq.dmq_rope_kv_cache(q, k, v, M, pos0, hq, hkv, qo, kc, vc, cache_len, freq_factors=f)
            dmq.dmq_attention_gqa(qo, kc, vc, out, M, pos0, hq, hkv, cache_len)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().view(np.uint16) for t in (qo, kc, vc, out)])
    for name, a, b in zip(("q_f16", "k_cache", "v_cache", "out"), outs[0], outs[1]):
        assert np.array_equal(a, b), f"{name}: {int((a != b).sum())} of {a.size} values differ"


def test_rope_kv_cache_freq_factors(dmq):
    # the factors as the kernel receives them (fp32); the oracle takes the same values
    f = np.random.default_rng(9).uniform(1.0, 32.0, D_HEAD // 2).astype(np.float32)
    q, k, v, qo, kc, vc, sent = _rope_case(dmq, 4, 5000, 24, 8, 5004, seed=99, freq_factors=f)
    _check_rope(q, k, v, qo, kc, vc, sent, 4, 5000, 24, 8, "rope with frequency factors", freq_factors=f)


def _attention_case(dmq, M, pos0, hq, hkv, cache_len, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    n = pos0 + M
    q = (rng.standard_normal((M, hq * D_HEAD)) * spread).astype(np.float16)
    kc = np.zeros((hkv, cache_len, D_HEAD), np.float16)
    vc = np.zeros((hkv, cache_len, D_HEAD), np.float16)
    kc[:, :n, :] = (rng.standard_normal((hkv, n, D_HEAD)) * spread).astype(np.float16)
    vc[:, :n, :] = rng.standard_normal((hkv, n, D_HEAD)).astype(np.float16)
    out = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    dmq.dmq_attention_gqa(dev(q), dev(kc), dev(vc), out, M, pos0, hq, hkv, cache_len)
    torch.cuda.synchronize()
    return q, kc, vc, out.cpu().numpy()


def _check_attention(q, kc, vc, out, M, pos0, hq, what):
    q3 = q.reshape(M, hq, D_HEAD).astype(np.float64)
    ref, mass = attn.attention_gqa(q3, kc, vc, pos0)
    got = out.reshape(M, hq, D_HEAD).astype(np.float64)
    # final fp16 rounding (2^-11 relative), fp32 exp / sums (5e-4 of the
    # output's scale sum p|v|), and the fp32 scores: a 128-term fp32 dot is
    # off by at most 128 * 2^-24 * sum |q k| / sqrt(128), which moves every
    # weight by that factor in the exponent (twice the largest such error
    # times sum p|v| bounds the output change)
    hkv = kc.shape[0]
    grp = hq // hkv
    ds = np.zeros((M, hq, 1))
    for h in range(hq):
        kabs = np.abs(kc[h // grp].astype(np.float64))
        for i in range(M):
            n = pos0 + i + 1
            ds[i, h, 0] = 128 * 2.0 ** -24 * np.max(kabs[:n] @ np.abs(q3[i, h])) / np.sqrt(D_HEAD)
    tol = 2.0 ** -10 * np.abs(ref) + (5e-4 + 2.0 * ds) * mass + 1e-6
    err = np.abs(got - ref)
    ok = err <= tol
    worst = float(np.max(err / tol))
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outputs outside the bound (worst {worst:.3g})"
    print(f"{what}: max err/bound = {worst:.3g}")


@pytest.mark.parametrize("M,pos0,hq,hkv,cache_len", [(1, 0, 24, 8, 16), (1, 1023, 24, 8, 1024), (1, 4096, 24, 8, 5000),
                                                     (7, 100, 24, 8, 128), (64, 0, 24, 8, 64), (3, 1500, 6, 2, 2048),
                                                     (33, 600, 8, 8, 700), (5, 511, 16, 2, 600),
                                                     (4, 20, 4, 4, 32), (2, 7, 5, 1, 9)])
def test_attention_gqa(dmq, M, pos0, hq, hkv, cache_len):
    """Decode (M = 1) at several cache lengths, chunk boundaries (512 keys),
    prefill blocks with and without an offset, and every group size from 1
    to 8 query heads per KV head."""
    q, kc, vc, out = _attention_case(dmq, M, pos0, hq, hkv, cache_len, seed=M * 13 + pos0)
    _check_attention(q, kc, vc, out, M, pos0, hq, f"attention M={M} pos0={pos0} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("M,pos0,hq,hkv", [(17, 0, 24, 8), (300, 50, 24, 8), (129, 1000, 6, 2), (200, 3, 8, 1)])
def test_attention_gqa_prefill_mfma(dmq, M, pos0, hq, hkv):
    """More than 16 queries run the MFMA kernel (128 queries per workgroup,
    32-key blocks): ragged query blocks, a cache offset, the causal diagonal
    inside blocks, group sizes 3, 1 and 8."""
    q, kc, vc, out = _attention_case(dmq, M, pos0, hq, hkv, pos0 + M + 5, seed=M + pos0)
    _check_attention(q, kc, vc, out, M, pos0, hq, f"attention prefill M={M} pos0={pos0} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("M", [1024, 2048])
def test_attention_gqa_prefill_full_size_sampled(dmq, M):
    """The Llama-3.2-3B prefill shape (1024 or 2048 queries from position 0,
    24 query heads over 8 KV heads), every output of a sample of query rows
    that covers every 128-query block and both ends."""
    hq, hkv = 24, 8
    q, kc, vc, out = _attention_case(dmq, M, 0, hq, hkv, M, seed=77 + M)
    rows = synthetic.row_sample(M, 24 * M // 1024, seed=3, tile=128)
    # the oracle on the sampled rows: each row's attention depends only on its
    # own query and the cache
    for r in rows:
        _check_attention(q[r:r + 1], kc, vc, out[r:r + 1], 1, int(r), hq, f"attention prefill {M} row {r}")


def test_attention_gqa_long_context_fallback(dmq):
    """Beyond 4096 pieces of 64 positions (262,144 cached positions) the
    decode attention runs its one-workgroup-per-KV-head kernel instead of the
    split pieces; the no-allocation call takes the same kernel (it needs no
    scratch there) and gives the same bits."""
    M, pos0, hq, hkv = 2, 262200, 4, 1
    cache_len = pos0 + M + 6
    q, kc, vc, out = _attention_case(dmq, M, pos0, hq, hkv, cache_len, seed=21)
    _check_attention(q, kc, vc, out, M, pos0, hq, "attention fallback past 262144 positions")
    o2 = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    dmq.dmq_attention_gqa_noalloc(dev(q), dev(kc), dev(vc), o2, M, pos0, hq, hkv, cache_len)
    torch.cuda.synchronize()
    assert np.array_equal(o2.cpu().numpy().view(np.uint16), out.view(np.uint16))


def test_attention_gqa_peaked_scores(dmq):
    """Large score spread (one key dominates, many weights underflow) and a
    run of 3 decode steps appending to the same cache."""
    q, kc, vc, out = _attention_case(dmq, 2, 900, 24, 8, 1024, seed=5, spread=4.0)
    _check_attention(q, kc, vc, out, 2, 900, 24, "attention peaked")


@pytest.mark.parametrize("M,pos0,hq,hkv", [(300, 20, 24, 8), (150, 0, 6, 2)])
def test_attention_gqa_prefill_rising_scores(dmq, M, pos0, hq, hkv):
    """Prefill (MFMA path) with scores that rise along the keys by about 45
    in natural units: every query's running maximum moves many times, by
    more and by less than 2^8 in the exp2 domain, and a large spread case
    (one key dominates, most weights underflow)."""
    rng = np.random.default_rng(M + hq)
    n = pos0 + M
    u = rng.standard_normal(D_HEAD)
    q = (rng.standard_normal((M, hq, D_HEAD)) * 0.5 + 2.0 * u).astype(np.float16).reshape(M, hq * D_HEAD)
    ramp = 2.0 * np.arange(n) / n
    kc = (rng.standard_normal((hkv, n, D_HEAD)) * 0.5 + ramp[None, :, None] * u).astype(np.float16)
    vc = rng.standard_normal((hkv, n, D_HEAD)).astype(np.float16)
    out = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    dmq.dmq_attention_gqa(dev(q), dev(kc), dev(vc), out, M, pos0, hq, hkv, n)
    torch.cuda.synchronize()
    _check_attention(q, kc, vc, out.cpu().numpy(), M, pos0, hq, f"attention rising M={M} pos0={pos0}")
    q2, kc2, vc2, out2 = _attention_case(dmq, M, pos0, hq, hkv, n, seed=M * 7, spread=4.0)
    _check_attention(q2, kc2, vc2, out2, M, pos0, hq, f"attention prefill peaked M={M}")


def test_residual_rmsnorm(dmq):
    rng = np.random.default_rng(21)
    for M, K in ((1, 3072), (5, 768), (64, 3072)):
        h = rng.standard_normal((M, K)).astype(np.float32)
        y = (rng.standard_normal((M, K)) * 3.0).astype(np.float32)
        g = _norm_weights(K, seed=K + M)
        ho = torch.empty((M, K), dtype=torch.float32, device=DEV)
        xn = torch.empty((M, K), dtype=torch.float16, device=DEV)
        dmq.dmq_residual_rmsnorm(dev(h), dev(y), dev(g), 1e-5, ho, xn, M, K)
        # in place, add only
        hin = dev(h)
        dmq.dmq_residual_rmsnorm(hin, dev(y), None, 0.0, hin, None, M, K)
        torch.cuda.synchronize()
        hgot = ho.cpu().numpy()
        assert np.array_equal(hgot, h + y), f"residual M={M}: h_out is not the fp32 sum"
        assert np.array_equal(hin.cpu().numpy(), h + y), f"residual M={M}: in-place add differs"
        xhat = attn.rmsnorm_f64(hgot, g, 1e-5)
        lo, hi = oracle.rmsnorm_f16_interval(xhat)
        got = xn.cpu().numpy().astype(np.float64)
        ok = (got >= lo) & (got <= hi)
        assert ok.all(), f"residual+rmsnorm M={M}: {int((~ok).sum())} normalized values outside the interval"


@pytest.mark.parametrize("M,K", [(1, 768), (1, 3072), (1, 3328), (1, 4096), (1, 8192), (1, 32768), (5, 768)])
def test_residual_rmsnorm_gemm(dmq, M, K):
    """Residual add + RMSNorm + projections in one call: at M = 1 the decode
    kernel forms the sum and the norm while staging x (one launch), above it
    the residual kernel runs first.  Plain Q4_K and Q6_K projections and a
    SwiGLU gate|up pair (h = silu(gate) * up in fp16).  K = 3328 gives uneven
    wave slices (13 blocks), K = 4096 is the largest one-pass staging (every
    lane's second chunk live), K = 8192 and 32768 take the two-pass staging,
    the last with the largest x slice the decode kernel takes (73.7 KB of
    LDS)."""
    rng = np.random.default_rng(M * 31 + K)
    h = rng.standard_normal((M, K)).astype(np.float32)
    ya = (rng.standard_normal((M, K)) * 2.0).astype(np.float32)
    g = _norm_weights(K, seed=K + 7)
    wq4 = synthetic.q4k_blocks(96, K, seed=K + 1)
    wq6 = synthetic.q6k_blocks(64, K, seed=K + 2)
    wgu = synthetic.q4k_blocks(1024, K, seed=K + 3)

    def run(with_xn):
        ho = torch.empty((M, K), dtype=torch.float32, device=DEV)
        xn = torch.empty((M, K), dtype=torch.float16, device=DEV) if with_xn else None
        y4 = torch.empty((M, 96), dtype=torch.float32, device=DEV)
        y6 = torch.empty((M, 64), dtype=torch.float32, device=DEV)
        hh = torch.empty((M, 512), dtype=torch.float16, device=DEV)
        projs = [("q4k", dev(wq4), y4, 96), ("q6k", dev(wq6), y6, 64), ("q4k", dev(wgu), hh, 1024, "swiglu")]
        dmq.dmq_residual_rmsnorm_gemm(dev(h), dev(ya), dev(g), 1e-5, ho, xn, projs, M, K)
        torch.cuda.synchronize()
        return ho.cpu().numpy(), (None if xn is None else xn.cpu().numpy()), y4.cpu().numpy(), \
            y6.cpu().numpy(), hh.cpu().numpy()

    ho, xnh, y4, y6, hh = run(True)
    assert np.array_equal(ho, h + ya), "h_out is not the fp32 sum"
    lo, hi = oracle.rmsnorm_f16_interval(attn.rmsnorm_f64(ho, g, 1e-5))
    xg = xnh.astype(np.float64)
    assert np.all((xg >= lo) & (xg <= hi)), "xn outside the RMSNorm interval"
    for fmt, wq, N, y in (("q4k", wq4, 96, y4), ("q6k", wq6, 64, y6)):
        ref, sc = oracle.gemm_quant(fmt, xnh, wq, N, K)
        err = np.abs(y.astype(np.float64) - ref)
        assert (err <= oracle.gemm_tolerance(sc)).all(), f"{fmt} projection out of bound"
    gu, sc = oracle.gemm_quant("q4k", xnh, wgu, 1024, K)
    eg = oracle.gemm_tolerance(sc)
    hlo, hhi = oracle.swiglu_interval(gu[:, :512], gu[:, 512:], eg[:, :512], eg[:, 512:])
    assert oracle.swiglu_accepts(hh.astype(np.float64), hlo, hhi).all(), "SwiGLU h outside the interval"
    if M == 1:
        # without xn the decode launch computes the same staged activations
        ho2, _, y42, y62, hh2 = run(False)
        assert np.array_equal(ho2, ho) and np.array_equal(y42, y4) and np.array_equal(y62, y6)
        assert np.array_equal(hh2, hh)


@pytest.mark.parametrize("M,pos0", [(1, 37), (16, 0), (5, 200)])
def test_decoder_layer_chain(dmq, M, pos0):
    """One decoder layer through the library on a small Llama-shaped layer
    (hidden 768 = 6 query heads x 128, 2 KV heads, FFN 1024): RMSNorm ->
    Q|K|V -> RoPE + cache -> attention -> O projection -> residual + RMSNorm
    -> SwiGLU FFN -> residual.  Each new stage is checked on its own GPU
    inputs, and the layer output against the fp64 oracle layer fed the same
    weights, inputs and cache (end to end, 1% of the output norm)."""
    Dm, hq, hkv, F = 768, 6, 2, 1024
    cache_len = pos0 + M + 3
    rng = np.random.default_rng(M * 7 + pos0)
    x = rng.standard_normal((M, Dm)).astype(np.float32)
    # small RMSNorm weights: the synthetic Q4_K/Q6_K weights are large (up to
    # ~20), so unit-scale inputs would give scores in the tens of thousands
    g1 = (0.02 * _norm_weights(Dm, 1)).astype(np.float32)
    # small FFN input weights: the synthetic Q4_K/Q6_K weights are large (up
    # to ~20), and the fp16 hidden values must stay finite for the
    # end-to-end comparison
    g2 = (0.05 * _norm_weights(Dm, 2)).astype(np.float32)
    wq_ = synthetic.q4k_blocks(hq * D_HEAD, Dm, seed=11)
    wk_ = synthetic.q4k_blocks(hkv * D_HEAD, Dm, seed=12)
    wv_ = synthetic.q6k_blocks(hkv * D_HEAD, Dm, seed=13)
    wo_ = synthetic.q4k_blocks(Dm, hq * D_HEAD, seed=14)
    wgu = synthetic.q4k_blocks(2 * F, Dm, seed=15)
    wd_ = synthetic.q6k_blocks(Dm, F, seed=16)
    # earlier positions of the cache: rotated keys and values of earlier tokens
    kc0 = np.zeros((hkv, cache_len, D_HEAD), np.float16)
    vc0 = np.zeros((hkv, cache_len, D_HEAD), np.float16)
    kc0[:, :pos0] = (rng.standard_normal((hkv, pos0, D_HEAD)) * 2).astype(np.float16)
    vc0[:, :pos0] = rng.standard_normal((hkv, pos0, D_HEAD)).astype(np.float16)

    t = lambda a: dev(a)  # noqa: E731
    xd = t(x)
    xn1 = torch.empty((M, Dm), dtype=torch.float16, device=DEV)
    dmq.dmq_residual_rmsnorm(xd, torch.zeros_like(xd), t(g1), 1e-5, torch.empty_like(xd), xn1, M, Dm)
    yq = torch.empty((M, hq * D_HEAD), dtype=torch.float32, device=DEV)
    yk = torch.empty((M, hkv * D_HEAD), dtype=torch.float32, device=DEV)
    yv = torch.empty((M, hkv * D_HEAD), dtype=torch.float32, device=DEV)
    dmq.dmq_gemm_group([("q4k", xn1, t(wq_.reshape(-1)), yq, M, hq * D_HEAD, Dm),
                        ("q4k", xn1, t(wk_.reshape(-1)), yk, M, hkv * D_HEAD, Dm),
                        ("q6k", xn1, t(wv_.reshape(-1)), yv, M, hkv * D_HEAD, Dm)])
    kc, vc = t(kc0), t(vc0)
    qr = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    dmq.dmq_rope_kv_cache(yq, yk, yv, M, pos0, hq, hkv, qr, kc, vc, cache_len)
    att = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    dmq.dmq_attention_gqa(qr, kc, vc, att, M, pos0, hq, hkv, cache_len)
    yo = torch.empty((M, Dm), dtype=torch.float32, device=DEV)
    dmq.dmq_gemm_q4k(att, t(wo_.reshape(-1)), yo, M, Dm, hq * D_HEAD)
    h1 = torch.empty((M, Dm), dtype=torch.float32, device=DEV)
    xn2 = torch.empty((M, Dm), dtype=torch.float16, device=DEV)
    dmq.dmq_residual_rmsnorm(xd, yo, t(g2), 1e-5, h1, xn2, M, Dm)
    hf = torch.empty((M, F), dtype=torch.float16, device=DEV)
    yd = torch.empty((M, Dm), dtype=torch.float32, device=DEV)
    dmq.dmq_ffn_swiglu_q4k(xn2, t(wgu.reshape(-1)), t(wd_.reshape(-1)), hf, yd, M, Dm, F)
    out = torch.empty((M, Dm), dtype=torch.float32, device=DEV)
    dmq.dmq_residual_rmsnorm(h1, yd, None, 0.0, out, None, M, Dm)
    torch.cuda.synchronize()
    cpu = lambda a: a.cpu().numpy()  # noqa: E731

    # stage checks on the GPU's own stage inputs
    q_, k_, v_ = cpu(yq), cpu(yk), cpu(yv)
    kc_, vc_ = cpu(kc), cpu(vc)
    pos = np.arange(pos0, pos0 + M)
    exact_q = attn.rope(q_.reshape(M, hq, D_HEAD), pos)
    lo, hi = oracle.f16_interval(exact_q, np.repeat(np.abs(q_.reshape(M, hq, D_HEAD)[..., 0::2])
                                                    + np.abs(q_.reshape(M, hq, D_HEAD)[..., 1::2]), 2, axis=-1) * 2.0 ** -21)
    qg = cpu(qr).reshape(M, hq, D_HEAD).astype(np.float64)
    assert np.all((qg >= lo) & (qg <= hi)), "layer: rotated queries outside the interval"
    assert np.array_equal(kc_[:, :pos0], kc0[:, :pos0]), "layer: earlier cache rows changed"
    _check_attention(cpu(qr), kc_, vc_, cpu(att), M, pos0, hq, "layer attention")
    ref_o, s_o = oracle.gemm_quant("q4k", cpu(att), wo_, Dm, hq * D_HEAD)
    assert_within(cpu(yo), ref_o, s_o, "layer O projection")
    assert np.array_equal(cpu(h1), x + cpu(yo)), "layer: first residual is not the fp32 sum"
    assert np.isfinite(cpu(hf).astype(np.float32)).all(), "layer: fp16 FFN hidden values overflowed"
    assert np.array_equal(cpu(out), cpu(h1) + cpu(yd)), "layer: second residual is not the fp32 sum"

    # end to end: the fp64 oracle layer on the same weights, input and cache
    xh1 = attn.rmsnorm_f64(x, g1, 1e-5)
    W = lambda fmt, wq, n, k: oracle.f16_bits_to_f64(oracle.dequant(fmt, wq, n, k))  # noqa: E731
    Wq = W("q4k", wq_, hq * D_HEAD, Dm); Wk = W("q4k", wk_, hkv * D_HEAD, Dm); Wv = W("q6k", wv_, hkv * D_HEAD, Dm)  # noqa: E702
    Wo = W("q4k", wo_, Dm, hq * D_HEAD); Wgu = W("q4k", wgu, 2 * F, Dm); Wd = W("q6k", wd_, Dm, F)  # noqa: E702
    Q = attn.rope((xh1 @ Wq.T).reshape(M, hq, D_HEAD), pos)
    Kn = attn.rope((xh1 @ Wk.T).reshape(M, hkv, D_HEAD), pos)
    Vn = (xh1 @ Wv.T).reshape(M, hkv, D_HEAD)
    Kc = kc0.astype(np.float64); Vc = vc0.astype(np.float64)  # noqa: E702
    Kc[:, pos0:pos0 + M] = Kn.transpose(1, 0, 2); Vc[:, pos0:pos0 + M] = Vn.transpose(1, 0, 2)  # noqa: E702
    A, _ = attn.attention_gqa(Q, Kc, Vc, pos0)
    H1 = attn.residual_add(x, A.reshape(M, -1) @ Wo.T)
    xh2 = attn.rmsnorm_f64(H1, g2, 1e-5)
    G = xh2 @ Wgu[:F].T
    U = xh2 @ Wgu[F:].T
    OUT = attn.residual_add(H1, (oracle.silu(G) * U) @ Wd.T)
    rel = np.linalg.norm(cpu(out) - OUT) / np.linalg.norm(OUT)
    print(f"layer M={M} pos0={pos0}: end-to-end relative error {rel:.3g}")
    assert rel < 1e-2, f"layer output differs from the fp64 oracle layer by {rel:.3g} of its norm"


# ------------------------------------------------------------ workspaces ---
# The split-K partial sums and the decode attention's partial states live in
# per-(device, stream) workspaces that grow with stream-ordered allocations:
# a growing call must neither wait for work queued before it nor free a
# buffer that work queued earlier (or a graph captured earlier) still uses.

def _sleeping(stream, cycles=200_000_000):
    """Queue a bounded spin kernel on `stream` and an event after it."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(cycles)
        done = torch.cuda.Event()
        done.record()
    return done


def test_workspace_growth_does_not_block(dmq):
    """On a fresh stream, behind a long spin kernel: a split-K GEMM (new
    workspace), a larger split-K GEMM (grown workspace) and two decode
    attention calls (new, then larger) each return while the spin kernel is
    still running, and give the bits of the same calls on the current
    stream."""
    import time
    gemms = []
    for fmt, M, N, K in (("q6k", 40, 37, 8192), ("q6k", 1024, 3072, 8192)):
        x = synthetic.activations(M, K, seed=M + K)
        wq = synthetic.weight_blocks(fmt, N, K, seed=N + K)
        gemms.append((fmt, M, N, K, dev(x), dev(wq.reshape(-1))))
    hq, hkv, L = 24, 8, 1024
    rng = np.random.default_rng(9)
    kc = dev(rng.standard_normal((hkv, L, D_HEAD)).astype(np.float16))
    vc = dev(rng.standard_normal((hkv, L, D_HEAD)).astype(np.float16))
    atts = [(M, L - M, dev(rng.standard_normal((M, hq * D_HEAD)).astype(np.float16))) for M in (1, 16)]

    def gemm(i, stream=None):
        fmt, M, N, K, xd, wd = gemms[i]
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        (dmq.dmq_gemm_q4k if fmt == "q4k" else dmq.dmq_gemm_q6k)(xd, wd, y, M, N, K, stream=stream)
        return y

    def att(i, stream=None):
        M, pos0, q = atts[i]
        out = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
        dmq.dmq_attention_gqa(q, kc, vc, out, M, pos0, hq, hkv, L, stream=stream)
        return out

    ref = [gemm(0), gemm(1), att(0), att(1)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    got, waits = [], []
    for call in (lambda s: gemm(0, s), lambda s: gemm(1, s), lambda s: att(0, s), lambda s: att(1, s)):
        done = _sleeping(side)
        t0 = time.perf_counter()
        with torch.cuda.stream(side):
            got.append(call(side))
        waits.append((time.perf_counter() - t0, done.query()))
        side.synchronize()
    for i, (dt, finished) in enumerate(waits):
        assert not finished, f"call {i} returned only after the work queued before it ({dt * 1e3:.1f} ms)"
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a, b), f"call {i}: bits differ from the same call on another stream"
    print("host time of the growing calls (ms):", [round(dt * 1e3, 2) for dt, _ in waits])


def test_graph_captured_before_growth_still_replays(dmq):
    """A graph captured with the stream's workspace at one size keeps
    working after a later call on that stream grew (replaced) it: replays,
    with eager work and synchronisations between them, give the eager
    result every time."""
    hq, hkv, L = 24, 8, 2048
    rng = np.random.default_rng(10)
    kc = dev(rng.standard_normal((hkv, L, D_HEAD)).astype(np.float16))
    vc = dev(rng.standard_normal((hkv, L, D_HEAD)).astype(np.float16))
    q1 = dev(rng.standard_normal((1, hq * D_HEAD)).astype(np.float16))
    q16 = dev(rng.standard_normal((16, hq * D_HEAD)).astype(np.float16))
    fmt, M, N, K = "q6k", 40, 37, 8192
    x = dev(synthetic.activations(M, K, seed=5))
    wq = dev(synthetic.weight_blocks(fmt, N, K, seed=6).reshape(-1))
    side = torch.cuda.Stream()
    o1 = torch.empty((1, hq * D_HEAD), dtype=torch.float16, device=DEV)
    o16 = torch.empty((16, hq * D_HEAD), dtype=torch.float16, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(side):
        dmq.dmq_attention_gqa(q1, kc, vc, o1, 1, 1000, hq, hkv, L, stream=side)
        dmq.dmq_gemm_q6k(x, wq, y, M, N, K, stream=side)
    side.synchronize()
    want1, wanty = o1.clone(), y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        dmq.dmq_attention_gqa(q1, kc, vc, o1, 1, 1000, hq, hkv, L, stream=side)
        dmq.dmq_gemm_q6k(x, wq, y, M, N, K, stream=side)
    # grow both workspaces of the stream: 16 queries, and a larger split-K GEMM
    Mb, Nb = 1024, 3072
    xb = dev(synthetic.activations(Mb, K, seed=7))
    wb = dev(synthetic.weight_blocks(fmt, Nb, K, seed=8).reshape(-1))
    yb = torch.empty((Mb, Nb), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(side):
        dmq.dmq_attention_gqa(q16, kc, vc, o16, 16, L - 16, hq, hkv, L, stream=side)
        dmq.dmq_gemm_q6k(xb, wb, yb, Mb, Nb, K, stream=side)
    side.synchronize()
    want16 = o16.clone()
    for r in range(4):
        o1.zero_()
        y.zero_()
        with torch.cuda.stream(side):
            graph.replay()
        side.synchronize()
        assert torch.equal(o1, want1) and torch.equal(y, wanty), f"replay {r} differs from the eager result"
        with torch.cuda.stream(side):   # eager work between replays
            dmq.dmq_attention_gqa(q16, kc, vc, o16, 16, L - 16, hq, hkv, L, stream=side)
        side.synchronize()
        assert torch.equal(o16, want16)


# ------------------------------------------- attention || FFN (layer) ---

def _layer_setup(M, pos0, cache_len, seed=5):
    """A small Llama-shaped layer (hidden 768 = 6 query heads x 128, 2 KV
    heads, FFN 1024) with its inputs, as in the decoder-layer chain test."""
    Dm, hq, hkv, F = 768, 6, 2, 1024
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, Dm)).astype(np.float32)
    g1 = (0.02 * _norm_weights(Dm, 1)).astype(np.float32)
    g2 = (0.05 * _norm_weights(Dm, 2)).astype(np.float32)
    g3 = (0.03 * _norm_weights(Dm, 3)).astype(np.float32)
    host = {"q": synthetic.q4k_blocks(hq * D_HEAD, Dm, seed=11), "k": synthetic.q4k_blocks(hkv * D_HEAD, Dm, seed=12),
            "v": synthetic.q6k_blocks(hkv * D_HEAD, Dm, seed=13), "o": synthetic.q4k_blocks(Dm, hq * D_HEAD, seed=14),
            "gate_up": synthetic.q4k_blocks(2 * F, Dm, seed=15), "down": synthetic.q6k_blocks(Dm, F, seed=16)}
    kc0 = np.zeros((hkv, cache_len, D_HEAD), np.float16)
    vc0 = np.zeros((hkv, cache_len, D_HEAD), np.float16)
    kc0[:, :pos0] = (rng.standard_normal((hkv, pos0, D_HEAD)) * 2).astype(np.float16)
    vc0[:, :pos0] = rng.standard_normal((hkv, pos0, D_HEAD)).astype(np.float16)
    return dict(Dm=Dm, hq=hq, hkv=hkv, F=F, x=x, g1=g1, g2=g2, g3=g3, host=host, kc0=kc0, vc0=vc0)


def _layer_run(dmq, S, M, pos0, cache_len, chunk, two_streams):
    Dm, hq, hkv, F = S["Dm"], S["hq"], S["hkv"], S["F"]
    e = lambda *shape, dt=torch.float32: torch.empty(shape, dtype=dt, device=DEV)  # noqa: E731
    xd = dev(S["x"])
    xn = e(M, Dm, dt=torch.float16)
    dmq.dmq_residual_rmsnorm(xd, torch.zeros_like(xd), dev(S["g1"]), 1e-5, e(M, Dm), xn, M, Dm)
    W = {k: dev(v.reshape(-1)) for k, v in S["host"].items()}
    W.update(fmt_v="q6k", g_ffn=dev(S["g2"]), g_next=dev(S["g3"]), k_cache=dev(S["kc0"]), v_cache=dev(S["vc0"]))
    B = {"h_in": xd, "xn_in": xn, "yq": e(M, hq * D_HEAD), "yk": e(M, hkv * D_HEAD), "yv": e(M, hkv * D_HEAD),
         "q_rot": e(M, hq * D_HEAD, dt=torch.float16), "attn": e(M, hq * D_HEAD, dt=torch.float16),
         "yo": e(M, Dm), "h_mid": e(M, Dm), "xn_ffn": e(M, Dm, dt=torch.float16), "h_ffn": e(M, F, dt=torch.float16),
         "y_down": e(M, Dm), "h_out": e(M, Dm), "xn_out": e(M, Dm, dt=torch.float16)}
    layer = dmq.make_layer(W, B, M, Dm, F, hq, hkv, cache_len)
    torch.cuda.synchronize()
    sa = torch.cuda.current_stream()
    sf = torch.cuda.Stream() if two_streams else sa
    dmq.dmq_layer_prefill(layer, M, pos0, Dm, F, hq, hkv, cache_len, 1e-5, chunk, stream_attn=sa, stream_ffn=sf)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in B.items()}
    out["k_cache"], out["v_cache"] = W["k_cache"].cpu().numpy(), W["v_cache"].cpu().numpy()
    return out, W, B


@pytest.mark.parametrize("M,pos0,chunk", [(300, 50, 64), (256, 0, 128), (40, 7, 16)])
def test_layer_prefill_two_streams_same_bits(dmq, M, pos0, chunk):
    """The attention side of chunk c+1 and the FFN of chunk c on two streams
    give exactly the bits of the same chunked schedule on one stream, in every
    output, scratch and cache buffer, and on a repeat."""
    cache_len = pos0 + M + 5
    S = _layer_setup(M, pos0, cache_len)
    serial, _, _ = _layer_run(dmq, S, M, pos0, cache_len, chunk, two_streams=False)
    for rep in range(2):
        conc, _, _ = _layer_run(dmq, S, M, pos0, cache_len, chunk, two_streams=True)
        for k in serial:
            assert np.array_equal(serial[k].view(np.uint8), conc[k].view(np.uint8)), f"{k} differs (repeat {rep})"
    assert np.isfinite(serial["h_ffn"].astype(np.float32)).all()


def test_layer_prefill_matches_single_calls_and_oracle(dmq):
    """One pass (chunk >= M) equals the layer composed of the single calls
    bit for bit; the two-stream chunked layer matches the fp64 oracle layer
    end to end (1% of the output norm, as the decoder-layer chain test)."""
    M, pos0 = 96, 30
    cache_len = pos0 + M + 2
    S = _layer_setup(M, pos0, cache_len, seed=6)
    Dm, hq, hkv, F = S["Dm"], S["hq"], S["hkv"], S["F"]
    one, W, B = _layer_run(dmq, S, M, pos0, cache_len, M, two_streams=False)
    # the same layer from the single calls
    e = lambda *shape, dt=torch.float32: torch.empty(shape, dtype=dt, device=DEV)  # noqa: E731
    kc, vc = dev(S["kc0"]), dev(S["vc0"])
    yq, yk, yv = e(M, hq * D_HEAD), e(M, hkv * D_HEAD), e(M, hkv * D_HEAD)
    dmq.dmq_gemm_group([("q4k", B["xn_in"], W["q"], yq, M, hq * D_HEAD, Dm), ("q4k", B["xn_in"], W["k"], yk, M, hkv * D_HEAD, Dm),
                        ("q6k", B["xn_in"], W["v"], yv, M, hkv * D_HEAD, Dm)])
    qr, att = e(M, hq * D_HEAD, dt=torch.float16), e(M, hq * D_HEAD, dt=torch.float16)
    dmq.dmq_rope_kv_cache(yq, yk, yv, M, pos0, hq, hkv, qr, kc, vc, cache_len)
    dmq.dmq_attention_gqa(qr, kc, vc, att, M, pos0, hq, hkv, cache_len)
    yo = e(M, Dm)
    dmq.dmq_gemm_group([("q4k", att, W["o"], yo, M, Dm, hq * D_HEAD)])
    h1, xn2 = e(M, Dm), e(M, Dm, dt=torch.float16)
    dmq.dmq_residual_rmsnorm(B["h_in"], yo, W["g_ffn"], 1e-5, h1, xn2, M, Dm)
    hf, yd = e(M, F, dt=torch.float16), e(M, Dm)
    dmq.dmq_ffn_swiglu_q4k(xn2, W["gate_up"], W["down"], hf, yd, M, Dm, F)
    ho, xo = e(M, Dm), e(M, Dm, dt=torch.float16)
    dmq.dmq_residual_rmsnorm(h1, yd, W["g_next"], 1e-5, ho, xo, M, Dm)
    torch.cuda.synchronize()
    for name, t in (("h_mid", h1), ("h_out", ho), ("xn_out", xo), ("h_ffn", hf), ("attn", att)):
        assert np.array_equal(one[name].view(np.uint8), t.cpu().numpy().view(np.uint8)), f"{name} differs from the single calls"
    assert np.array_equal(one["k_cache"].view(np.uint16), kc.cpu().numpy().view(np.uint16))
    # end to end against the fp64 oracle layer, for the two-stream chunked run
    conc, _, _ = _layer_run(dmq, S, M, pos0, cache_len, 32, two_streams=True)
    x = S["x"]
    pos = np.arange(pos0, pos0 + M)
    Wd = lambda fmt, wq, n, k: oracle.f16_bits_to_f64(oracle.dequant(fmt, wq, n, k))  # noqa: E731
    H = S["host"]
    xh1 = attn.rmsnorm_f64(x, S["g1"], 1e-5)
    Q = attn.rope((xh1 @ Wd("q4k", H["q"], hq * D_HEAD, Dm).T).reshape(M, hq, D_HEAD), pos)
    Kn = attn.rope((xh1 @ Wd("q4k", H["k"], hkv * D_HEAD, Dm).T).reshape(M, hkv, D_HEAD), pos)
    Vn = (xh1 @ Wd("q6k", H["v"], hkv * D_HEAD, Dm).T).reshape(M, hkv, D_HEAD)
    Kc = S["kc0"].astype(np.float64); Vc = S["vc0"].astype(np.float64)  # noqa: E702
    Kc[:, pos0:pos0 + M] = Kn.transpose(1, 0, 2); Vc[:, pos0:pos0 + M] = Vn.transpose(1, 0, 2)  # noqa: E702
    A, _ = attn.attention_gqa(Q, Kc, Vc, pos0)
    H1 = attn.residual_add(x, A.reshape(M, -1) @ Wd("q4k", H["o"], Dm, hq * D_HEAD).T)
    xh2 = attn.rmsnorm_f64(H1, S["g2"], 1e-5)
    Wgu = Wd("q4k", H["gate_up"], 2 * F, Dm)
    OUT = attn.residual_add(H1, (oracle.silu(xh2 @ Wgu[:F].T) * (xh2 @ Wgu[F:].T)) @ Wd("q6k", H["down"], Dm, F).T)
    rel = np.linalg.norm(conc["h_out"] - OUT) / np.linalg.norm(OUT)
    print(f"layer prefill (two streams, chunk 32): end-to-end relative error {rel:.3g}")
    assert rel < 1e-2
