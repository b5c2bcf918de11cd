"""dmq_attention_gqa_noalloc against dmq_attention_gqa, through the C ABI.

The no-allocation variant keeps the decode path's partial softmax states in a
fixed per-GPU scratch array instead of the stream's workspace; it runs the
same kernels, so its outputs must be the same bits.  Two calls in a row, the
second smaller than the first (the scratch keeps the first call's contents),
then a prefill call (no scratch) and a decode call on a second stream.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D_HEAD = 128
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dmq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_q4_amd
    return dequant_gemm_q4_amd


def _case(M, pos0, hq, hkv, L, seed):
    rng = np.random.default_rng(seed)
    n = pos0 + M
    kc = np.zeros((hkv, L, D_HEAD), np.float16)
    vc = np.zeros((hkv, L, D_HEAD), np.float16)
    kc[:, :n] = rng.standard_normal((hkv, n, D_HEAD)).astype(np.float16)
    vc[:, :n] = rng.standard_normal((hkv, n, D_HEAD)).astype(np.float16)
    q = rng.standard_normal((M, hq * D_HEAD)).astype(np.float16)
    t = lambda a: torch.from_numpy(a).to(DEV)   # noqa: E731
    return t(q), t(kc), t(vc)


def _both(dmq, M, pos0, hq, hkv, L, seed, stream=None):
    q, kc, vc = _case(M, pos0, hq, hkv, L, seed)
    a = torch.empty((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    b = torch.full((M, hq * D_HEAD), float("nan"), dtype=torch.float16, device=DEV)
    dmq.dmq_attention_gqa(q, kc, vc, a, M, pos0, hq, hkv, L, stream=stream)
    dmq.dmq_attention_gqa_noalloc(q, kc, vc, b, M, pos0, hq, hkv, L, stream=stream)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_attention_matches_allocating_call(dmq):
    print(f"noalloc: M=16 pos0=3000 then M=1 pos0=500, then prefill M=40, then a second stream", flush=True)
    cases = [(16, 3000, 24, 8, 4096, 1), (1, 500, 24, 8, 1024, 2), (40, 7, 24, 8, 64, 3), (3, 70, 6, 2, 80, 4)]
    for M, pos0, hq, hkv, L, seed in cases:
        a, b = _both(dmq, M, pos0, hq, hkv, L, seed)
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a, b), f"M={M} pos0={pos0}: the no-allocation call's bits differ"
    side = torch.cuda.Stream()
    a, b = _both(dmq, 2, 900, 24, 8, 1024, 5, stream=side)
    assert torch.equal(a, b), "second stream: bits differ"


def test_noalloc_attention_rejects_oversize(dmq):
    hq, M = 24, 16
    pieces = dmq.DMQ_NOALLOC_SCRATCH_BYTES // (M * hq * (D_HEAD + 2) * 4) + 1
    L = 64 * pieces
    q = torch.zeros((M, hq * D_HEAD), dtype=torch.float16, device=DEV)
    kc = torch.zeros((8, L, D_HEAD), dtype=torch.float16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(dmq.DmqError) as e:
        dmq.dmq_attention_gqa_noalloc(q, kc, kc, out, M, L - M, hq, 8, L)
    assert e.value.status == dmq.DMQ_ERR_SCRATCH
