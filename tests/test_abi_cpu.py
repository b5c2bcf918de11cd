"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/dmq.h, and rejects bad arguments on the host before
any HIP call (so nothing here touches a device, with or without a GPU)."""
import ctypes
import os
import re

import pytest

import dequant_gemm_q4_amd as dmq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmq.h")

A16 = 0x10000          # a 16-byte aligned address that is never dereferenced
MIS = 0x10008          # 8 mod 16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dmq_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 16, names
    assert set(names) == set(dmq.EXPORTS)
    raw = ctypes.CDLL(dmq.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_noalloc_attention_validation():
    """The no-allocation attention call checks like dmq_attention_gqa, and a
    decode call whose partial states exceed the fixed scratch is rejected
    with DMQ_ERR_SCRATCH before anything touches a device."""
    f = L.dmq_attention_gqa_noalloc
    Q, KC, VC, O = (A16 + 0x10000000 * i for i in range(4))   # 256 MiB apart: no overlaps
    assert f(None, KC, VC, O, 1, 0, 24, 8, 16, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(Q, KC, VC, Q, 1, 0, 24, 8, 16, None) == dmq.DMQ_ERR_INVALID_ARG          # out is q
    assert f(Q, KC, VC, O, 1, 16, 24, 8, 16, None) == dmq.DMQ_ERR_INVALID_ARG         # past the cache
    assert f(Q, KC, VC, O, 1, 0, 24, 7, 16, None) == dmq.DMQ_ERR_INVALID_ARG          # heads not grouped
    assert f(Q + 8, KC, VC, O, 1, 0, 24, 8, 16, None) == dmq.DMQ_ERR_ALIGNMENT
    rec = 520                                                   # bytes per (query, head, piece)
    cap_pieces = dmq.DMQ_NOALLOC_SCRATCH_BYTES // (16 * 24 * rec)
    L_big = 64 * (cap_pieces + 1)
    assert f(Q, KC, VC, O, 16, L_big - 16, 24, 8, L_big, None) == dmq.DMQ_ERR_SCRATCH
    assert "scratch" in dmq.status_string(dmq.DMQ_ERR_SCRATCH)


def test_layer_prefill_validation():
    """dmq_layer_prefill checks its sizes, formats and pointers on the host
    before it records an event or enqueues a kernel."""
    f = L.dmq_layer_prefill
    w = dmq.LayerWeights()
    for i, n in enumerate(("wq", "wk", "wv", "wo", "w_gate_up", "w_down", "g_ffn", "k_cache", "v_cache")):
        setattr(w, n, A16 + 0x100000 * (i + 1))
    b = dmq.LayerBuffers()
    for i, n in enumerate(("h_in", "xn_in", "yq", "yk", "yv", "q_rot", "attn", "yo", "h_mid", "xn_ffn", "h_ffn",
                           "y_down", "h_out", "xn_out")):
        setattr(b, n, A16 + 0x1000000 * (i + 1))
    args = lambda **k: dict(dict(M=8, pos0=0, D=768, F=1024, hq=6, hkv=2, L=64, chunk=4), **k)  # noqa: E731

    def call(wp, bp, a, theta=500000.0):
        return f(wp, bp, a["M"], a["pos0"], a["D"], a["F"], a["hq"], a["hkv"], a["L"], theta, 1e-5, a["chunk"],
                 None, None)
    assert call(None, ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    assert call(ctypes.byref(w), None, args()) == dmq.DMQ_ERR_INVALID_ARG
    assert call(ctypes.byref(w), ctypes.byref(b), args(D=700)) == dmq.DMQ_ERR_INVALID_ARG     # D % 256
    assert call(ctypes.byref(w), ctypes.byref(b), args(F=0)) == dmq.DMQ_ERR_INVALID_ARG
    assert call(ctypes.byref(w), ctypes.byref(b), args(hq=3)) == dmq.DMQ_ERR_INVALID_ARG      # 3*128 % 256
    assert call(ctypes.byref(w), ctypes.byref(b), args(chunk=0)) == dmq.DMQ_ERR_INVALID_ARG
    assert call(ctypes.byref(w), ctypes.byref(b), args(M=0)) == dmq.DMQ_ERR_INVALID_ARG
    w.fmt_v = 7
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    w.fmt_v = 0
    b.h_mid = A16 + 8
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_ALIGNMENT
    b.h_mid = None
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    b.h_mid = A16 + 0x20000000
    w.g_next = A16 + 0x30000000
    b.xn_out = None                                          # g_next without xn_out
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    b.xn_out = A16 + 0x40000000
    # the single calls' requirements, checked before anything is enqueued
    assert call(ctypes.byref(w), ctypes.byref(b), args(hkv=4)) == dmq.DMQ_ERR_INVALID_ARG   # 6 % 4 heads
    assert call(ctypes.byref(w), ctypes.byref(b), args(pos0=60)) == dmq.DMQ_ERR_INVALID_ARG  # past the cache
    assert call(ctypes.byref(w), ctypes.byref(b), args(), theta=1.0) == dmq.DMQ_ERR_INVALID_ARG
    w.k_cache = A16 + 0x800008
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_ALIGNMENT
    w.k_cache = A16 + 0x800000
    # written buffers overlapping each other, a cache or a weight array
    yk = b.yk
    b.yk = b.yq
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    b.yk = yk
    yo = b.yo
    b.yo = w.wq
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    b.yo = w.v_cache
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    b.yo = yo
    h_out = b.h_out
    b.h_out = b.h_in
    assert call(ctypes.byref(w), ctypes.byref(b), args()) == dmq.DMQ_ERR_INVALID_ARG
    b.h_out = h_out


def test_version_and_status_strings():
    assert dmq.dmq_version() == 1
    for st in (0, -1, -2, -3, -4):
        assert dmq.status_string(st) and "unknown" not in dmq.status_string(st)
    assert "unknown" in dmq.status_string(42)


L = dmq.lib


def _no_gpu():
    """True when no HIP device is visible (counting devices does not
    initialise one).  Only then may a test make a call whose arguments pass
    the host checks: with a device it would launch on these fake pointers."""
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.parametrize("fn", ["dmq_gemm_q4k", "dmq_gemm_q6k"])
def test_gemm_validation(fn):
    f = getattr(L, fn)
    assert f(None, A16, A16, 4, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, None, A16, 4, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, None, 4, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, A16, 0, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, A16, 4, 0, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, A16, 4, 4, 0, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, A16, 4, 4, 300, None) == dmq.DMQ_ERR_INVALID_ARG      # K % 256
    assert f(A16, A16, A16, -1, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, A16, 1 << 31, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(MIS, A16, A16, 4, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT         # x
    assert f(A16, A16, MIS, 4, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT         # y
    assert f(A16, A16 + 1, A16, 4, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT     # odd weights


def test_weight_alignment_rules():
    # Q4_K blocks need 16-byte alignment, Q6_K only 2
    assert L.dmq_gemm_q4k(A16, A16 + 2, A16, 4, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT
    assert L.dmq_dequant_q4k(A16 + 8, A16, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT
    assert L.dmq_dequant_q6k(A16 + 1, A16, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT


@pytest.mark.parametrize("fn", ["dmq_dequant_q4k", "dmq_dequant_q6k"])
def test_dequant_validation(fn):
    f = getattr(L, fn)
    assert f(None, A16, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, None, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, 0, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, A16, 4, 128, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(A16, MIS, 4, 256, None) == dmq.DMQ_ERR_ALIGNMENT


def test_ffn_validation():
    f = L.dmq_ffn_swiglu_q4k
    assert f(A16, A16, A16, None, A16, 4, 256, 256, None) == dmq.DMQ_ERR_INVALID_ARG   # h
    assert f(A16, A16, A16, A16, None, 4, 256, 256, None) == dmq.DMQ_ERR_INVALID_ARG   # y
    assert f(A16, A16, A16, A16, A16, 4, 300, 256, None) == dmq.DMQ_ERR_INVALID_ARG    # D % 256
    assert f(A16, A16, A16, A16, A16, 4, 256, 100, None) == dmq.DMQ_ERR_INVALID_ARG    # F % 256
    assert f(A16, A16, A16, MIS, A16, 4, 256, 256, None) == dmq.DMQ_ERR_ALIGNMENT      # h
    assert f(A16, A16, A16 + 1, A16, A16, 4, 256, 256, None) == dmq.DMQ_ERR_ALIGNMENT  # down


def _desc(fmt=0, M=4, N=4, K=256, x=A16, wq=A16, y=A16, reserved=0):
    d = dmq.GemmDesc()
    d.format, d.reserved, d.x_f16, d.wq, d.y, d.M, d.N, d.K = fmt, reserved, x, wq, y, M, N, K
    return d


def test_group_validation():
    g = L.dmq_gemm_group
    arr = (dmq.GemmDesc * 2)(_desc(), _desc())
    assert g(arr, 0, None) == dmq.DMQ_ERR_INVALID_ARG
    assert g(arr, 65, None) == dmq.DMQ_ERR_INVALID_ARG
    assert g(None, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.GemmDesc * 1)(_desc(reserved=1))
    assert g(bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.GemmDesc * 1)(_desc(fmt=7))
    assert g(bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.GemmDesc * 2)(_desc(), _desc(K=100))
    assert g(bad, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.GemmDesc * 2)(_desc(), _desc(y=MIS))
    assert g(bad, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    # decode (M = 1) and prefill problems cannot share one call
    mixed = (dmq.GemmDesc * 2)(_desc(M=1), _desc(M=8))
    assert g(mixed, 2, None) == dmq.DMQ_ERR_INVALID_ARG


def test_binding_rejects_host_tensors_and_bad_sizes():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 256, dtype=torch.float16)
    w = torch.zeros(4 * 144, dtype=torch.uint8)
    y = torch.zeros(4, 4, dtype=torch.float32)
    with pytest.raises(ValueError):
        dmq.dmq_gemm_q4k(x, w, y, 4, 4, 256)          # CPU tensors are refused
    with pytest.raises(ValueError):
        dmq.make_group([("q4k", x, w, y, 4, 4, 512)])  # K mismatch is caught first


def test_gemm_k_limit():
    # the GEMM kernels take K up to 2^20
    assert L.dmq_gemm_q4k(A16, A16, A16, 4, 4, (1 << 20) + 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert L.dmq_gemm_q6k(A16, A16, A16, 1, 4, (1 << 20) + 256, None) == dmq.DMQ_ERR_INVALID_ARG


def _proj(fmt=0, N=4, wq=A16, y=A16, flags=0):
    d = dmq.ProjDesc()
    d.format, d.flags, d.wq, d.y, d.N = fmt, flags, wq, y, N
    return d


def test_rmsnorm_gemm_validation():
    f = L.dmq_rmsnorm_gemm
    p = (dmq.ProjDesc * 2)(_proj(), _proj(fmt=1))
    X, G, XN = A16, A16 + 0x1000, A16 + 0x2000
    assert f(X, G, 1e-5, XN, 4, 256, p, 0, None) == dmq.DMQ_ERR_INVALID_ARG      # count
    assert f(X, G, 1e-5, XN, 4, 256, p, 65, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(X, G, 1e-5, XN, 4, 256, None, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(None, G, 1e-5, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG    # x
    assert f(X, None, 1e-5, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG    # g
    assert f(X, G, -1.0, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG       # eps < 0
    assert f(X, G, float("nan"), XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(X, G, float("inf"), XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(X, G, 1e-5, XN, 4, 300, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG       # K % 256
    assert f(X, G, 1e-5, XN, 0, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG       # M
    assert f(X, G, 1e-5, None, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG     # xn needed for M > 1
    assert f(X, G, 1e-5, X, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG        # xn == x
    assert f(MIS, G, 1e-5, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    assert f(X, G + 8, 1e-5, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    assert f(X, G, 1e-5, XN + 8, 4, 256, p, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    bad = (dmq.ProjDesc * 1)(_proj(flags=2))                   # unknown flag
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.ProjDesc * 1)(_proj(flags=1))                   # SwiGLU pair: N/2 not a multiple of 256
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.ProjDesc * 1)(_proj(fmt=1, N=512, flags=1))     # SwiGLU pair in Q6_K
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.ProjDesc * 1)(_proj(fmt=5))
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.ProjDesc * 1)(_proj(N=0))
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.ProjDesc * 1)(_proj(y=MIS))
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_ALIGNMENT
    bad = (dmq.ProjDesc * 1)(_proj(wq=A16 + 2))                # Q4_K weights need 16 bytes
    assert f(X, G, 1e-5, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_ALIGNMENT


def test_residual_rmsnorm_gemm_validation():
    f = L.dmq_residual_rmsnorm_gemm
    p = (dmq.ProjDesc * 2)(_proj(), _proj(fmt=1))
    H, Y, G, HO, XN = (A16 + 0x1000 * i for i in range(5))
    # M = 4, K = 256: 4 KiB of fp32 per residual buffer, 2 KiB of xn
    assert f(H, Y, G, 1e-5, HO, XN, 4, 256, p, 0, None) == dmq.DMQ_ERR_INVALID_ARG      # count
    assert f(H, Y, G, 1e-5, HO, XN, 4, 256, None, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(None, Y, G, 1e-5, HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, None, G, 1e-5, HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, None, 1e-5, HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, 1e-5, None, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, float("nan"), HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, 1e-5, HO, XN, 4, 300, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG       # K % 256
    assert f(H, Y, G, 1e-5, HO, None, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG     # xn needed for M > 1
    assert f(H, Y, G, 1e-5, H, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG        # h_out is h_in
    assert f(H, Y, G, 1e-5, H + 0x800, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG  # overlaps h_in
    assert f(H, Y, G, 1e-5, Y, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG        # h_out is y_add
    assert f(H, Y, G, 1e-5, HO, HO + 0x400, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG  # xn inside h_out
    assert f(H, Y, HO + 0x200, 1e-5, HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG  # g inside h_out
    assert f(H, Y, XN + 0x100, 1e-5, HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_INVALID_ARG  # g inside xn
    assert f(MIS, Y, G, 1e-5, HO, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    assert f(H, Y, G, 1e-5, HO + 8, XN, 4, 256, p, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    assert f(H, Y, G, 1e-5, HO, XN + 8, 4, 256, p, 2, None) == dmq.DMQ_ERR_ALIGNMENT
    bad = (dmq.ProjDesc * 1)(_proj(flags=1))                   # SwiGLU pair: N/2 not a multiple of 256
    assert f(H, Y, G, 1e-5, HO, XN, 4, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG
    bad = (dmq.ProjDesc * 1)(_proj(N=0))
    assert f(H, Y, G, 1e-5, HO, None, 1, 256, bad, 1, None) == dmq.DMQ_ERR_INVALID_ARG  # decode path too


def test_projection_outputs_must_not_overlap_inputs_or_each_other():
    """In one launch some workgroups write a projection's output while others
    still read the activations, the norm weights and the residual buffers
    (and write the other outputs): every such overlap is rejected.  Each
    case below is valid except for the one overlap it names (M = 4, K = 256:
    2 KiB of fp16 x / xn, 4 KiB of fp32 residual rows, 1 KiB of g; a plain
    projection with N = 4 writes 64 bytes, a SwiGLU pair with N = 512
    writes 4 * 256 fp16 = 2 KiB)."""
    X, G, XN = A16, A16 + 0x1000, A16 + 0x2000
    Y0, Y1 = A16 + 0x8000, A16 + 0x9000

    def rms(*projs):
        arr = (dmq.ProjDesc * len(projs))(*projs)
        return L.dmq_rmsnorm_gemm(X, G, 1e-5, XN, 4, 256, arr, len(projs), None)
    for y in (X + 0x7c0, G + 0x20, XN, XN + 0x7f0):
        assert rms(_proj(y=y)) == dmq.DMQ_ERR_INVALID_ARG, hex(y)
    assert rms(_proj(y=Y0), _proj(y=Y0 + 0x30)) == dmq.DMQ_ERR_INVALID_ARG           # outputs overlap
    assert rms(_proj(y=Y0), _proj(N=512, flags=1, y=Y0 - 0x7f0)) == dmq.DMQ_ERR_INVALID_ARG  # into h's 2 KiB
    if _no_gpu():   # disjoint: passes the host checks (and then finds no device)
        assert rms(_proj(y=Y0), _proj(y=Y1)) == dmq.DMQ_ERR_UNSUPPORTED

    H, Yad, HO = A16 + 0x3000, A16 + 0x4000, A16 + 0x5000

    def res(*projs, xn=XN, M=4):
        arr = (dmq.ProjDesc * len(projs))(*projs)
        return L.dmq_residual_rmsnorm_gemm(H, Yad, G, 1e-5, HO, xn, M, 256, arr, len(projs), None)
    for y in (H + 0xff0, Yad, HO + 0x800, G, XN + 0x10):
        assert res(_proj(y=y)) == dmq.DMQ_ERR_INVALID_ARG, hex(y)
    assert res(_proj(y=Yad + 0x10), xn=None, M=1) == dmq.DMQ_ERR_INVALID_ARG          # the decode path too
    assert res(_proj(y=Y0), _proj(y=Y0)) == dmq.DMQ_ERR_INVALID_ARG
    if _no_gpu():
        assert res(_proj(y=Y0), _proj(y=Y1)) == dmq.DMQ_ERR_UNSUPPORTED


def test_rope_kv_cache_validation():
    f = L.dmq_rope_kv_cache
    Q, K, V, QO, KC, VC = (A16 + 0x1000 * i for i in range(6))
    ok = dict(q=Q, k=K, v=V, M=4, pos0=0, hq=24, hkv=8, theta=500000.0, ff=None, qo=QO, kc=KC, vc=VC, L=16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["M"], a["pos0"], a["hq"], a["hkv"], a["theta"], a["ff"], a["qo"],
                 a["kc"], a["vc"], a["L"], None)
    for bad in (dict(q=None), dict(k=None), dict(v=None), dict(qo=None), dict(kc=None), dict(vc=None),
                dict(M=0), dict(pos0=-1), dict(pos0=13), dict(L=0), dict(hq=25), dict(hkv=0), dict(hq=72),
                dict(theta=1.0), dict(theta=float("nan")), dict(theta=-5.0)):
        assert call(**bad) == dmq.DMQ_ERR_INVALID_ARG, bad
    for bad in (dict(q=MIS), dict(k=MIS), dict(v=MIS), dict(qo=MIS), dict(kc=MIS), dict(vc=MIS),
                dict(ff=A16 + 2)):
        assert call(**bad) == dmq.DMQ_ERR_ALIGNMENT, bad


def test_rope_attention_gqa_validation():
    """The fused RoPE + cache append + attention call makes the checks of
    both calls, and rejects an output over any other buffer.  M = 2, 24
    query and 8 KV heads of 128, cache of 16 positions: q fp32 24 KiB, k and
    v fp32 8 KiB each, q_f16 and the output 12 KiB each, each cache 32 KiB."""
    f = L.dmq_rope_attention_gqa
    Q, K, V, QO, KC, VC, O = (A16 + 0x100000 * i for i in range(7))   # 1 MiB apart: no overlaps
    ok = dict(q=Q, k=K, v=V, M=2, pos0=0, hq=24, hkv=8, theta=500000.0, ff=None, qo=QO, kc=KC, vc=VC, L=16, o=O)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["M"], a["pos0"], a["hq"], a["hkv"], a["theta"], a["ff"], a["qo"],
                 a["kc"], a["vc"], a["L"], a["o"], None)
    for bad in (dict(q=None), dict(k=None), dict(v=None), dict(qo=None), dict(kc=None), dict(vc=None), dict(o=None),
                dict(M=0), dict(pos0=-1), dict(pos0=15), dict(L=0), dict(hq=25), dict(hkv=0), dict(hq=72),
                dict(theta=1.0), dict(theta=float("nan"))):
        assert call(**bad) == dmq.DMQ_ERR_INVALID_ARG, bad
    for bad in (dict(q=MIS), dict(k=MIS), dict(v=MIS), dict(qo=MIS), dict(kc=MIS), dict(vc=MIS), dict(o=MIS),
                dict(ff=A16 + 2)):
        assert call(**bad) == dmq.DMQ_ERR_ALIGNMENT, bad
    for bad in (dict(o=QO), dict(o=QO + 0x2ff0), dict(o=KC + 0x7ff0), dict(o=VC), dict(o=Q + 0x10),
                dict(qo=K), dict(kc=V + 0x1ff0), dict(vc=KC + 0x10), dict(kc=O - 0x7ff0)):
        assert call(**bad) == dmq.DMQ_ERR_INVALID_ARG, bad
    if _no_gpu():
        assert call() == dmq.DMQ_ERR_UNSUPPORTED
        assert call(M=1, pos0=15) == dmq.DMQ_ERR_UNSUPPORTED


def test_attention_gqa_validation():
    f = L.dmq_attention_gqa
    Q, KC, VC, O = (A16 + 0x1000 * i for i in range(4))
    ok = dict(q=Q, kc=KC, vc=VC, o=O, M=2, pos0=3, hq=24, hkv=8, L=8)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kc"], a["vc"], a["o"], a["M"], a["pos0"], a["hq"], a["hkv"], a["L"], None)
    for bad in (dict(q=None), dict(kc=None), dict(vc=None), dict(o=None), dict(o=Q), dict(M=0),
                dict(pos0=7), dict(pos0=-1), dict(hq=20), dict(hq=80, hkv=8), dict(hkv=0)):
        assert call(**bad) == dmq.DMQ_ERR_INVALID_ARG, bad
    for bad in (dict(q=MIS), dict(kc=MIS), dict(vc=MIS), dict(o=MIS)):
        assert call(**bad) == dmq.DMQ_ERR_ALIGNMENT, bad


def test_residual_rmsnorm_validation():
    f = L.dmq_residual_rmsnorm
    H, Y, G, HO, XN = (A16 + 0x1000 * i for i in range(5))
    assert f(None, Y, G, 1e-5, HO, XN, 2, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, None, G, 1e-5, HO, XN, 2, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, 1e-5, None, XN, 2, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, 1e-5, HO, None, 2, 256, None) == dmq.DMQ_ERR_INVALID_ARG    # g needs xn
    assert f(H, Y, G, -1.0, HO, XN, 2, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, float("nan"), HO, XN, 2, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(H, Y, G, 1e-5, HO, XN, 2, 300, None) == dmq.DMQ_ERR_INVALID_ARG      # K % 256
    assert f(H, Y, G, 1e-5, HO, XN, 0, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(MIS, Y, G, 1e-5, HO, XN, 2, 256, None) == dmq.DMQ_ERR_ALIGNMENT
    assert f(H, Y, G + 8, 1e-5, HO, XN, 2, 256, None) == dmq.DMQ_ERR_ALIGNMENT
    assert f(H, Y, G, 1e-5, HO, XN + 8, 2, 256, None) == dmq.DMQ_ERR_ALIGNMENT
    # without g, a missing xn or a bad eps is no error: checked here through
    # another argument's error, so no call ever reaches the device
    assert f(H, Y, None, float("nan"), HO, None, 2, 300, None) == dmq.DMQ_ERR_INVALID_ARG
    assert f(MIS, Y, None, float("nan"), HO, None, 2, 256, None) == dmq.DMQ_ERR_ALIGNMENT


def test_outputs_overlapping_inputs_are_rejected():
    """The GEMM, grouped GEMM, FFN and dequant calls reject an output that
    shares a byte with an input of the same launch or with another output
    (some workgroups would write it while others still read it).  M = 4,
    N = 4, K = 256: x is 2 KiB, y 64 bytes, a Q4_K weight array 4 blocks of
    144 bytes, a Q6_K one 4 blocks of 210 bytes."""
    X, W, Y = A16, A16 + 0x1000, A16 + 0x2000
    g = L.dmq_gemm_q4k
    for y in (X, X + 0x7f0, W, W + 0x230):
        assert g(X, W, y, 4, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG, hex(y)
    assert L.dmq_gemm_q6k(X, W, W + 0x340, 4, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG   # Q6_K: 840 bytes
    if _no_gpu():
        assert g(X, W, Y, 4, 4, 256, None) == dmq.DMQ_ERR_UNSUPPORTED
        assert L.dmq_gemm_q6k(X, W, W + 0x350, 4, 4, 256, None) == dmq.DMQ_ERR_UNSUPPORTED

    def group(*ps):
        arr = (dmq.GemmDesc * len(ps))()
        for i, (x, w, y) in enumerate(ps):
            arr[i].format, arr[i].x_f16, arr[i].wq, arr[i].y = 0, x, w, y
            arr[i].M, arr[i].N, arr[i].K = 4, 4, 256
        return L.dmq_gemm_group(arr, len(ps), None)
    assert group((X, W, Y), (X, W, Y + 0x30)) == dmq.DMQ_ERR_INVALID_ARG     # two outputs share bytes
    assert group((X, W, Y), (Y, W, Y + 0x100)) == dmq.DMQ_ERR_INVALID_ARG    # one's output is another's x
    assert group((X, W, Y), (X, Y - 0x10, Y + 0x100)) == dmq.DMQ_ERR_INVALID_ARG   # ... or its weights
    if _no_gpu():
        assert group((X, W, Y), (X, W, Y + 0x40)) == dmq.DMQ_ERR_UNSUPPORTED   # shared inputs are fine

    # FFN, M = 4, D = 256, F = 256: h is 2 KiB of fp16, y 4 KiB of fp32
    WGU, WD, H, YF = A16 + 0x10000, A16 + 0x20000, A16 + 0x30000, A16 + 0x40000
    ffn = lambda x=X, h=H, y=YF: L.dmq_ffn_swiglu_q4k(x, WGU, WD, h, y, 4, 256, 256, None)  # noqa: E731
    assert ffn(h=X + 0x10) == dmq.DMQ_ERR_INVALID_ARG
    assert ffn(y=H + 0x7f0) == dmq.DMQ_ERR_INVALID_ARG
    assert ffn(y=WD) == dmq.DMQ_ERR_INVALID_ARG
    assert ffn(h=WGU + 0x400) == dmq.DMQ_ERR_INVALID_ARG
    if _no_gpu():
        assert ffn() == dmq.DMQ_ERR_UNSUPPORTED

    # dequant: 4 rows of 256 weights, 2 KiB of fp16 out
    assert L.dmq_dequant_q4k(W, W + 0x200, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG
    assert L.dmq_dequant_q6k(W, W - 0x7f0, 4, 256, None) == dmq.DMQ_ERR_INVALID_ARG


def test_layer_step_overlaps_are_rejected():
    """RoPE + cache append, attention and residual + RMSNorm reject outputs
    that share bytes with what they read.  M = 2, 6 query heads and 2 KV
    heads of 128, cache of 16 positions: q fp32 6 KiB, q_f16 3 KiB, each
    cache 8 KiB, attention output 3 KiB; residual rows K = 256."""
    Q, K_, V, QH, KC, VC, O = (A16 + 0x10000 * i for i in range(7))
    rope = lambda qh=QH, kc=KC, vc=VC, q=Q: L.dmq_rope_kv_cache(  # noqa: E731
        q, K_, V, 2, 0, 6, 2, 500000.0, None, qh, kc, vc, 16, None)
    assert rope(qh=Q + 0x1000) == dmq.DMQ_ERR_INVALID_ARG          # q_f16 over q
    assert rope(kc=V + 0x100) == dmq.DMQ_ERR_INVALID_ARG           # cache over v
    assert rope(vc=KC + 0x1ff0) == dmq.DMQ_ERR_INVALID_ARG         # the two caches
    att = lambda out=O, q=QH: L.dmq_attention_gqa(q, KC, VC, out, 2, 14, 6, 2, 16, None)  # noqa: E731
    assert att(out=QH + 0x100) == dmq.DMQ_ERR_INVALID_ARG
    assert att(out=VC + 0x1ff0) == dmq.DMQ_ERR_INVALID_ARG
    assert L.dmq_attention_gqa_noalloc(QH, KC, VC, KC, 2, 14, 6, 2, 16, None) == dmq.DMQ_ERR_INVALID_ARG
    H, Yr, G, XN, HO = (A16 + 0x100000 + 0x10000 * i for i in range(5))
    res = lambda ho=HO, xn=XN, g=G: L.dmq_residual_rmsnorm(H, Yr, g, 1e-5, ho, xn, 4, 256, None)  # noqa: E731
    assert res(ho=H + 0x10) == dmq.DMQ_ERR_INVALID_ARG              # partly over h_in
    assert res(xn=Yr + 0x3f0) == dmq.DMQ_ERR_INVALID_ARG            # xn over y
    assert res(xn=HO + 0x200) == dmq.DMQ_ERR_INVALID_ARG            # xn over h_out
    assert res(ho=G - 0x10) == dmq.DMQ_ERR_INVALID_ARG              # h_out over g
    if _no_gpu():
        assert res(ho=H) == dmq.DMQ_ERR_UNSUPPORTED                # in place: allowed
        assert res(ho=Yr) == dmq.DMQ_ERR_UNSUPPORTED
        assert rope() == dmq.DMQ_ERR_UNSUPPORTED
        assert att() == dmq.DMQ_ERR_UNSUPPORTED
