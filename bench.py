"""Benchmark: prefill TFLOP/s of the fused Q4_K / Q6_K dequant-GEMM at M=1024.

One step = one pass of the prefill hot path over one batch: the seven
projection GEMMs of one Llama-3.2-3B-shaped decoder layer (Q, K, V, O, gate,
up in Q4_K, down in Q6_K) at M = 1024 tokens, issued as one grouped launch of
the library (dmq_gemm_group).  Weights rotate over several independently
seeded layers (more bytes than the 256 MB Infinity Cache) so every step
streams its weights from HBM.  Inputs are resident in HBM before timing.

Prints one JSON line (rank 0, one GPU).  Extra keys:
  roofline      -- the GEMM kernel against the fp16 dense MFMA peak, from HIP
                   events around every launch on the launch stream;
  cpu_baseline  -- the CPU oracle on a bounded sample of the same workload;
  decode        -- the M = 1 decode kernel on one layer (GB/s of weights).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synthetic  # noqa: E402

import hashlib  # noqa: E402

PEAK_FP16_TFLOPS = 2516.6      # MI355X dense fp16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
M_PREFILL = 1024
ROTATE_LAYERS = 5              # 5 x 63.1 MB of weights > 256 MB Infinity Cache
DECODE_ROTATE = 8              # decode: 8 x 63.1 MB
SETTLE_MS = 150.0              # untimed GPU work before any timed region (clock settling)


# HBM bytes per launch of the grouped prefill call (the GEMM kernel and the
# split-K combine), from rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled by
# the same counters' reading for a plain copy of known size
# (profiles/gemm_kernel_layer_m1024_traffic.md).  Valid
# only for the kernel sources they were taken with: a changed source reports
# traffic as null until the counters are taken again.
TRAFFIC_SOURCES = ("dequant_gemm_q4_amd/csrc/gemm.hip", "dequant_gemm_q4_amd/csrc/dmq_common.h")
TRAFFIC = {"sources_sha256": "1033dacbb2758a9c331803b657681d1bfaab1b5f342691ebb532f7982cc0340d", "bytes_per_launch": 619616247}
COPY_PROBE_BYTES = 256 << 20


def sources_sha256():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_probe(torch, reps=3):
    """A plain device-to-device copy of COPY_PROBE_BYTES (for calibrating the
    FETCH_SIZE / WRITE_SIZE counters: it reads and writes exactly that much),
    then timed copies of 64 MiB and 256 MiB as a plain-bandwidth reference."""
    src = torch.randint(0, 255, (COPY_PROBE_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    out = {"copy_probe_bytes": COPY_PROBE_BYTES, "reps": reps}
    for n in (64 << 20, 256 << 20):
        a, b = src[:n], dst[:n]
        for _ in range(3):
            b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        out[f"copy_{n >> 20}MiB_read_plus_write_GBps"] = round(2 * n / ms / 1e6, 1)
    print(json.dumps(out), flush=True)


def vendor_gemm_probe(torch):
    """Dense fp16 GEMMs through torch.matmul (the vendor BLAS) on the layer's
    shapes at M = 1024: a reference for what a dense, dequant-free fp16 GEMM
    reaches on this GPU (fp16 output, fp32 accumulation)."""
    out = {}
    M = M_PREFILL
    tot_fl, tot_ms = 0.0, 0.0
    for name, fmt, N, K in synthetic.LAYER_PROJECTIONS:
        a = torch.randn(M, K, device="cuda", dtype=torch.float16)
        w = torch.randn(N, K, device="cuda", dtype=torch.float16)
        wt = w.t()
        f = lambda: torch.matmul(a, wt)   # noqa: E731
        settle(torch, f, 5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        fl = 2.0 * M * N * K
        out[f"{name}_{N}x{K}_TFLOPs"] = round(fl / ms / 1e9, 1)
        tot_fl += fl
        tot_ms += ms
    out["layer_sequential_TFLOPs"] = round(tot_fl / tot_ms / 1e9, 1)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
    settle(torch, lambda: torch.matmul(a, a), 3, chunk=3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.matmul(a, a)
    e1.record()
    torch.cuda.synchronize()
    out["square_8192_fp16_out_TFLOPs"] = round(2 * 8192 ** 3 / (e0.elapsed_time(e1) / 10) / 1e9, 1)
    # graphics clock and socket power while the square GEMM runs
    out["square_8192_clock_power"] = ClockSampler(torch).run_while(lambda: torch.matmul(a, a))
    print(json.dumps({"vendor_gemm_probe": out}), flush=True)


def _timed(torch, fn, reps=20, warm=5):
    """Mean ms of fn() over reps launches (HIP events on the current stream),
    after at least `warm` untimed calls and SETTLE_MS of GPU time."""
    settle(torch, fn, warm, chunk=max(1, min(25, warm)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


SWEEP_PARTS = ("config0", "ffn", "layers", "rmsnorm", "lmhead", "chain", "overlap")


def sweep(torch, dmq, parts=SWEEP_PARTS):
    """The other configurations of the scope table, one JSON line each:
    config 0 (one Q projection at M=16), config 3 (fused SwiGLU FFN at
    M=1024, x ~ N(0,1) and the sigma=1/16 companion), config 4 (one layer's
    seven GEMMs at M = 1024 / 2048 / 4096, weights rotated over 5 layers,
    and the Q6_K LM head on 1024 rows).  `parts` selects which."""
    if "config0" in parts:
        sweep_config0(torch, dmq)
    if "ffn" in parts:
        sweep_ffn(torch, dmq)
    if "layers" in parts:
        sweep_layers(torch, dmq)
    if "rmsnorm" in parts:
        sweep_rmsnorm(torch, dmq)
    if "lmhead" in parts:
        sweep_lmhead(torch, dmq)
    if "chain" in parts:
        layer_chain_sweep(torch, dmq)
    if "overlap" in parts:
        layer_overlap_sweep(torch, dmq)


def sweep_config0(torch, dmq):
    dev = "cuda"
    # config 0: one Q projection, M = 16, weights rotated (64 copies > 256 MB cache)
    M, N, K = 16, 3072, 3072
    x = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(0, 0, 0))).to(dev)
    ws = [torch.from_numpy(synthetic.q4k_blocks(N, K, seed=synthetic.weight_seed(0, layer, 0)).reshape(-1)).to(dev)
          for layer in range(64)]
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    it = [0]

    def c0():
        dmq.dmq_gemm_q4k(x, ws[it[0] % 64], y, M, N, K)
        it[0] += 1
    ms = _timed(torch, c0, reps=64)
    # the same 64 launches replayed from a HIP graph: no host launch gaps
    gms = time_graph(torch, lambda w: dmq.dmq_gemm_q4k(x, w, y, M, N, K), ws, 4)
    wbytes = N * (K // 256) * 144
    print(json.dumps({"sweep": "config0 Q4_K GEMM M=16 N=K=3072, 64 rotating weight copies",
                      "us": round(ms * 1e3, 2), "TFLOP/s": round(2 * M * N * K / ms / 1e9, 2),
                      "weight_GB/s": round(wbytes / ms / 1e6, 1),
                      "graph_us": round(gms * 1e3, 2), "graph_weight_GB/s": round(wbytes / gms / 1e6, 1)}), flush=True)
    del ws
    # one layer's seven projections at M = 16, 2 and 3 in one grouped launch
    # (M = 2 on the two-row decode kernel, the others on the small-M kernel),
    # 8 rotating layers, graph replay
    for M, kern in ((16, "small-M"), (2, "two-row decode"), (3, "small-M")):
        xs, ys = {}, {}
        for idx, (name, fmt, N, K) in enumerate(synthetic.LAYER_PROJECTIONS):
            xs[name] = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(0, 0, idx))).to(dev)
            ys[name] = torch.empty((M, N), dtype=torch.float32, device=dev)
        layers = [layer_problems(torch, dmq, 0, layer, M, xs, ys) for layer in range(8)]
        per = time_graph(torch, dmq.dmq_gemm_group, [g for g, _ in layers], 20, per_replay=True)
        us = float(np.median(per)) * 1e3
        print(json.dumps({"sweep": f"layer GEMMs M={M} (grouped {kern} launch, 8 rotating layers, graph replay)",
                          "us_per_layer": round(us, 2), "weight_GB/s": round(weight_bytes() / us / 1e3, 1),
                          "TFLOP/s": round(flops_of(M) / us / 1e6, 2), "ms_per_layer": stats(per)}), flush=True)
        del layers


def sweep_ffn(torch, dmq):
    dev = "cuda"
    # config 3: fused FFN, M = 1024, D = 3072, F = 8192
    M, D, F = 1024, 3072, 8192
    wgu = torch.from_numpy(synthetic.q4k_blocks(2 * F, D, seed=synthetic.weight_seed(3, 0, 4)).reshape(-1)).to(dev)
    wd = torch.from_numpy(synthetic.q6k_blocks(D, F, seed=synthetic.weight_seed(3, 0, 6)).reshape(-1)).to(dev)
    h = torch.empty((M, F), dtype=torch.float16, device=dev)
    yf = torch.empty((M, D), dtype=torch.float32, device=dev)
    for sigma in (1.0, 1.0 / 16):
        xf = torch.from_numpy(synthetic.activations(M, D, seed=synthetic.act_seed(3, 0, 4), sigma=sigma)).to(dev)
        ms = _timed(torch, lambda: dmq.dmq_ffn_swiglu_q4k(xf, wgu, wd, h, yf, M, D, F))
        hf = h.float()
        fl = 2.0 * M * (2 * F * D + D * F)
        print(json.dumps({"sweep": f"config3 SwiGLU FFN M=1024 D=3072 F=8192 x~N(0,{sigma:g}^2)",
                          "us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                          "h_overflow_fraction": round(float((~torch.isfinite(hf)).float().mean()), 4)}), flush=True)
    del wgu, wd, h, yf



def sweep_layers(torch, dmq):
    dev = "cuda"
    # config 4: one layer's seven GEMMs at M = 1024, 2048, 4096 (grouped launch)
    for M in (1024, 2048, 4096):
        xs, ys = {}, {}
        for idx, (name, fmt, N, K) in enumerate(synthetic.LAYER_PROJECTIONS):
            xs[name] = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(4, 0, idx),
                                                              unit_rms=True)).to(dev)
            ys[name] = torch.empty((M, N), dtype=torch.float32, device=dev)
        layers = [layer_problems(torch, dmq, 4, layer, M, xs, ys) for layer in range(ROTATE_LAYERS)]
        it = [0]

        def c4():
            dmq.dmq_gemm_group(layers[it[0] % ROTATE_LAYERS][0])
            it[0] += 1
        ms = _timed(torch, c4)
        print(json.dumps({"sweep": f"config4 layer GEMMs M={M} (grouped launch, 5 rotating layers)",
                          "ms": round(ms, 4), "TFLOP/s": round(flops_of(M) / ms / 1e9, 1),
                          "pct_fp16_peak": round(100 * flops_of(M) / ms / 1e9 / PEAK_FP16_TFLOPS, 2)}), flush=True)
        del layers, xs, ys



def sweep_rmsnorm(torch, dmq):
    dev = "cuda"
    # RMSNorm ahead of the Q|K|V projections (K = 3072): the normalize-then-
    # GEMM call against the same three GEMMs on already normalized input, at
    # M = 1024 (norm kernel + grouped GEMM) and M = 1 (norm fused into the
    # decode kernel's x staging; graph replays over 8 weight copies)
    K = 3072
    g = torch.from_numpy(np.random.default_rng(77).uniform(0.5, 1.5, K).astype(np.float32)).to(dev)
    qkv = [(i, N) for i, N in enumerate((3072, 1024, 1024))]
    for M in (1024, 1):
        x = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(2, 0, 0), sigma=1.5)).to(dev)
        xn = torch.empty((M, K), dtype=torch.float16, device=dev)
        ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _, N in qkv]
        nl = 8 if M == 1 else 5
        ws = [[torch.from_numpy(synthetic.q4k_blocks(N, K, seed=synthetic.weight_seed(2, layer, i)).reshape(-1)).to(dev)
               for i, N in qkv] for layer in range(nl)]
        projs = [dmq.make_projs([("q4k", w, y, N) for w, y, (_, N) in zip(wl, ys, qkv)], K) for wl in ws]
        groups = [dmq.make_group([("q4k", xn, w, y, M, N, K) for w, y, (_, N) in zip(wl, ys, qkv)]) for wl in ws]
        out_xn = None if M == 1 else xn
        fused = lambda p: dmq.dmq_rmsnorm_gemm(x, g, 1e-5, out_xn, p, M, K)   # noqa: E731
        if M == 1:
            t_norm = time_graph(torch, fused, projs, 8)
            t_plain = time_graph(torch, dmq.dmq_gemm_group, groups, 8)
        else:
            it = [0]

            def run(fn, lst):
                fn(lst[it[0] % len(lst)])
                it[0] += 1
            t_norm = _timed(torch, lambda: run(fused, projs))
            t_plain = _timed(torch, lambda: run(dmq.dmq_gemm_group, groups))
        fl = 2.0 * M * K * sum(N for _, N in qkv)
        print(json.dumps({"sweep": f"RMSNorm + Q|K|V projections M={M} K={K} "
                                   f"({'graph replay' if M == 1 else 'host-launched'})",
                          "us_with_norm": round(t_norm * 1e3, 2), "us_gemms_only": round(t_plain * 1e3, 2),
                          "norm_overhead_us": round((t_norm - t_plain) * 1e3, 2),
                          "TFLOP/s_with_norm": round(fl / t_norm / 1e9, 1)}), flush=True)
        del ws, projs, groups



def sweep_lmhead(torch, dmq):
    dev = "cuda"
    # config 4: tied LM head, Q6_K 3072 -> 128256 on 1024 rows
    name, fmt, N, K = synthetic.LM_HEAD
    M = 1024
    wl = torch.from_numpy(synthetic.lm_head_weights(4).reshape(-1)).to(dev)
    xl = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(4, 0, synthetic.LM_HEAD_INDEX),
                                                unit_rms=True)).to(dev)
    yl = torch.empty((M, N), dtype=torch.float32, device=dev)
    ms = _timed(torch, lambda: dmq.dmq_gemm_q6k(xl, wl, yl, M, N, K), reps=10, warm=2)
    print(json.dumps({"sweep": "config4 LM head Q6_K N=128256 K=3072 M=1024",
                      "ms": round(ms, 4), "TFLOP/s": round(2.0 * M * N * K / ms / 1e9, 1)}), flush=True)


def layer_chain_sweep(torch, dmq):
    """A whole decoder layer through the library (RMSNorm -> Q|K|V -> RoPE +
    KV cache -> attention -> O projection -> residual + RMSNorm -> SwiGLU FFN
    -> residual), Llama-3.2-3B shapes, weights rotated over several seeded
    layers: the decode step (M = 1, graph replay) at two context lengths and
    the M = 1024 prefill (host-launched); the attention kernel alone; the
    decode LM head."""
    dev = "cuda"
    D, F, HQ, HKV, HD = synthetic.HIDDEN, synthetic.FFN, synthetic.N_HEADS, synthetic.N_KV_HEADS, synthetic.HEAD_DIM
    rng = np.random.default_rng(1234)
    g1 = torch.from_numpy((0.02 * rng.uniform(0.5, 1.5, D)).astype(np.float32)).to(dev)
    g2 = torch.from_numpy((0.05 * rng.uniform(0.5, 1.5, D)).astype(np.float32)).to(dev)

    def weights(layer):
        w = {name: (fmt, wq) for name, fmt, N, K, wq in synthetic.layer_weights(4, layer)}
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(dev)  # noqa: E731
        return {"q": t(w["q"][1]), "k": t(w["k"][1]), "v": t(w["v"][1]), "o": t(w["o"][1]),
                "gu": t(np.concatenate([w["gate"][1], w["up"][1]], axis=0)), "down": t(w["down"][1])}

    def buffers(M):
        e = lambda *shape, dt=torch.float32: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        x = torch.from_numpy(rng.standard_normal((M, D)).astype(np.float32)).to(dev)
        return {"x": x, "zero": torch.zeros_like(x), "h0": e(M, D), "xn1": e(M, D, dt=torch.float16),
                "yq": e(M, HQ * HD), "yk": e(M, HKV * HD), "yv": e(M, HKV * HD),
                "qr": e(M, HQ * HD, dt=torch.float16), "att": e(M, HQ * HD, dt=torch.float16), "yo": e(M, D),
                "h1": e(M, D), "xn2": e(M, D, dt=torch.float16), "hf": e(M, F, dt=torch.float16), "yd": e(M, D),
                "out": e(M, D)}

    # one layer of a stack: xn1 = RMSNorm(x) comes from the previous layer's
    # last call (residual add fused with this layer's input RMSNorm), which
    # this layer's last call repeats for the next one (in place on x)
    def step(W, B, kc, vc, M, pos0, L):
        dmq.dmq_gemm_group(W["qkv"])
        dmq.dmq_rope_kv_cache(B["yq"], B["yk"], B["yv"], M, pos0, HQ, HKV, B["qr"], kc, vc, L)
        dmq.dmq_attention_gqa(B["qr"], kc, vc, B["att"], M, pos0, HQ, HKV, L)
        dmq.dmq_gemm_q4k(B["att"], W["o"], B["yo"], M, D, HQ * HD)
        dmq.dmq_residual_rmsnorm(B["x"], B["yo"], g2, 1e-5, B["h1"], B["xn2"], M, D)
        dmq.dmq_ffn_swiglu_q4k(B["xn2"], W["gu"], W["down"], B["hf"], B["yd"], M, D, F)
        dmq.dmq_residual_rmsnorm(B["h1"], B["yd"], g1, 1e-5, B["x"], B["xn1"], M, D)

    # the same layer with the residual adds fused into the projections that
    # follow them (dmq_residual_rmsnorm_gemm): at M = 1 the decode kernel
    # forms h = h_in + y and its RMSNorm while it stages x.  The residual
    # stream alternates between x and h1; this layer's first call adds the
    # previous layer's FFN output.
    def step_fused(W, B, kc, vc, M, pos0, L, rope_in_attention=False):
        dmq.dmq_residual_rmsnorm_gemm(B["h1"], B["yd"], g1, 1e-5, B["x"], None, W["qkv_p"], M, D)
        if rope_in_attention:   # RoPE + cache append inside the attention call (one launch fewer at M = 1)
            dmq.dmq_rope_attention_gqa(B["yq"], B["yk"], B["yv"], M, pos0, HQ, HKV, B["qr"], kc, vc, L, B["att"])
        else:
            dmq.dmq_rope_kv_cache(B["yq"], B["yk"], B["yv"], M, pos0, HQ, HKV, B["qr"], kc, vc, L)
            dmq.dmq_attention_gqa(B["qr"], kc, vc, B["att"], M, pos0, HQ, HKV, L)
        dmq.dmq_gemm_q4k(B["att"], W["o"], B["yo"], M, D, HQ * HD)
        dmq.dmq_residual_rmsnorm_gemm(B["x"], B["yo"], g2, 1e-5, B["h1"], None, W["gu_p"], M, D)
        dmq.dmq_gemm_q6k(B["hf"], W["down"], B["yd"], M, D, F)

    def make(nl, M, L):
        Ws = [weights(l) for l in range(nl)]
        B = buffers(M)
        for W in Ws:
            W["qkv"] = dmq.make_group([("q4k", B["xn1"], W["q"], B["yq"], M, HQ * HD, D),
                                       ("q4k", B["xn1"], W["k"], B["yk"], M, HKV * HD, D),
                                       ("q4k", B["xn1"], W["v"], B["yv"], M, HKV * HD, D)])
            W["qkv_p"] = dmq.make_projs([("q4k", W["q"], B["yq"], HQ * HD), ("q4k", W["k"], B["yk"], HKV * HD),
                                         ("q4k", W["v"], B["yv"], HKV * HD)], D)
            W["gu_p"] = dmq.make_projs([("q4k", W["gu"], B["hf"], 2 * F, "swiglu")], D)
        caches = [(torch.zeros((HKV, L, HD), dtype=torch.float16, device=dev),
                   torch.zeros((HKV, L, HD), dtype=torch.float16, device=dev)) for _ in range(nl)]
        for kc, vc in caches:   # earlier tokens' keys and values
            kc.normal_()
            vc.normal_()
        dmq.dmq_residual_rmsnorm(B["x"], B["zero"], g1, 1e-5, B["h0"], B["xn1"], M, D)
        return Ws, B, caches

    # decode step, 8 rotating layers, graph replay
    for L in (1024, 4096):
        pos0 = L - 1
        Ws, B, caches = make(8, 1, L)
        items = list(zip(Ws, caches))
        us = time_graph(torch, lambda it: step(it[0], B, it[1][0], it[1][1], 1, pos0, L), items, 8) * 1e3
        B["h1"].copy_(B["x"])
        B["yd"].zero_()
        uf = time_graph(torch, lambda it: step_fused(it[0], B, it[1][0], it[1][1], 1, pos0, L), items, 8) * 1e3
        ur = time_graph(torch, lambda it: step_fused(it[0], B, it[1][0], it[1][1], 1, pos0, L, True), items, 8) * 1e3
        # the attention kernel alone at this context
        ua = time_graph(torch, lambda it: dmq.dmq_attention_gqa(B["qr"], it[1][0], it[1][1], B["att"], 1, pos0,
                                                                HQ, HKV, L), items, 8) * 1e3
        kv_bytes = 2 * HKV * L * HD * 2
        print(json.dumps({"sweep": f"decode step, one Llama-3.2-3B layer, all kernels (graph replay, 8 rotating layers), "
                                   f"context {L}", "us_per_layer": round(us, 2),
                          "fused_residual_us_per_layer": round(uf, 2),
                          "fused_residual_and_rope_us_per_layer": round(ur, 2),
                          "attention_us": round(ua, 2), "attention_kv_GB/s": round(kv_bytes / ua / 1e3, 1)}),
              flush=True)
        del Ws, B, caches, items
    # LM head at M = 1 (decode): 323 MB of Q6_K
    name, fmt, N, K = synthetic.LM_HEAD
    wl = torch.from_numpy(synthetic.lm_head_weights(4).reshape(-1)).to(dev)
    x1 = torch.from_numpy(synthetic.activations(1, K, seed=3)).to(dev)
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    ul = time_graph(torch, lambda w: dmq.dmq_gemm_q6k(x1, w, y1, 1, N, K), [wl], 8) * 1e3
    print(json.dumps({"sweep": "decode LM head Q6_K 128256x3072, M=1 (graph replay)", "us": round(ul, 2),
                      "GB/s": round(wl.numel() / ul / 1e3, 1)}), flush=True)
    del wl
    # prefill M = 1024 from position 0, 3 rotating layers, host-launched
    M, L = 1024, 1024
    Ws, B, caches = make(3, M, L)
    it = [0]

    def one():
        W, (kc, vc) = Ws[it[0] % 3], caches[it[0] % 3]
        it[0] += 1
        step(W, B, kc, vc, M, 0, L)
    ms = _timed(torch, one, reps=10, warm=3)
    it[0] = 0
    ma = _timed(torch, lambda: dmq.dmq_attention_gqa(B["qr"], caches[0][0], caches[0][1], B["att"], M, 0, HQ, HKV, L),
                reps=10, warm=2)
    att_flop = 4.0 * HQ * HD * (M * (M + 1) / 2)
    gemm_flop = flops_of(M)
    print(json.dumps({"sweep": "prefill, one Llama-3.2-3B layer, all kernels (host-launched, 3 rotating layers), M=1024",
                      "ms_per_layer": round(ms, 4), "attention_ms": round(ma, 4),
                      "attention_TFLOP/s": round(att_flop / ma / 1e9, 2),
                      "layer_TFLOP/s": round((gemm_flop + att_flop) / ms / 1e9, 1)}), flush=True)


def layer_overlap_sweep(torch, dmq):
    """dmq_layer_prefill on Llama-3.2-3B shapes (weights rotated over 3 seeded
    layers): the attention side of chunk c+1 overlapped with the FFN of chunk
    c on two streams, against the same chunked schedule on one stream and
    against one pass over all rows."""
    dev = "cuda"
    D, F, HQ, HKV, HD = synthetic.HIDDEN, synthetic.FFN, synthetic.N_HEADS, synthetic.N_KV_HEADS, synthetic.HEAD_DIM
    rng = np.random.default_rng(4321)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    g = [t((s_ * rng.uniform(0.5, 1.5, D)).astype(np.float32)) for s_ in (0.02, 0.05, 0.02)]
    for M in (1024, 4096):
        L = M
        e = lambda *shape, dt=torch.float32: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        x = t(rng.standard_normal((M, D)).astype(np.float32))
        xn = e(M, D, dt=torch.float16)
        dmq.dmq_residual_rmsnorm(x, torch.zeros_like(x), g[0], 1e-5, e(M, D), xn, M, D)
        B = {"h_in": x, "xn_in": xn, "yq": e(M, HQ * HD), "yk": e(M, HKV * HD), "yv": e(M, HKV * HD),
             "q_rot": e(M, HQ * HD, dt=torch.float16), "attn": e(M, HQ * HD, dt=torch.float16), "yo": e(M, D),
             "h_mid": e(M, D), "xn_ffn": e(M, D, dt=torch.float16), "h_ffn": e(M, F, dt=torch.float16),
             "y_down": e(M, D), "h_out": e(M, D), "xn_out": e(M, D, dt=torch.float16)}
        layers = []
        for layer in range(3):
            w = {name: wq for name, fmt, N, K, wq in synthetic.layer_weights(4, layer)}
            W = {"q": t(w["q"].reshape(-1)), "k": t(w["k"].reshape(-1)), "v": t(w["v"].reshape(-1)),
                 "o": t(w["o"].reshape(-1)), "gate_up": t(np.concatenate([w["gate"], w["up"]]).reshape(-1)),
                 "down": t(w["down"].reshape(-1)), "g_ffn": g[1], "g_next": g[2],
                 "k_cache": torch.zeros((HKV, L, HD), dtype=torch.float16, device=dev),
                 "v_cache": torch.zeros((HKV, L, HD), dtype=torch.float16, device=dev)}
            layers.append((W, dmq.make_layer(W, B, M, D, F, HQ, HKV, L)))
        side = torch.cuda.Stream()
        res = {}
        plan = [("one_pass", M, False)]
        for ch in (M // 2, M // 4, 256):
            plan += [(f"chunk{ch}_one_stream", ch, False), (f"chunk{ch}_two_streams", ch, True)]
        for label, chunk, two in plan:
            it = [0]

            def one():
                dmq.dmq_layer_prefill(layers[it[0] % 3][1], M, 0, D, F, HQ, HKV, L, 1e-5, chunk,
                                      stream_attn=torch.cuda.current_stream(),
                                      stream_ffn=side if two else None)
                it[0] += 1
            res[label] = _timed(torch, one, reps=10, warm=3)
        att_flop = 4.0 * HQ * HD * (M * (M + 1) / 2)
        fl = flops_of(M) + att_flop
        best = min((k for k in res if k.endswith("two_streams")), key=lambda k: res[k])
        gains = {k.replace("_two_streams", ""): round(res[k.replace("two_streams", "one_stream")] / res[k], 3)
                 for k in res if k.endswith("two_streams")}
        print(json.dumps({"sweep": f"prefill layer, attention || FFN on two streams (dmq_layer_prefill), M={M}",
                          **{f"{k}_ms": round(v, 4) for k, v in res.items()},
                          "two_stream_gain_over_one_stream": gains,
                          "best_two_streams": best, "best_vs_one_pass": round(res["one_pass"] / res[best], 3),
                          "TFLOP/s_one_pass": round(fl / res["one_pass"] / 1e9, 1),
                          "TFLOP/s_best_two_streams": round(fl / res[best] / 1e9, 1)}), flush=True)
        del layers, B


def layer_problems(torch, dmq, config, layer, M, xs, ys):
    probs = []
    for name, fmt, N, K, wq in synthetic.layer_weights(config, layer):
        w = torch.from_numpy(wq.reshape(-1)).cuda()
        probs.append((fmt, xs[name], w, ys[name], M, N, K))
    return dmq.make_group(probs), probs


def flops_of(M):
    return sum(2.0 * M * N * K for _, _, N, K in synthetic.LAYER_PROJECTIONS)


def weight_bytes():
    size = {"q4k": 144, "q6k": 210}
    return sum(N * (K // 256) * size[f] for _, f, N, K in synthetic.LAYER_PROJECTIONS)


def settle(torch, fn, min_launches, min_ms=SETTLE_MS, chunk=25, cap=20000):
    """Untimed warm-up: call fn() at least min_launches times and until
    min_ms of GPU time have run back to back.  From idle, the GPU needs tens
    of milliseconds of continuous work before its clock settles (the first
    launches of the M=1024 layer take up to 1.8x the settled time).  Returns
    (launches run, GPU ms, mean ms of the first min(chunk, n) launches)."""
    n, ms, first = 0, 0.0, None
    while (n < min_launches or ms < min_ms) and n < cap:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(chunk):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        if first is None:
            first = t / chunk
        n += chunk
        ms += t
    return n, ms, first


def stats(ms_list):
    """Median, 95th percentile, min, max and coefficient of variation of a
    list of per-run times (ms)."""
    a = np.asarray(ms_list, dtype=np.float64)
    return {"n": int(a.size), "median": round(float(np.median(a)), 5), "p95": round(float(np.percentile(a, 95)), 5),
            "min": round(float(a.min()), 5), "max": round(float(a.max()), 5),
            "cv": round(float(a.std() / a.mean()), 4) if a.size > 1 else 0.0}


def device_record(torch):
    """What the run ran on: device name and architecture, compute units,
    memory, ROCm / HIP / torch versions."""
    p = torch.cuda.get_device_properties(0)
    rec = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "memory_GiB": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        with open("/opt/rocm/.info/version") as f:
            rec["rocm"] = f.read().strip()
    except OSError:
        rec["rocm"] = None
    return rec


class ClockSampler:
    """Graphics clock and power while the caller keeps the GPU busy, two ways.

    * Shader clock from the GPU itself: torch.cuda._sleep(n) spins one wave
      for n cycles of the shader-clock counter (s_memtime); a long spin on a
      side stream, timed with events while the load runs, gives n / t.
    * amdsmi's metrics table (per-XCD current graphics clocks, socket power,
      energy accumulator).  The table is refreshed only now and then, so a
      sample counts only when its firmware timestamp differs from the one
      before it; average power is the energy accumulator's growth between the
      first and the last refresh seen, over the host time between them.
    Reports None for a part (and why) where it cannot be measured."""

    SPIN = 50_000_000   # cycles: 21-29 ms at 1.7-2.4 GHz

    def __init__(self, torch):
        self.refreshes, self.error, self.handle = [], None, None
        self.spin_mhz = None
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            p = torch.cuda.get_device_properties(0)
            bus = getattr(p, "pci_bus_id", None)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if bus is None or int(bdf.split(":")[1], 16) == int(bus):
                    self.handle = h
                    break
            if self.handle is None:
                self.error = "device not found among amdsmi handles"
        except Exception as e:   # noqa: BLE001
            self.error = f"amdsmi unavailable: {type(e).__name__}: {e}"

    def _read(self):
        """(firmware timestamp, mean per-XCD current graphics clock in MHz,
        socket power in W or None, energy accumulator or None)."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        v = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        clk = float(np.mean(v)) if v else float(m["current_gfxclk"])
        pw = m.get("current_socket_power")
        en = m.get("energy_accumulator")
        return (m.get("firmware_timestamp"), clk, float(pw) if isinstance(pw, (int, float)) else None,
                int(en) if isinstance(en, int) else None)

    def _spin_clock(self, torch, stream, busy_fn, reps=3):
        """Shader clock in MHz from a timed clock-counter spin of SPIN cycles
        on `stream` (median of `reps`).  Before each spin, enough calls of
        the load are queued to outlast it even at 1 GHz; the spin's start
        may wait for a workgroup of the load to finish (well under 1% of
        the spin)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            busy_fn()
        e1.record()
        e1.synchronize()
        per_call_ms = max(e0.elapsed_time(e1) / 20, 1e-3)
        calls = int(1.5 * (self.SPIN / 1e6) / per_call_ms) + 1
        est = []
        for _ in range(reps):
            for _ in range(calls):
                busy_fn()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                s0.record()
                torch.cuda._sleep(self.SPIN)
                s1.record()
            torch.cuda.synchronize()
            est.append(self.SPIN / (s0.elapsed_time(s1) * 1e3))
        return float(np.median(est))

    def run_while(self, busy_fn, seconds=3.0):
        """Call busy_fn() repeatedly (it enqueues GPU work) for `seconds`;
        amdsmi is polled from a second thread, and the spins run on a side
        stream once a quarter of the time has passed (clock settled)."""
        import threading
        import torch
        stop = threading.Event()
        t0 = time.perf_counter()

        def sample():
            last = None
            while not stop.is_set():
                try:
                    ts, clk, pw, en = self._read()
                except Exception as e:   # noqa: BLE001
                    self.error = f"{type(e).__name__}: {e}"
                    return
                now = time.perf_counter()
                if last is not None and ts != last and now - t0 > seconds / 4:
                    self.refreshes.append((now, clk, pw, en))
                last = ts
                time.sleep(0.005)
        t = None
        if self.handle is not None:
            t = threading.Thread(target=sample)
            t.start()
        side = torch.cuda.Stream()
        spun = False
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                busy_fn()
            if not spun and time.perf_counter() - t0 > seconds / 4:
                self.spin_mhz = self._spin_clock(torch, side, busy_fn)
                spun = True
            torch.cuda.synchronize()
        stop.set()
        if t is not None:
            t.join()
        return self.result()

    def result(self):
        out = {"spin_MHz": round(self.spin_mhz, 1) if self.spin_mhz else None,
               "spin_source": "torch.cuda._sleep spin of 5e7 shader-clock cycles on a side stream under the load, event-timed"}
        r = self.refreshes
        if not r:
            out.update({"amdsmi_MHz": None, "amdsmi_refreshes": 0,
                        "amdsmi_error": self.error or "metrics table not refreshed during the window"})
            return out
        clk = [c for _, c, _, _ in r]
        pw = [p for _, _, p, _ in r if p is not None]
        out.update({"amdsmi_MHz": round(float(np.median(clk)), 1), "amdsmi_min_MHz": round(min(clk), 1),
                    "amdsmi_max_MHz": round(max(clk), 1),
                    "socket_power_W": round(float(np.median(pw)), 1) if pw else None,
                    "amdsmi_refreshes": len(r)})
        en = [(tt, e) for tt, _, _, e in r if e is not None]
        if len(en) >= 2 and en[-1][0] > en[0][0]:
            res_uj = self.amdsmi.amdsmi_get_energy_count(self.handle)["counter_resolution"]
            out["energy_avg_power_W"] = round((en[-1][1] - en[0][1]) * res_uj * 1e-6 / (en[-1][0] - en[0][0]), 1)
        return out


def time_launches(torch, launch, groups, steps, warmup):
    """Run `launch(group)` over the rotating groups on the current stream.
    The `steps` timed launches run back to back between one pair of events
    (total_ms).  A second pass of the same launches, each between its own
    pair of events, gives the per-launch distribution; it is not part of
    total_ms, since an event recorded between two launches costs GPU time
    of its own.  Returns (total_ms, [per-launch ms], warm-up record)."""
    it = [0]

    def one():
        launch(groups[it[0] % len(groups)])
        it[0] += 1
    nw, wms, cold = settle(torch, one, warmup)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        launch(groups[i % len(groups)])
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        launch(groups[i % len(groups)])
        ev[i][1].record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return total, per, {"launches": nw, "gpu_ms": round(wms, 1), "first_ms_per_step": round(cold, 4)}


def time_graph(torch, launch, groups, replays, per_replay=False):
    """Capture one launch per group into a HIP graph and time `replays`
    replays (kernels back to back, no host launch gaps), each between its own
    pair of events.  Returns ms per launch (mean over the replays), or with
    per_replay the list of per-replay ms per launch."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for g in groups:
            launch(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    # captured on the stream that ran the launches above, so that any
    # per-stream workspace the library keeps already exists
    with torch.cuda.graph(graph, stream=side):
        for g in groups:
            launch(g)
    settle(torch, graph.replay, 2, chunk=5)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) / len(groups) for a, b in ev]
    return per if per_replay else float(np.mean(per))


def cpu_baseline(rows_sample: int):
    """The oracle (dequant + fp64 matmul) on `rows_sample` rows of every
    projection of one layer, timed on this host; scaled to TFLOP/s."""
    import oracle
    oracle.build()
    items = []
    for idx, (name, fmt, N, K, wq) in enumerate(synthetic.layer_weights(2, 0)):
        x = synthetic.activations(rows_sample, K, seed=synthetic.act_seed(2, 0, idx), unit_rms=True)
        items.append((fmt, x, wq, N, K))
    t = time.perf_counter()
    for fmt, x, wq, N, K in items:
        oracle.gemm_quant(fmt, x, wq, N, K)
    dt = time.perf_counter() - t
    fl = flops_of(rows_sample)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {rows_sample} of {M_PREFILL} rows of all 7 projections of one layer "
                      f"(exact dequant + fp64 matmul; {fl / 1e9:.1f} GFLOP in {dt:.1f} s)"}


def counters_workload(torch, dmq, reps=5):
    """A short run for counter collection (rocprofv3 --pmc): `reps` launches
    each of the M = 1024 prefill layer (one grouped GEMM call), the M = 1
    decode layer (one grouped GEMV launch), config 0 (M = 16 small-M kernel)
    and a plain device copy of COPY_PROBE_BYTES (the reference that scales
    FETCH_SIZE / WRITE_SIZE to bytes), with no warm-up loops."""
    xs, ys, dxs, dys = {}, {}, {}, {}
    for idx, (name, fmt, N, K) in enumerate(synthetic.LAYER_PROJECTIONS):
        xs[name] = torch.from_numpy(synthetic.activations(M_PREFILL, K, seed=synthetic.act_seed(2, 0, idx),
                                                          unit_rms=True)).cuda()
        ys[name] = torch.empty((M_PREFILL, N), dtype=torch.float32, device="cuda")
        dxs[name] = torch.from_numpy(synthetic.activations(1, K, seed=synthetic.act_seed(1, 0, idx))).cuda()
        dys[name] = torch.empty((1, N), dtype=torch.float32, device="cuda")
    pre = [layer_problems(torch, dmq, 2, layer, M_PREFILL, xs, ys) for layer in range(ROTATE_LAYERS)]
    dec = [layer_problems(torch, dmq, 1, layer, 1, dxs, dys) for layer in range(DECODE_ROTATE)]
    M, N, K = 16, 3072, 3072
    x0 = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(0, 0, 0))).cuda()
    w0 = [torch.from_numpy(synthetic.q4k_blocks(N, K, seed=synthetic.weight_seed(0, layer, 0)).reshape(-1)).cuda()
          for layer in range(8)]
    y0 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for i in range(reps):
        dmq.dmq_gemm_group(pre[i % len(pre)][0])
    for i in range(reps):
        dmq.dmq_gemm_group(dec[i % len(dec)][0])
    for i in range(reps):
        dmq.dmq_gemm_q4k(x0, w0[i % len(w0)], y0, M, N, K)
    torch.cuda.synchronize()
    src = torch.randint(0, 255, (COPY_PROBE_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counters_workload": {"reps": reps, "copy_bytes": COPY_PROBE_BYTES}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=1024, help="rows of the CPU-oracle sample (0: skip)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain copy of known size (counter calibration) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="only measure the other configurations (M=16, FFN, M sweep, LM head, layer chain) and exit")
    ap.add_argument("--sweep-part", choices=SWEEP_PARTS, action="append",
                    help="with --sweep: only these parts (repeatable)")
    ap.add_argument("--layer", action="store_true",
                    help="only time whole decoder layers (decode step and prefill) through the library and exit")
    ap.add_argument("--counters", action="store_true",
                    help="only run a few launches of each hot kernel and a calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--vendor-gemm-probe", action="store_true",
                    help="only time dense fp16 torch.matmul on the layer shapes (reference) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dequant_gemm_q4_amd as dmq
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.vendor_gemm_probe:
        vendor_gemm_probe(torch)
        return
    if args.counters:
        counters_workload(torch, dmq)
        return
    if args.sweep:
        sweep(torch, dmq, tuple(args.sweep_part) if args.sweep_part else SWEEP_PARTS)
        return
    if args.layer:
        layer_chain_sweep(torch, dmq)
        layer_overlap_sweep(torch, dmq)
        return
    M = M_PREFILL

    # activations and outputs (shared by the rotating layers), weights per layer
    xs, ys = {}, {}
    for idx, (name, fmt, N, K) in enumerate(synthetic.LAYER_PROJECTIONS):
        xs[name] = torch.from_numpy(synthetic.activations(M, K, seed=synthetic.act_seed(2, 0, idx),
                                                          unit_rms=True)).cuda()
        ys[name] = torch.empty((M, N), dtype=torch.float32, device="cuda")
    # keep (descriptor array, tensors) pairs: the arrays hold raw device pointers
    layers = [layer_problems(torch, dmq, 2, layer, M, xs, ys) for layer in range(ROTATE_LAYERS)]
    groups = [g for g, _ in layers]
    total_ms, per, warm = time_launches(torch, dmq.dmq_gemm_group, groups, args.steps, args.warmup)
    flops = flops_of(M)
    value = flops * args.steps / (total_ms / 1e3) / 1e12
    kern_ms = float(np.mean(per))
    achieved = flops / (kern_ms / 1e3) / 1e12

    out = {
        "metric": "prefill TFLOP/s of fused Q4_K dequant-GEMM at M=1024 (% FP16 MFMA peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        # the untimed warm-up actually run: at least `warmup` steps and SETTLE_MS
        # of GPU time; first_ms_per_step is its first 25 steps, from an idle GPU
        "warmup_run": warm,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.2-3B decoder layer prefill: 7 projection GEMMs (Q/K/V/O/gate/up Q4_K, "
                               "down Q6_K) at M=1024 in one grouped launch, weights rotated over 5 layers",
                   "M": M, "flop_per_step": flops, "weight_bytes_per_step": weight_bytes(),
                   "pct_fp16_peak": round(100.0 * value / PEAK_FP16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": (TRAFFIC["bytes_per_launch"] if TRAFFIC["sources_sha256"] == sources_sha256() else None),
                     "kernel": "dmq::gemm_kernel<3,8,2,false,8> (grouped Q4_K/Q6_K prefill launch) + "
                               "dmq::splitk_reduce_kernel (piece-order sum of the split down projection)",
                     "launch_ms": round(kern_ms, 4)},
        # per-step times (events around each of the K timed steps): the pages'
        # protocol reports medians and 95th percentiles over repeated runs
        "step_ms": stats(per),
        "device": device_record(torch),
        "seeds": {"weights": "1000003*config + 1009*layer + projection (0..6 = q,k,v,o,gate,up,down)",
                  "activations": "weight seed + 500000000", "config": 2, "layers": list(range(ROTATE_LAYERS)),
                  "generator": "numpy PCG64"},
    }
    # achieved graphics clock and socket power, sampled while the same step
    # runs again (untimed)
    it = [0]

    def again():
        dmq.dmq_gemm_group(groups[it[0] % len(groups)])
        it[0] += 1
    out["sclk_during_step"] = ClockSampler(torch).run_while(again)

    if not args.no_decode:
        dxs, dys = {}, {}
        for idx, (name, fmt, N, K) in enumerate(synthetic.LAYER_PROJECTIONS):
            dxs[name] = torch.from_numpy(synthetic.activations(1, K, seed=synthetic.act_seed(1, 0, idx))).cuda()
            dys[name] = torch.empty((1, N), dtype=torch.float32, device="cuda")
        del groups, layers
        dlayers = [layer_problems(torch, dmq, 1, layer, 1, dxs, dys) for layer in range(DECODE_ROTATE)]
        dgroups = [g for g, _ in dlayers]
        dsteps = max(args.steps, 50)
        d_total, d_per, _ = time_launches(torch, dmq.dmq_gemm_group, dgroups, dsteps, args.warmup)
        wb = weight_bytes()
        d_ms = float(np.mean(d_per))
        # a decode loop replays its launches from a graph: time that too, 20
        # replays of the 8 rotating layers, each replay between its own events
        g_per = time_graph(torch, dmq.dmq_gemm_group, dgroups, 20, per_replay=True)
        g_ms = float(np.median(g_per))
        # the cost of a launch itself: a one-wave kernel (torch's spin kernel,
        # one cycle) launched back to back on the same stream, no events
        # between the launches; every decode launch carries this much
        for _ in range(50):
            torch.cuda._sleep(1)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(dsteps):
            torch.cuda._sleep(1)
        f1.record()
        f1.synchronize()
        floor_us = 1e3 * f0.elapsed_time(f1) / dsteps
        out["decode"] = {"workload": "M=1, one layer's 7 projections in one grouped launch, 8 rotating layers",
                         "us_per_layer": round(1e3 * d_total / dsteps, 2),
                         "launch_floor_us": round(floor_us, 2),
                         "GB/s": round(wb / (d_total / dsteps / 1e3) / 1e9, 1),
                         "kernel_GB/s": round(wb / (d_ms / 1e3) / 1e9, 1),
                         "kernel_ms": stats(d_per),
                         "graph_us_per_layer": round(1e3 * g_ms, 2),
                         "graph_GB/s": round(wb / (g_ms / 1e3) / 1e9, 1),
                         "graph_ms_per_layer": stats(g_per),
                         # launches back to back on one stream, no events between them
                         "frac_hbm": round(wb / (d_total / dsteps / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                         "seeds": {"config": 1, "layers": list(range(DECODE_ROTATE))}}

    if args.cpu_rows > 0:
        out["cpu_baseline"] = cpu_baseline(args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
