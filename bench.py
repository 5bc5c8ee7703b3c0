"""Benchmark of the MXSens hot path on one MI355X.

Headline (default): one step = one Llama-2-70B block (one of the 80), every
stage of the path on synthetic, seeded inputs resident in HBM before timing
starts: calibrate over 128 x 2048 tokens for each of the block's four layer
inputs (q/k/v share one, o, gate/up share one, down; 27.9 GB of bf16), score,
allocate (5/15/80 % 8/6/4-bit), quantize W for the seven weights (q 8192 x
8192, k and v 1024 x 8192, o 8192 x 8192, gate and up 28672 x 8192, down
8192 x 28672), quantize X and the mixed GEMM at M = 2048 for all seven, and
MXINT4 quantisation of K and V (2048 tokens x 8 heads x 128).

Prints one JSON line. `value` is the block's GEMM work (2 M N K summed over
the seven layers) over the block step time, in TOPS, with mxs_mixed_gemm
(int8 block sums for the 4-bit blocks, exact bf16 products for the 8- and
6-bit blocks). The step is timed twice: eagerly (every call from Python,
`eager`) and as one HIP graph of the step's calls, captured once and
replayed (`graph`); `value` and `ms_per_step` are the replay's when every
output of the replayed step equals the eager step's bit for bit, else the
eager step's. `stages` gives every stage's time per step, GB/s (and
TOPS) and fraction of its peak, from HIP events around every call on the
library's stream in the eager steps; `roofline` is for the stage with the
largest share of the step, `roofline_gemm` and `roofline_calibrate` for the
GEMM and calibration calls; `variant_mx`, `variant_fused` and
`variant_prepared` repeat the step with mxs_mixed_gemm_mx (fp6 block-scaled
MFMA prefill), mxs_mixed_gemm_fused (X quantized inside the product) and
mxs_prepare_weights + mxs_mixed_gemm_prepared (W's operand built once per
weight, a prepare_w stage). `cpu_baseline` is the
CPU oracle on a bounded sample of the step, extrapolated (all host cores,
and one core in a child process). Extra keys: `q_proj_step` (the Llama-3-8B
q_proj-shaped layer step), `mlp_gemm` (Llama-3-8B MLP GEMMs at 4096 tokens),
`decode` (70B MLP decode GEMMs at 1, 8 and 32 tokens, cache-cold) and
`mixed_vs_uniform` (mixed_gemm under the all-4-bit and the 5/15/80 % maps,
q_proj prefill and 70B up-projection decode, warm and cold).

`roofline.traffic` comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counters
stored in profiles/ and is reported only while the kernel source is
unchanged since they were taken.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]
       python bench.py --workload q_proj   (the Llama-3-8B q_proj layer step alone)
       python bench.py --copy-probe   (a plain device copy of known size, to
                                       scale the HBM byte counters)
       python bench.py --overhead     (mixed_gemm under the all-4-bit, 4.03-bit,
                                       binary 4/8 and 5/15/80 % maps, prefill and
                                       decode: one JSON line per map)
       python bench.py --layerwise    (layer sensitivities and the layer-wise budget
                                       for the seven linear layers of a 70B block)
       python bench.py --attention    (one query token over the MXINT4 K/V cache,
                                       70B heads, 2048 / 8192 / 32768 tokens)
       python bench.py --decode       (decode-shape GEMMs of the 70B MLP at 1, 8
                                       and 32 tokens: one JSON line per case)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
INT8_PEAK = 5.0e15         # OP/s, MI355X dense int8 MFMA
FP6_PEAK = 10.1e15         # FLOP/s, MI355X dense fp6 / fp4 MFMA (the prefill GEMM's instruction)


GEMM_SOURCE = os.path.join(ROOT, "bit_gemm_hdiag_amd", "csrc", "mxs_gemm.hip")
GEMM_TRAFFIC = os.path.join(ROOT, "profiles", "mixed_gemm_q_proj_2048x4096x4096.traffic.txt")
COPY_BYTES = 1 << 29


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(key="traffic_bytes_per_call"):
    """HBM bytes per q_proj mixed_gemm call (key traffic_bytes_per_call_mx:
    per mixed_gemm_mx call) from the stored counter summary, or None when the
    summary is missing or the GEMM source changed since it was taken."""
    return stored_traffic(GEMM_TRAFFIC, key, GEMM_SOURCE)


def copy_probe(torch):
    """A plain device-to-device copy of COPY_BYTES, for counter scaling."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": COPY_BYTES, "dispatches": 3}), flush=True)


def decode_cases(mx, synth, torch, reps=20):
    """70B MLP decode GEMMs (up 28672 x 8192, down 8192 x 28672, 5/15/80 %) at
    1, 8 and 32 tokens: one dict per case."""
    out = []
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[4]
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    for li, lay in enumerate(cfg["layers"]):
        N, K = lay["N"], lay["K"]
        bp8, bp6 = lay["budget"]
        seed = 4000 + 100 * li
        gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
        Wt = synth.weights(N, K, seed + synth.ROLE_W, device=dev)
        n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
        perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(dev)
        Wq = mx.mxs_quantize(Wt, perm, n8, n6, n4)
        del Wt
        wbytes = N * (32 * n8 + 24 * n6 + 16 * n4 + K // 32)
        for M in cfg["Ms"]:
            X = synth.activations(M, K, seed + synth.ROLE_X, gains, device=dev)
            Aq = mx.mxs_quantize(X, perm, n8, n6, n4)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ws = torch.empty(max(1, mx.mxs_mixed_gemm_workspace(Aq, Wq)), dtype=torch.uint8, device=dev)
            fn = lambda: mx.mxs_mixed_gemm(Aq, Wq, Y, ws=ws)
            tc = time_cold(torch, fn, reps, flush)
            tg = time_graph(torch, fn, reps)
            out.append({"case": f"decode {lay['name']} {N}x{K}", "tokens": M, "us": tc * 1e6,
                        "warm_graph_us": tg * 1e6, "w_bytes": wbytes, "GBps": wbytes / tc / 1e9,
                        "hbm_frac": wbytes / tc / HBM_PEAK, "warm_hbm_frac": wbytes / tg / HBM_PEAK})
            log(json.dumps(out[-1]))
            del X, Aq, Y, ws
        del Wq
    return out


def overhead_cases(mx, synth, torch, reps=20, brief=False):
    """Cost of the mixed map against uniform MXINT4: mixed_gemm on the same
    layer under the all-4-bit map, the 4.03-bit map (one 8-bit block), the
    binary 4/8 map of the same 8-bit share (5 %), and the 5/15/80 % map, for
    the q_proj prefill (2048 x 4096 x 4096) and the 70B up-projection decode
    (1 token, 28672 x 8192). brief: only the all-4-bit and 5/15/80 % maps and
    mxs_mixed_gemm, returned instead of printed."""
    dev = torch.device("cuda:0")
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    rows = []
    for case, M, N, K, seed in (("prefill q_proj", 2048, 4096, 4096, 5000), ("decode 70B up", 1, 28672, 8192, 5100)):
        nb = K // 32
        gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
        W = synth.weights(N, K, seed + synth.ROLE_W, device=dev)
        X = synth.activations(M, K, seed + synth.ROLE_X, gains, device=dev)
        perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(dev)
        base = None
        maps = (("uniform 4-bit", (0, 0)), ("one 8-bit block", ((10000 + nb - 1) // nb, 0)),
                ("binary 4/8 (5 % 8-bit)", (500, 0)), ("5/15/80 %", (500, 1500)))
        if brief:
            maps = (maps[0], maps[3])
        for name, (bp8, bp6) in maps:
            n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
            Wq = mx.mxs_quantize(W, perm, n8, n6, n4)
            Aq = mx.mxs_quantize(X, perm, n8, n6, n4)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            out = {"case": case, "map": name, "blocks": [n8, n6, n4], "avg_bits": (8 * n8 + 6 * n6 + 4 * n4) / nb}
            for entry in ("mxs_mixed_gemm",) if brief else ("mxs_mixed_gemm", "mxs_mixed_gemm_mx"):
                wsf = getattr(mx, entry + "_workspace")
                ws = torch.empty(max(1, wsf(Aq, Wq)), dtype=torch.uint8, device=dev)
                f = getattr(mx, entry)
                fn = lambda: f(Aq, Wq, Y, ws=ws)
                out[entry + "_us"] = time_graph(torch, fn, reps) * 1e6
                out[entry + "_cold_us"] = time_cold(torch, fn, reps, flush) * 1e6
            if base is None:
                base = out
            for k in ("mxs_mixed_gemm_us", "mxs_mixed_gemm_mx_us", "mxs_mixed_gemm_cold_us"):
                if k in out:
                    out[k.replace("_us", "_vs_uniform")] = out[k] / base[k]
            if brief:
                rows.append(out)
            else:
                print(json.dumps(out), flush=True)
            del Wq, Aq, Y
        del W, X
    return rows


FP32_MFMA_PEAK = 157.3e12   # FLOP/s, MI355X dense fp32 matrix


def layerwise_cases(mx, synth, torch, T=256, B=4.5, reps=10):
    """Layer-wise allocation for the seven linear layers of one 70B block:
    each layer's sensitivity S (uniform-MXINT4 output error on T calibration
    tokens: two quantize calls, the mixed GEMM and mxs_output_error), then
    mxs_layer_budget at average width B. The output-error kernel is timed
    against the fp32 matrix-core peak (2 T N K flops of the dense product)."""
    dev = torch.device("cuda:0")
    layers = [("q_proj", 8192, 8192), ("k_proj", 1024, 8192), ("v_proj", 1024, 8192), ("o_proj", 8192, 8192),
              ("gate_proj", 28672, 8192), ("up_proj", 28672, 8192), ("down_proj", 8192, 28672)]
    S, rows, Ks = [], [], []
    for i, (name, N, K) in enumerate(layers):
        seed = 6000 + 16 * i
        inp = {"q_proj": 0, "k_proj": 0, "v_proj": 0, "o_proj": 1, "gate_proj": 2, "up_proj": 2, "down_proj": 3}[name]
        gains = synth.outlier_gains(K, 6000 + 16 * inp + synth.ROLE_CHANNELS)
        X = synth.activations(T, K, 6000 + 16 * inp + synth.ROLE_CALIB, gains, device=dev)
        W = synth.weights(N, K, seed + synth.ROLE_W, device=dev)
        nb = K // 32
        A4 = mx.qmat_alloc(T, K, 0, 0, nb, dev)
        W4 = mx.qmat_alloc(N, K, 0, 0, nb, dev)
        Yq = torch.empty((T, N), dtype=torch.float32, device=dev)
        ws_g = torch.empty(max(1, mx.mxs_mixed_gemm_workspace(A4, W4)), dtype=torch.uint8, device=dev)
        err = torch.empty(1, dtype=torch.float64, device=dev)
        ws_e = torch.empty(mx.mxs_output_error_workspace(T, N), dtype=torch.uint8, device=dev)

        def pipeline():
            mx.mxs_quantize(X, None, 0, 0, nb, out=A4)
            mx.mxs_quantize(W, None, 0, 0, nb, out=W4)
            mx.mxs_mixed_gemm(A4, W4, Yq, ws=ws_g)
            mx.mxs_output_error(X, W, Yq, err=err, ws=ws_e)

        pipeline()
        s_l = err.cpu().item()
        t_err = time_graph(torch, lambda: mx.mxs_output_error(X, W, Yq, err=err, ws=ws_e), reps)
        t_all = time_graph(torch, pipeline, reps)
        flops = 2 * T * N * K
        S.append(s_l); rows.append(N); Ks.append(K)
        print(json.dumps({"case": "layerwise 70B block", "layer": name, "N": N, "K": K, "tokens": T, "S": s_l,
                          "output_error_us": t_err * 1e6, "output_error_TFLOPs": flops / t_err / 1e12,
                          "fp32_mfma_frac": flops / t_err / FP32_MFMA_PEAK, "sensitivity_us": t_all * 1e6}),
              flush=True)
        del X, W, A4, W4, Yq
    t0 = time.perf_counter()
    blocks, R = mx.mxs_layer_budget(S, rows, Ks, B)
    t_budget = time.perf_counter() - t0
    bits = sum(r * 32 * (8 * b[0] + 6 * b[1] + 4 * b[2]) for r, b in zip(rows, blocks))
    print(json.dumps({"case": "layerwise 70B block budget", "B": B, "R": R, "blocks": blocks,
                      "avg_bits": bits / sum(r * k for r, k in zip(rows, Ks)), "host_us": t_budget * 1e6}),
          flush=True)


def attention_cases(mx, synth, torch, reps=20):
    """Attention of one query token over the MXINT4 K/V cache, Llama-2-70B
    heads (64 query heads on 8 KV heads, head dimension 128), at 2048, 8192
    and 32768 cached tokens: bytes = the K and V codes and scales, read once."""
    dev = torch.device("cuda:0")
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    Hq, Hkv, D = 64, 8, 128
    for T in (2048, 8192, 32768):
        seed = 9000 + T
        kc, ks = mx.mxs_quantize_kv(synth.kv(T, Hkv, D, seed, device=dev))
        vc, vs = mx.mxs_quantize_kv(synth.kv(T, Hkv, D, seed + 1, device=dev))
        q = torch.randn(Hq, D, generator=torch.Generator().manual_seed(seed)).to(dev)
        out = torch.empty(Hq, D, dtype=torch.float32, device=dev)
        ws = torch.empty(mx.mxs_attend_kv4_workspace(T, Hq, Hkv, D), dtype=torch.uint8, device=dev)
        fn = lambda: mx.mxs_attend_kv4(q, (kc, ks), (vc, vs), D ** -0.5, out=out, ws=ws)
        tc = time_cold(torch, fn, reps, flush)
        tg = time_graph(torch, fn, reps)
        nbytes = 2 * T * Hkv * (D // 2 + D // 32)
        print(json.dumps({"case": "attention over MXINT4 K/V, 70B heads 64/8 x 128", "tokens": T,
                          "kv_bytes": nbytes, "us": tc * 1e6, "warm_graph_us": tg * 1e6,
                          "GBps": nbytes / tc / 1e9, "hbm_frac": nbytes / tc / HBM_PEAK,
                          "warm_hbm_frac": nbytes / tg / HBM_PEAK}), flush=True)


def build_workload(mx, synth, torch, dev):
    cfg = synth.CONFIGS[2]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    bp8, bp6 = cfg["budget"]
    seed = 2000
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    w = dict(
        M=M, N=N, K=K, bp8=bp8, bp6=bp6, calib_rows=cfg["calib_rows"], kv_shape=cfg["kv"],
        Xc=synth.activations(cfg["calib_rows"], K, seed + synth.ROLE_CALIB, gains, device=dev),
        X=synth.activations(M, K, seed + synth.ROLE_X, gains, device=dev),
        W=synth.weights(N, K, seed + synth.ROLE_W, device=dev),
        Kc=synth.kv(cfg["kv"]["T"], cfg["kv"]["H"], cfg["kv"]["D"], seed + synth.ROLE_KV, device=dev),
        Vc=synth.kv(cfg["kv"]["T"], cfg["kv"]["H"], cfg["kv"]["D"], seed + synth.ROLE_KV + 8, device=dev),
    )
    n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
    w["blocks"] = (n8, n6, n4)
    u8 = dict(dtype=torch.uint8, device=dev)
    w["hdiag"] = torch.zeros(K, dtype=torch.float64, device=dev)
    w["score"] = torch.empty(K, dtype=torch.float64, device=dev)
    w["bits"] = torch.empty(K, **u8)
    w["perm"] = torch.empty(K, dtype=torch.int32, device=dev)
    w["ws_cal"] = torch.empty(max(1, mx.mxs_calibrate_workspace(w["calib_rows"], K)), **u8)
    w["ws_sc"] = torch.empty(max(1, mx.mxs_score_workspace(N, K)), **u8)
    w["Aq"] = mx.qmat_alloc(M, K, n8, n6, n4, dev)
    w["Wq"] = mx.qmat_alloc(N, K, n8, n6, n4, dev)
    w["Y"] = torch.empty((M, N), dtype=torch.float32, device=dev)
    w["ws_g"] = torch.empty(max(1, mx.mxs_mixed_gemm_workspace(w["Aq"], w["Wq"])), **u8)
    w["ws_gx"] = torch.empty(max(1, mx.mxs_mixed_gemm_mx_workspace(w["Aq"], w["Wq"])), **u8)
    w["ws_gf"] = torch.empty(max(1, mx.mxs_mixed_gemm_fused_workspace(M, w["X"].dtype, w["Wq"])), **u8)
    T, H, D = cfg["kv"]["T"], cfg["kv"]["H"], cfg["kv"]["D"]
    w["kc"] = [torch.empty((T, H, D // 2), **u8) for _ in range(2)]
    w["ks"] = [torch.empty((T, H, D // 32), **u8) for _ in range(2)]
    return w


def stage_fns(mx, w, variant=None):
    """The step's stages; variant "mx": the GEMM stage is mixed_gemm_mx;
    variant "fused": quantize_x and the GEMM are one mixed_gemm_fused call."""
    n8, n6, n4 = w["blocks"]
    if variant == "mx":
        gemm = lambda: mx.mxs_mixed_gemm_mx(w["Aq"], w["Wq"], w["Y"], ws=w["ws_gx"])
    elif variant == "fused":
        gemm = lambda: mx.mxs_mixed_gemm_fused(w["X"], w["perm"], w["Wq"], w["Y"], ws=w["ws_gf"])
    else:
        gemm = lambda: mx.mxs_mixed_gemm(w["Aq"], w["Wq"], w["Y"], ws=w["ws_g"])
    stages = [
        ("calibrate", lambda: (w["hdiag"].zero_(), mx.mxs_calibrate(w["Xc"], w["hdiag"], ws=w["ws_cal"]))),
        ("score", lambda: mx.mxs_score(w["W"], w["hdiag"], w["score"], ws=w["ws_sc"])),
        ("allocate", lambda: mx.mxs_allocate(w["score"], w["bp8"], w["bp6"], w["bits"], w["perm"])),
        ("quantize_w", lambda: mx.mxs_quantize(w["W"], w["perm"], n8, n6, n4, out=w["Wq"])),
        ("quantize_x", lambda: mx.mxs_quantize(w["X"], w["perm"], n8, n6, n4, out=w["Aq"])),
        ("mixed_gemm", gemm),
        ("quantize_kv", lambda: (mx.mxs_quantize_kv(w["Kc"], w["kc"][0], w["ks"][0]),
                                 mx.mxs_quantize_kv(w["Vc"], w["kc"][1], w["ks"][1]))),
    ]
    return [st for st in stages if not (variant == "fused" and st[0] == "quantize_x")]


def algorithmic_work(w):
    """Bytes (or ops) each stage must move (or do) by definition."""
    M, N, K = w["M"], w["N"], w["K"]
    n8, n6, n4 = w["blocks"]
    nb = K // 32
    packed = 32 * n8 + 24 * n6 + 16 * n4 + nb          # bytes per quantised row
    T, H, D = w["kv_shape"]["T"], w["kv_shape"]["H"], w["kv_shape"]["D"]
    return {
        "calibrate": dict(bytes=w["calib_rows"] * K * 2 + 16 * K),
        "score": dict(bytes=N * K * 2 + 24 * K),
        "allocate": dict(bytes=K * 8 + K * 5),
        "quantize_w": dict(bytes=N * K * 2 + N * packed + 4 * K),
        "quantize_x": dict(bytes=M * K * 2 + M * packed + 4 * K),
        "mixed_gemm": dict(ops=2 * M * N * K, bytes=(M + N) * packed + 4 * M * N),
        "quantize_kv": dict(bytes=2 * T * H * D * (2 + 0.5 + 1 / 32)),
    }


def time_stage(torch, fn, reps):
    for _ in range(3):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps * 1e-3


FLUSH_BYTES = 512 << 20   # more than the 256 MB Infinity Cache in front of HBM


def time_cold(torch, fn, reps, flush):
    """Median time of single calls, each after a read pass over a buffer
    larger than the Infinity Cache, so the call's inputs come from HBM rather
    than from the cache that repeated calls would leave warm. The pass only
    reads, so the cache holds no dirty lines that the call would have to
    write back."""
    fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        torch.amax(flush)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2] * 1e-3


def time_graph(torch, fn, reps):
    """Mean time per call of reps back-to-back calls replayed from one HIP
    graph: the device time of the calls without the Python launch path."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (2 * reps) * 1e-3


def cpu_baseline(w, torch, min_seconds=10.0, max_reps=20):
    """The CPU oracle over the whole step (every stage, every row), repeated
    until about min_seconds of CPU work; the mean step time gives the rate."""
    import oracle
    oracle.build()
    K, N, M = w["K"], w["N"], w["M"]
    n8, n6, n4 = w["blocks"]
    Xc = w["Xc"].float().cpu().numpy()
    Wh = w["W"].float().cpu().numpy()
    Xh = w["X"].float().cpu().numpy()
    kv = [w["Kc"].float().cpu().numpy(), w["Vc"].float().cpu().numpy()]
    tot = {}
    reps = 0
    t_all = time.perf_counter()
    while reps < max_reps and (reps == 0 or time.perf_counter() - t_all < min_seconds):
        t = {}
        t0 = time.perf_counter(); h = oracle.calibrate(Xc); t["calibrate"] = time.perf_counter() - t0
        t0 = time.perf_counter(); s = oracle.score(Wh, h); t["score"] = time.perf_counter() - t0
        t0 = time.perf_counter(); bits, perm = oracle.allocate(s, w["bp8"], w["bp6"]); t["allocate"] = time.perf_counter() - t0
        t0 = time.perf_counter(); Wq = oracle.quantize(Wh, perm, n8, n6, n4); t["quantize_w"] = time.perf_counter() - t0
        t0 = time.perf_counter(); Aq = oracle.quantize(Xh, perm, n8, n6, n4); t["quantize_x"] = time.perf_counter() - t0
        t0 = time.perf_counter(); oracle.mixed_gemm(Aq, Wq); t["mixed_gemm"] = time.perf_counter() - t0
        t0 = time.perf_counter(); [oracle.quantize_kv(x) for x in kv]; t["quantize_kv"] = time.perf_counter() - t0
        for k, v in t.items():
            tot[k] = tot.get(k, 0.0) + v
        reps += 1
    stage = {k: v / reps for k, v in tot.items()}
    step = sum(stage.values())
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=2 * M * N * K / step / 1e12, unit="TOPS", cores=cores, kind="oracle",
                sample=f"the whole step (every stage, all {M} token rows) run {reps} times back to back, "
                       f"{time.perf_counter() - t_all:.1f} s of CPU work in total; value from the mean step",
                step_s=step, stage_s=stage)


# ----------------------------------------------------------------------------
# The Llama-2-70B block step (the headline workload)
BLOCK_INPUT_K = {0: 8192, 1: 8192, 2: 8192, 3: 28672}   # q/k/v, o, gate/up, down inputs
BLOCK_INPUT_OF = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}


def packed_row_bytes(K, blocks):
    n8, n6, n4 = blocks
    return 32 * n8 + 24 * n6 + 16 * n4 + K // 32


def block_workload(mx, synth, torch, dev):
    """Every input of one 70B block resident in HBM: the four layer inputs'
    calibration tokens (128 x 2048 each) and prefill tokens (2048), the seven
    bf16 weights, K and V of 2048 x 8 x 128, and every output buffer."""
    cfg = synth.CONFIGS[5]
    M, T = cfg["M"], cfg["calib_rows"]
    bp8, bp6 = cfg["budget"]
    u8 = dict(dtype=torch.uint8, device=dev)
    w = dict(M=M, T=T, bp8=bp8, bp6=bp6, inputs={}, layers=[])
    for inp, K in BLOCK_INPUT_K.items():
        seed = 5000 + 16 * inp
        gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
        log(f"input {inp}: calibration {T} x {K} bf16")
        w["inputs"][inp] = dict(
            K=K, Xc=synth.activations(T, K, seed + synth.ROLE_CALIB, gains, device=dev),
            X=synth.activations(M, K, seed + synth.ROLE_X, gains, device=dev),
            hdiag=torch.zeros(K, dtype=torch.float64, device=dev),
            ws=torch.empty(max(1, mx.mxs_calibrate_workspace(T, K)), **u8))
    for li, lay in enumerate(cfg["layers"]):
        N, K = lay["N"], lay["K"]
        blocks = mx.mxs_budget_blocks(K, bp8, bp6)
        w["layers"].append(dict(
            name=lay["name"], N=N, K=K, inp=BLOCK_INPUT_OF[lay["name"]], blocks=blocks,
            W=synth.weights(N, K, 5500 + 16 * li + synth.ROLE_W, device=dev),
            score=torch.empty(K, dtype=torch.float64, device=dev), bits=torch.empty(K, **u8),
            perm=torch.empty(K, dtype=torch.int32, device=dev),
            ws_sc=torch.empty(max(1, mx.mxs_score_workspace(N, K)), **u8),
            Wq=mx.qmat_alloc(N, K, *blocks, dev), Aq=mx.qmat_alloc(M, K, *blocks, dev)))
        L = w["layers"][-1]
        L["wp"] = torch.empty(max(1, mx.mxs_prepare_weights_size(L["Wq"])), **u8)
    maxN = max(L["N"] for L in w["layers"])
    ybuf = torch.empty(M * maxN, dtype=torch.float32, device=dev)
    for L in w["layers"]:
        L["Y"] = ybuf[:M * L["N"]].view(M, L["N"])
    w["ws_g"] = torch.empty(max(max(mx.mxs_mixed_gemm_workspace(L["Aq"], L["Wq"]) for L in w["layers"]), 1), **u8)
    w["ws_gx"] = torch.empty(max(max(mx.mxs_mixed_gemm_mx_workspace(L["Aq"], L["Wq"]) for L in w["layers"]), 1), **u8)
    w["ws_gf"] = torch.empty(max(max(mx.mxs_mixed_gemm_fused_workspace(M, torch.bfloat16, L["Wq"])
                                     for L in w["layers"]), 1), **u8)
    w["ws_gp"] = torch.empty(max(max(mx.mxs_mixed_gemm_prepared_workspace(L["Aq"], L["Wq"]) for L in w["layers"]), 1),
                             **u8)
    # the layer's K and V stacked as one [2 T, H, D] tensor: one quantize_kv launch
    kv = cfg["kv"]
    w["kv_shape"] = kv
    w["KV"] = torch.cat([synth.kv(kv["T"], kv["H"], kv["D"], 5000 + synth.ROLE_KV, device=dev),
                         synth.kv(kv["T"], kv["H"], kv["D"], 5000 + synth.ROLE_KV + 8, device=dev)])
    w["kvc"] = torch.empty((2 * kv["T"], kv["H"], kv["D"] // 2), **u8)
    w["kvs"] = torch.empty((2 * kv["T"], kv["H"], kv["D"] // 32), **u8)
    return w


def block_calls(mx, w, variant=None):
    """One block step as (stage, label, fn, work) in stream order; work is the
    call's algorithmic bytes (and ops for the GEMM). By default the GEMMs are
    mxs_mixed_gemm (both operands prepared inside every call). variant
    "prepared": each weight's prefill operand is built once after its
    quantisation (a prepare_w stage) and the GEMMs are
    mxs_mixed_gemm_prepared; "fused": quantize_x + GEMM become one
    mxs_mixed_gemm_fused call per layer; "mx": the GEMMs are
    mxs_mixed_gemm_mx."""
    M, T = w["M"], w["T"]
    calls = []
    for inp, I in w["inputs"].items():
        K = I["K"]
        calls.append(("calibrate", f"input {inp}",
                      lambda I=I: (I["hdiag"].zero_(), mx.mxs_calibrate(I["Xc"], I["hdiag"], ws=I["ws"])),
                      dict(bytes=T * K * 2 + 16 * K)))
    for L in w["layers"]:
        h = w["inputs"][L["inp"]]["hdiag"]
        calls.append(("score", L["name"], lambda L=L, h=h: mx.mxs_score(L["W"], h, L["score"], ws=L["ws_sc"]),
                      dict(bytes=L["N"] * L["K"] * 2 + 24 * L["K"])))
    for L in w["layers"]:
        calls.append(("allocate", L["name"],
                      lambda L=L: mx.mxs_allocate(L["score"], w["bp8"], w["bp6"], L["bits"], L["perm"]),
                      dict(bytes=13 * L["K"])))
    for L in w["layers"]:
        pr = packed_row_bytes(L["K"], L["blocks"])
        calls.append(("quantize_w", L["name"], lambda L=L: mx.mxs_quantize(L["W"], L["perm"], *L["blocks"], out=L["Wq"]),
                      dict(bytes=L["N"] * L["K"] * 2 + L["N"] * pr + 4 * L["K"])))
    if variant == "prepared":
        for L in w["layers"]:
            pr = packed_row_bytes(L["K"], L["blocks"])
            calls.append(("prepare_w", L["name"], lambda L=L: mx.mxs_prepare_weights(L["Wq"], out=L["wp"]),
                          dict(bytes=L["N"] * pr + mx.mxs_prepare_weights_size(L["Wq"]))))
    for L in w["layers"]:
        pr = packed_row_bytes(L["K"], L["blocks"])
        X = w["inputs"][L["inp"]]["X"]
        gemm_work = dict(ops=2 * M * L["N"] * L["K"], bytes=(M + L["N"]) * pr + 4 * M * L["N"])
        if variant == "fused":
            calls.append(("mixed_gemm", L["name"],
                          lambda L=L, X=X: mx.mxs_mixed_gemm_fused(X, L["perm"], L["Wq"], L["Y"], ws=w["ws_gf"]),
                          gemm_work))
            continue
        calls.append(("quantize_x", L["name"], lambda L=L, X=X: mx.mxs_quantize(X, L["perm"], *L["blocks"], out=L["Aq"]),
                      dict(bytes=M * L["K"] * 2 + M * pr + 4 * L["K"])))
        if variant == "mx":
            fn = lambda L=L: mx.mxs_mixed_gemm_mx(L["Aq"], L["Wq"], L["Y"], ws=w["ws_gx"])
        elif variant == "prepared":
            fn = lambda L=L: mx.mxs_mixed_gemm_prepared(L["Aq"], L["Wq"], L["wp"], L["Y"], ws=w["ws_gp"])
        else:
            fn = lambda L=L: mx.mxs_mixed_gemm(L["Aq"], L["Wq"], L["Y"], ws=w["ws_g"])
        calls.append(("mixed_gemm", L["name"], fn, gemm_work))
    kv = w["kv_shape"]
    kvb = 2 * kv["T"] * kv["H"] * kv["D"] * (2 + 0.5 + 1 / 32)
    calls.append(("quantize_kv", "K and V", lambda: mx.mxs_quantize_kv(w["KV"], w["kvc"], w["kvs"]), dict(bytes=kvb)))
    return calls


def run_block_steps(torch, calls, steps, warmup):
    """warmup untimed steps, then `steps` timed steps between two
    synchronisations; every call is also bracketed by HIP events on the
    current stream (the stream the library launches on). Returns the step
    time and per-stage totals (seconds per step, work per step, calls)."""
    for _ in range(warmup):
        for _, _, fn, _ in calls:
            fn()
    torch.cuda.synchronize()
    ev = []
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        for stage, label, fn, work in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev.append((stage, label, a, b, work))
    e.record()
    torch.cuda.synchronize()
    step_s = s.elapsed_time(e) / steps * 1e-3
    stages = {}
    for stage, label, a, b, work in ev:
        d = stages.setdefault(stage, dict(s=0.0, bytes=0.0, ops=0.0, calls=0, by_call={}))
        t = a.elapsed_time(b) * 1e-3
        d["s"] += t / steps
        d["bytes"] += work.get("bytes", 0) / steps
        d["ops"] += work.get("ops", 0) / steps
        d["calls"] += 1
        d["by_call"][label] = d["by_call"].get(label, 0.0) + t / steps
    for d in stages.values():
        d["calls"] //= steps
    return step_s, stages


def run_block_graph(torch, calls, steps, warmup):
    """The same step captured once in a HIP graph and replayed: `warmup`
    untimed replays, then `steps` timed replays between two
    synchronisations. Every replay launches every kernel of the step; what
    it drops is the host's per-call work (Python, argument marshalling,
    launch calls), which leaves the GPU idle between short kernels."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, _, fn, _ in calls:
            fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    step_s = s.elapsed_time(e) / steps * 1e-3
    del g
    return step_s


def block_outputs(w):
    """Copies of everything a block step writes (Hdiag, scores, bit maps,
    permutations, planes, Y, K/V codes and scales)."""
    out = [I["hdiag"].clone() for I in w["inputs"].values()]
    for L in w["layers"]:
        out += [L["score"].clone(), L["bits"].clone(), L["perm"].clone(), L["Y"].clone()]
        for q in (L["Wq"], L["Aq"]):
            out += [t.clone() for t in (q.q8, q.q6, q.q4, q.sc) if t is not None]
    return out + [w["kvc"].clone(), w["kvs"].clone()]


def run_block_steps_concurrent(torch, calls, w, steps, warmup):
    """The same step with two streams (default priority): the four
    calibrations run in order on one, each layer's score, allocate,
    quantize and GEMM on the other as soon as its input's Hdiag is ready,
    so the HBM-bound calibration of an input overlaps the matrix-core work
    of the layers of the inputs before it. Steps join at their ends (the
    next step's calibration overwrites Hdiag). Returns the step time."""
    cal = {label: fn for stage, label, fn, _ in calls if stage == "calibrate"}
    per_layer = {}
    for stage, label, fn, _ in calls:
        if stage not in ("calibrate", "quantize_kv"):
            per_layer.setdefault(label, []).append(fn)
    kv = [fn for stage, _, fn, _ in calls if stage == "quantize_kv"]
    s_cal, s_lay = torch.cuda.Stream(), torch.cuda.Stream()

    def step():
        cur = torch.cuda.current_stream()
        s_cal.wait_stream(cur)
        s_lay.wait_stream(cur)
        ready = {}
        with torch.cuda.stream(s_cal):
            for inp in sorted(w["inputs"]):
                cal[f"input {inp}"]()
                ev = torch.cuda.Event()
                ev.record(s_cal)
                ready[inp] = ev
        with torch.cuda.stream(s_lay):
            waited = set()
            for L in w["layers"]:
                if L["inp"] not in waited:
                    s_lay.wait_event(ready[L["inp"]])
                    waited.add(L["inp"])
                for fn in per_layer[L["name"]]:
                    fn()
            for fn in kv:
                fn()
        cur.wait_stream(s_cal)
        cur.wait_stream(s_lay)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps * 1e-3


def stage_summary(stages):
    out = {}
    for name, d in stages.items():
        o = dict(ms=d["s"] * 1e3, calls=d["calls"], GBps=d["bytes"] / d["s"] / 1e9,
                 hbm_frac=d["bytes"] / d["s"] / HBM_PEAK,
                 us_by_call={k: v * 1e6 for k, v in d["by_call"].items()})
        if d["ops"]:
            o["TOPS"] = d["ops"] / d["s"] / 1e12
            o["int8_mfma_frac"] = d["ops"] / d["s"] / INT8_PEAK
        out[name] = o
    return out


def stored_traffic(path, key, source, sha_key="source_sha256"):
    """Bytes per call from a stored counter summary (key = value lines), or
    None when the summary is missing or `source` changed since it was taken
    (its hash no longer equals the summary's `sha_key`)."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get(sha_key) != sha:
            return None
        return float(kv[key])
    except (OSError, KeyError, ValueError):
        return None


BLOCK_TRAFFIC = os.path.join(ROOT, "profiles", "70b_block.traffic.txt")
COLSUM_SOURCE = os.path.join(ROOT, "bit_gemm_hdiag_amd", "csrc", "mxs_colsum.hip")


def roofline_of(stage, d, prepared=False):
    """Roofline object of one stage's calls: algorithmic work per call over
    the mean call duration (Σ work / Σ time over the timed calls). prepared:
    the GEMM calls are mxs_mixed_gemm_prepared (their own stored traffic)."""
    per_call_s = d["s"] / d["calls"]
    if d["ops"]:
        ach = d["ops"] / d["s"]
        key = "mixed_gemm_prepared_bytes_per_call" if prepared else "mixed_gemm_bytes_per_call"
        r = dict(bound="mfma", achieved=ach / 1e12, peak=INT8_PEAK / 1e12, unit="TOP/s", frac=ach / INT8_PEAK,
                 traffic=stored_traffic(BLOCK_TRAFFIC, key, GEMM_SOURCE),
                 algorithmic_ops_per_launch=d["ops"] / d["calls"])
    else:
        ach = d["bytes"] / d["s"]
        r = dict(bound="hbm", achieved=ach / 1e9, peak=HBM_PEAK / 1e9, unit="GB/s", frac=ach / HBM_PEAK,
                 traffic=(stored_traffic(BLOCK_TRAFFIC, "calibrate_bytes_per_call", COLSUM_SOURCE,
                                         "colsum_source_sha256") if stage == "calibrate" else None))
    r.update(stage=stage, launch_us=per_call_s * 1e6, algorithmic_bytes_per_launch=d["bytes"] / d["calls"],
             launches_per_step=d["calls"])
    return r


def mlp_gemms(mx, synth, torch, reps=10):
    """The Llama-3-8B MLP GEMMs at 4096 tokens (gate/up 14336 x 4096 at
    3/10/87 %, down 4096 x 14336 at 8/20/72 %), mxs_mixed_gemm,
    mxs_mixed_gemm_prepared (W prepared once, outside the timing) and
    mxs_mixed_gemm_mx, graph-replayed back to back (inputs of 60-240 MB).
    The channel map is the method's own: calibrate over 8 x 2048 tokens,
    score, allocate."""
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[3]
    M = cfg["M"]
    out = {}
    for li, lay in enumerate(cfg["layers"]):
        if lay["name"] == "up":
            continue          # the same shape and budget as gate
        N, K = lay["N"], lay["K"]
        seed = 3000 + 16 * li
        gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
        blocks = mx.mxs_budget_blocks(K, *lay["budget"])
        W = synth.weights(N, K, seed + synth.ROLE_W, device=dev)
        h = mx.mxs_calibrate(synth.activations(cfg["calib_rows"], K, seed + synth.ROLE_CALIB, gains, device=dev))
        _, perm = mx.mxs_allocate(mx.mxs_score(W, h), *lay["budget"])
        Wq = mx.mxs_quantize(W, perm, *blocks)
        del W
        Aq = mx.mxs_quantize(synth.activations(M, K, seed + synth.ROLE_X, gains, device=dev), perm, *blocks)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ops = 2 * M * N * K
        d = dict(shape=f"{M}x{N}x{K}", blocks=list(blocks))
        wp = mx.mxs_prepare_weights(Wq)
        for entry in ("mxs_mixed_gemm", "mxs_mixed_gemm_prepared", "mxs_mixed_gemm_mx"):
            ws = torch.empty(max(1, getattr(mx, entry + "_workspace")(Aq, Wq)), dtype=torch.uint8, device=dev)
            f = getattr(mx, entry)
            if entry == "mxs_mixed_gemm_prepared":
                t = time_graph(torch, lambda: f(Aq, Wq, wp, Y, ws=ws), reps)
            else:
                t = time_graph(torch, lambda: f(Aq, Wq, Y, ws=ws), reps)
            d[entry] = dict(us=t * 1e6, TOPS=ops / t / 1e12, int8_mfma_frac=ops / t / INT8_PEAK)
            del ws
        del wp
        out[lay["name"]] = d
        log("mlp", json.dumps(d))
        del Wq, Aq, Y
    return out


def block_cpu_sample(w, torch):
    """Host copies of a bounded sample of the block step for the CPU oracle,
    with the factor that scales each stage's sample to the whole step."""
    M, T = w["M"], w["T"]
    S = dict(calib=[], layers=[], kv=[], scale={})
    tc = 16384
    for inp, I in w["inputs"].items():
        S["calib"].append(I["Xc"][:tc].float().cpu().numpy())
    S["scale"]["calibrate"] = T / tc
    wr = 2                    # score and quantize W on 1/2 of every weight's rows
    xr = 2                    # quantize X on 1/2 of the tokens
    gr = 512                  # GEMM on 512 tokens against the sampled weight rows
    for L in w["layers"]:
        X = w["inputs"][L["inp"]]["X"]
        S["layers"].append(dict(name=L["name"], K=L["K"], blocks=L["blocks"],
                                inp_id=L["inp"], W=L["W"][:L["N"] // wr].float().cpu().numpy(),
                                X=X[:M // xr].float().cpu().numpy()))
    S["scale"].update(score=wr, quantize_w=wr, quantize_x=xr, mixed_gemm=(M / gr) * wr, allocate=1,
                      quantize_kv=1)
    S["gemm_rows"] = gr
    T = w["kv_shape"]["T"]
    S["kv"] = [w["KV"][:T].float().cpu().numpy(), w["KV"][T:].float().cpu().numpy()]
    S["bp"] = (w["bp8"], w["bp6"])
    return S


def oracle_stage_times(S, sub=1):
    """The CPU oracle over the sample S (each stage's rows cut by `sub` more),
    in the step's order; returns seconds per stage scaled to the whole step."""
    import numpy as np
    import oracle
    oracle.build()
    t = {}

    def timed(stage, f):
        t0 = time.perf_counter()
        r = f()
        t[stage] = t.get(stage, 0.0) + (time.perf_counter() - t0) * S["scale"][stage] * sub
        return r
    hd = [timed("calibrate", lambda X=X: oracle.calibrate(np.ascontiguousarray(X[:X.shape[0] // sub])))
          for X in S["calib"]]
    bp8, bp6 = S["bp"]
    for L in S["layers"]:
        W = np.ascontiguousarray(L["W"][:max(1, L["W"].shape[0] // sub)])
        X = np.ascontiguousarray(L["X"][:max(1, L["X"].shape[0] // sub)])
        sc = timed("score", lambda: oracle.score(W, hd[L["inp_id"]]))
        _, perm = timed("allocate", lambda: oracle.allocate(sc, bp8, bp6))
        Wq = timed("quantize_w", lambda: oracle.quantize(W, perm, *L["blocks"]))
        Aq = timed("quantize_x", lambda: oracle.quantize(X, perm, *L["blocks"]))
        g = max(1, S["gemm_rows"] // sub)
        Ag = {k: (v[:g] if isinstance(v, np.ndarray) else v) for k, v in Aq.items()}
        timed("mixed_gemm", lambda: oracle.mixed_gemm(Ag, Wq))
    for kv in S["kv"]:
        timed("quantize_kv", lambda kv=kv: oracle.quantize_kv(np.ascontiguousarray(kv[:max(1, kv.shape[0] // sub)])))
    return t


def save_sample(S, sub, path):
    """The sample as one .npz of arrays plus a JSON file of the rest."""
    import numpy as np
    arrays = {f"calib{i}": X for i, X in enumerate(S["calib"])}
    arrays.update({f"kv{i}": X for i, X in enumerate(S["kv"])})
    meta = dict(sub=sub, scale=S["scale"], gemm_rows=S["gemm_rows"], bp=list(S["bp"]), layers=[])
    for i, L in enumerate(S["layers"]):
        arrays[f"W{i}"], arrays[f"X{i}"] = L["W"], L["X"]
        meta["layers"].append(dict(name=L["name"], K=L["K"], blocks=list(L["blocks"]), inp_id=L["inp_id"]))
    np.savez(os.path.join(path, "sample.npz"), **arrays)
    with open(os.path.join(path, "sample.json"), "w") as f:
        json.dump(meta, f)


def load_sample(path):
    import numpy as np
    with open(os.path.join(path, "sample.json")) as f:
        meta = json.load(f)
    z = np.load(os.path.join(path, "sample.npz"))
    n_in = sum(1 for k in z.files if k.startswith("calib"))
    S = dict(calib=[z[f"calib{i}"] for i in range(n_in)], kv=[z["kv0"], z["kv1"]], scale=meta["scale"],
             gemm_rows=meta["gemm_rows"], bp=tuple(meta["bp"]), layers=[])
    for i, L in enumerate(meta["layers"]):
        S["layers"].append(dict(name=L["name"], K=L["K"], blocks=tuple(L["blocks"]), inp_id=L["inp_id"],
                                W=z[f"W{i}"], X=z[f"X{i}"]))
    return S, meta["sub"]


def oracle_child(path):
    """1-thread oracle timing in a child process (OMP_NUM_THREADS=1): loads the
    sample the parent saved and prints the scaled stage times."""
    S, sub = load_sample(path)
    print(json.dumps(oracle_stage_times(S, sub)), flush=True)


def block_cpu_baseline(w, torch, gemm_ops):
    """The CPU oracle on a bounded sample of the block step, on all host cores
    and on one core; stage times are extrapolated to the whole step."""
    import shutil
    import subprocess
    import tempfile
    S = block_cpu_sample(w, torch)
    t0 = time.perf_counter()
    t_all = oracle_stage_times(S)
    wall_all = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    step_all = sum(t_all.values())
    res = dict(value=gemm_ops / step_all / 1e12, unit="TOPS", cores=cores, kind="oracle",
               sample=(f"extrapolated: calibrate on 16384 of the 262144 tokens of each input (x16), score and "
                       f"quantize W on 1/2 of every weight's rows (x2), quantize X on 1024 of 2048 tokens (x2), "
                       f"the GEMM on 512 tokens x 1/2 of the weight rows (x8), K/V in full; "
                       f"{wall_all:.1f} s of CPU work on {cores} threads"),
               step_s=step_all, stage_s=t_all)
    sub = 8
    tmp = tempfile.mkdtemp(prefix="mxs_oracle_")
    try:
        save_sample(S, sub, tmp)
        env = dict(os.environ, OMP_NUM_THREADS="1")
        t0 = time.perf_counter()
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-child", tmp], env=env,
                           capture_output=True, text=True, timeout=600)
        wall_one = time.perf_counter() - t0
        if r.returncode == 0:
            t_one = json.loads(r.stdout.strip().splitlines()[-1])
            step_one = sum(t_one.values())
            res["one_core"] = dict(value=gemm_ops / step_one / 1e12, cores=1, step_s=step_one, stage_s=t_one,
                                   sample=f"the same sample cut 8x further (x8 more extrapolation), "
                                          f"{wall_one:.1f} s wall in a child process with OMP_NUM_THREADS=1")
        else:
            res["one_core"] = dict(error=r.stderr[-500:])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return res


def block_line(mx, synth, torch, args):
    """The headline: one Llama-2-70B block step per `step`."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("building the 70B block workload")
    w = block_workload(mx, synth, torch, dev)
    M = w["M"]
    gemm_ops = sum(2 * M * L["N"] * L["K"] for L in w["layers"])
    log(f"warmup {args.warmup}, timing {args.steps} block steps")
    calls = block_calls(mx, w, args.block_variant)
    eager_s, stages = run_block_steps(torch, calls, args.steps, args.warmup)
    log(f"block step {eager_s * 1e3:.3f} ms (eager)")
    ref = block_outputs(w)
    graph_s = run_block_graph(torch, calls, args.steps, args.warmup)
    same = all(torch.equal(a, b) for a, b in zip(ref, block_outputs(w)))
    del ref
    log(f"block step {graph_s * 1e3:.3f} ms (graph replay, outputs equal to the eager step: {same})")
    step_s = graph_s if same else eager_s
    dominant = max(stages, key=lambda k: stages[k]["s"])
    out = {
        "metric": "mixed MXINT GEMM TOPS & quantize GB/s, % of MI355X roofline (1 GPU)",
        "value": gemm_ops / step_s / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded outlier-channel activations, Student-t weights, bf16)",
        "config": {"workload": "Llama-2-70B block (one of 80): calibrate 128x2048 tokens for each of the 4 layer "
                               "inputs (K 8192 x3, 28672), score/allocate/quantize W for q 8192x8192, k and v "
                               "1024x8192, o 8192x8192, gate and up 28672x8192, down 8192x28672 (5/15/80% "
                               "8/6/4-bit), quantize X and mixed GEMM at M=2048 for all 7, MXINT4 K and V "
                               "2048x8x128; one step = one block",
                   "global_batch": M, "seq_len": M, "parallelism": "none (1 GPU)",
                   "pipeline_80_layers_s": step_s * 80, "gemm_variant": args.block_variant or "mxs_mixed_gemm",
                   "launch": "the step's calls captured once in a HIP graph and replayed" if same else "eager"},
        "gemm_ops_per_step": gemm_ops,
        "eager": dict(value=gemm_ops / eager_s / 1e12, ms_per_step=eager_s * 1e3),
        "graph": dict(value=gemm_ops / graph_s / 1e12, ms_per_step=graph_s * 1e3, outputs_equal_eager=same),
        "stages": stage_summary(stages),
        "roofline": roofline_of(dominant, stages[dominant]),
        "roofline_gemm": roofline_of("mixed_gemm", stages["mixed_gemm"], prepared=args.block_variant == "prepared"),
        "roofline_calibrate": roofline_of("calibrate", stages["calibrate"]),
    }
    if not args.no_extras:
        for variant, key, entry in (("mx", "variant_mx", "mxs_mixed_gemm_mx (fp6 block-scaled MFMA prefill)"),
                                    ("fused", "variant_fused", "mxs_mixed_gemm_fused (X quantized inside the "
                                                               "product; no quantize_x stage)"),
                                    ("prepared", "variant_prepared", "mxs_prepare_weights once per weight after "
                                                                     "its quantisation (prepare_w stage), then "
                                                                     "mxs_mixed_gemm_prepared")):
            log(f"the block step with {entry}")
            sv, st = run_block_steps(torch, block_calls(mx, w, variant), max(3, args.steps // 2), 2)
            g = st["mixed_gemm"]
            out[key] = dict(entry=entry, value=gemm_ops / sv / 1e12, ms_per_step=sv * 1e3,
                            gemm_ms_per_step=g["s"] * 1e3, gemm_TOPS=g["ops"] / g["s"] / 1e12,
                            int8_peak_frac=g["ops"] / g["s"] / INT8_PEAK,
                            fp6_peak_frac=g["ops"] / g["s"] / FP6_PEAK if variant == "mx" else None)
            if variant == "prepared":
                p = st["prepare_w"]
                out[key].update(prepare_w_ms_per_step=p["s"] * 1e3,
                                roofline_gemm=roofline_of("mixed_gemm", g, prepared=True))
        log("the block step on two streams (calibration beside the layers' work)")
        sc = run_block_steps_concurrent(torch, block_calls(mx, w), w, max(3, args.steps // 2), 2)
        out["variant_two_streams"] = dict(
            entry="the same calls (mxs_mixed_gemm) on two streams: calibrations in order on one, each layer's "
                  "score/allocate/quantize/GEMM on the other once its input's Hdiag is ready",
            value=gemm_ops / sc / 1e12, ms_per_step=sc * 1e3)
    if not args.no_cpu:
        log("cpu baseline (oracle, sampled)")
        out["cpu_baseline"] = block_cpu_baseline(w, torch, gemm_ops)
    del w
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("q_proj layer step (Llama-3-8B)")
        qa = argparse.Namespace(**vars(args))
        qa.no_cpu = True
        q = q_proj_line(mx, synth, torch, qa)
        out["q_proj_step"] = {k: q[k] for k in ("value", "ms_per_step", "gemm_tops", "quantize_gbps", "roofline",
                                                 "variant_mx", "variant_fused", "stages")}
        out["mlp_gemm"] = mlp_gemms(mx, synth, torch)
        out["decode"] = decode_cases(mx, synth, torch)
        log("mixed map against uniform MXINT4 (q_proj prefill, 70B up decode)")
        out["mixed_vs_uniform"] = overhead_cases(mx, synth, torch, reps=10, brief=True)
    return out


def q_proj_line(mx, synth, torch, args):
    """The q_proj-shaped layer step (2048 x 4096 x 4096) as one JSON object."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("building workload")
    w = build_workload(mx, synth, torch, dev)

    def run_steps(stages):
        """Warm up, then time args.steps whole steps; the GEMM call is also
        timed with events on its own inside every timed step."""
        gemm_ev = []

        def step(timed=False):
            for name, fn in stages:
                if timed and name == "mixed_gemm":
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn()
                    b.record()
                    gemm_ev.append((a, b))
                else:
                    fn()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            step(timed=True)
        e.record()
        torch.cuda.synchronize()
        step_s = s.elapsed_time(e) / args.steps * 1e-3
        gemm_s = sum(a.elapsed_time(b) for a, b in gemm_ev) / len(gemm_ev) * 1e-3
        return step_s, gemm_s

    stages = stage_fns(mx, w)
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    step_s, gemm_call_s = run_steps(stages)
    log(f"step {step_s * 1e3:.3f} ms, mixed_gemm call {gemm_call_s * 1e6:.1f} us")
    log("the same step with mixed_gemm_mx")
    step_x, gemm_x = run_steps(stage_fns(mx, w, variant="mx"))
    log(f"step {step_x * 1e3:.3f} ms, mixed_gemm_mx call {gemm_x * 1e6:.1f} us")
    log("the same step with mixed_gemm_fused (no quantize_x stage)")
    step_f, gemm_f = run_steps(stage_fns(mx, w, variant="fused"))
    log(f"step {step_f * 1e3:.3f} ms, mixed_gemm_fused call {gemm_f * 1e6:.1f} us")

    work = algorithmic_work(w)
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    stage_out = {}
    extra = [("mixed_gemm_mx", dict(stage_fns(mx, w, variant="mx"))["mixed_gemm"]),
             ("mixed_gemm_fused", dict(stage_fns(mx, w, variant="fused"))["mixed_gemm"])]
    for name, fn in stages + extra:
        t = time_cold(torch, fn, max(args.stage_reps, 9), flush)
        tw = time_stage(torch, fn, args.stage_reps)
        tg = time_graph(torch, fn, args.stage_reps)
        wk = work["mixed_gemm" if name in ("mixed_gemm_mx", "mixed_gemm_fused") else name]
        d = dict(ms=t * 1e3, warm_ms=tw * 1e3, warm_graph_ms=tg * 1e3)
        if "bytes" in wk:
            d["GBps"] = wk["bytes"] / t / 1e9
            d["hbm_frac"] = wk["bytes"] / t / HBM_PEAK
        if "ops" in wk:
            d["TOPS"] = wk["ops"] / t / 1e12
            d["int8_mfma_frac"] = wk["ops"] / t / INT8_PEAK
            if name == "mixed_gemm_mx":
                d["fp6_mfma_frac"] = wk["ops"] / t / FP6_PEAK
        stage_out[name] = d
        log(name, json.dumps(d))

    gemm = stage_out["mixed_gemm"]
    M, N, K = w["M"], w["N"], w["K"]
    ops = 2 * M * N * K
    achieved = ops / gemm_call_s / 1e12
    roofline = dict(bound="mfma", achieved=achieved, peak=INT8_PEAK / 1e12, unit="TOP/s",
                    frac=achieved * 1e12 / INT8_PEAK, traffic=measured_traffic(),
                    kernel="mixed_gemm call: k_gemm_prep + k_gemm_a2r (int8 MFMA for 4-bit blocks, bf16 MFMA for 8- and 6-bit blocks)",
                    algorithmic_ops_per_launch=ops, launch_us=gemm_call_s * 1e6,
                    algorithmic_bytes_per_launch=work["mixed_gemm"]["bytes"])
    ach_x = ops / gemm_x / 1e12
    variant = {"entry": "mxs_mixed_gemm_mx (prefill on the block-scaled fp6 MFMA: k_mx_prep + k_gemm_mx)",
               "value": ops / step_x / 1e12, "ms_per_step": step_x * 1e3, "launch_us": gemm_x * 1e6,
               "achieved": ach_x, "unit": "TFLOP/s", "peak": FP6_PEAK / 1e12,
               "frac": ach_x * 1e12 / FP6_PEAK, "int8_peak_frac": ach_x * 1e12 / INT8_PEAK,
               "traffic": measured_traffic("traffic_bytes_per_call_mx")}
    qx = stage_out["quantize_x"]
    ach_f = ops / gemm_f / 1e12
    fused = {"entry": "mxs_mixed_gemm_fused (X quantized into the prefill operand: k_quant_prep + "
                      "k_gemm_prep of W + k_gemm_a2r; the step drops its quantize_x stage)",
             "value": ops / step_f / 1e12, "ms_per_step": step_f * 1e3, "launch_us": gemm_f * 1e6,
             "achieved": ach_f, "unit": "TOP/s", "peak": INT8_PEAK / 1e12, "frac": ach_f * 1e12 / INT8_PEAK,
             "cold_us": stage_out["mixed_gemm_fused"]["ms"] * 1e3,
             "unfused_cold_us": (qx["ms"] + stage_out["mixed_gemm"]["ms"]) * 1e3}
    out = {
        "metric": "mixed MXINT GEMM TOPS & quantize GB/s, % of MI355X roofline (1 GPU)",
        "value": ops / step_s / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded outlier-channel activations, Student-t weights, bf16)",
        "config": {"workload": "Llama-3-8B q_proj prefill layer: calibrate 8x2048 tokens, score/allocate/"
                               "quantize W 4096x4096, quantize X 2048x4096, mixed GEMM 2048x4096x4096 "
                               "(5/15/80% 8/6/4-bit, 6/20/102 blocks), MXINT4 K and V 2048x8x128",
                   "global_batch": M, "seq_len": M, "parallelism": "none (1 GPU)"},
        "gemm_tops": gemm["TOPS"],
        "quantize_gbps": {"w": stage_out["quantize_w"]["GBps"], "x": qx["GBps"],
                          "kv": stage_out["quantize_kv"]["GBps"]},
        "stages": stage_out,
        "roofline": roofline,
        "variant_mx": variant,
        "variant_fused": fused,
    }
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, torch)
    return out




def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="70B block step only (no variants, no q_proj / MLP / decode keys)")
    ap.add_argument("--workload", choices=("70b_block", "q_proj"), default="70b_block")
    ap.add_argument("--block-variant", choices=("mx", "fused", "prepared"), default=None,
                    help="run the block step's timed steps with this GEMM variant (for profiling it; "
                         "the headline is the default step)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--overhead", action="store_true")
    ap.add_argument("--layerwise", action="store_true")
    ap.add_argument("--attention", action="store_true")
    ap.add_argument("--oracle-child", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.oracle_child:
        oracle_child(args.oracle_child)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(the hot path would shard by rows and columns; no collective is built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    import bit_gemm_hdiag_amd as mx
    from bit_gemm_hdiag_amd import synth
    if args.decode:
        for d in decode_cases(mx, synth, torch):
            print(json.dumps(d), flush=True)
        return
    if args.overhead:
        overhead_cases(mx, synth, torch)
        return
    if args.layerwise:
        layerwise_cases(mx, synth, torch)
        return
    if args.attention:
        attention_cases(mx, synth, torch)
        return
    if args.workload == "q_proj":
        print(json.dumps(q_proj_line(mx, synth, torch, args)), flush=True)
        return
    print(json.dumps(block_line(mx, synth, torch, args)), flush=True)


if __name__ == "__main__":
    main()
