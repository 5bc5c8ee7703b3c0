"""Benchmark of the MXSens hot path on one MI355X.

One step = one pass of every stage over the Llama-3-8B q_proj-shaped layer
(synthetic, seeded): calibrate over 8 x 2048 tokens, score, allocate,
quantize W, quantize X, the mixed 8/6/4-bit GEMM (2048 x 4096 x 4096) and
MXINT4 quantisation of K and V (2048 tokens x 8 heads x 128). Inputs are
resident in HBM before timing starts.

Prints one JSON line. `value` is the whole step's throughput in GEMM TOPS
(2 M N K per step over the step time) with mxs_mixed_gemm (int8 block sums);
per-stage times, TOPS and GB/s are in `stages` (`ms`: median of single
calls, each after a read pass over 512 MB that evicts the 256 MB Infinity Cache,
so inputs come from HBM; `warm_ms`: back-to-back calls through the Python
binding; `warm_graph_ms`: the same calls replayed from one HIP graph; both
warm figures re-read inputs the cache holds); `roofline` is for the
dominant kernel; `variant_mx` repeats the step with mxs_mixed_gemm_mx
(prefill on the block-scaled fp6 matrix cores) and `variant_fused` with
mxs_mixed_gemm_fused (X quantized inside the product, no quantize_x stage);
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same step.

The dominant kernel's roofline uses the mixed_gemm call's own duration,
timed with HIP events on its stream inside every timed step; its HBM
traffic comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counters stored in
profiles/ and is reported only while the GEMM source is unchanged since.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
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
                                       and 32 tokens: one JSON line per case, GB/s
                                       of packed W + scale bytes against HBM peak,
                                       median of single calls after an Infinity
                                       Cache flush; `warm_graph_us` is the same
                                       calls replayed back to back from a graph)
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
    """HBM bytes per mixed_gemm call (key traffic_bytes_per_call_mx: per
    mixed_gemm_mx call) from the stored counter summary, or None when the
    summary is missing or the GEMM source changed since it was taken."""
    try:
        kv = {}
        with open(GEMM_TRAFFIC) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        with open(GEMM_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("source_sha256") != sha:
            return None
        return float(kv[key])
    except (OSError, KeyError, ValueError):
        return None


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
    """70B MLP decode GEMMs (up 28672 x 8192, down 8192 x 28672, 5/15/80 %)."""
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
            print(json.dumps({"case": f"decode {lay['name']} {N}x{K}", "tokens": M, "us": tc * 1e6,
                              "warm_graph_us": tg * 1e6, "w_bytes": wbytes, "GBps": wbytes / tc / 1e9,
                              "hbm_frac": wbytes / tc / HBM_PEAK, "warm_hbm_frac": wbytes / tg / HBM_PEAK}),
                  flush=True)


def overhead_cases(mx, synth, torch, reps=20):
    """Cost of the mixed map against uniform MXINT4: mixed_gemm on the same
    layer under the all-4-bit map, the 4.03-bit map (one 8-bit block), the
    binary 4/8 map of the same 8-bit share (5 %), and the 5/15/80 % map, for
    the q_proj prefill (2048 x 4096 x 4096) and the 70B up-projection decode
    (1 token, 28672 x 8192)."""
    dev = torch.device("cuda:0")
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    for case, M, N, K, seed in (("prefill q_proj", 2048, 4096, 4096, 5000), ("decode 70B up", 1, 28672, 8192, 5100)):
        nb = K // 32
        gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
        W = synth.weights(N, K, seed + synth.ROLE_W, device=dev)
        X = synth.activations(M, K, seed + synth.ROLE_X, gains, device=dev)
        perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(dev)
        base = None
        for name, (bp8, bp6) in (("uniform 4-bit", (0, 0)), ("one 8-bit block", ((10000 + nb - 1) // nb, 0)),
                                 ("binary 4/8 (5 % 8-bit)", (500, 0)), ("5/15/80 %", (500, 1500))):
            n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
            Wq = mx.mxs_quantize(W, perm, n8, n6, n4)
            Aq = mx.mxs_quantize(X, perm, n8, n6, n4)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            out = {"case": case, "map": name, "blocks": [n8, n6, n4], "avg_bits": (8 * n8 + 6 * n6 + 4 * n4) / nb}
            for entry in ("mxs_mixed_gemm", "mxs_mixed_gemm_mx"):
                wsf = getattr(mx, entry + "_workspace")
                ws = torch.empty(max(1, wsf(Aq, Wq)), dtype=torch.uint8, device=dev)
                f = getattr(mx, entry)
                fn = lambda: f(Aq, Wq, Y, ws=ws)
                out[entry + "_us"] = time_graph(torch, fn, reps) * 1e6
                out[entry + "_cold_us"] = time_cold(torch, fn, reps, flush) * 1e6
            if base is None:
                base = out
            for k in ("mxs_mixed_gemm_us", "mxs_mixed_gemm_mx_us", "mxs_mixed_gemm_cold_us"):
                out[k.replace("_us", "_vs_uniform")] = out[k] / base[k]
            print(json.dumps(out), flush=True)
            del Wq, Aq, Y
        del W, X


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--stage-reps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--overhead", action="store_true")
    ap.add_argument("--layerwise", action="store_true")
    ap.add_argument("--attention", action="store_true")
    args = ap.parse_args()
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
        decode_cases(mx, synth, torch)
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
                    kernel="mixed_gemm call: k_gemm_prep + k_gemm_dma (int8 MFMA)",
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
                      "k_gemm_prep of W + k_gemm_dma; the step drops its quantize_x stage)",
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
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
