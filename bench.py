"""Benchmark of the block-scaled FP4 hot path on one MI355X.

One step runs every stage of the path once on seeded synthetic inputs that are
already resident in HBM:
  quantize  MX and NV quantization of the 4096x4096 weight and 2048x4096
            activation of the single-linear workload, the lossless MX->NV remap
            and an MX dequantize of the weight;
  gemm      the 4096^3 W4A4 MXFP4 GEMM (activations quantized on the fly,
            weights pre-quantized, fp32 accumulation, bf16 output);
  moe       the MoE layer at hidden 4096 (384 experts, top-6, intermediate
            2048, 8192 tokens, MXFP4 weights and activations).
Each stage is bracketed by HIP events on the stream the kernels run on.  The
input of every HBM-bound stage rotates through copies whose total exceeds the
256 MB last-level cache, so each launch reads HBM, not cache.

Output: one JSON line.  `value` is the W4A4 GEMM throughput (TFLOP/s), the
first quantity of the metric; the quantize GB/s and MoE tokens/s are in
`components`; `roofline` describes the kernel with the largest share of the
step time and `rooflines` every timed kernel.  `cpu_baseline` times the CPU
oracle on a bounded sample of the GEMM workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "W4A4 GEMM TFLOPS (% FP4 MFMA peak); quantize GB/s; MoE tokens/s at h=4096"
PEAK_HBM_GBS = 8000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_BF16_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-moe", action="store_true", help="skip the MoE stage (profiling runs)")
    p.add_argument("--only", default="", help="comma list of stages to run (profiling runs)")
    return p.parse_args()


class Stage:
    def __init__(self, name, launch, bound, work, unit_work, kernel=None, per_launch=1):
        self.name, self.launch, self.bound = name, launch, bound
        self.work = work            # algorithmic bytes (hbm) or flops (mfma) per launch
        self.unit_work = unit_work  # description of the per-unit figure
        self.kernel = kernel or name
        self.times = []             # ms per launch


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import block_scaled_fp4_mx_amd as F
    import workloads as W

    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    def rot_copies(t, per_copy_bytes):
        n = max(2, int(np.ceil(1.5 * MALL_BYTES / per_copy_bytes)))
        return [t.clone() for _ in range(n)]

    # ---------------------------------------------------------------- inputs
    wl2 = W.workload2()
    W2 = wl2.W.to(dev)
    A2 = wl2.A.to(dev)
    pair_bytes = (W2.numel() + A2.numel()) * 2
    nrot2 = max(2, int(np.ceil(1.5 * MALL_BYTES / pair_bytes)))
    W2s = [W2.clone() for _ in range(nrot2)]
    A2s = [A2.clone() for _ in range(nrot2)]

    def qbufs(x, blk):
        r, k = x.shape
        return (torch.empty((r, k // 2), dtype=torch.uint8, device=dev),
                torch.empty((r, k // blk), dtype=torch.uint8, device=dev))

    W2mx, A2mx = qbufs(W2, 32), qbufs(A2, 32)
    W2nv, A2nv = qbufs(W2, 16), qbufs(A2, 16)
    tsW = torch.zeros(1, dtype=torch.float32, device=dev)
    tsA = torch.zeros(1, dtype=torch.float32, device=dev)
    nvws = torch.empty(F.fp4_quantize_nv_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    rem_s = torch.empty((4096, 4096 // 16), dtype=torch.uint8, device=dev)
    rem_ts = torch.zeros(1, dtype=torch.float32, device=dev)
    rem_n = torch.zeros(1, dtype=torch.int32, device=dev)
    deq = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    # pre-quantized weight codes rotate for the remap and dequant inputs
    W2mx_rot = []
    for i in range(nrot2):
        c, s = qbufs(W2, 32)
        F.fp4_quantize_mx(W2s[i], c, s)
        W2mx_rot.append((c, s))

    wl3 = W.workload3()
    A3 = wl3.A.to(dev)
    A3s = rot_copies(A3, A3.numel() * 2)
    W3 = wl3.W.to(dev)
    W3q = qbufs(W3, 32)
    F.fp4_quantize_mx(W3, *W3q)
    A3q = qbufs(A3, 32)
    C3 = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    del W3

    st = {"i": 0}

    def cur(lst):
        return lst[st["i"] % len(lst)]

    M2 = 4096 * 4096
    M2a = 2048 * 4096
    stages = [
        Stage("quantize_mx_W", lambda: F.fp4_quantize_mx(cur(W2s), *W2mx), "hbm", M2 * (2 + 0.5 + 1 / 32),
              "2.53125 B/elem (2 bf16 in, 0.5 codes, 1/32 scale)", "mx_quantize_kernel"),
        Stage("quantize_mx_A", lambda: F.fp4_quantize_mx(cur(A2s), *A2mx), "hbm", M2a * (2 + 0.5 + 1 / 32),
              "2.53125 B/elem", "mx_quantize_kernel"),
        Stage("quantize_nv_W", lambda: F.fp4_quantize_nv(cur(W2s), *W2nv, tsW, False, nvws), "hbm",
              M2 * (2 + 0.5 + 1 / 16), "2.5625 B/elem (2 in, 0.5 codes, 1/16 scale; tensor amax re-read not counted)",
              "nv_amax+nv_quantize"),
        Stage("quantize_nv_A", lambda: F.fp4_quantize_nv(cur(A2s), *A2nv, tsA, False, nvws), "hbm",
              M2a * (2 + 0.5 + 1 / 16), "2.5625 B/elem", "nv_amax+nv_quantize"),
        Stage("remap_W", lambda: F.fp4_remap_mx_to_nv(cur(W2mx_rot)[0], cur(W2mx_rot)[1], rem_s, rem_ts, rem_n),
              "hbm", M2 * (1 / 32 + 1 / 16), "0.09375 B/elem (scale bytes in and out)", "remap kernels"),
        Stage("dequant_mx_W", lambda: F.fp4_dequant(F.FMT_MX, cur(W2mx_rot)[0], cur(W2mx_rot)[1], None, deq), "hbm",
              M2 * (0.5 + 1 / 32 + 2), "2.53125 B/elem (codes+scale in, bf16 out)", "dequant_kernel"),
        Stage("gemm_quantize_A", lambda: F.fp4_quantize_mx(cur(A3s), *A3q), "hbm", 4096 * 4096 * (2 + 0.5 + 1 / 32),
              "2.53125 B/elem", "mx_quantize_kernel"),
        Stage("gemm_mx_4096", lambda: F.fp4_gemm(F.FMT_MX, A3q[0], A3q[1], W3q[0], W3q[1], C3), "mfma",
              2.0 * 4096 ** 3, "2*M*N*K flop", "gemm_mx_kernel"),
    ]

    moe = None
    if not args.no_moe:
        moe = build_moe(torch, F, W, dev)
        if moe is not None:
            stages.append(Stage("moe_h4096", moe["launch"], moe["bound"], moe["work"], moe["unit"], "moe (all kernels)"))

    if args.only:
        keep = set(args.only.split(","))
        stages = [s for s in stages if s.name in keep]

    for _ in range(args.warmup):
        for s in stages:
            s.launch()
        st["i"] += 1
    torch.cuda.synchronize()

    # one event pair per stage per step; the queue stays full between steps, so
    # no event interval includes host launch latency
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in stages]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for s, (e0, e1) in zip(stages, evs[k]):
            e0.record(stream)
            s.launch()
            e1.record(stream)
        st["i"] += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for k in range(args.steps):
        for s, (e0, e1) in zip(stages, evs[k]):
            s.times.append(e0.elapsed_time(e1))
    ms_per_step = wall * 1e3 / args.steps

    rooflines = {}
    for s in stages:
        avg_ms = float(np.mean(s.times))
        if s.bound == "hbm":
            ach = s.work / (avg_ms * 1e-3) / 1e9
            rooflines[s.name] = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                     frac=round(ach / PEAK_HBM_GBS, 4), traffic=None, avg_us=round(avg_ms * 1e3, 2),
                                     best_us=round(min(s.times) * 1e3, 2), work_per_launch=s.work,
                                     per_unit=s.unit_work, kernel=s.kernel)
        else:
            peak = s.bound == "mfma_bf16" and PEAK_BF16_TFLOPS or PEAK_FP4_TFLOPS
            ach = s.work / (avg_ms * 1e-3) / 1e12
            rooflines[s.name] = dict(bound="mfma", achieved=round(ach, 1), peak=peak, unit="TFLOP/s",
                                     frac=round(ach / peak, 4), traffic=None, avg_us=round(avg_ms * 1e3, 2),
                                     best_us=round(min(s.times) * 1e3, 2), work_per_launch=s.work,
                                     per_unit=s.unit_work, kernel=s.kernel)
    dom = max(stages, key=lambda s: np.mean(s.times))
    gemm = rooflines.get("gemm_mx_4096")
    value = gemm["achieved"] if gemm else None
    comps = {}
    if gemm:
        comps["gemm_tflops"] = gemm["achieved"]
        comps["gemm_frac_fp4_peak"] = gemm["frac"]
        qa = rooflines.get("gemm_quantize_A")
        if qa:
            comps["gemm_with_onthefly_quantize_tflops"] = round(
                2.0 * 4096 ** 3 / ((gemm["avg_us"] + qa["avg_us"]) * 1e-6) / 1e12, 1)
    for n in ("quantize_mx_W", "quantize_mx_A", "quantize_nv_W", "quantize_nv_A"):
        if n in rooflines:
            comps[n + "_GBps"] = rooflines[n]["achieved"]
    if moe is not None and "moe_h4096" in rooflines:
        comps["moe_tokens_per_s"] = round(8192 / (rooflines["moe_h4096"]["avg_us"] * 1e-6), 1)
        comps["moe_active_experts"] = moe["active"]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1",
        "data": "synthetic",
        "config": {"workload": "linear 4096x4096 W + 2048x4096 A quantize/remap/dequant; "
                               "W4A4 MXFP4 GEMM 4096^3 (bf16 out, fp32 accumulate); "
                               "MoE hidden 4096, 384 experts, top-6, inter 2048, 8192 tokens (MXFP4)",
                   "accumulate": "fp32"},
        "components": comps,
        "roofline": {k: v for k, v in rooflines[dom.name].items()
                     if k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} | {"kernel": dom.name},
        "rooflines": rooflines,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


def build_moe(torch, F, W, dev):
    """MoE workload at hidden 4096; returns None while the library reports the
    MoE entry point as unsupported."""
    m = W.moe_workload(4)
    T, H, I, E = 8192, m.hidden, m.inter, m.num_experts
    X = m.X.to(dev)
    ids = torch.from_numpy(m.ids).to(dev)
    wts = torch.from_numpy(m.weights).to(dev)
    active = sorted(set(m.ids.ravel().tolist()))
    w13c = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13s = torch.full((E, 2 * I, H // 32), 127, dtype=torch.uint8, device=dev)
    w2c = torch.zeros((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2s = torch.full((E, H, I // 32), 127, dtype=torch.uint8, device=dev)
    for e, a, b in W.expert_weights_device(4, E, H, I, dev):
        if e in active:
            F.fp4_quantize_mx(a, w13c[e], w13s[e])
            F.fp4_quantize_mx(b, w2c[e], w2s[e])
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(F.fp4_moe_workspace_bytes(F.FMT_MX, T, H, 6, E, I), dtype=torch.uint8, device=dev)
    launch = lambda: F.fp4_moe_grouped_gemm(F.FMT_MX, X, ids, wts, E, I, w13c, w13s, w2c, w2s, out, ws)
    try:
        launch()
        torch.cuda.synchronize()
    except F.Fp4Error as e:
        if e.status == -4:
            return None
        raise
    counts = np.bincount(m.ids.ravel(), minlength=E)
    flops = float(6 * counts.sum() * H * I)
    return dict(launch=launch, bound="mfma", work=flops, unit="6*H*I flop per routed slot", active=len(active))


def cpu_baseline():
    """The CPU oracle on a bounded sample of the GEMM workload: 64 rows of A
    quantized and multiplied by the full quantized W (4096x4096), fp64."""
    import workloads as W
    from oracle import gemm as G
    from oracle import quant as Q
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        threads = os.cpu_count() or 1
    wl = W.workload3()
    ab = W.bf16_bits(wl.A)[:64]
    wb = W.bf16_bits(wl.W)
    t0 = time.perf_counter()
    ea = Q.mx_quantize(ab)
    eb = tuple(np.concatenate(p) for p in zip(*[Q.mx_quantize(wb[i:i + 512]) for i in range(0, 4096, 512)]))
    G.gemm_ref("mx", *ea, *eb)
    dt = time.perf_counter() - t0
    flops = 2.0 * 64 * 4096 * 4096
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "64x4096 A rows times the full 4096x4096 W of the 4096^3 GEMM: MX-quantize both "
                      "(fp64 numpy) and the exact fp64 product with its error bound; "
                      f"{dt:.1f} s on {os.cpu_count()} host cores"}


if __name__ == "__main__":
    main()
