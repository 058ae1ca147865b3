"""Benchmark of the block-scaled FP4 hot path on one MI355X.

One step runs every stage of the path once, on seeded synthetic inputs that
are already resident in HBM:
  quantize  MX and NV quantization of the 4096x4096 weight and the 2048x4096
            activation of the single-linear workload (NV with the tensor scale
            computed, and for the activation also with a calibrated one), the
            lossless MX->NV remap and an MX dequantize of the weight; the QAT
            fake-quant node (fused quantize -> dequantize, MX and NV) of the
            weight and its straight-through backward into fp32 master
            gradients;
  kv        MXFP4 KV-cache append of a 16384-token prefill (d = 512) into
            scattered cache slots, and indexer-style FP4 QK scores of 64
            queries against 32768 cached keys (fp32 scores);
  gemm      the 4096^3 W4A4 MXFP4 GEMM (activations quantized on the fly,
            weights pre-quantized, fp32 accumulation, bf16 output), the same
            product in NVFP4, and the W4A8 variant (MXFP8 activations quantized
            on the fly times the MXFP4 weights);
  moe       the MoE layer at hidden 4096 (384 experts, top-6, intermediate
            2048, 8192 tokens, MXFP4 weights and activations), and the NVFP4
            MoE layer at hidden 7168 (intermediate 3072) on a decode batch of
            64 tokens and on a prefill batch of 16384 tokens.
The input of every HBM-bound stage rotates through copies whose total exceeds
the 256 MB last-level cache, so each launch reads HBM, not cache.

Timing.  W warmup steps, then K steps of the whole path back to back, with no
markers in between; ms_per_step is their wall time between two device
synchronizations.  Then each stage is launched K times back to back between
two HIP events recorded on its stream, behind a spin kernel that keeps the
device busy while the host queues the launches (so host launch latency never
shows): the stage's duration is the event interval over K.  An event marker
costs the device about 6 us, so it is kept out of these intervals.  For the
MoE stages a second pass records the entry point's stage events between its
kernels, which gives each kernel's duration (each interval then also holds one
marker, small against these kernels).

Output: one JSON line.  `value` is the W4A4 GEMM throughput (TFLOP/s), the
first quantity of the metric; the quantize GB/s and the MoE tokens/s are in
`components`.  `roofline` describes the kernel with the largest share of the
step time (algorithmic work per launch over its event-measured duration) and
`rooflines` every timed stage and MoE kernel.  `traffic` comes from
rocprofv3 FETCH_SIZE / WRITE_SIZE counters recorded in profiles/traffic.json
(written by profile_counters.sh), scaled by what the same counters read for a
plain copy of known size; it is null when the kernel sources changed since.
`cpu_baseline` times the CPU oracle on the whole GEMM workload (its
`per_workload` list: every workload, the MoE ones on bounded token samples).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import glob
import json
import os
import sys
import time

import numpy as np

METRIC = "W4A4 GEMM TFLOPS (% FP4 MFMA peak); quantize GB/s; MoE tokens/s at h=4096"
PEAK_HBM_GBS = 8000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
MALL_BYTES = 256 << 20
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")
MOE_KERNELS = ("quantize_x", "routing", "gate_up", "down", "combine")
SPACER_CYCLES = 16_000_000
TIMING_BLOCKS = 5              # per-stage timing blocks of `steps` launches each


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-moe", action="store_true", help="skip the MoE stages")
    p.add_argument("--only", default="", help="comma list of stages to run (profiling runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy per step (counter calibration runs)")
    return p.parse_args()


def source_digest():
    """Digest of the kernel sources, so recorded counters can be matched to the
    code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "block_scaled_fp4_mx_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Stage:
    def __init__(self, name, launch, bound, work, per_unit, kernel, moe=None):
        self.name, self.launch, self.bound = name, launch, bound
        self.work = work            # algorithmic bytes (hbm) or flops (mfma) per launch
        self.per_unit = per_unit    # the per-unit figure the work is built from
        self.kernel = kernel        # kernel name(s) as rocprofv3 reports them
        self.moe = moe              # MoE: dict with the stage events and per-kernel work
        self.times = []             # ms per launch
        self.best = None            # ms per launch of the fastest timing block


def roofline_entry(bound, work, ms, per_unit, kernel, extra=None):
    if bound == "hbm":
        ach = work / (ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    else:
        ach = work / (ms * 1e-3) / 1e12
        peak = {"mfma_bf16": PEAK_BF16_TFLOPS, "mfma_fp8": PEAK_FP8_TFLOPS}.get(bound, PEAK_FP4_TFLOPS)
        unit = "TFLOP/s"
    e = dict(bound="mfma" if bound.startswith("mfma") else bound, achieved=round(ach, 1), peak=peak, unit=unit,
             frac=round(ach / peak, 4), traffic=None, avg_us=round(ms * 1e3, 2), work_per_launch=work,
             per_unit=per_unit, kernel=kernel)
    if extra:
        e.update(extra)
    return e


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("source_digest") == source_digest() else None


def main():
    t_start = time.perf_counter()
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU runs are not part of it "
                                   "(--gpus must be 1)", "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import block_scaled_fp4_mx_amd as F
    import workloads as W

    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    def progress(msg):
        print(f"[bench] {msg} ({time.perf_counter() - t_start:.0f} s)", file=sys.stderr, flush=True)

    def rot_copies(t, per_copy_bytes):
        n = max(2, int(np.ceil(1.5 * MALL_BYTES / per_copy_bytes)))
        return [t.clone() for _ in range(n)]

    def qbufs(x, blk):
        r, k = x.shape
        return (torch.empty((r, k // 2), dtype=torch.uint8, device=dev),
                torch.empty((r, k // blk), dtype=torch.uint8, device=dev))

    # ---------------------------------------------------------------- inputs
    wl2 = W.workload2()
    W2, A2 = wl2.W.to(dev), wl2.A.to(dev)
    pair_bytes = (W2.numel() + A2.numel()) * 2
    nrot2 = max(2, int(np.ceil(1.5 * MALL_BYTES / pair_bytes)))
    W2s = [W2.clone() for _ in range(nrot2)]
    A2s = [A2.clone() for _ in range(nrot2)]
    W2mx, A2mx = qbufs(W2, 32), qbufs(A2, 32)
    W2nv, A2nv = qbufs(W2, 16), qbufs(A2, 16)
    tsW = torch.zeros(1, dtype=torch.float32, device=dev)
    tsA = torch.zeros(1, dtype=torch.float32, device=dev)
    tsA_cal = (A2.abs().max().float() / 2688.0).reshape(1).contiguous()   # a calibrated activation scale
    tsW_cal = (W2.abs().max().float() / 2688.0).reshape(1).contiguous()
    nvws = torch.empty(F.fp4_quantize_nv_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    rem_s = torch.empty((4096, 4096 // 16), dtype=torch.uint8, device=dev)
    rem_ts = torch.zeros(1, dtype=torch.float32, device=dev)
    rem_n = torch.zeros(1, dtype=torch.int32, device=dev)
    smax_ws = torch.empty(F.fp4_scale_max_workspace_bytes(4096, 4096), dtype=torch.uint8, device=dev)
    deq = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    fp8_v = torch.empty((4096, 4096), dtype=torch.uint8, device=dev)
    fp8_s = torch.empty((4096, 4096 // 32), dtype=torch.uint8, device=dev)
    fp8_ts = torch.zeros(1, dtype=torch.float32, device=dev)
    fp8_n = torch.zeros(1, dtype=torch.int32, device=dev)
    fq_out = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    masters = rot_copies(torch.zeros((4096, 4096), dtype=torch.float32, device=dev), 4096 * 4096 * 4)
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

    def nv_quantized(x):
        c, s = qbufs(x, 16)
        ts = torch.zeros(1, dtype=torch.float32, device=dev)
        F.fp4_quantize_nv(x, c, s, ts, False, nvws)
        return c, s, ts

    A3n, W3n = nv_quantized(A3), nv_quantized(W3)
    del W3
    # KV cache: prefill append (16384 tokens, d 512) into a permuted slot order,
    # and scores of 64 query latents against 32768 cached keys
    KV_T, KV_D, KV_N, KV_Q = 16384, 512, 32768, 64
    kv_x = rot_copies(W.to_bf16(np.random.default_rng(7).standard_normal((KV_T, KV_D))).to(dev), KV_T * KV_D * 2)
    kv_slots = torch.from_numpy(np.random.default_rng(8).permutation(KV_N)[:KV_T].astype(np.int32)).to(dev)
    kv_cc = torch.empty((KV_N, KV_D // 2), dtype=torch.uint8, device=dev)
    kv_cs = torch.empty((KV_N, KV_D // 32), dtype=torch.uint8, device=dev)
    keys = W.to_bf16(np.random.default_rng(9).standard_normal((KV_N, KV_D))).to(dev)
    F.fp4_kv_append_mx(keys, torch.arange(KV_N, dtype=torch.int32, device=dev), kv_cc, kv_cs)
    n_kv = max(2, int(np.ceil(1.5 * MALL_BYTES / (KV_N * (KV_D // 2 + KV_D // 32)))))
    kv_caches = [(kv_cc.clone(), kv_cs.clone()) for _ in range(n_kv)]     # contiguous codes, scales
    kv_q = qbufs(W.to_bf16(np.random.default_rng(10).standard_normal((KV_Q, KV_D))).to(dev), 32)
    F.fp4_quantize_mx(W.to_bf16(np.random.default_rng(10).standard_normal((KV_Q, KV_D))).to(dev), *kv_q)
    kv_scores = torch.empty((KV_Q, KV_N), dtype=torch.float32, device=dev)
    del keys

    def kv_score():
        cc, cs = cur(kv_caches)
        F.fp4_gemm(F.FMT_MX, kv_q[0], kv_q[1], cc, cs, kv_scores)

    A3q8 = (torch.empty((4096, 4096), dtype=torch.uint8, device=dev),
            torch.empty((4096, 4096 // 32), dtype=torch.uint8, device=dev))

    st = {"i": 0}

    def cur(lst):
        return lst[st["i"] % len(lst)]

    M2, M2a = 4096 * 4096, 2048 * 4096
    MXB, NVB, MX8B = 2 + 0.5 + 1 / 32, 2 + 0.5 + 1 / 16, 2 + 1 + 1 / 32
    stages = [
        Stage("quantize_mx_W", lambda: F.fp4_quantize_mx(cur(W2s), *W2mx), "hbm", M2 * MXB,
              "2.53125 B/elem (2 bf16 in, 0.5 codes, 1/32 scale out)", "mx_quantize_kernel"),
        Stage("quantize_mx_A", lambda: F.fp4_quantize_mx(cur(A2s), *A2mx), "hbm", M2a * MXB,
              "2.53125 B/elem", "mx_quantize_kernel"),
        Stage("quantize_nv_W", lambda: F.fp4_quantize_nv(cur(W2s), *W2nv, tsW, False, nvws), "hbm", M2 * NVB,
              "2.5625 B/elem (2 in, 0.5 codes, 1/16 scale out); the tensor-amax read is not counted",
              "nv_amax_kernel + nv_quantize_kernel"),
        Stage("quantize_nv_A", lambda: F.fp4_quantize_nv(cur(A2s), *A2nv, tsA, False, nvws), "hbm", M2a * NVB,
              "2.5625 B/elem; the tensor-amax read is not counted", "nv_amax_kernel + nv_quantize_kernel"),
        Stage("quantize_nv_A_calibrated", lambda: F.fp4_quantize_nv(cur(A2s), *A2nv, tsA_cal, True, nvws), "hbm",
              M2a * NVB, "2.5625 B/elem (calibrated s_t: one pass)", "nv_quantize_kernel"),
        Stage("quantize_nv_W_calibrated", lambda: F.fp4_quantize_nv(cur(W2s), *W2nv, tsW_cal, True, nvws), "hbm",
              M2 * NVB, "2.5625 B/elem (supplied s_t: the second pass alone)", "nv_quantize_kernel"),
        Stage("remap_W", lambda: F.fp4_remap_mx_to_nv(cur(W2mx_rot)[0], cur(W2mx_rot)[1], rem_s, rem_ts, rem_n,
                                                      workspace=smax_ws),
              "hbm", M2 * (1 / 32 + 1 / 16), "0.09375 B/elem (scale bytes in and out)",
              "scale_max_kernel + remap_kernel"),
        Stage("dequant_fp8_W", lambda: F.fp4_mx_dequant_fp8(cur(W2mx_rot)[0], cur(W2mx_rot)[1], fp8_v, fp8_ts, fp8_n,
                                                            fp8_s, workspace=smax_ws), "hbm", M2 * (0.5 + 1 / 32 + 1 + 1 / 32),
              "1.5625 B/elem (codes + UE8M0 scale in, E4M3 value + E4M3 block scale out)",
              "scale_max_kernel + fp8_dequant_kernel"),
        Stage("dequant_mx_W", lambda: F.fp4_dequant(F.FMT_MX, cur(W2mx_rot)[0], cur(W2mx_rot)[1], None, deq), "hbm",
              M2 * (0.5 + 1 / 32 + 2), "2.53125 B/elem (codes + scale in, bf16 out)", "dequant_kernel"),
        Stage("fake_quant_mx_W", lambda: F.fp4_fake_quant(F.FMT_MX, cur(W2s), fq_out), "hbm", M2 * 4.0,
              "4 B/elem (2 bf16 in, 2 bf16 out)", "mx_quantize_kernel<true, 1> (bf16 out)"),
        Stage("fake_quant_nv_W", lambda: F.fp4_fake_quant(F.FMT_NV, cur(W2s), fq_out, tsW, False, nvws), "hbm",
              M2 * 4.0, "4 B/elem; the tensor-amax read is not counted", "nv_amax_kernel + nv_quantize_kernel<true, 1> (bf16 out)"),
        Stage("ste_backward_W", lambda: F.fp4_ste_backward(cur(W2s), cur(masters), accumulate=True), "hbm", M2 * 10.0,
              "10 B/elem (2 bf16 gradient, 4 fp32 master read, 4 written)", "ste_backward_kernel"),
        Stage("kv_append_prefill16384", lambda: F.fp4_kv_append_mx(cur(kv_x), kv_slots, kv_cc, kv_cs), "hbm",
              KV_T * KV_D * MXB + KV_T * 4, "2.53125 B/elem + 4 B slot id per token",
              "mx_quantize_kernel<true, 3>"),
        Stage("indexer_scores_64x32768", kv_score, "hbm",
              KV_N * KV_D * (0.5 + 1 / 32) + KV_Q * KV_D * (0.5 + 1 / 32) + KV_Q * KV_N * 4,
              "cached key codes + scales (0.53125 B/elem) + query codes + fp32 scores out",
              "gemm_mx_skinny_kernel<4, 1>"),
        Stage("gemm_quantize_A", lambda: F.fp4_quantize_mx(cur(A3s), *A3q), "hbm", 4096 * 4096 * MXB,
              "2.53125 B/elem", "mx_quantize_kernel"),
        Stage("gemm_mx_4096", lambda: F.fp4_gemm(F.FMT_MX, A3q[0], A3q[1], W3q[0], W3q[1], C3), "mfma",
              2.0 * 4096 ** 3, "2*M*N*K flop", "gemm_mx_256_kernel"),
        Stage("gemm_nv_4096", lambda: F.fp4_gemm(F.FMT_NV, A3n[0], A3n[1], W3n[0], W3n[1], C3, A3n[2], W3n[2]),
              "mfma_bf16", 2.0 * 4096 ** 3, "2*M*N*K flop (fp16 MFMA on the exact expansion; 16-bit peak)",
              "gemm_nv_tile_kernel"),
        Stage("gemm_quantize_A_mxfp8", lambda: F.fp4_quantize_mxfp8(cur(A3s), *A3q8), "hbm", 4096 * 4096 * MX8B,
              "3.03125 B/elem (2 bf16 in, 1 E4M3 code, 1/32 scale out)", "mxfp8_quantize_kernel"),
        Stage("gemm_w4a8_4096", lambda: F.fp4_gemm_w4a8(A3q8[0], A3q8[1], W3q[0], W3q[1], C3), "mfma_fp8",
              2.0 * 4096 ** 3, "2*M*N*K flop (E4M3 x E2M1 MFMA; FP8 peak)", "gemm_w4a8_256_kernel"),
    ]
    want = set(args.only.split(",")) if args.only else None
    progress("linear and GEMM inputs ready")
    if not args.no_moe:
        if want is None or "moe_h4096" in want:
            stages.append(build_moe_h4096(torch, F, W, dev))
            progress("build_moe_h4096 done")
        if want is None or "moe_h7168_decode64" in want:
            stages.append(build_moe_decode(torch, F, W, dev))
            progress("build_moe_decode done")
        if want is None or "moe_h7168_prefill16384" in want:
            stages.append(build_moe_prefill(torch, F, W, dev))
            progress("build_moe_prefill done")
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        stages.append(Stage("copy_256MiB", lambda: dst.copy_(src), "hbm", 2.0 * (256 << 20),
                            "256 MiB read + 256 MiB written", "copy"))
    if want is not None:
        stages = [s for s in stages if s.name in want]

    progress(f"{len(stages)} stages built")
    # No Python garbage collection while launches are queued: a collection pause
    # longer than the spacer's cushion lets the device idle inside a timed block
    # (seen as one block of a stage running ~40x slower).
    gc.disable()
    for _ in range(args.warmup):
        for s in stages:
            s.launch()
        st["i"] += 1
    torch.cuda.synchronize()
    progress("warmup done")

    # timed steps: the whole path, back to back, with no markers in between
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for s in stages:
            s.launch()
        st["i"] += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    progress("timed steps done")

    # per-stage durations: `steps` launches of the stage between two events on
    # its stream, queued behind a spin kernel so the host's launch rate never
    # leaves the device idle between them
    def spacer():
        torch.cuda._sleep(SPACER_CYCLES)

    moe_marks = {}
    for s in stages:
        # TIMING_BLOCKS blocks of `steps` launches: the mean over all launches,
        # and the best block's mean (events between single launches would
        # disturb the short kernels)
        s.times = []
        for _ in range(args.steps):          # one untimed block first: the stage's first launches after the
            s.launch()                       # previous stage have shown one-off stalls of milliseconds
            st["i"] += 1
        for _ in range(TIMING_BLOCKS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            spacer()
            e0.record(stream)
            for _ in range(args.steps):
                s.launch()
                st["i"] += 1
            e1.record(stream)
            torch.cuda.synchronize()
            s.times.append(e0.elapsed_time(e1) / args.steps)
        s.best = min(s.times)
        if s.moe:
            # the MoE entry point records its stage events between its kernels
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
            for row in evs:                 # materialize the events the library records
                for e in row:
                    e.record(stream)
            spacer()
            for k in range(args.steps):
                s.moe["set_events"]([e.cuda_event for e in evs[k]])
                s.launch()
            torch.cuda.synchronize()
            s.moe["set_events"]([None] * 6)
            moe_marks[s.name] = evs

    gc.enable()
    progress("per-stage timing done")
    traffic = load_traffic()
    rooflines = {}
    kernel_rows = []                        # (ms, name, entry) for the dominant-kernel choice
    for s in stages:
        ms = float(np.mean(s.times))
        e = roofline_entry(s.bound, s.work, ms, s.per_unit, s.kernel,
                           {"best_us": round(s.best * 1e3, 2), "block_us": [round(t * 1e3, 2) for t in s.times]})
        if s.moe:
            e["kernels"] = {}
            evs = moe_marks[s.name]
            for i, kname in enumerate(MOE_KERNELS):
                kms = float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
                bound, work, unit = s.moe["work"][kname]
                ke = roofline_entry(bound, work, kms, unit, s.moe["kernel_names"][kname])
                e["kernels"][kname] = ke
                kernel_rows.append((kms, f"{s.name}.{kname}", ke))
        else:
            kernel_rows.append((ms, s.name, e))
        rooflines[s.name] = e
    if traffic:
        for _, name, e in kernel_rows:
            t = traffic.get("kernels", {}).get(name)
            if t is not None:
                e["traffic"] = t["bytes_per_launch"]
            mf = traffic.get("mfma", {}).get(name)
            if mf is not None:
                e["mfma_busy"] = mf["mfma_busy"]
                e["lds_bank_conflicts_per_access"] = mf["lds_bank_conflicts_per_access"]

    dom_ms, dom_name, dom = max(kernel_rows, key=lambda r: r[0])
    comps = {}
    gemm = rooflines.get("gemm_mx_4096")
    value = gemm["achieved"] if gemm else None
    if gemm:
        comps["gemm_tflops"] = gemm["achieved"]
        comps["gemm_frac_fp4_peak"] = gemm["frac"]
        qa = rooflines.get("gemm_quantize_A")
        if qa:
            comps["gemm_with_onthefly_quantize_tflops"] = round(
                2.0 * 4096 ** 3 / ((gemm["avg_us"] + qa["avg_us"]) * 1e-6) / 1e12, 1)
    if "gemm_w4a8_4096" in rooflines:
        g8 = rooflines["gemm_w4a8_4096"]
        comps["gemm_w4a8_tflops"] = g8["achieved"]
        comps["gemm_w4a8_frac_fp8_peak"] = g8["frac"]
        q8 = rooflines.get("gemm_quantize_A_mxfp8")
        if q8:
            comps["gemm_w4a8_with_onthefly_quantize_tflops"] = round(
                2.0 * 4096 ** 3 / ((g8["avg_us"] + q8["avg_us"]) * 1e-6) / 1e12, 1)
    if "gemm_nv_4096" in rooflines:
        comps["gemm_nv_tflops"] = rooflines["gemm_nv_4096"]["achieved"]
        comps["gemm_nv_frac_16bit_peak"] = rooflines["gemm_nv_4096"]["frac"]
    for n in ("quantize_mx_W", "quantize_mx_A", "quantize_nv_W", "quantize_nv_A", "quantize_nv_A_calibrated",
              "remap_W", "dequant_mx_W", "dequant_fp8_W", "gemm_quantize_A", "gemm_quantize_A_mxfp8", "fake_quant_mx_W", "fake_quant_nv_W", "ste_backward_W",
              "kv_append_prefill16384", "indexer_scores_64x32768"):
        if n in rooflines:
            comps[n + "_GBps"] = rooflines[n]["achieved"]
    # the two passes of the NV quantize with a computed s_t: pass 2 alone is the
    # supplied-s_t stage; pass 1 (the tensor amax, 2 B read per element) is the rest
    for t, n_el in (("W", M2), ("A", M2a)):
        full, cal = rooflines.get(f"quantize_nv_{t}"), rooflines.get(f"quantize_nv_{t}_calibrated")
        if full and cal and full["avg_us"] > cal["avg_us"]:
            comps[f"quantize_nv_{t}_pass1_amax_GBps"] = round(n_el * 2.0 / ((full["avg_us"] - cal["avg_us"]) * 1e-6) / 1e9, 1)
            comps[f"quantize_nv_{t}_pass2_GBps"] = cal["achieved"]
    if "moe_h4096" in rooflines:
        m = rooflines["moe_h4096"]
        comps["moe_h4096_tokens_per_s"] = round(8192 / (m["avg_us"] * 1e-6), 1)
        comps["moe_h4096_tflops"] = m["achieved"]
    if "moe_h7168_decode64" in rooflines:
        m = rooflines["moe_h7168_decode64"]
        comps["moe_h7168_decode_tokens_per_s"] = round(64 / (m["avg_us"] * 1e-6), 1)
        comps["moe_h7168_decode_weight_GBps"] = m["achieved"]
        comps["moe_h7168_decode_frac_hbm"] = m["frac"]
    if "moe_h7168_prefill16384" in rooflines:
        m = rooflines["moe_h7168_prefill16384"]
        comps["moe_h7168_prefill_tokens_per_s"] = round(16384 / (m["avg_us"] * 1e-6), 1)
        comps["moe_h7168_prefill_tflops"] = m["achieved"]
        comps["moe_h7168_prefill_frac_16bit_peak"] = m["frac"]
        comps["moe_h7168_prefill_frac_fp4_peak"] = round(m["achieved"] / PEAK_FP4_TFLOPS, 4)
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
        "config": {"workload": "W4A4 MXFP4 GEMM M=N=K=4096 (bf16 out, fp32 accumulate) for value; per step also "
                               "MX/NV quantize of linear 4096x4096 W and 2048x4096 A, MX->NV remap, MX dequant, "
                               "MX -> FP8 dequant, "
                               "MX/NV fake-quant of W and its STE backward, MXFP4 KV-cache append (16384 x 512) "
                               "and FP4 indexer scores (64 x 32768 x 512), "
                               "NVFP4 and W4A8 (MXFP8 x MXFP4) GEMMs at 4096^3, "
                               "MoE hidden 4096 (384 experts, top-6, inter 2048, 8192 tokens, MXFP4) and "
                               "NVFP4 MoE hidden 7168 (inter 3072) at 64 decode and 16384 prefill tokens",
                   "accumulate": "fp32", "traffic_source": "profiles/traffic.json" if traffic else None},
        "components": comps,
        "roofline": {k: v for k, v in dom.items() if k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
                    | {"kernel": dom_name},
        "rooflines": rooflines,
        "gpu": gpu_info(torch),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


def moe_stage(torch, F, name, fmt, m, E, w13c, w13s, w2c, w2s, w13ts, w2ts, act, out, ws, weight_bytes, flops_gu,
              flops_dn, bound):
    """A MoE stage: one fp4_moe_grouped_gemm call with stage events."""
    dbg = F.MoeDebug()
    X = m.X.to("cuda")
    ids = torch.from_numpy(m.ids).to("cuda")
    wts = torch.from_numpy(m.weights).to("cuda")
    T, H = X.shape
    I, k = m.inter, m.ids.shape[1]

    def set_events(handles):
        for i, h in enumerate(handles):
            dbg.stage_events[i] = h

    def launch():
        F.fp4_moe_grouped_gemm(fmt, X, ids, wts, E, I, w13c, w13s, w2c, w2s, out, ws, w13_tensor_scales=w13ts,
                               w2_tensor_scales=w2ts, act_tensor_scales=act, debug=dbg)

    S = T * k
    blk = 32 if fmt == F.FMT_MX else 16
    qb = 2 + 0.5 + 1 / blk
    work = {
        "quantize_x": ("hbm", T * H * qb, f"{qb} B/elem of x"),
        "routing": ("hbm", S * 4 * 4, "16 B per slot (ids in, perm/slot_pos/placement out)"),
        "gate_up": (bound, flops_gu, "4*H*I flop per routed slot (g and u)"),
        "down": (bound, flops_dn, "2*H*I flop per routed slot"),
        "combine": ("hbm", S * H * 4 + T * H * 2, "4 B per slot per hidden column in, 2 B per token column out"),
    }
    nv_gu, nv_dn = (("moe_gate_up_nv_kernel<32, 3>", "moe_down_nv_kernel<32, 3>") if T <= 128 else
                    ("moe_gate_up_nvw_kernel", "moe_down_nvw_kernel"))   # the launcher's decode / wide NV tiles
    names = {"quantize_x": "mx_quantize_kernel" if fmt == F.FMT_MX else "nv_quantize_kernel",
             "routing": "route_count_kernel + route_scan_kernel + route_place_kernel",
             "gate_up": "moe_gate_up_mx256_kernel" if fmt == F.FMT_MX else
             (f"expand_nv16_kernel (x) + {nv_gu}" if T <= 128 else nv_gu),
             "down": "moe_down_mx256_kernel" if fmt == F.FMT_MX else nv_dn,
             "combine": "combine_kernel"}
    if bound == "hbm":
        # decode: the expert weights dominate the bytes of both GEMMs
        work["gate_up"] = ("hbm", weight_bytes * 2 / 3, "active experts' w1/w3 codes + scales")
        work["down"] = ("hbm", weight_bytes / 3, "active experts' w2 codes + scales")
        total_work, unit = weight_bytes, "active experts' weight bytes (codes + scales) per launch"
    else:
        total_work, unit = flops_gu + flops_dn, "6*H*I flop per routed slot"
    return Stage(name, launch, bound, total_work, unit, "MoE (all kernels)",
                 moe={"set_events": set_events, "work": work, "kernel_names": names})


def build_moe_h4096(torch, F, W, dev):
    """MXFP4 MoE layer at hidden 4096 (8192 tokens)."""
    m = W.moe_workload(4)
    T, H, I, E = 8192, m.hidden, m.inter, 384
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
    S = int(m.ids.size)
    per_expert = 3 * H * I * (0.5 + 1 / 32)
    return moe_stage(torch, F, "moe_h4096", F.FMT_MX, m, E, w13c, w13s, w2c, w2s, None, None, None, out, ws,
                     len(active) * per_expert, 4.0 * S * H * I, 2.0 * S * H * I, "mfma")


def build_moe_decode(torch, F, W, dev):
    """NVFP4 MoE layer at hidden 7168 on a decode batch of 64 tokens: the
    active experts' weights stream from HBM."""
    return build_moe_nv(torch, F, W, dev, 64, "moe_h7168_decode64", "hbm")


def build_moe_prefill(torch, F, W, dev):
    """NVFP4 MoE layer at hidden 7168 on a prefill batch of 16384 tokens: both
    grouped GEMMs are bound by the fp16 MFMA the exact NV expansion feeds."""
    return build_moe_nv(torch, F, W, dev, 16384, "moe_h7168_prefill16384", "mfma_bf16")


def build_moe_nv(torch, F, W, dev, tokens, name, bound):
    """NVFP4 MoE layer at hidden 7168 (inter 3072, 384 experts, top-6).  The
    activation tensor scales are calibrated: s_x from amax(x), s_h from amax(h)
    of one calibration call."""
    m = W.moe_workload(5, tokens)
    T, H, I, E = tokens, m.hidden, m.inter, 384
    active = sorted(set(m.ids.ravel().tolist()))
    w13c = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13s = torch.zeros((E, 2 * I, H // 16), dtype=torch.uint8, device=dev)
    w2c = torch.zeros((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2s = torch.zeros((E, H, I // 16), dtype=torch.uint8, device=dev)
    w13ts = torch.zeros(E, dtype=torch.float32, device=dev)
    w2ts = torch.zeros(E, dtype=torch.float32, device=dev)
    nvws = torch.empty(F.fp4_quantize_nv_workspace_bytes(1, 1), dtype=torch.uint8, device=dev)
    for e, a, b in W.expert_weights_device(5, E, H, I, dev):
        if e in active:
            F.fp4_quantize_nv(a, w13c[e], w13s[e], w13ts[e:e + 1], False, nvws)
            F.fp4_quantize_nv(b, w2c[e], w2s[e], w2ts[e:e + 1], False, nvws)
    X = m.X.to(dev)
    act = torch.tensor([float(X.abs().max()) / 2688.0, 1.0], dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(F.fp4_moe_workspace_bytes(F.FMT_NV, T, H, 6, E, I), dtype=torch.uint8, device=dev)
    S = int(m.ids.size)
    # calibration call: amax of h over this batch
    h = torch.empty((S, I), dtype=torch.bfloat16, device=dev)
    dbg = F.MoeDebug()
    dbg.h_bf16 = h.data_ptr()
    F.fp4_moe_grouped_gemm(F.FMT_NV, X, torch.from_numpy(m.ids).to(dev), torch.from_numpy(m.weights).to(dev), E, I,
                           w13c, w13s, w2c, w2s, out, ws, w13_tensor_scales=w13ts, w2_tensor_scales=w2ts,
                           act_tensor_scales=act, debug=dbg)
    torch.cuda.synchronize()
    act[1] = float(h.float().abs().max()) / 2688.0
    del h
    per_expert = 3 * H * I * (0.5 + 1 / 16)
    return moe_stage(torch, F, name, F.FMT_NV, m, E, w13c, w13s, w2c, w2s, w13ts, w2ts, act, out, ws,
                     len(active) * per_expert, 4.0 * S * H * I, 2.0 * S * H * I, bound)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in pools] or [os.cpu_count() or 1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('num_threads')} threads" for i in pools
                                 if i.get("user_api") == "blas"})) or "none found"
    except Exception:
        threads, blas = os.cpu_count() or 1, "unknown"
    return int(threads), blas


def _rows(fn, bits, n=512):
    return tuple(np.concatenate(p) for p in zip(*[fn(bits[i:i + n]) for i in range(0, bits.shape[0], n)]))


def _cpu_moe(workload, tokens, sample_tokens, fmt):
    """The MoE oracle (moe_forward) on the first `sample_tokens` tokens of the
    workload's batch.  Expert weights are pre-quantized inputs of the path, so
    the touched experts get seeded random codes and scales (the oracle's time
    does not depend on their values) and the routing ids are renumbered to them."""
    import workloads as W
    from oracle import moe as M
    m = W.moe_workload(workload, tokens)
    xb = W.bf16_bits(m.X[:sample_tokens])
    ids = m.ids[:sample_tokens]
    touched = np.unique(ids)
    local = np.searchsorted(touched, ids).astype(np.int32)
    n, H, I = len(touched), m.hidden, m.inter
    blk = 32 if fmt == "mx" else 16
    rng = np.random.default_rng(5)
    w13c = rng.integers(0, 256, (n, 2 * I, H // 2), dtype=np.uint8)
    w2c = rng.integers(0, 256, (n, H, I // 2), dtype=np.uint8)
    lo, hi = (118, 128) if fmt == "mx" else (0x28, 0x48)      # UE8M0 bytes / finite E4M3 bytes
    w13s = rng.integers(lo, hi, (n, 2 * I, H // blk), dtype=np.uint8)
    w2s = rng.integers(lo, hi, (n, H, I // blk), dtype=np.uint8)
    st = (np.full(n, 1e-3, np.float32), np.full(n, 1e-3, np.float32)) if fmt == "nv" else (None, None)
    act = (np.float32(2e-3), np.float32(1e-3)) if fmt == "nv" else (None, None)
    t0 = time.perf_counter()
    M.moe_forward(fmt, xb, local, m.weights[:sample_tokens], w13c, w13s, w2c, w2s, st[0], st[1], act_st=act)
    dt = time.perf_counter() - t0
    return dt, n


def cpu_baseline():
    """The CPU oracle, as it stands, timed on the host cores for every
    workload: the whole W4A4 GEMM (the `value` workload), the linear workload's
    quantizers and remap, the tiny workload, and bounded token samples of the
    three MoE workloads (stated in each entry's `sample`)."""
    import workloads as W
    from oracle import gemm as G
    from oracle import quant as Q
    threads, blas = _blas_threads()
    base = {"cores": threads, "kind": "oracle"}
    per = []
    # tiny workload: MX quantize of A and W and the GEMM
    wl1 = W.workload1()
    a1, w1 = W.bf16_bits(wl1.A), W.bf16_bits(wl1.W)
    t0 = time.perf_counter()
    G.gemm_ref("mx", *Q.mx_quantize(a1), *Q.mx_quantize(w1))
    dt = time.perf_counter() - t0
    per.append(dict(base, workload="tiny MXFP4 quantize + GEMM 32x512x256", value=round(dt * 1e6, 1),
                    unit="us per pass", sample="whole workload"))
    # linear workload: quantizers and remap
    wl2 = W.workload2()
    for name, bits in (("W 4096x4096", W.bf16_bits(wl2.W)), ("A 2048x4096", W.bf16_bits(wl2.A))):
        n = bits.size
        t0 = time.perf_counter()
        mq = _rows(Q.mx_quantize, bits)
        t_mx = time.perf_counter() - t0
        t0 = time.perf_counter()
        Q.nv_quantize(bits)
        t_nv = time.perf_counter() - t0
        t0 = time.perf_counter()
        Q.remap_mx_to_nv(*mq)
        t_rm = time.perf_counter() - t0
        per.append(dict(base, workload=f"linear {name}: MX quantize", value=round(n * 2.53125 / t_mx / 1e9, 4),
                        unit="GB/s", sample="whole tensor"))
        per.append(dict(base, workload=f"linear {name}: NV quantize (computed s_t)",
                        value=round(n * 2.5625 / t_nv / 1e9, 4), unit="GB/s", sample="whole tensor"))
        per.append(dict(base, workload=f"linear {name}: MX->NV remap", value=round(n * 0.09375 / t_rm / 1e9, 4),
                        unit="GB/s", sample="whole tensor"))
    # GEMM workload: A quantized, exact fp64 product and its bound, W pre-quantized
    wl = W.workload3()
    ab = W.bf16_bits(wl.A)
    eb = _rows(Q.mx_quantize, W.bf16_bits(wl.W))
    t0 = time.perf_counter()
    ea = _rows(Q.mx_quantize, ab)
    G.gemm_ref("mx", *ea, *eb)
    dt_gemm = time.perf_counter() - t0
    flops = 2.0 * 4096 ** 3
    gemm = dict(base, workload="W4A4 MXFP4 GEMM 4096^3", value=round(flops / dt_gemm / 1e12, 6), unit="TFLOP/s",
                sample="the whole 4096^3 W4A4 MXFP4 GEMM: MX-quantize A (fp64 numpy) and the exact fp64 product "
                       f"with its error bound, W pre-quantized; {dt_gemm:.1f} s")
    per.append(gemm)
    # MoE workloads on token samples
    for wl_, T, ns, fmt, label in ((4, None, 8, "mx", "MoE h4096 MXFP4, 8192 tokens"),
                                   (5, 64, 4, "nv", "MoE h7168 NVFP4, decode 64 tokens"),
                                   (5, 16384, 4, "nv", "MoE h7168 NVFP4, prefill 16384 tokens")):
        dt, ne = _cpu_moe(wl_, T, ns, fmt)
        per.append(dict(base, workload=label, value=round(ns / dt, 4), unit="tokens/s",
                        sample=f"the first {ns} tokens of the batch ({ns * 6} routed slots, {ne} experts): "
                               f"{dt:.1f} s; tokens/s = {ns} / time, extrapolated to the batch by token count "
                               "(each expert's weights are dequantized once per call, so a whole batch "
                               "would amortize that over more tokens)"))
    out = dict(gemm)
    out["sample"] = gemm["sample"] + f" (on {os.cpu_count()} host cores)"
    out.update(cpu_model=cpu_model(), os_cpu_count=os.cpu_count(), blas=blas, per_workload=per)
    return out


def gpu_info(torch):
    """Device name, architecture, compute units and the engine clock levels the
    driver lists (the stage times above run at whatever level the power
    manager picks; the peaks assume 2.4 GHz)."""
    info = {}
    try:
        p = torch.cuda.get_device_properties(0)
        info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count}
        rate = getattr(p, "clock_rate", None)
        if rate:
            info["max_sclk_mhz"] = round(rate / 1000)
    except Exception:
        pass
    levels = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                levels += [int(t.lower().split("mhz")[0].split()[-1]) for t in f.read().split("\n") if "mhz" in t.lower()]
        except (OSError, ValueError, IndexError):
            continue
    if levels:
        info["sclk_levels_mhz"] = sorted(set(levels))
    return info


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
