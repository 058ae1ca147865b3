"""Summaries of the rocprofv3 output that profile_counters.sh collects.

Writes into the profiles directory:
  kernel_stats_bench.txt      per-kernel call counts and durations of one
                              benchmark run (--kernel-trace --stats);
  traffic_bench_stages.txt    HBM bytes per launch of the main stages and MoE
                              kernels (FETCH_SIZE, WRITE_SIZE), each scaled by
                              what the same counter reads for a plain 256 MiB
                              device copy (256 MiB read, 256 MiB written);
  mfma_lds_bench_stages.txt   matrix-core busy fraction, MFMA operations and
                              LDS bank conflicts per launch of the MFMA-bound
                              stages' kernels;
  traffic.json                the traffic and matrix-core figures for bench.py,
                              tagged with the digest of the kernel sources they
                              were taken on.
usage: python3 profile_summary.py <raw output dir> <profiles dir>
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
from bench import source_digest  # noqa: E402

TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o run -- "
             "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline")
PMC_CMD = ("rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <out>/pmc_<stage>_<counter> -o run -- "
           "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration --only <stage>")
MFMA_CMD = ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_INSTS_VALU_MFMA_MOPS_F16 "
            "SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE "
            "--output-format csv -d <out>/mfma_<stage> -o run -- python3 bench.py --steps 3 --warmup 1 "
            "--no-cpu-baseline --only <stage>")
MFMA_CTRS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_INSTS_VALU_MFMA_MOPS_F16",
             "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS",
             "GRBM_GUI_ACTIVE")
SIMDS = 1024          # 256 compute units x 4 SIMDs
XCCS = 8              # GRBM_GUI_ACTIVE is counted once per XCC; the sum over them is 8x the busy cycles
MFMA_ROWS = {
    "gemm_mx_4096": ("gemm_mx_4096", "gemm_mx_256_kernel", 2.0 * 4096 ** 3),
    "gemm_nv_4096": ("gemm_nv_4096", "gemm_nv_tile_kernel", 2.0 * 4096 ** 3),
    "gemm_w4a8_4096": ("gemm_w4a8_4096", "gemm_w4a8_256_kernel", 2.0 * 4096 ** 3),
    "moe_h4096.gate_up": ("moe_h4096", "moe_gate_up_mx256_kernel", 4.0 * 49152 * 4096 * 2048),
    "moe_h4096.down": ("moe_h4096", "moe_down_mx256_kernel", 2.0 * 49152 * 4096 * 2048),
    "moe_h7168_decode64.gate_up": ("moe_h7168_decode64", "moe_gate_up_nv_kernel", 4.0 * 384 * 7168 * 3072),
    "moe_h7168_decode64.down": ("moe_h7168_decode64", "moe_down_nv_kernel", 2.0 * 384 * 7168 * 3072),
    "moe_h7168_prefill16384.gate_up": ("moe_h7168_prefill16384", "moe_gate_up_nvw_kernel", 4.0 * 98304 * 7168 * 3072),
    "moe_h7168_prefill16384.down": ("moe_h7168_prefill16384", "moe_down_nvw_kernel", 2.0 * 98304 * 7168 * 3072),
}
COPY_BYTES = 256 << 20

# bench row -> (profiled stage, [(kernel-name substring, grid size or None)]); the
# row's bytes per launch are the sum over its kernels of the mean per dispatch
ROWS = {
    "gemm_mx_4096": ("gemm_mx_4096", [("gemm_mx_256_kernel", None)]),
    "quantize_mx_W": ("quantize_mx_W", [("mx_quantize_kernel", None)]),
    "quantize_nv_W": ("quantize_nv_W", [("nv_amax_kernel", None), ("nv_quantize_kernel", None)]),
    "dequant_fp8_W": ("dequant_fp8_W", [("scale_max_kernel", None), ("fp8_dequant_kernel", None)]),
    "moe_h4096.gate_up": ("moe_h4096", [("moe_gate_up_mx256_kernel", None)]),
    "moe_h4096.down": ("moe_h4096", [("moe_down_mx256_kernel", None)]),
    "moe_h4096.combine": ("moe_h4096", [("combine_kernel", None)]),
    "moe_h7168_decode64.gate_up": ("moe_h7168_decode64", [("moe_gate_up_nv_kernel", None),
                                                          ("expand_nv16_kernel", 64 * 7168 // 16)]),
    "moe_h7168_decode64.down": ("moe_h7168_decode64", [("moe_down_nv_kernel", None)]),
    "moe_h7168_decode64.combine": ("moe_h7168_decode64", [("combine_kernel", None)]),
    # prefill: both fp16 expansions run at the capped grid, so only the tile kernels are attributed
    "moe_h7168_prefill16384.gate_up": ("moe_h7168_prefill16384", [("moe_gate_up_nvw_kernel", None)]),
    "moe_h7168_prefill16384.down": ("moe_h7168_prefill16384", [("moe_down_nvw_kernel", None)]),
    "moe_h7168_prefill16384.combine": ("moe_h7168_prefill16384", [("combine_kernel", None)]),
    "gemm_nv_4096": ("gemm_nv_4096", [("gemm_nv_tile_kernel", None)]),
    "gemm_w4a8_4096": ("gemm_w4a8_4096", [("gemm_w4a8_256_kernel", None)]),
    "gemm_quantize_A_mxfp8": ("gemm_quantize_A_mxfp8", [("mxfp8_quantize_kernel", None)]),
    "fake_quant_mx_W": ("fake_quant_mx_W", [("mx_quantize_kernel<true, 1>", None)]),
    "ste_backward_W": ("ste_backward_W", [("ste_backward_kernel", None)]),
    "indexer_scores_64x32768": ("indexer_scores_64x32768", [("gemm_mx_skinny_kernel", None)]),
}


def short(name):
    n = name.replace("(anonymous namespace)::", "").replace("fp4::", "")
    return n.split("(")[0][:70]


def read_counter(raw, stage, counter, folder=None):
    """Per dispatch: (kernel name, grid size, value) of one counter of a pass
    (values summed over the counter's instances)."""
    folder = folder or f"pmc_{stage}_{counter}"
    files = glob.glob(os.path.join(raw, folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        return []
    vals = {}
    for r in csv.DictReader(open(files[0])):
        if r.get("Counter_Name") != counter:
            continue
        key = r["Dispatch_Id"]
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", "0")) or 0)
        ent = vals.setdefault(key, [r["Kernel_Name"], grid, 0.0])
        ent[2] += float(r["Counter_Value"])
    return list(vals.values())


def mean_for(disp, sub, grid):
    v = [x[2] for x in disp if sub in x[0] and (grid is None or x[1] == grid)]
    return (sum(v) / len(v), len(v)) if v else (None, 0)


def main(raw, prof):
    os.makedirs(prof, exist_ok=True)
    # ---- kernel durations
    stats = glob.glob(os.path.join(raw, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        rows = list(csv.DictReader(open(stats[0])))
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        with open(os.path.join(prof, "kernel_stats_bench.txt"), "w") as f:
            f.write("Kernel durations of one benchmark run on MI355X (rocprofv3 kernel trace).\n")
            f.write(f"command: {TRACE_CMD}\n")
            f.write("The run includes input setup (quantizing the rotating copies and the MoE expert weights),\n"
                    "1 warmup step, 5 timed steps and the per-stage timing launches.\n\n")
            f.write(f"{'kernel':72s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} {'total ms':>10s}\n")
            for r in rows:
                if "fp4::" not in r["Name"] and "copy" not in r["Name"].lower():
                    continue
                f.write(f"{short(r['Name']):72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                        f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                        f"{float(r['TotalDurationNs']) / 1e6:10.3f}\n")
    prev = {}
    try:
        with open(os.path.join(prof, "traffic.json")) as f:
            prev = json.load(f)
    except (OSError, ValueError):
        pass
    keep = prev if prev.get("source_digest") == source_digest() else {}
    out = {"source_digest": source_digest(), "counter_units": "KiB per dispatch"}
    t = traffic_summary(raw, prof)
    if t is not None:
        out.update(t)
    elif "kernels" in keep:
        out.update({k: keep[k] for k in ("copy_calibration", "kernels") if k in keep})
    m = mfma_summary(raw, prof)
    if m is not None:
        out["mfma"] = m
    elif "mfma" in keep:
        out["mfma"] = keep["mfma"]
    with open(os.path.join(prof, "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)


def traffic_summary(raw, prof):
    cf = read_counter(raw, "copy_256MiB", "FETCH_SIZE")
    cw = read_counter(raw, "copy_256MiB", "WRITE_SIZE")
    big = lambda d: max((x for x in d if "copy" in x[0].lower() or "Copy" in x[0]), key=lambda x: x[2], default=None)
    bf, bw = big(cf), big(cw)
    if not bf or not bw:
        print("no copy calibration found; traffic not written")
        return None
    ff = COPY_BYTES / (bf[2] * 1024.0)
    fw = COPY_BYTES / (bw[2] * 1024.0)
    out = {"copy_calibration": {"kernel": short(bf[0]), "fetch_kib": bf[2], "write_kib": bw[2],
                                "factor_fetch": ff, "factor_write": fw}, "kernels": {}}
    lines = []
    for row, (stage, parts) in ROWS.items():
        fd, wd = read_counter(raw, stage, "FETCH_SIZE"), read_counter(raw, stage, "WRITE_SIZE")
        fsum = wsum = 0.0
        ok = True
        detail = []
        for sub, grid in parts:
            fm, fn = mean_for(fd, sub, grid)
            wm, wn = mean_for(wd, sub, grid)
            if fm is None or wm is None:
                ok = False
                break
            fsum += fm * 1024.0 * ff
            wsum += wm * 1024.0 * fw
            detail.append(f"{sub}{'' if grid is None else f'[grid {grid}]'}: FETCH {fm:.0f} KiB x{fn}, WRITE {wm:.0f} KiB x{wn}")
        if not ok:
            continue
        out["kernels"][row] = {"fetch_bytes": round(fsum), "write_bytes": round(wsum),
                               "bytes_per_launch": round(fsum + wsum)}
        lines.append(f"{row:30s} read {fsum / 1e6:10.2f} MB  written {wsum / 1e6:10.2f} MB  total "
                     f"{(fsum + wsum) / 1e6:10.2f} MB   ({'; '.join(detail)})")
    with open(os.path.join(prof, "traffic_bench_stages.txt"), "w") as f:
        f.write("HBM traffic per launch of bench.py stages on MI355X (rocprofv3 counters, one counter per pass).\n")
        f.write(f"command (per stage and counter): {PMC_CMD}\n")
        f.write(f"calibration: a 256 MiB device copy ({short(bf[0])}) reads FETCH_SIZE {bf[2]:.0f} KiB and "
                f"WRITE_SIZE {bw[2]:.0f} KiB; bytes = counter * 1024 * (256 MiB / copy's counter bytes), "
                f"factors {ff:.4f} (fetch) and {fw:.4f} (write).\n")
        f.write(f"kernel sources digest: {source_digest()}\n\n")
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return out


def mfma_summary(raw, prof):
    """Per kernel, means over its dispatches: matrix-core busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (GRBM_GUI_ACTIVE per XCC
    x 1024 SIMDs)), matrix operations (MOPS x 512) against the algorithmic
    flops, and LDS bank-conflict cycles per LDS access cycle."""
    res, lines = {}, []
    for row, (stage, sub, flops) in MFMA_ROWS.items():
        vals = {}
        for c in MFMA_CTRS:
            d = read_counter(raw, stage, c, folder=f"mfma_{stage}")
            m, n = mean_for(d, sub, None)
            if m is None:
                break
            vals[c] = m
        if len(vals) != len(MFMA_CTRS):
            continue
        gui = vals["GRBM_GUI_ACTIVE"] / XCCS
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMDS) if gui else None
        ops = 512.0 * (vals["SQ_INSTS_VALU_MFMA_MOPS_F6F4"] + vals["SQ_INSTS_VALU_MFMA_MOPS_F16"] +
                       vals["SQ_INSTS_VALU_MFMA_MOPS_F8"])
        lds = vals["SQ_LDS_IDX_ACTIVE"] - vals["SQ_LDS_BANK_CONFLICT"]
        conf = vals["SQ_LDS_BANK_CONFLICT"] / lds if lds > 0 else None
        res[row] = {"mfma_busy": round(busy, 4) if busy is not None else None, "gui_active_cycles": round(gui),
                    "mfma_ops": ops, "algorithmic_flops": flops,
                    "lds_bank_conflicts_per_access": round(conf, 4) if conf is not None else None,
                    "raw": vals}
        lines.append(f"{row:32s} MFMA busy {100 * busy:6.1f}%  matrix ops {ops:.4g} (algorithmic {flops:.4g}, "
                     f"x{ops / flops:.3f})  LDS bank conflicts {conf if conf is None else round(conf, 4)} per access "
                     f"({vals['SQ_LDS_BANK_CONFLICT']:.4g} conflict / {vals['SQ_LDS_IDX_ACTIVE']:.4g} active cycles)  "
                     f"GUI active {gui:.4g} cycles")
    if not res:
        print("no matrix-core counters found")
        return None
    with open(os.path.join(prof, "mfma_lds_bench_stages.txt"), "w") as f:
        f.write("Matrix-core utilisation and LDS bank conflicts per launch of the MFMA-bound kernels of bench.py "
                "on MI355X (rocprofv3 counters, one pass per stage).\n")
        f.write(f"command (per stage): {MFMA_CMD}\n")
        f.write("MFMA busy = sum of SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs / (GRBM_GUI_ACTIVE per XCC x 1024); "
                "matrix ops = 512 x (MOPS_F6F4 + MOPS_F16 + MOPS_F8); LDS bank conflicts per access = "
                "SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT).  Means over the kernel's "
                "dispatches in the run (setup calls included).\n")
        f.write(f"kernel sources digest: {source_digest()}\n\n")
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return res

if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
