"""Measured peak rates of the MI355X units the block-scaled FP4 kernels are
bound by (block_scaled_fp4_mx_amd/probes/peak.hip): matrix-core rate of each
MFMA shape the kernels issue, device copy bandwidth, and the per-CU rate of the
global-to-LDS DMA that feeds the LDS-staged GEMM tiles, and the LDS read rate.  These are the
denominators the roofline figures in bench.py can be read against, next to the
data-sheet peaks.

    python peak_probe.py [--quick] [--out FILE]

prints one JSON line; --out also writes a short text summary.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "block_scaled_fp4_mx_amd", "probes", "libfp4_peak.so")

MFMA = [  # kind, name, data-sheet dense peak in TFLOP/s
    (0, "scaled MFMA 16x16x128, E2M1 x E2M1 (MX GEMM, MX MoE tiles)", 10100.0),
    (1, "scaled MFMA 32x32x64, E2M1 x E2M1", 10100.0),
    (2, "scaled MFMA 16x16x128, E2M1 x E4M3 (W4A8 GEMM)", 5000.0),
    (3, "MFMA 16x16x32 f16 (NV tiles, expanded operands)", 2500.0),
]


def load():
    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is missing: build with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB)
    d = ctypes.c_double
    lib.peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(d)]
    lib.peak_copy.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.POINTER(d)]
    lib.peak_lds_dma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(d)]
    lib.peak_lds_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(d)]
    for f in (lib.peak_mfma, lib.peak_copy, lib.peak_lds_dma, lib.peak_lds_read):
        f.restype = ctypes.c_int
    return lib


def run(quick=False):
    lib = load()
    out = ctypes.c_double()

    def call(fn, *args):
        rc = fn(*args, ctypes.byref(out))
        if rc != 0:
            raise RuntimeError(f"{fn.__name__}{args} failed with {rc}")
        return out.value

    iters = 200 if quick else 2000
    reps = 2 if quick else 5
    res = {"mfma": [], "copy": None, "lds_dma": None, "lds_read": None}
    for kind, name, spec in MFMA:
        rates = {g: round(call(lib.peak_mfma, kind, g, iters, reps), 1) for g in (256, 512)}
        best = max(rates.values())
        res["mfma"].append({"kind": name, "tflops_256_groups": rates[256], "tflops_512_groups": rates[512],
                            "spec_tflops": spec, "frac_of_spec": round(best / spec, 4)})
        print(f"{name:60s} {rates[256]:9.1f} / {rates[512]:9.1f} TFLOP/s  ({best / spec:.1%} of {spec:.0f})",
              file=sys.stderr, flush=True)
    nbytes = (32 if quick else 256) << 20
    gbps = call(lib.peak_copy, nbytes, reps * 4)
    res["copy"] = {"bytes": nbytes, "gbps": round(gbps, 1), "spec_gbps": 8000.0, "frac_of_spec": round(gbps / 8000.0, 4)}
    print(f"device copy of {nbytes >> 20} MiB (read + write)                     {gbps:9.1f} GB/s", file=sys.stderr,
          flush=True)
    dma = {}
    for g in (1, 256):
        dma[g] = round(call(lib.peak_lds_dma, g, iters, reps), 2)
    res["lds_dma"] = {"gbps_per_workgroup_alone": dma[1], "gbps_per_workgroup_256": dma[256],
                      "gbps_total_256": round(dma[256] * 256, 1)}
    print(f"global_load_lds_dwordx4 per workgroup: alone {dma[1]:.1f} GB/s, 256 at once {dma[256]:.1f} GB/s each "
          f"({dma[256] * 256 / 1000:.2f} TB/s in all)", file=sys.stderr, flush=True)
    rd = round(call(lib.peak_lds_read, 256, iters * 4, reps), 1)
    res["lds_read"] = {"gbps_per_workgroup_256": rd, "bytes_per_clock_at_2400mhz": round(rd / 2.4, 1)}
    print(f"ds_read_b128 per workgroup (256 at once): {rd:.1f} GB/s ({rd / 2.4:.1f} B per 2.4 GHz clock)",
          file=sys.stderr, flush=True)
    return res


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--quick", action="store_true", help="short runs (tests)")
    p.add_argument("--out", default="", help="also write a text summary to this file")
    a = p.parse_args()
    res = run(a.quick)
    print(json.dumps(res))
    if a.out:
        with open(a.out, "w") as f:
            f.write("Measured peak rates on MI355X (block_scaled_fp4_mx_amd/probes/peak.hip).\n")
            f.write(f"command: python peak_probe.py{' --quick' if a.quick else ''} --out <file>\n\n")
            f.write("Matrix cores, from registers (8 waves per workgroup, independent accumulators, random operands\n"
                    "and scale bytes), at 256 and 512 workgroups:\n")
            for m in res["mfma"]:
                f.write(f"  {m['kind']:60s} {m['tflops_256_groups']:9.1f} / {m['tflops_512_groups']:9.1f} TFLOP/s"
                        f"  {m['frac_of_spec']:.1%} of the {m['spec_tflops']:.0f} TFLOP/s figure\n")
            c = res["copy"]
            f.write(f"\nDevice copy of {c['bytes'] >> 20} MiB: {c['gbps']:.1f} GB/s read + write "
                    f"({c['frac_of_spec']:.1%} of 8000 GB/s)\n")
            d = res["lds_dma"]
            f.write(f"\nglobal_load_lds_dwordx4 from an L2-resident 1 MiB source, 64 KiB per workgroup per round:\n"
                    f"  one workgroup alone {d['gbps_per_workgroup_alone']:.1f} GB/s; 256 workgroups "
                    f"{d['gbps_per_workgroup_256']:.1f} GB/s each, {d['gbps_total_256']:.1f} GB/s in all\n")
            r = res["lds_read"]
            f.write(f"\nds_read_b128, 8 waves per workgroup, 256 workgroups: {r['gbps_per_workgroup_256']:.1f} GB/s per "
                    f"workgroup ({r['bytes_per_clock_at_2400mhz']:.1f} B per clock at 2.4 GHz)\n")


if __name__ == "__main__":
    main()
