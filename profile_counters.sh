#!/bin/bash
# rocprofv3 profiles of bench.py's stages on an MI355X: kernel durations of
# the whole benchmark, then HBM traffic (FETCH_SIZE, then WRITE_SIZE, one
# counter per pass) of the main stages and of a plain 256 MiB device copy that
# calibrates the counters.  Raw output goes to $PROFILE_OUT (default
# gpurun_out/profile); profile_summary.py writes the text summaries and
# profiles/traffic.json that bench.py reads.
set -euo pipefail
R=$(cd "$(dirname "$0")" && pwd)
OUT=${PROFILE_OUT:-$R/gpurun_out/profile}
mkdir -p "$OUT"
cd /tmp
export TMPDIR=/tmp

echo "kernel trace of the whole benchmark"
timeout -k 10 900 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
    python3 "$R/bench.py" --steps 5 --warmup 1 --no-cpu-baseline > "$OUT/trace.log" 2>&1

for grp in copy_256MiB gemm_mx_4096 gemm_nv_4096 gemm_w4a8_4096 gemm_quantize_A_mxfp8 quantize_mx_W quantize_nv_W \
           fake_quant_mx_W ste_backward_W indexer_scores_64x32768 \
           moe_h4096 moe_h7168_decode64 moe_h7168_prefill16384; do
    for ctr in FETCH_SIZE WRITE_SIZE; do
        echo "counter $ctr on $grp"
        timeout -s KILL 400 rocprofv3 --pmc "$ctr" --output-format csv -d "$OUT/pmc_${grp}_${ctr}" -o run -- \
            python3 "$R/bench.py" --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration --only "$grp" \
            > "$OUT/pmc_${grp}_${ctr}.log" 2>&1
    done
done

python3 "$R/profile_summary.py" "$OUT" "$R/profiles"
