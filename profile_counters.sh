#!/bin/bash
# rocprofv3 profiles of bench.py's stages on an MI355X: kernel durations of
# the whole benchmark, HBM traffic (FETCH_SIZE, then WRITE_SIZE, one counter
# per pass) of the main stages and of a plain 256 MiB device copy that
# calibrates the counters, and the matrix-core busy cycles, MFMA operation
# counts and LDS bank conflicts of the MFMA-bound stages.  The summaries go to
# $PROFILE_SUMMARY_DIR (default profiles/), merged with a traffic.json there
# that was taken on the same kernel sources.  Raw output goes to $PROFILE_OUT (default
# gpurun_out/profile); profile_summary.py writes the text summaries and
# profiles/traffic.json that bench.py reads.
set -euo pipefail
R=$(cd "$(dirname "$0")" && pwd)
OUT=${PROFILE_OUT:-$R/gpurun_out/profile}
mkdir -p "$OUT"
cd /tmp
export TMPDIR=/tmp

# PROFILE_PARTS picks the parts to run (default all): trace, traffic, mfma.
PARTS=${PROFILE_PARTS:-trace traffic mfma}

if [[ " $PARTS " == *" trace "* ]]; then
    echo "kernel trace of the whole benchmark"
    timeout -k 10 900 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
        python3 "$R/bench.py" --steps 5 --warmup 1 --no-cpu-baseline > "$OUT/trace.log" 2>&1
fi

if [[ " $PARTS " == *" traffic "* ]]; then
    for grp in copy_256MiB gemm_mx_4096 gemm_nv_4096 gemm_w4a8_4096 gemm_quantize_A_mxfp8 quantize_mx_W quantize_nv_W \
               dequant_fp8_W fake_quant_mx_W ste_backward_W indexer_scores_64x32768 \
               moe_h4096 moe_h7168_decode64 moe_h7168_prefill16384; do
        for ctr in FETCH_SIZE WRITE_SIZE; do
            echo "counter $ctr on $grp"
            timeout -s KILL 400 rocprofv3 --pmc "$ctr" --output-format csv -d "$OUT/pmc_${grp}_${ctr}" -o run -- \
                python3 "$R/bench.py" --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration --only "$grp" \
                > "$OUT/pmc_${grp}_${ctr}.log" 2>&1
        done
    done
fi

# matrix-core and LDS counters of the MFMA-bound stages, one pass (7 SQ + 1 GRBM counters)
MFMA_CTRS="SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE"
if [[ " $PARTS " == *" mfma "* ]]; then
    for grp in gemm_mx_4096 gemm_nv_4096 gemm_w4a8_4096 moe_h4096 moe_h7168_decode64 moe_h7168_prefill16384; do
        echo "matrix-core and LDS counters on $grp"
        timeout -s KILL 400 rocprofv3 --pmc $MFMA_CTRS --output-format csv -d "$OUT/mfma_${grp}" -o run -- \
            python3 "$R/bench.py" --steps 3 --warmup 1 --no-cpu-baseline --only "$grp" \
            > "$OUT/mfma_${grp}.log" 2>&1
    done
fi

python3 "$R/profile_summary.py" "$OUT" "${PROFILE_SUMMARY_DIR:-$R/profiles}"
