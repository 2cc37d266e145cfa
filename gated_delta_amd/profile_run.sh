#!/bin/bash
# Collects the rocprofv3 kernel summaries and the counter passes behind
# profiles/: kernel trace + stats of the bench's timed steps (and, in passes
# of their own, of the one-pass multi-token decode, the output norm and gate,
# the prologue, the decode step with the prologue in front, the
# per-channel-decay prefill, the segmented state pass and the prefill fused
# with the output norm and gate), then one FETCH_SIZE and one
# WRITE_SIZE pass over the prefill alone, each of those, and a plain device
# copy of known size (the counter calibration), then one pass of the MFMA
# counters over the prefill.
#   usage: gated_delta_amd/profile_run.sh OUTDIR
# Raw rocprofv3 output lands in OUTDIR/prof_*; then
#   python gated_delta_amd/profile_summary.py OUTDIR
# condenses it into profiles/.
set -o pipefail
R="$(cd "$(dirname "$0")/.." && pwd)"
OUT="$(mkdir -p "${1:?output directory}" && cd "$1" && pwd)"
cd /tmp && export TMPDIR=/tmp
echo "== kernel trace + stats: python bench.py --steps 20 --warmup 3 --no-cpu --no-extras --processes 1"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace" -o trace \
    -- python -u "$R/bench.py" --steps 20 --warmup 3 --no-cpu --no-extras --processes 1 \
    > "$OUT/prof_trace.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode decode_tokens --steps 20 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_dt" -o trace \
    -- python -u "$R/bench.py" --mode decode_tokens --steps 20 --no-cpu \
    > "$OUT/prof_trace_dt.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode output_norm_gate --steps 20 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_ep" -o trace \
    -- python -u "$R/bench.py" --mode output_norm_gate --steps 20 --no-cpu \
    > "$OUT/prof_trace_ep.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode prologue --steps 20 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_pro" -o trace \
    -- python -u "$R/bench.py" --mode prologue --steps 20 --no-cpu \
    > "$OUT/prof_trace_pro.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode decode_prologue --steps 10 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_dp" -o trace \
    -- python -u "$R/bench.py" --mode decode_prologue --steps 10 --no-cpu \
    > "$OUT/prof_trace_dp.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode prefill_diag --steps 10 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_diag" -o trace \
    -- python -u "$R/bench.py" --mode prefill_diag --steps 10 --no-cpu \
    > "$OUT/prof_trace_diag.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode segments --steps 10 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_seg" -o trace \
    -- python -u "$R/bench.py" --mode segments --steps 10 --no-cpu \
    > "$OUT/prof_trace_seg.log" 2>&1 || exit $?
echo "== kernel trace + stats: python bench.py --mode prefill_norm_gate --steps 10 --no-cpu"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_png" -o trace \
    -- python -u "$R/bench.py" --mode prefill_norm_gate --steps 10 --no-cpu \
    > "$OUT/prof_trace_png.log" 2>&1 || exit $?
for ctr in FETCH_SIZE WRITE_SIZE; do
  for mode in prefill copy decode_tokens output_norm_gate prologue decode_prologue prefill_diag; do
    echo "== pmc $ctr: python bench.py --mode $mode --steps 2 --warmup 1 --no-cpu"
    timeout -s KILL 120 rocprofv3 --pmc $ctr --output-format csv -d "$OUT/prof_${ctr}_$mode" -o pmc \
        -- python -u "$R/bench.py" --mode $mode --steps 2 --warmup 1 --no-cpu \
        > "$OUT/prof_${ctr}_$mode.log" 2>&1 || exit $?
  done
done
MFMA="SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES"
echo "== pmc MFMA counters: python bench.py --mode prefill --steps 2 --warmup 1 --no-cpu"
timeout -s KILL 120 rocprofv3 --pmc $MFMA --output-format csv -d "$OUT/prof_MFMA_prefill" -o pmc \
    -- python -u "$R/bench.py" --mode prefill --steps 2 --warmup 1 --no-cpu \
    > "$OUT/prof_MFMA_prefill.log" 2>&1 || exit $?
for cfg in 1 2 4; do
  echo "== kernel trace + stats: python bench.py --mode prefill_config --config $cfg --steps 10 --warmup 2 --no-cpu"
  timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/prof_trace_c$cfg" -o trace \
      -- python -u "$R/bench.py" --mode prefill_config --config $cfg --steps 10 --warmup 2 --no-cpu \
      > "$OUT/prof_trace_c$cfg.log" 2>&1 || exit $?
  echo "== pmc MFMA counters: python bench.py --mode prefill_config --config $cfg --steps 2 --warmup 1 --no-cpu"
  timeout -s KILL 120 rocprofv3 --pmc $MFMA --output-format csv -d "$OUT/prof_MFMA_c$cfg" -o pmc \
      -- python -u "$R/bench.py" --mode prefill_config --config $cfg --steps 2 --warmup 1 --no-cpu \
      > "$OUT/prof_MFMA_c$cfg.log" 2>&1 || exit $?
done
echo "== done"
