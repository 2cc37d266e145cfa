"""Condense the rocprofv3 output of profile_run.sh into profiles/.

usage: python gated_delta_amd/profile_summary.py OUTDIR

Writes
  profiles/kernels_rda_prefill_T16384_H16_decode_B256_H16.txt
      per-kernel call count and average / total duration of the bench's
      timed steps (kernel trace + stats);
  profiles/kernels_rda_decode_tokens_B256_T3_H16.txt
      the same for the one-pass multi-token decode (bench --mode decode_tokens);
  profiles/kernels_rda_output_norm_gate_rows262144.txt
      the same for the output norm and gate (bench --mode output_norm_gate);
  profiles/kernels_rda_prologue_T16384_H16.txt
      the same for the prologue (bench --mode prologue);
  profiles/kernels_rda_decode_step_prologue_B256_H16.txt
      the same for the decode step with the prologue in front, beside the
      plain decode step (bench --mode decode_prologue);
  profiles/kernels_rda_prefill_diag_T16384_H16.txt
      the same for the per-channel-decay prefill (bench --mode prefill_diag);
  profiles/kernels_rda_prefill_segmented_T16384_H2.txt
      the same for the segmented state pass beside the one-pass walk on the
      long prompt's first two heads (bench --mode segments);
  profiles/kernels_rda_prefill_norm_gate_T16384_H16.txt
      the same for the prefill alone, followed by the output norm and gate,
      and fused with it (bench --mode prefill_norm_gate);
  profiles/hbm_traffic.txt
      FETCH_SIZE and WRITE_SIZE per dispatch of every prefill kernel, each
      scaled by what the same counter reads for a device copy of known size,
      as bytes per launch (read by bench.py for its roofline entry), with the
      hash of the kernel sources they were taken on.
"""
import csv
import glob
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


sys.path.insert(0, ROOT)
from gated_delta_amd.srchash import kernel_source_hash as source_hash  # noqa: E402


# HIP kernel -> the stage name bench.py reports it under
STAGE = {"chunk_table_kernel": "rda_chunk_table", "prep_bf16_kernel": "rda_prep",
         "walk_bf16_kernel": "rda_walk", "decode_step_kernel": "rda_decode_step",
         "decode_tokens_kernel": "rda_decode_tokens", "norm_gate_kernel": "rda_output_norm_gate",
         "prologue_kernel": "rda_prologue", "prep_diag_kernel": "rda_prep_diag",
         "walk_diag_kernel": "rda_walk_diag", "segment_combine_kernel": "rda_segment_combine",
         "prep_kernel": "rda_prep", "walk_kernel": "rda_walk",
         "decode_prologue_kernel": "rda_decode_step_prologue"}

# the other prefill workloads: bench --mode prefill_config --config N
CONFIGS = {1: ("T64_H1_fp32", "one fp32 head of 64 tokens (S0 = 0)"),
           2: ("T2048_H16", "T=2048 x H=16, bf16 q/k/v, S0 = 0"),
           4: ("varlen8_T32768_H16", "8 packed sequences, 32768 tokens x H=16 in all, bf16 "
                                     "q/k/v, S0 per sequence")}


def short(name: str) -> str:
    n = name.replace("rda::(anonymous namespace)::", "").replace("void ", "")
    n = n.replace("rda::", "")
    return n.split("(")[0].split("<")[0].strip()


def find(d, pattern):
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        sys.exit(f"no {pattern} under {d}")
    return hits[0]


PREP_KERNELS = ("prep_bf16_kernel", "prep_kernel", "prep_diag_kernel")


def counter(d, name):
    """Average per-dispatch value of counter `name` by kernel (first launch of
    each kernel skipped when it ran more than once)."""
    rows = list(csv.DictReader(open(find(d, "*counter_collection.csv"))))
    by = {}
    for r in rows:
        if r["Counter_Name"] != name:
            continue
        by.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v[1:] if len(v) > 1 else v) for k, v in by.items()}


def counter_per_call(d, name):
    """Counter `name` summed per prefill call, by kernel: a call starts at each
    dispatch of a prep kernel (every prefill plan launches one per call); the
    first call is skipped.  Returns ({kernel: value per call}, {kernel:
    launches per call}), or empty dicts when the pass ran no prep kernel."""
    rows = [r for r in csv.DictReader(open(find(d, "*counter_collection.csv")))
            if r["Counter_Name"] == name]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    starts = [i for i, r in enumerate(rows) if short(r["Kernel_Name"]) in PREP_KERNELS]
    if len(starts) < 2:
        return {}, {}
    kept = rows[starts[1]:]
    calls = len(starts) - 1
    tot, cnt = {}, {}
    for r in kept:
        k = short(r["Kernel_Name"])
        tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
        cnt[k] = cnt.get(k, 0) + 1
    return {k: v / calls for k, v in tot.items()}, {k: v / calls for k, v in cnt.items()}


def calls_in_trace(rows):
    """Prefill calls in a kernel-trace pass: the dispatches of its prep kernel."""
    return sum(int(r["Calls"]) for r in rows if short(r["Name"]) in PREP_KERNELS)


def kernel_table(trace_dir, path, header, templates=False):
    """Write the per-kernel call count / average / total of one kernel-trace
    pass to `path` under `header`; returns the stats rows.  templates: keep
    the template arguments in the names (instantiations listed apart)."""
    rows = list(csv.DictReader(open(find(trace_dir, "*kernel_stats.csv"))))
    name = short
    if templates:
        def name(n):
            n = n.replace("rda::(anonymous namespace)::", "").replace("void ", "")
            return n.replace("rda::", "").split("(")[0].strip()
    ncalls = calls_in_trace(rows)
    lines = header + [f"# kernel sources: {source_hash()}"]
    if ncalls:
        lines.append(f"# prefill calls in the pass: {ncalls} (dispatches of the prep kernel); "
                     "us_per_call = total_us / calls")
    lines.append(f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'total_us':>12s} {'pct':>6s}"
                 + (f" {'us_per_call':>12s}" if ncalls else ""))
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{name(r['Name'])[:40]:40s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['TotalDurationNs']) / 1e3:12.1f} "
                     f"{float(r['Percentage']):6.2f}"
                     + (f" {float(r['TotalDurationNs']) / 1e3 / ncalls:12.2f}" if ncalls else ""))
    open(path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return rows


def main():
    out = sys.argv[1]
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)

    # ---- kernel trace summary ------------------------------------------------
    rows = kernel_table(
        os.path.join(out, "prof_trace"),
        os.path.join(prof, "kernels_rda_prefill_T16384_H16_decode_B256_H16.txt"),
        ["# rocprofv3 kernel trace, the bench's timed steps: RDA prefill T=16384 H=16",
         "# d=128 (bf16 q/k/v, fp32 state) + one RDA decode step B=256 H=16; 3 warmup + 20",
         "# timed steps, then 20 per-stage prefill calls (each followed by a decode step)",
         "# command: gated_delta_amd/profile_run.sh OUTDIR, whose first pass is",
         "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace -o trace \\",
         "#     -- python bench.py --steps 20 --warmup 3 --no-cpu --no-extras --processes 1",
         "# then python gated_delta_amd/profile_summary.py OUTDIR"])
    if os.path.isdir(os.path.join(out, "prof_trace_dt")):
        kernel_table(
            os.path.join(out, "prof_trace_dt"),
            os.path.join(prof, "kernels_rda_decode_tokens_B256_T3_H16.txt"),
            ["# rocprofv3 kernel trace, the one-pass multi-token decode: rda_decode_tokens on",
             "# B=256 sequences x H=16 heads, T=3 tokens (one token plus two drafts), bf16",
             "# q/k/v, per-sequence accept counts, fp32 states in place; 20 calls, each after a",
             "# 512 MiB read (reduce_kernel: the cache flush) and followed by a state restore",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose second pass is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_dt -o trace \\",
             "#     -- python bench.py --mode decode_tokens --steps 20 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"])

    if os.path.isdir(os.path.join(out, "prof_trace_ep")):
        kernel_table(
            os.path.join(out, "prof_trace_ep"),
            os.path.join(prof, "kernels_rda_output_norm_gate_rows262144.txt"),
            ["# rocprofv3 kernel trace, the output norm and gate: rda_output_norm_gate on the",
             "# long prompt's 16384 x 16 = 262144 output rows of 128 (fp32 o, bf16 gate, bf16",
             "# out, sigmoid gate, weight); 20 calls, each after a 512 MiB read (reduce_kernel:",
             "# the cache flush)",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose third pass is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_ep -o trace \\",
             "#     -- python bench.py --mode output_norm_gate --steps 20 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"])

    if os.path.isdir(os.path.join(out, "prof_trace_pro")):
        kernel_table(
            os.path.join(out, "prof_trace_pro"),
            os.path.join(prof, "kernels_rda_prologue_T16384_H16.txt"),
            ["# rocprofv3 kernel trace, the prologue: rda_prologue on the long prompt, 16384",
             "# tokens x 16 heads (bf16 raw q, k, v; conv width 4 with a history; SiLU; q/k",
             "# norm; write gate; b and the floored decay); 20 calls, each after a 512 MiB",
             "# read (reduce_kernel: the cache flush)",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose fourth pass is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_pro -o trace \\",
             "#     -- python bench.py --mode prologue --steps 20 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"])

    if os.path.isdir(os.path.join(out, "prof_trace_dp")):
        kernel_table(
            os.path.join(out, "prof_trace_dp"),
            os.path.join(prof, "kernels_rda_decode_step_prologue_B256_H16.txt"),
            ["# rocprofv3 kernel trace, the decode step with the prologue in front:",
             "# rda_decode_step_prologue on B=256 sequences x H=16 heads (bf16 raw q, k, v;",
             "# conv width 4, SiLU, the history updated in place; fp32 states in place),",
             "# then rda_decode_step on the same states; 11 calls of each, each after a",
             "# 512 MiB read (reduce_kernel: the cache flush)",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose pass for it is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_dp -o trace \\",
             "#     -- python bench.py --mode decode_prologue --steps 10 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"])

    if os.path.isdir(os.path.join(out, "prof_trace_diag")):
        kernel_table(
            os.path.join(out, "prof_trace_diag"),
            os.path.join(prof, "kernels_rda_prefill_diag_T16384_H16.txt"),
            ["# rocprofv3 kernel trace, the per-channel-decay prefill: rda_prefill_diag on the",
             "# long prompt, 16384 tokens x 16 heads (bf16 q/k/v, a decay per key channel,",
             "# S0 ~ N(0, 0.02)), the overlapped plan in chunk ranges: chunk table, prep_diag",
             "# (the first range), walk_diag once per range (each launch also preps the next",
             "# range on the CUs the walk leaves idle); 11 calls, each after a 512 MiB read",
             "# (reduce_kernel: the cache flush); us_per_call sums a call's launches",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose fifth pass is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_diag -o trace \\",
             "#     -- python bench.py --mode prefill_diag --steps 10 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"])

    if os.path.isdir(os.path.join(out, "prof_trace_seg")):
        kernel_table(
            os.path.join(out, "prof_trace_seg"),
            os.path.join(prof, "kernels_rda_prefill_segmented_T16384_H2.txt"),
            ["# rocprofv3 kernel trace, the segmented state pass: rda_prefill on the long",
             "# prompt's first 2 heads (16384 tokens x 2 heads, bf16 q/k/v, S0 ~ N(0, 0.02)),",
             "# P = 8 segments: prep, walk_bf16_kernel<false> (every segment from zero and",
             "# from the identity), segment_combine_kernel, walk_bf16_kernel<true> (outputs);",
             "# then the same inputs through the one-pass walk (cu_seqlens = {0, T}: chunk",
             "# table, prep, walk_bf16_kernel<true>); then the same two ways with a",
             "# per-channel decay (prep_diag_kernel, walk_diag_kernel<false>, the combine,",
             "# walk_diag_kernel<true>); 11 calls of each, each after a 512 MiB read",
             "# (reduce_kernel: the cache flush).  The <true> walks average the output pass",
             "# and the one-pass walk; the combine averages the two decays.",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose sixth pass is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_seg -o trace \\",
             "#     -- python bench.py --mode segments --steps 10 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"], templates=True)

    if os.path.isdir(os.path.join(out, "prof_trace_png")):
        kernel_table(
            os.path.join(out, "prof_trace_png"),
            os.path.join(prof, "kernels_rda_prefill_norm_gate_T16384_H16.txt"),
            ["# rocprofv3 kernel trace, the long prompt (16384 x 16, bf16 q/k/v, S0 ~ N(0,",
             "# 0.02)) three ways: rda_prefill alone, rda_prefill then rda_output_norm_gate",
             "# (bf16 gate and out), and rda_prefill_norm_gate (the fused form, whose norm",
             "# pass is norm_gate_kernel<..., true>); 11 calls of each, each after a 512 MiB",
             "# read (reduce_kernel: the cache flush)",
             "# command: gated_delta_amd/profile_run.sh OUTDIR, whose seventh pass is",
             "#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_png -o trace \\",
             "#     -- python bench.py --mode prefill_norm_gate --steps 10 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"], templates=True)

    # ---- HBM traffic -------------------------------------------------------------
    n = 1 << 30   # bytes the calibration copy reads and writes per launch
    f_copy = counter(os.path.join(out, "prof_FETCH_SIZE_copy"), "FETCH_SIZE")
    w_copy = counter(os.path.join(out, "prof_WRITE_SIZE_copy"), "WRITE_SIZE")
    fk = max(f_copy, key=f_copy.get)
    wk = max(w_copy, key=w_copy.get)
    f_scale = n / (f_copy[fk] * 1024.0)
    w_scale = n / (w_copy[wk] * 1024.0)
    fetch = counter(os.path.join(out, "prof_FETCH_SIZE_prefill"), "FETCH_SIZE")
    write = counter(os.path.join(out, "prof_WRITE_SIZE_prefill"), "WRITE_SIZE")
    fetch_call, per_call = counter_per_call(os.path.join(out, "prof_FETCH_SIZE_prefill"),
                                            "FETCH_SIZE")
    write_call, _ = counter_per_call(os.path.join(out, "prof_WRITE_SIZE_prefill"), "WRITE_SIZE")
    # the multi-token decode and the output norm and gate, from passes of
    # their own (only their own kernel: the flush and restores are not theirs)
    for mode, kern in (("decode_tokens", "decode_tokens_kernel"),
                       ("output_norm_gate", "norm_gate_kernel"), ("prologue", "prologue_kernel"),
                       ("decode_prologue", "decode_prologue_kernel"),
                       ("prefill_diag", "prep_diag_kernel"), ("prefill_diag", "walk_diag_kernel")):
        fd = os.path.join(out, f"prof_FETCH_SIZE_{mode}")
        wd = os.path.join(out, f"prof_WRITE_SIZE_{mode}")
        if os.path.isdir(fd) and os.path.isdir(wd):
            fm, wm = counter(fd, "FETCH_SIZE"), counter(wd, "WRITE_SIZE")
            if kern in fm and kern in wm:
                fetch[kern], write[kern] = fm[kern], wm[kern]
            # a prefill mode: also per call (the per-channel walk runs once per
            # chunk range of the overlapped plan)
            fcm, pcm = counter_per_call(fd, "FETCH_SIZE")
            wcm, _ = counter_per_call(wd, "WRITE_SIZE")
            if kern in fcm and kern in wcm:
                fetch_call[kern], write_call[kern], per_call[kern] = fcm[kern], wcm[kern], pcm[kern]
    lines = ["# HBM bytes per launch of the prefill kernels, RDA prefill T=16384 H=16 d=128",
             "# (bf16 q/k/v), of the one-pass multi-token decode (B=256 T=3 H=16), of the",
             "# output norm and gate (262144 rows), of the prologue (T=16384 H=16, conv",
             "# width 4), of the decode step with the prologue in front (B=256 H=16) and of",
             "# the per-channel-decay prefill's two kernels (T=16384 H=16).",
             "# FETCH_SIZE and WRITE_SIZE (KiB per",
             "# dispatch) from one rocprofv3 --pmc pass each, scaled by what the same counter",
             "# reads for a plain device copy of 1 GiB (bench.py --mode copy):",
             f"#   copy FETCH_SIZE = {f_copy[fk]:.0f} KiB -> scale {f_scale:.3f};"
             f" copy WRITE_SIZE = {w_copy[wk]:.0f} KiB -> scale {w_scale:.3f}",
             "# command: gated_delta_amd/profile_run.sh OUTDIR (passes",
             "#   rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d OUTDIR/prof_<ctr>_<mode> -o pmc \\",
             "#     -- python bench.py --mode prefill|copy|decode_tokens|output_norm_gate|prologue|\\",
             "#        decode_prologue|prefill_diag \\",
             "#        --steps 2 --warmup 1 --no-cpu)",
             "# then python gated_delta_amd/profile_summary.py OUTDIR",
             f"source_hash = {source_hash()}",
             f"fetch_scale = {f_scale:.4f}",
             f"write_scale = {w_scale:.4f}"]
    for k in sorted(set(fetch) | set(write)):
        fb = fetch.get(k, 0.0) * 1024.0 * f_scale
        wb = write.get(k, 0.0) * 1024.0 * w_scale
        name = STAGE.get(k, k)
        lines.append(f"{name}.kernel = {k}")
        lines.append(f"{name}.fetch_bytes = {fb:.0f}")
        lines.append(f"{name}.write_bytes = {wb:.0f}")
        lines.append(f"{name}.bytes_per_launch = {fb + wb:.0f}")
        if k in fetch_call and k in write_call:
            # per prefill call (the walk runs twice per call in the plan that
            # preps later chunks beside it)
            fcb = fetch_call[k] * 1024.0 * f_scale
            wcb = write_call[k] * 1024.0 * w_scale
            lines.append(f"{name}.launches_per_call = {per_call[k]:.2f}")
            lines.append(f"{name}.bytes_per_call = {fcb + wcb:.0f}")
    path = os.path.join(prof, "hbm_traffic.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))

    # ---- MFMA counters -------------------------------------------------------------
    mdir = os.path.join(out, "prof_MFMA_prefill")
    if os.path.isdir(mdir):
        mfma_summary(mdir, rows, os.path.join(prof, "mfma_rda_prefill_T16384_H16.txt"),
                     "RDA prefill T=16384", "H=16 d=128 (bf16 q/k/v)",
                     "--mode prefill --steps 2 --warmup 1 --no-cpu",
                     "prof_MFMA_prefill")
    for cid, (tag, what) in CONFIGS.items():
        tdir = os.path.join(out, f"prof_trace_c{cid}")
        mdir = os.path.join(out, f"prof_MFMA_c{cid}")
        if not (os.path.isdir(tdir) and os.path.isdir(mdir)):
            continue
        crows = kernel_table(
            tdir, os.path.join(prof, f"kernels_rda_prefill_{tag}.txt"),
            [f"# rocprofv3 kernel trace, the prefill workload {what}; 12 calls",
             f"# command: gated_delta_amd/profile_run.sh OUTDIR, whose pass for this workload is",
             f"#   rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/prof_trace_c{cid} -o trace \\",
             f"#     -- python bench.py --mode prefill_config --config {cid} --steps 10 --warmup 2 --no-cpu",
             "# then python gated_delta_amd/profile_summary.py OUTDIR"])
        mfma_summary(mdir, crows, os.path.join(prof, f"mfma_rda_prefill_{tag}.txt"),
                     "the prefill workload", what,
                     f"--mode prefill_config --config {cid} --steps 2 --warmup 1 --no-cpu",
                     f"prof_MFMA_c{cid}")


def mfma_summary(mdir, rows, path, what1, what2, bench_args, dname):
    """Executed MFMA work per launch of each kernel from one counter pass,
    with its rate over the kernel's average duration in `rows` (the kernel
    trace of the same workload)."""
    avg_us = {short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in rows}
    ncalls = calls_in_trace(rows)
    call_us = {short(r["Name"]): float(r["TotalDurationNs"]) / 1e3 / ncalls for r in rows} \
        if ncalls else {}
    m16_call, per_call = counter_per_call(mdir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    m32_call, _ = counter_per_call(mdir, "SQ_INSTS_VALU_MFMA_MOPS_F32")
    mops16 = counter(mdir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    mops32 = counter(mdir, "SQ_INSTS_VALU_MFMA_MOPS_F32")
    inst16 = counter(mdir, "SQ_INSTS_VALU_MFMA_BF16")
    busy = counter(mdir, "SQ_VALU_MFMA_BUSY_CYCLES")
    cu = counter(mdir, "SQ_BUSY_CU_CYCLES")
    lines = [f"# MFMA work executed per launch of the prefill kernels, {what1}",
             f"# {what2}, from one rocprofv3 --pmc pass:",
             "#   rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 \\",
             "#     SQ_INSTS_VALU_MFMA_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES \\",
             f"#     --output-format csv -d OUTDIR/{dname} -o pmc \\",
             f"#     -- python bench.py {bench_args}",
             "# (part of gated_delta_amd/profile_run.sh OUTDIR; then",
             "# python gated_delta_amd/profile_summary.py OUTDIR).  MOPS count 512 flops each;",
             "# the executed work includes the hi/lo split products.  Per call: every launch",
             "# of the kernel in one prefill call (a call starts at its prep kernel; the",
             "# first call skipped).  The rate divides the work per call by the kernel's",
             "# time per call in the kernel trace summary (its total over the calls); the",
             "# fraction is of the 2.5 PFLOP/s dense bf16 peak.  mfma_busy_per_simd = MFMA busy cycles",
             "# (summed over a CU's four SIMDs) / (4 x CU busy cycles).",
             f"source_hash = {source_hash()}"]
    for k in sorted(mops16):
        name = STAGE.get(k, k)
        f16 = mops16[k] * 512.0
        f32 = mops32.get(k, 0.0) * 512.0
        lines.append(f"{name}.kernel = {k}")
        lines.append(f"{name}.mfma_bf16_instructions = {inst16.get(k, 0.0):.0f}")
        lines.append(f"{name}.mfma_bf16_flops = {f16:.0f}")
        lines.append(f"{name}.mfma_f32_flops = {f32:.0f}")
        if k in m16_call:
            # per prefill call: every launch of the kernel in one call, over
            # the kernel's time per call in the trace
            c16 = m16_call[k] * 512.0
            c32 = m32_call.get(k, 0.0) * 512.0
            lines.append(f"{name}.launches_per_call = {per_call[k]:.2f}")
            lines.append(f"{name}.mfma_bf16_flops_per_call = {c16:.0f}")
            lines.append(f"{name}.mfma_f32_flops_per_call = {c32:.0f}")
            if call_us.get(k, 0) > 0:
                rate = (c16 + c32) / (call_us[k] * 1e-6) / 1e12
                lines.append(f"{name}.us_per_call = {call_us[k]:.2f}")
                lines.append(f"{name}.mfma_tflops = {rate:.2f}")
                lines.append(f"{name}.mfma_frac_of_bf16_peak = {rate / 2500.0:.4f}")
        elif k in avg_us and avg_us[k] > 0:
            rate = (f16 + f32) / (avg_us[k] * 1e-6) / 1e12
            lines.append(f"{name}.mfma_tflops = {rate:.2f}")
            lines.append(f"{name}.mfma_frac_of_bf16_peak = {rate / 2500.0:.4f}")
        if cu.get(k):
            # the busy count sums a CU's four SIMDs (16 cycles per 16x16x32
            # instruction), the CU count one per CU: per-SIMD utilisation
            lines.append(f"{name}.mfma_busy_per_simd = {busy.get(k, 0.0) / (4 * cu[k]):.4f}")
    open(path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
