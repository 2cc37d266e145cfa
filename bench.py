"""Benchmark of the RDA token mixer hot path on one MI355X.

One step = one rda_prefill over the long-prompt workload (T = 16384 tokens,
H = 16 heads, d = 128, bf16 q/k/v, fp32 gates, S0 ~ N(0, 0.02)) plus one
rda_decode_step over the decode batch (B = 256 sequences x 16 heads, fp32
128 x 128 states updated in place; step i uses the (i mod 128)-th of 128
pre-drawn bf16 tokens).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line:
  value      prefill tokens/s on the long-prompt workload: T / the mean time of
             one rda_prefill call between HIP events on its stream (prep,
             then walk; the decode step between calls streams 512 MiB, so no
             prefill starts with its inputs in the Infinity Cache)
  decode     decode state bandwidth (algorithmic bytes / kernel time) of the
             steps between prefill calls, and of 128 steps back to back
             (back_to_back_128)
  roofline   the kernel with the largest time per step, against its bound
  kernels    every kernel's average duration (HIP events on its stream), from
             calls of rda_prefill_profiled; for one sequence without offsets
             the prep kernel writes the chunk table, so no table kernel runs
  cpu_baseline  the fp64 oracle on the same prefill inputs, host cores
  parity     rel-L2 / max-abs of this run's prefill output vs the oracle
The oracle runs only in this CPU leg (skipped with --no-cpu): the baseline
timing, and the parity figures of this run's outputs (parity, and the parity
entries of other_prefill_workloads, prefill_segmented, prefill_diag,
prologue, output_norm_gate and decode_tokens).
  also       the prefill back to back without the flush (ms_per_call_unflushed)
             and after a read-only 512 MiB flush (ms_per_call_read_flushed),
             the practical HBM rate of an in-place read-modify-write of 256 MiB
             (hbm_practical, and decode.frac_of_practical), and the three other
             prefill workloads -- one fp32 head of 64 tokens, T = 2048 x 16
             heads, 8 packed sequences of 32768 tokens x 16 heads -- each with
             time, algorithmic MFMA / HBM fractions and parity against the oracle
             (other_prefill_workloads); rda_decode_tokens on the decode batch
             with one token plus two drafts per sequence: one-pass verify +
             commit, read-only verify and commit-only, each with its state
             bandwidth (decode_tokens); the output norm and gate on the long
             prompt's 262144 output rows (output_norm_gate); the prologue on
             the long prompt and on the decode batch (prologue), and the
             whole block -- prologue, prefill, output norm and gate -- as
             tokens/s (output_norm_gate.block_tokens_per_s); the long prompt
             with a per-channel decay and the per-channel decode step
             (prefill_diag); the long prompt with 1, 2 and 4 of its heads
             (one GPU's share under head sharding), segmented state pass
             against the one-pass walk, and the same for the per-channel
             decay on 2 heads (prefill_segmented)

Usage: python bench.py [--gpus 1] [--steps 128] [--warmup 5] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("RDA prefill tokens/s (H=16,d=128,T=16384) + decode state HBM GB/s, 1 GPU")
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, vendor figure
D = 128
C = 64
# Algorithmic work per unit (token-head for prefill, (batch, head) for decode)
PREFILL_IN_BYTES = 3 * D * 2 + 2 * 4        # bf16 q, k, v + fp32 a, b   = 776
PREFILL_OUT_BYTES = D * 4                   # fp32 o                     = 512
PREFILL_BYTES = PREFILL_IN_BYTES + PREFILL_OUT_BYTES          # 1288
STATE_BYTES = D * D * 4                     # one fp32 state             = 65536
PREFILL_FLOPS = 6 * D * D + 5 * C * D + C * C // 3            # 140,629 (triangle-aware)
DECODE_BYTES = 2 * STATE_BYTES + PREFILL_IN_BYTES + PREFILL_OUT_BYTES   # 132,360


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0 = all)")
    ap.add_argument("--mode", choices=["bench", "prefill", "decode", "decode_tokens",
                                       "output_norm_gate", "prologue", "prefill_diag",
                                       "segments", "copy", "prefill_config",
                                       "decode_prologue", "prefill_norm_gate"],
                    default="bench",
                    help="prefill/decode: run only that part (for profiling); decode_tokens / "
                         "output_norm_gate / prologue / prefill_diag / segments: only the "
                         "one-pass multi-token decode / the output norm and gate / the long "
                         "prompt's prologue / its per-channel-decay prefill / its first two "
                         "heads through the segmented and the one-pass state pass, --steps "
                         "calls after a cache flush each; copy: a plain device copy of known "
                         "size (counter calibration); prefill_config: --steps calls of the "
                         "prefill workload --config (1 = one fp32 head of 64 tokens, 2 = "
                         "2048 x 16, 4 = 8 packed sequences of 32768 x 16 in all); "
                         "prefill_norm_gate: the long prompt's prefill alone, followed by "
                         "the output norm and gate, and with both fused")
    ap.add_argument("--config", type=int, choices=[1, 2, 4], default=2)
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps and the per-stage calls (the kernel trace "
                         "of exactly what the kernels entry reports)")
    ap.add_argument("--processes", type=int, default=3,
                    help="fresh processes timing the headline steps (this one included); "
                         "value is the median of their per-call times")
    ap.add_argument("--child", action="store_true",
                    help="internal: one extra timing process (headline steps only)")
    return ap.parse_args()


def spawn_timing_processes(args, n):
    """Runs the headline steps (W warmup + K timed, no extras, no oracle) in
    n fresh child processes, one after another, before this process touches
    the GPU; returns each child's parsed JSON line (None for a failed one)."""
    res = []
    for i in range(n):
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--child", "--steps",
               str(args.steps), "--warmup", str(args.warmup), "--no-cpu", "--no-extras",
               "--mode", args.mode]
        print(f"[bench] timing process {i + 2} of {n + 1}", file=sys.stderr, flush=True)
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
            lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
            res.append(json.loads(lines[-1]) if r.returncode == 0 and lines else None)
            if r.returncode != 0:
                print(r.stderr[-2000:], file=sys.stderr, flush=True)
        except (subprocess.TimeoutExpired, ValueError) as e:
            print(f"[bench] timing process failed: {e}", file=sys.stderr, flush=True)
            res.append(None)
    return res


from gated_delta_amd.srchash import kernel_source_hash  # noqa: E402


def read_profile(fname: str, key: str):
    """A value from a committed counter summary under profiles/, or None when
    the summary is missing or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    val = kv.get(key)
    return float(val) if val else None


def read_traffic(kernel: str):
    """HBM bytes of one kernel (FETCH_SIZE + WRITE_SIZE, calibrated) per
    prefill call when the summary has that figure (every launch in a call),
    else per launch."""
    per_call = read_profile("hbm_traffic.txt", f"{kernel}.bytes_per_call")
    return per_call if per_call is not None else read_profile("hbm_traffic.txt",
                                                              f"{kernel}.bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the RDA "
              "path here is a single-GPU kernel set; multi-GPU sharding is a design note, "
              "not a runnable mode.", file=sys.stderr)
        sys.exit(2)

    # the other fresh processes of the timing protocol run first, before this
    # process initialises the GPU (they are started as children, never exec'd)
    children = []
    if args.mode == "bench" and not args.child and args.processes > 1:
        children = spawn_timing_processes(args, args.processes - 1)

    import numpy as np
    import torch

    from gated_delta_amd import rda, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.mode == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.mode == "prefill_config":
        pc = synth.CONFIGS[args.config]()
        tok = (lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)) if pc.bf16 else \
            (lambda x: torch.from_numpy(x).to(dev))
        qc, kc, vc = tok(pc.q), tok(pc.k), tok(pc.v)
        ac, bc = torch.from_numpy(pc.a).to(dev), torch.from_numpy(pc.b).to(dev)
        S0c = torch.from_numpy(pc.S0).to(dev) if pc.S0 is not None else None
        for _ in range(args.warmup + args.steps):
            rda.rda_prefill(qc, kc, vc, ac, bc, cu_seqlens=pc.cu_seqlens, S0=S0c)
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "config": args.config, "T": pc.total_tokens,
                          "H": pc.num_heads, "calls": args.warmup + args.steps}), flush=True)
        return

    if args.mode in ("decode_tokens", "output_norm_gate", "prologue", "prefill_diag",
                     "segments", "decode_prologue", "prefill_norm_gate"):
        timed = make_timer(torch, np, stream)
        flush_buf = torch.ones((128 << 20,), dtype=torch.float32, device=dev)
        flush = lambda: flush_buf.sum()
        if args.mode == "prefill_norm_gate":
            res = fused_norm_gate_measurement(args, torch, np, rda, synth, dev, timed, flush,
                                              reps=args.steps)
        elif args.mode == "decode_prologue":
            res = decode_prologue_measurement(args, {}, torch, np, rda, synth, dev, timed, flush,
                                              reps=args.steps)
        elif args.mode == "decode_tokens":
            res = decode_tokens_measurements(args, {}, torch, np, rda, synth, dev, stream, timed,
                                             flush, reps=args.steps,
                                             modes=("verify_commit_in_place",))
        elif args.mode == "output_norm_gate":
            res = epilogue_measurements(args, {}, torch, np, rda, synth, dev, timed, flush,
                                        16384, 16, reps=args.steps)
        elif args.mode == "segments":
            res = segment_measurements(args, torch, np, rda, synth, dev, stream, timed, flush,
                                       reps=args.steps, heads=(2,))
        elif args.mode == "prologue":
            res = prologue_measurements(args, {}, torch, np, rda, synth, dev, timed, flush,
                                        16384, 16, reps=args.steps, decode=False)
        else:
            res = diag_measurements(args, {}, torch, np, rda, synth, dev, timed, flush,
                                    reps=args.steps, decode=False)
        print(json.dumps({"mode": args.mode, **res}), flush=True)
        return

    # ---- inputs (host draw, then resident on the device) --------------------
    t = time.time()
    p = synth.config3()
    T, H = p.total_tokens, p.num_heads
    q = torch.from_numpy(p.q).to(torch.bfloat16).to(dev)
    k = torch.from_numpy(p.k).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(p.v).to(torch.bfloat16).to(dev)
    a = torch.from_numpy(p.a).to(dev)
    b = torch.from_numpy(p.b).to(dev)
    S0 = torch.from_numpy(p.S0).to(dev)
    o = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    Sf = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(rda.rda_prefill_workspace_bytes(1, T, H), dtype=torch.uint8, device=dev)
    log(f"prefill inputs ready ({time.time() - t:.1f}s)")

    B, DH, NTOK = 256, 16, 128
    do_decode = args.mode in ("bench", "decode")
    do_prefill = args.mode in ("bench", "prefill")
    if do_decode:
        t = time.time()
        S_dec = torch.from_numpy(synth.decode_state(B, DH)).to(dev)
        toks = []
        for i in range(NTOK):
            x = synth.decode_step_inputs(i, B, DH)
            toks.append(tuple(torch.from_numpy(getattr(x, n)).to(torch.bfloat16).to(dev)
                              for n in "qkv") + (torch.from_numpy(x.a).to(dev),
                                                 torch.from_numpy(x.b).to(dev)))
        o_dec = torch.empty((B, DH, D), dtype=torch.float32, device=dev)
        log(f"decode inputs ready ({time.time() - t:.1f}s)")

    def make_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)      # materialise the underlying HIP events
        return evs

    K, W = args.steps, args.warmup

    def one_step(i, call_ev=None, dec_ev=None):
        if do_prefill:
            if call_ev is not None:
                call_ev[0].record(stream)
            rda.rda_prefill(q, k, v, a, b, S0=S0, o=o, S_final=Sf, workspace=ws)
            if call_ev is not None:
                call_ev[1].record(stream)
        if do_decode:
            qt, kt, vt, at, bt = toks[i % NTOK]
            if dec_ev is not None:
                dec_ev[0].record(stream)
            rda.rda_decode_step(qt, kt, vt, at, bt, S_dec, o=o_dec)
            if dec_ev is not None:
                dec_ev[1].record(stream)

    for i in range(W):
        one_step(i)
    torch.cuda.synchronize()

    call_evs = [make_events(2) for _ in range(K)]
    dec_evs = [make_events(2) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        one_step(W + i, call_evs[i] if do_prefill else None, dec_evs[i] if do_decode else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-stage breakdown: the same calls with an event pair around each
    # stage (rda_prefill_profiled runs the same kernels), after the timed
    # steps because the events between launches add about 6 us to a call; a
    # decode step between calls streams 512 MiB, as in the timed loop
    KB = min(K, 20)
    stage_evs = [make_events(2 * rda.RDA_NUM_STAGES) for _ in range(KB)]
    if do_prefill:
        torch.cuda.synchronize()
        for i in range(KB):
            rda.rda_prefill(q, k, v, a, b, S0=S0, o=o, S_final=Sf, workspace=ws,
                            stage_events=stage_evs[i])
            if do_decode:
                qt, kt, vt, at, bt = toks[i % NTOK]
                rda.rda_decode_step(qt, kt, vt, at, bt, S_dec, o=o_dec)
        torch.cuda.synchronize()

    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": wall * 1e3 / K, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "RDA long-prompt prefill T=16384 H=16 d=128 (bf16 q/k/v, "
                                  "fp32 gates, S0~N(0,0.02)) + RDA decode step B=256 H=16 "
                                  "d=128 (fp32 states in place)",
                      "prefill": {"T": T, "H": H, "d": D, "chunk": C, "qkv": "bf16",
                                  "state": "fp32", "o": "fp32"},
                      "decode": {"B": B, "H": DH, "d": D, "tokens_cycled": NTOK}}}

    kernels = {}
    if do_prefill:
        st = np.array([[stage_evs[i][2 * s].elapsed_time(stage_evs[i][2 * s + 1])
                        for s in range(rda.RDA_NUM_STAGES)] for i in range(KB)])   # ms
        call = np.array([call_evs[i][0].elapsed_time(call_evs[i][1]) for i in range(K)])
        units = T * H
        call_s = float(np.mean(call)) * 1e-3
        out["value"] = T / call_s
        out["unit"] = "tokens/s"
        out["prefill"] = {"ms_per_call": call_s * 1e3, "tokens_per_s": T / call_s,
                          "hbm_roofline_tokens_per_s": PEAK_HBM_GBPS * 1e9 / (PREFILL_BYTES * H),
                          "algorithmic_TFLOPs": PREFILL_FLOPS * units / call_s / 1e12,
                          "mfma_frac_algorithmic": PREFILL_FLOPS * units / call_s / 1e12
                          / PEAK_BF16_TFLOPS,
                          "hbm_frac_algorithmic": (PREFILL_BYTES * units + 2 * H * STATE_BYTES)
                          / call_s / 1e9 / PEAK_HBM_GBPS}
        # MFMA work rocprofv3 counted per launch (hi/lo split products
        # included), over this run's call time
        mf = [read_profile("mfma_rda_prefill_T16384_H16.txt", f"{n}.mfma_{t}_flops_per_call")
              for n in ("rda_prep", "rda_walk") for t in ("bf16", "f32")]
        if all(x is not None for x in mf):
            out["prefill"]["mfma_frac_executed_rocprof"] = sum(mf) / call_s / 1e12 / PEAK_BF16_TFLOPS
        else:
            out["prefill"]["mfma_frac_executed_rocprof"] = None
        names = {0: "rda_chunk_table", 1: "rda_prep", 2: "rda_walk"}
        # the walk streams q, k, v again and writes o and the states, so it is
        # charged the whole path's algorithmic bytes (1288 B per token-head
        # plus S0 and S_final); the prep's figure is the inputs it reads
        # itself (q, k, a, b).  Times are per call: in the plan that preps
        # the later chunks beside the walk, the prep stage is the prep of the
        # first chunks and the walk stage the walk launches (the first also
        # preps the rest on the CUs the walk leaves idle).
        kb = {0: 0.0, 1: (2 * D * 2 + 2 * 4) * units,
              2: PREFILL_BYTES * units + 2 * H * STATE_BYTES}
        for s in range(rda.RDA_NUM_STAGES):
            if s == rda.RDA_STAGE_TABLE:
                continue    # no cu_seqlens: the table is written by the prep kernel
            ms = float(np.mean(st[:, s]))
            kernels[names[s]] = {"us_per_call": ms * 1e3, "alg_bytes": kb[s],
                                 "launches_per_call": read_profile(
                                     "hbm_traffic.txt", f"{names[s]}.launches_per_call")}
    if do_decode:
        dms = np.array([dec_evs[i][0].elapsed_time(dec_evs[i][1]) for i in range(K)])
        dsec = float(np.mean(dms)) * 1e-3
        dbytes = DECODE_BYTES * B * DH
        gbps = dbytes / dsec / 1e9
        out["decode"] = {"value": gbps, "unit": "GB/s", "us_per_step": dsec * 1e6,
                         "frac_of_peak": gbps / PEAK_HBM_GBPS, "bytes_per_step": dbytes,
                         "tokens_per_s": B / dsec}
        kernels["rda_decode_step"] = {"us_per_call": dsec * 1e6, "alg_bytes": dbytes,
                                      "launches_per_call": 1}
        if "value" not in out:
            out["value"], out["unit"] = gbps, "GB/s"
        if not args.no_extras:
            # 128 decode steps back to back (the serving loop), one event pair
            # around all of them
            torch.cuda.synchronize()
            e0, e1 = make_events(2)
            e0.record(stream)
            for i in range(NTOK):
                qt, kt, vt, at, bt = toks[i]
                rda.rda_decode_step(qt, kt, vt, at, bt, S_dec, o=o_dec)
            e1.record(stream)
            torch.cuda.synchronize()
            bsec = e0.elapsed_time(e1) * 1e-3 / NTOK
            out["decode"]["back_to_back_128"] = {"us_per_step": bsec * 1e6,
                                                 "GBps": dbytes / bsec / 1e9,
                                                 "frac_of_peak": dbytes / bsec / 1e9
                                                 / PEAK_HBM_GBPS}
    out["kernels"] = kernels

    # roofline of the kernel with the largest time per step (per call: all
    # of its launches in one call)
    dom = max(kernels, key=lambda n: kernels[n]["us_per_call"])
    kd = kernels[dom]
    ach = kd["alg_bytes"] / (kd["us_per_call"] * 1e-6) / 1e9
    tr = read_traffic(dom)
    out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS,
                       "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS, "traffic": tr,
                       "alg_bytes_per_call": kd["alg_bytes"], "us_per_call": kd["us_per_call"],
                       "launches_per_call": kd["launches_per_call"]}
    if do_prefill:
        # the whole call (every kernel of rda_prefill) against the same bytes
        whole = (PREFILL_BYTES * T * H + 2 * H * STATE_BYTES) / (out["prefill"]["ms_per_call"]
                                                                 * 1e-3) / 1e9
        out["roofline"]["whole_call"] = {"achieved": whole, "frac": whole / PEAK_HBM_GBPS}

    if do_prefill and not args.child and args.mode == "bench":
        # the timing protocol: the median over fresh processes of each
        # process's mean per-call time (this process is one of them)
        per = [c["prefill"]["ms_per_call"] if c and "prefill" in c else None for c in children]
        per.append(out["prefill"]["ms_per_call"])
        ok = [x for x in per if x is not None]
        med = float(np.median(ok))
        out["protocol"] = {"processes": len(per), "processes_ok": len(ok),
                           "warmup_steps": W, "timed_steps": K,
                           "ms_per_call_per_process": per, "ms_per_call_median": med,
                           "this_process_ms_per_call": out["prefill"]["ms_per_call"]}
        if do_decode:
            dper = [c["decode"]["us_per_step"] if c and "decode" in c else None
                    for c in children] + [out["decode"]["us_per_step"]]
            out["protocol"]["decode_us_per_step_per_process"] = dper
            out["protocol"]["decode_us_per_step_median"] = float(
                np.median([x for x in dper if x is not None]))
        out["value"] = T / (med * 1e-3)
        out["prefill"]["tokens_per_s"] = out["value"]

    if args.mode == "bench" and not args.no_extras and not args.child:
        extra_measurements(args, out, torch, np, rda, synth, dev, stream, q, k, v, a, b, S0,
                           o, Sf, ws, T, H)

    if do_prefill:
        o_h = o.cpu().numpy().astype(np.float64)
        S_h = Sf.cpu().numpy().astype(np.float64)
    if do_prefill and not args.no_cpu:
        import oracle
        thr = oracle.threads_used(args.cpu_threads)
        t = time.perf_counter()
        ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0, threads=args.cpu_threads)
        cpu_s = time.perf_counter() - t
        # one core: the same prefill on a quarter of the prompt's tokens (every
        # head), the oracle's per-core rate scaled to the whole prompt
        Tq = T // 4
        sl = lambda x: np.ascontiguousarray(x[:Tq])
        t = time.perf_counter()
        oracle.prefill(sl(p.q), sl(p.k), sl(p.v), sl(p.a), sl(p.b), S0=p.S0, threads=1)
        one_s = time.perf_counter() - t
        cpu_model = None
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        out["cpu_baseline"] = {"value": T / cpu_s, "unit": "tokens/s", "cores": thr,
                               "cpu_model": cpu_model, "visible_cpus": os.cpu_count(),
                               "kind": "oracle",
                               "sample": f"the full long-prompt prefill (T={T}, H={H}, d={D}, "
                                         f"fp64 sequential recurrence, OpenMP over the {H} "
                                         f"heads), {cpu_s:.1f} s on {os.cpu_count()} visible "
                                         "host CPUs",
                               "single_core": {"value": Tq / one_s, "unit": "tokens/s",
                                               "cores": 1,
                                               "sample": f"the first {Tq} tokens of the same "
                                                         f"prompt, all {H} heads, one thread, "
                                                         f"{one_s:.1f} s"}}
        out["parity"] = {"o_rel_l2": float(np.linalg.norm(o_h - ro) / np.linalg.norm(ro)),
                         "o_max_abs": float(np.max(np.abs(o_h - ro))),
                         "S_rel_l2": float(np.linalg.norm(S_h - rS) / np.linalg.norm(rS))}
    print(json.dumps(out), flush=True)


# counter summaries of the other prefill workloads under profiles/
CONFIG_PROFILE = {1: "T64_H1_fp32", 2: "T2048_H16", 4: "varlen8_T32768_H16"}


def hbm_roofline(alg_bytes, sec, traffic=None):
    """An HBM roofline entry: algorithmic bytes over the measured time
    against the 8 TB/s peak (traffic: counted HBM bytes per launch, when a
    counter summary for the current kernels exists)."""
    ach = alg_bytes / sec / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBPS, "alg_bytes": alg_bytes, "traffic": traffic}


def make_timer(torch, np, stream):
    """timed(fn, reps, flush=None): median seconds of `fn` between HIP events
    on `stream`, each call preceded by `flush()` when given."""
    def timed(fn, reps, flush=None):
        ts = []
        for _ in range(reps):
            if flush is not None:
                flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ts])) * 1e-3   # s
    return timed


def extra_measurements(args, out, torch, np, rda, synth, dev, stream, q, k, v, a, b, S0, o, Sf,
                       ws, T, H):
    """The other figures the measurement plan asks for beside the headline:
    the prefill without the cache flush between calls, the practical HBM
    rate of an in-place read-modify-write of the decode's size, and the three
    other prefill workloads (time, algorithmic fractions, parity)."""
    timed = make_timer(torch, np, stream)

    # prefill back to back, inputs left in the Infinity Cache by the call before
    warm = timed(lambda: rda.rda_prefill(q, k, v, a, b, S0=S0, o=o, S_final=Sf, workspace=ws), 10)
    out["prefill"]["ms_per_call_unflushed"] = warm * 1e3
    out["prefill"]["tokens_per_s_unflushed"] = T / warm

    # practical HBM ceiling: in-place scaling of 256 MiB of fp32 (read + write)
    scratch = torch.ones((64 << 20,), dtype=torch.float32, device=dev)
    hs = timed(lambda: scratch.mul_(1.0), 10)
    hbm_gbps = 2 * scratch.numel() * 4 / hs / 1e9
    out["hbm_practical"] = {"GBps": hbm_gbps, "frac_of_peak": hbm_gbps / PEAK_HBM_GBPS,
                            "how": "in-place scaling of a 256 MiB fp32 buffer (read + write)"}
    if "decode" in out:
        out["decode"]["frac_of_practical"] = out["decode"]["value"] / hbm_gbps

    # evicts the Infinity Cache by reading 512 MiB: a read-only flush, so the
    # timed call does not pay for writing back the flush's own dirty lines
    flush_buf = torch.ones((128 << 20,), dtype=torch.float32, device=dev)
    flush = lambda: flush_buf.sum()
    # the headline prefill again, each call after the read-only flush (no
    # input in the cache and no dirty lines of other work left to write back)
    clean = timed(lambda: rda.rda_prefill(q, k, v, a, b, S0=S0, o=o, S_final=Sf, workspace=ws),
                  10, flush)
    out["prefill"]["ms_per_call_read_flushed"] = clean * 1e3
    out["prefill"]["tokens_per_s_read_flushed"] = T / clean

    configs = {}
    for cid, name in ((1, "single_head_fp32_T64"), (2, "nano_layer_T2048_H16"),
                      (4, "varlen_8_seqs_T32768_H16")):
        pc = synth.CONFIGS[cid]()
        Tc, Hc = pc.total_tokens, pc.num_heads
        tok = (lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)) if pc.bf16 else \
            (lambda x: torch.from_numpy(x).to(dev))
        qc, kc, vc = tok(pc.q), tok(pc.k), tok(pc.v)
        ac, bc = torch.from_numpy(pc.a).to(dev), torch.from_numpy(pc.b).to(dev)
        S0c = torch.from_numpy(pc.S0).to(dev) if pc.S0 is not None else None
        cuc = pc.cu_seqlens
        oc, Sfc = rda.rda_prefill(qc, kc, vc, ac, bc, cu_seqlens=cuc, S0=S0c)
        wsc = torch.empty(rda.rda_prefill_workspace_bytes(pc.num_seqs, Tc, Hc), dtype=torch.uint8,
                          device=dev)
        cu_dev = torch.from_numpy(cuc.astype(np.int32)).to(dev) if cuc is not None else None
        # the C entry point itself: the binding's check of cu_seqlens reads it
        # back to the host, which would put a device sync inside the timing
        cargs = [rda._ptr(qc), rda._ptr(kc), rda._ptr(vc), 0 if pc.bf16 else 1, rda._ptr(ac),
                 rda._ptr(bc), rda._ptr(cu_dev), pc.num_seqs, Tc, Hc, D, D, rda._ptr(S0c),
                 rda._ptr(oc), rda._ptr(Sfc), rda._ptr(wsc), wsc.numel(), stream.cuda_stream]

        def call():
            if rda.lib().rda_prefill(*cargs) != 0:
                raise RuntimeError("rda_prefill failed")
        sec = timed(call, 10, flush)
        graph_ms = None
        if cid == 1:
            # launch-bound: the same call captured once in a HIP graph, replayed
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                call()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                gcargs = list(cargs)
                gcargs[-1] = torch.cuda.current_stream().cuda_stream
                if rda.lib().rda_prefill(*gcargs) != 0:
                    raise RuntimeError("rda_prefill failed")
            torch.cuda.synchronize()
            graph_ms = timed(graph.replay, 10, flush) * 1e3
        units = Tc * Hc
        entry = {"T": Tc, "H": Hc, "N": pc.num_seqs, "qkv": "bf16" if pc.bf16 else "fp32",
                 "ms_per_call": sec * 1e3, "tokens_per_s": Tc / sec,
                 "mfma_frac_algorithmic": PREFILL_FLOPS * units / sec / 1e12 / PEAK_BF16_TFLOPS,
                 "hbm_frac_algorithmic": (PREFILL_BYTES * units +
                                          (2 if S0c is not None else 1) * pc.num_seqs * Hc *
                                          STATE_BYTES) / sec / 1e9 / PEAK_HBM_GBPS}
        entry["roofline"] = hbm_roofline((PREFILL_BYTES * units + (2 if S0c is not None else 1)
                                          * pc.num_seqs * Hc * STATE_BYTES), sec)
        mf = [read_profile(f"mfma_rda_prefill_{CONFIG_PROFILE[cid]}.txt", f"{n}.mfma_{t}_flops")
              for n in ("rda_prep", "rda_walk") for t in ("bf16", "f32")]
        entry["mfma_frac_executed_rocprof"] = (
            sum(x for x in mf if x is not None) / sec / 1e12 / PEAK_BF16_TFLOPS
            if any(x is not None for x in mf) else None)
        if graph_ms is not None:
            entry["ms_per_call_graph_replay"] = graph_ms
        if not args.no_cpu:
            import oracle
            ro, rS = oracle.prefill(pc.q, pc.k, pc.v, pc.a, pc.b, cu_seqlens=cuc, S0=pc.S0,
                                    threads=args.cpu_threads)
            oh = oc.cpu().numpy().astype(np.float64)
            Sh = Sfc.cpu().numpy().astype(np.float64)
            entry["parity"] = {"o_rel_l2": float(np.linalg.norm(oh - ro) / np.linalg.norm(ro)),
                               "o_max_abs": float(np.max(np.abs(oh - ro))),
                               "S_rel_l2": float(np.linalg.norm(Sh - rS) / np.linalg.norm(rS))}
        configs[name] = entry
        if cid == 4:
            entry["lengths"] = [int(x) for x in np.diff(cuc)]
    out["other_prefill_workloads"] = configs
    out["prefill_segmented"] = segment_measurements(args, torch, np, rda, synth, dev, stream,
                                                    timed, flush)
    out["prefill_diag"] = diag_measurements(args, out, torch, np, rda, synth, dev, timed, flush)
    out["prologue"] = prologue_measurements(args, out, torch, np, rda, synth, dev, timed, flush,
                                            T, H)
    out["output_norm_gate"] = epilogue_measurements(args, out, torch, np, rda, synth, dev, timed,
                                                    flush, T, H)
    out["prefill_norm_gate"] = fused_norm_gate_measurement(args, torch, np, rda, synth, dev,
                                                           timed, flush)
    out["decode_tokens"] = decode_tokens_measurements(args, out, torch, np, rda, synth, dev,
                                                      stream, timed, flush)
    del scratch, flush_buf


def diag_measurements(args, out, torch, np, rda, synth, dev, timed, flush, reps=10,
                      decode=True):
    """The per-channel-decay prefill on the long prompt (T = 16384, H = 16,
    bf16 q/k/v, per-channel decay, S0 ~ N(0, 0.02)) as tokens/s after a cache
    flush, with parity against the oracle; with `decode`, the per-channel
    decode step on the decode batch (256 x 16 states) as state GB/s."""
    T, H = 16384, 16
    p = synth.config3()
    alpha = synth.diag_alpha(T, H)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    dv = lambda a: torch.from_numpy(a).to(dev)
    q, k, v = bf(p.q), bf(p.k), bf(p.v)
    al, b, S0 = dv(alpha), dv(p.b), dv(p.S0)
    o = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    Sf = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(rda.rda_prefill_diag_workspace_bytes(1, T, H), dtype=torch.uint8, device=dev)
    sec = timed(lambda: rda.rda_prefill_diag(q, k, v, al, b, S0=S0, o=o, S_final=Sf,
                                             workspace=ws), reps, flush)
    res = {"T": T, "H": H, "ms_per_call": sec * 1e3, "tokens_per_s": T / sec,
           "workspace_bytes": ws.numel()}
    # per token-head: bf16 q, k, v, fp32 decay vector, b and o; S0 and S_final
    diag_bytes = T * H * (3 * D * 2 + D * 4 + 4 + D * 4) + 2 * H * STATE_BYTES
    tr = [read_traffic(n) for n in ("rda_prep_diag", "rda_walk_diag")]
    res["roofline"] = hbm_roofline(diag_bytes, sec, sum(tr) if None not in tr else None)
    if "prefill" in out:
        res["vs_scalar_decay"] = out["prefill"]["ms_per_call"] / (sec * 1e3)
    if not args.no_cpu:
        import oracle
        ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0,
                                     threads=args.cpu_threads)
        oh, Sh = o.cpu().numpy().astype(np.float64), Sf.cpu().numpy().astype(np.float64)
        res["parity"] = {"o_rel_l2": float(np.linalg.norm(oh - ro) / np.linalg.norm(ro)),
                         "o_max_abs": float(np.max(np.abs(oh - ro))),
                         "S_rel_l2": float(np.linalg.norm(Sh - rS) / np.linalg.norm(rS))}
    if decode:
        B = 256
        S_dec = dv(synth.decode_state(B, H))
        x = synth.decode_step_inputs(0, B, H)
        xq, xk, xv = (torch.from_numpy(getattr(x, n)).to(torch.bfloat16).to(dev) for n in "qkv")
        ad, bd = dv(synth.diag_alpha(B, H, key=(11,))), dv(x.b)
        od = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        dsec = timed(lambda: rda.rda_decode_step_diag(xq, xk, xv, ad, bd, S_dec, o=od), reps,
                     flush)
        dbytes = B * H * (2 * STATE_BYTES + PREFILL_IN_BYTES + PREFILL_OUT_BYTES + D * 4)
        res["decode"] = {"B": B, "us_per_step": dsec * 1e6, "GBps": dbytes / dsec / 1e9,
                         "frac_of_peak": dbytes / dsec / 1e9 / PEAK_HBM_GBPS,
                         "roofline": hbm_roofline(dbytes, dsec)}
    return res


PROLOGUE_K = 4   # conv width: three cached raw tokens per tensor


def prologue_measurements(args, out, torch, np, rda, synth, dev, timed, flush, T, H, reps=10,
                          decode=True):
    """rda_prologue on the long prompt (T x H token-heads, conv width 4, SiLU,
    bf16 raw q, k, v in and q, k, v out, fp32 gates) and, with `decode`, on
    the decode batch (256 sequences x 16 heads, one token, history updated
    in place), each timed after a cache flush with its algorithmic
    bandwidth; with the other stages measured, the whole block on the long
    prompt (prologue, prefill, output norm and gate) as tokens/s."""
    K = PROLOGUE_K
    x = synth.prologue_inputs(T, H, K)
    dv = lambda a: torch.from_numpy(a).to(dev)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    args_dev = (bf(x.xq), bf(x.xk), bf(x.xv), dv(x.conv_w), dv(x.beta_raw), dv(x.g_log))
    delta, hin = dv(x.delta), bf(x.hist)
    hout = torch.empty_like(hin)
    res_out = []

    def call():
        res_out[:] = rda.rda_prologue(*args_dev, delta=delta, hist_in=hin, hist_out=hout)
    sec = timed(call, reps, flush)
    tok_bytes = 3 * D * 2 * 2 + 3 * 4 + 2 * 4     # raw in + bf16 out, 3 gates in, a and b out
    hist_bytes = 2 * 3 * (K - 1) * H * D * 2      # one sequence's history in and out
    nbytes = T * H * tok_bytes + hist_bytes
    res = {"T": T, "H": H, "conv_width": K, "conv_act": "silu", "us_per_call": sec * 1e6,
           "GBps": nbytes / sec / 1e9, "frac_of_peak": nbytes / sec / 1e9 / PEAK_HBM_GBPS,
           "bytes_per_call": nbytes, "traffic": read_traffic("rda_prologue")}
    res["roofline"] = hbm_roofline(nbytes, sec, res["traffic"])
    if not args.no_cpu:
        import oracle
        rows = np.arange(0, T, max(T // 512, 1))    # every 32nd token's full row
        ref = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw, x.delta, x.g_log,
                              hist_in=x.hist)
        got = [t.float().cpu().numpy()[rows].astype(np.float64) for t in res_out[:3]]
        rel = [float(np.linalg.norm(g - r[rows]) / np.linalg.norm(r[rows]))
               for g, r in zip(got, ref[:3])]
        res["parity_sampled"] = {"q_rel_l2": rel[0], "k_rel_l2": rel[1], "v_rel_l2": rel[2]}
    if decode:
        B = 256
        xd = synth.prologue_inputs(B, H, K, N=B, key=(9,))
        dargs = tuple(f(a) for f, a in ((bf, xd.xq), (bf, xd.xk), (bf, xd.xv), (dv, xd.conv_w),
                                        (dv, xd.beta_raw), (dv, xd.g_log)))
        ddelta, dh = dv(xd.delta), bf(xd.hist)
        dsec = timed(lambda: rda.rda_prologue(*dargs, delta=ddelta, hist_in=dh, hist_out=dh,
                                              num_seqs=B), reps, flush)
        dbytes = B * H * tok_bytes + B * hist_bytes
        res["decode"] = {"B": B, "us_per_call": dsec * 1e6, "GBps": dbytes / dsec / 1e9,
                         "bytes_per_call": dbytes, "roofline": hbm_roofline(dbytes, dsec)}
        res["decode_fused"] = decode_prologue_measurement(args, out, torch, np, rda, synth, dev,
                                                          timed, flush, reps)
        if "decode" in out:
            res["decode_fused"]["prologue_plus_decode_step_us"] = (
                dsec * 1e6 + out["decode"]["us_per_step"])
    return res


def decode_prologue_measurement(args, out, torch, np, rda, synth, dev, timed, flush, reps=10,
                                B=256, H=16):
    """rda_decode_step_prologue on the decode batch (B sequences x H heads,
    conv width 4, SiLU, the history updated in place, fp32 states in place),
    timed after a cache flush, with its algorithmic bandwidth: the state read
    and written, the raw token and the gates' inputs read, the history read
    and written, o written."""
    K = PROLOGUE_K
    x = synth.prologue_inputs(B, H, K, N=B, key=(9,))
    dv = lambda a: torch.from_numpy(a).to(dev)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    xq, xk, xv, w, br, gl = (bf(x.xq), bf(x.xk), bf(x.xv), dv(x.conv_w), dv(x.beta_raw),
                             dv(x.g_log))
    dl, hist = dv(x.delta), bf(x.hist)
    S = dv(synth.decode_state(B, H))
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    sec = timed(lambda: rda.rda_decode_step_prologue(xq, xk, xv, w, br, gl, S, delta=dl,
                                                     hist_in=hist, hist_out=hist, o=o),
                reps, flush)
    nbytes = B * H * (2 * STATE_BYTES + 3 * D * 2 + 3 * 4 + D * 4) + \
        B * 2 * 3 * (K - 1) * H * D * 2
    # the plain decode step on the same states, timed the same way
    xd = synth.decode_step_inputs(0, B, H)
    q, k, v = (bf(getattr(xd, nm)) for nm in "qkv")
    a, b = dv(xd.a), dv(xd.b)
    psec = timed(lambda: rda.rda_decode_step(q, k, v, a, b, S, o=o), reps, flush)
    return {"B": B, "H": H, "conv_width": K, "us_per_step": sec * 1e6,
            "GBps": nbytes / sec / 1e9, "bytes_per_step": nbytes,
            "roofline": hbm_roofline(nbytes, sec, read_traffic("rda_decode_step_prologue")),
            "plain_decode_step_us_same_timing": psec * 1e6}


def epilogue_measurements(args, out, torch, np, rda, synth, dev, timed, flush, T, H, reps=10):
    """rda_output_norm_gate on the long prompt's output rows (T x H rows of
    128: fp32 o, bf16 gate, bf16 out, sigmoid gate), timed after a cache
    flush, with its algorithmic bandwidth, and the prefill plus the
    epilogue as tokens/s."""
    rows = T * H
    x = synth.epilogue_inputs(rows)
    o = torch.from_numpy(x.o).to(dev)
    g = torch.from_numpy(x.g).to(torch.bfloat16).to(dev)
    w = torch.from_numpy(x.weight).to(dev)
    y = torch.empty((rows, D), dtype=torch.bfloat16, device=dev)
    sec = timed(lambda: rda.rda_output_norm_gate(o, g, weight=w, out=y), reps, flush)
    nbytes = rows * (D * 4 + D * 2 + D * 2)
    res = {"rows": rows, "us_per_call": sec * 1e6, "GBps": nbytes / sec / 1e9,
           "frac_of_peak": nbytes / sec / 1e9 / PEAK_HBM_GBPS, "bytes_per_call": nbytes,
           "traffic": read_traffic("rda_output_norm_gate")}
    res["roofline"] = hbm_roofline(nbytes, sec, res["traffic"])
    if "hbm_practical" in out:
        res["frac_of_practical"] = res["GBps"] / out["hbm_practical"]["GBps"]
    if "prefill" in out:
        tot = out["prefill"]["ms_per_call"] * 1e-3 + sec
        res["prefill_plus_epilogue_tokens_per_s"] = T / tot
        if "prologue" in out:
            tot += out["prologue"]["us_per_call"] * 1e-6
            res["block_tokens_per_s"] = T / tot     # prologue + prefill + norm and gate
    if not args.no_cpu:
        import oracle
        pick = np.random.default_rng(11).choice(rows, size=2048, replace=False)
        ref = oracle.output_norm_gate(x.o[pick], x.g[pick], x.weight, 1e-5, "sigmoid")
        got = y.float().cpu().numpy()[pick].astype(np.float64)
        res["parity_sampled"] = {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                                 "max_rel": float(np.max(np.abs(got - ref) /
                                                         np.maximum(np.abs(ref), 1e-30)))}
    return res


def fused_norm_gate_measurement(args, torch, np, rda, synth, dev, timed, flush, reps=10):
    """The long prompt (16384 x 16, bf16 q/k/v, S0 ~ N(0, 0.02)) three ways,
    each timed after a cache flush: rda_prefill alone (fp32 o), the same
    followed by rda_output_norm_gate (bf16 out, sigmoid gate), and
    rda_prefill_norm_gate (the fused form: no fp32 o)."""
    p = synth.config3()
    T, H = p.total_tokens, p.num_heads
    q, k, v = (torch.from_numpy(getattr(p, n)).to(torch.bfloat16).to(dev) for n in "qkv")
    a, b, S0 = (torch.from_numpy(getattr(p, n)).to(dev) for n in ("a", "b", "S0"))
    x = synth.epilogue_inputs(T * H, key=(12,))
    g = torch.from_numpy(x.g.reshape(T, H, D)).to(torch.bfloat16).to(dev)
    w = torch.from_numpy(x.weight).to(dev)
    o = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    Sf = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    y = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rda.rda_prefill_norm_gate_workspace_bytes(1, T, H), dtype=torch.uint8,
                     device=dev)
    pre = lambda: rda.rda_prefill(q, k, v, a, b, S0=S0, o=o, S_final=Sf, workspace=ws)
    two = lambda: (pre(), rda.rda_output_norm_gate(o, g, weight=w, out=y))
    fused = lambda: rda.rda_prefill_norm_gate(q, k, v, a, b, g, S0=S0, weight=w, out=y,
                                              S_final=Sf, workspace=ws)
    for fn in (pre, two, fused):   # warm
        fn()
    t_pre, t_two, t_fused = (timed(fn, reps, flush) for fn in (pre, two, fused))
    elems = T * H * D
    return {"T": T, "H": H, "prefill_only_ms": t_pre * 1e3,
            "prefill_then_norm_gate_ms": t_two * 1e3, "fused_ms": t_fused * 1e3,
            "fused_over_prefill_only": t_fused / t_pre,
            "fused_tokens_per_s": T / t_fused,
            # output-side HBM bytes: fp32 o written and read back plus the gate
            # and the bf16 out, against the slice form (2.25 B per element
            # written and read) plus the gate and the bf16 out
            "output_bytes_two_calls": elems * (4 + 4 + 2 + 2),
            "output_bytes_fused": elems * (2.25 + 2.25 + 2 + 2)}


def segment_measurements(args, torch, np, rda, synth, dev, stream, timed, flush, reps=10,
                         heads=(1, 2, 4)):
    """The long prompt (T = 16384) with few heads -- one GPU's share of its 16
    heads at 16-, 8- and 4-way head sharding -- where rda_prefill takes the
    segmented state pass (one sequence, no offsets).  Timed beside the
    one-pass walk on the same inputs (cu_seqlens = [0, T] selects it), each
    call after the read-only flush; parity of the segmented call against the
    oracle."""
    p = synth.config3()
    T = p.total_tokens
    res = {"T": T}
    cu_one = torch.tensor([0, T], dtype=torch.int32, device=dev)
    for H in heads:
        sl = lambda x: np.ascontiguousarray(x[:, :H])
        qh, kh, vh = (torch.from_numpy(sl(getattr(p, n))).to(torch.bfloat16).to(dev) for n in "qkv")
        ah, bh = torch.from_numpy(sl(p.a)).to(dev), torch.from_numpy(sl(p.b)).to(dev)
        S0h = torch.from_numpy(np.ascontiguousarray(p.S0[:, :H])).to(dev)
        oh = torch.empty((T, H, D), dtype=torch.float32, device=dev)
        Sfh = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
        ws = torch.empty(rda.rda_prefill_workspace_bytes(1, T, H), dtype=torch.uint8, device=dev)
        entry = {}
        for name, cu in (("segmented", None), ("one_pass", cu_one)):
            cargs = [rda._ptr(qh), rda._ptr(kh), rda._ptr(vh), 0, rda._ptr(ah), rda._ptr(bh),
                     rda._ptr(cu), 1, T, H, D, D, rda._ptr(S0h), rda._ptr(oh), rda._ptr(Sfh),
                     rda._ptr(ws), ws.numel(), stream.cuda_stream]

            def call(cargs=cargs):
                if rda.lib().rda_prefill(*cargs) != 0:
                    raise RuntimeError("rda_prefill failed")
            call()
            sec = timed(call, reps, flush)
            entry[name] = {"ms_per_call": sec * 1e3, "tokens_per_s": T / sec}
        entry["speedup"] = entry["one_pass"]["ms_per_call"] / entry["segmented"]["ms_per_call"]
        if not args.no_cpu and H == 2:
            import oracle
            torch.cuda.synchronize()
            rda.rda_prefill(qh, kh, vh, ah, bh, S0=S0h, o=oh, S_final=Sfh, workspace=ws,
                            stream=stream)
            torch.cuda.synchronize()
            ro, rS = oracle.prefill(sl(p.q), sl(p.k), sl(p.v), sl(p.a), sl(p.b),
                                    S0=np.ascontiguousarray(p.S0[:, :H]), threads=args.cpu_threads)
            og = oh.cpu().numpy().astype(np.float64)
            Sg = Sfh.cpu().numpy().astype(np.float64)
            entry["parity"] = {"o_rel_l2": float(np.linalg.norm(og - ro) / np.linalg.norm(ro)),
                               "S_rel_l2": float(np.linalg.norm(Sg - rS) / np.linalg.norm(rS))}
        res[f"H{H}"] = entry
    # the per-channel decay on the long prompt's first 2 heads, the same way
    H = 2
    sl = lambda x: np.ascontiguousarray(x[:, :H])
    alpha = synth.diag_alpha(T, H, key=(10,))
    qh, kh, vh = (torch.from_numpy(sl(getattr(p, n))).to(torch.bfloat16).to(dev) for n in "qkv")
    alh, bh = torch.from_numpy(alpha).to(dev), torch.from_numpy(sl(p.b)).to(dev)
    S0h = torch.from_numpy(np.ascontiguousarray(p.S0[:, :H])).to(dev)
    oh = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    Sfh = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(rda.rda_prefill_diag_workspace_bytes(1, T, H), dtype=torch.uint8, device=dev)
    entry = {}
    for name, cu in (("segmented", None), ("one_pass", cu_one)):
        cargs = [rda._ptr(qh), rda._ptr(kh), rda._ptr(vh), 0, rda._ptr(alh), rda._ptr(bh),
                 rda._ptr(cu), 1, T, H, D, D, rda._ptr(S0h), rda._ptr(oh), rda._ptr(Sfh),
                 rda._ptr(ws), ws.numel(), stream.cuda_stream]

        def call(cargs=cargs):
            if rda.lib().rda_prefill_diag(*cargs) != 0:
                raise RuntimeError("rda_prefill_diag failed")
        call()
        sec = timed(call, reps, flush)
        entry[name] = {"ms_per_call": sec * 1e3, "tokens_per_s": T / sec}
    entry["speedup"] = entry["one_pass"]["ms_per_call"] / entry["segmented"]["ms_per_call"]
    if not args.no_cpu:
        import oracle
        torch.cuda.synchronize()
        rda.rda_prefill_diag(qh, kh, vh, alh, bh, S0=S0h, o=oh, S_final=Sfh, workspace=ws,
                             stream=stream)
        torch.cuda.synchronize()
        ro, rS = oracle.prefill_diag(sl(p.q), sl(p.k), sl(p.v), alpha, sl(p.b),
                                     S0=np.ascontiguousarray(p.S0[:, :H]),
                                     threads=args.cpu_threads)
        og = oh.cpu().numpy().astype(np.float64)
        Sg = Sfh.cpu().numpy().astype(np.float64)
        entry["parity"] = {"o_rel_l2": float(np.linalg.norm(og - ro) / np.linalg.norm(ro)),
                           "S_rel_l2": float(np.linalg.norm(Sg - rS) / np.linalg.norm(rS))}
    res["per_channel_H2"] = entry
    return res


def decode_tokens_measurements(args, out, torch, np, rda, synth, dev, stream, timed, flush,
                               reps=10, modes=None):
    """rda_decode_tokens on the decode batch with one token plus two drafts
    (B = 256 sequences x 16 heads, T = 3, per-sequence accept counts): the
    one-pass verify + commit in place, a read-only verify, and a commit-only
    call, each timed after a cache flush, with algorithmic state bandwidth."""
    B, T, H = 256, 3, 16
    x = synth.decode_tokens_inputs(B, T, H)
    S0 = synth.decode_state(B, H)
    qd, kd, vd = (torch.from_numpy(getattr(x, n)).to(torch.bfloat16).to(dev) for n in "qkv")
    ad, bd = torch.from_numpy(x.a).to(dev), torch.from_numpy(x.b).to(dev)
    acc = torch.from_numpy(x.accept).to(dev)
    S = torch.from_numpy(S0).to(dev)
    od = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    n_acc = float(np.mean(x.accept))
    tok_in = 3 * D * 2 + 2 * 4                  # bf16 q, k, v + fp32 a, b per token-head
    st_bytes = B * H * STATE_BYTES
    # the per-channel decay variant: alpha [B, T, H, 128] fp32 in place of a
    alpha = synth.diag_alpha(B * T, H, key=(11,)).reshape(B, T, H, D)
    ald = torch.from_numpy(alpha).to(dev)
    tok_in_diag = tok_in + (D - 1) * 4
    table = {
        # name: (entry point, decay, S_out, accept, o, algorithmic bytes)
        "verify_commit_in_place": ("rda_decode_tokens", ad, S, acc, od,
                                   2 * st_bytes + B * H * T * (tok_in + D * 4)),
        "verify_only": ("rda_decode_tokens", ad, None, None, od,
                        st_bytes + B * H * T * (tok_in + D * 4)),
        "commit_only": ("rda_decode_tokens", ad, S, acc, None,
                        2 * st_bytes + B * H * n_acc * (tok_in - D * 2)),
        "diag_verify_commit_in_place": ("rda_decode_tokens_diag", ald, S, acc, od,
                                        2 * st_bytes + B * H * T * (tok_in_diag + D * 4)),
    }
    res = {"B": B, "T": T, "H": H, "mean_accept": n_acc}
    S_copy = S.clone()
    for name, (fn, dec, So, ac, o_, nbytes) in table.items():
        if modes is not None and name not in modes:
            continue
        cargs = [rda._ptr(qd) if o_ is not None else None, rda._ptr(kd), rda._ptr(vd), 0,
                 rda._ptr(dec), rda._ptr(bd), B, T, H, D, D, rda._ptr(S), rda._ptr(So),
                 rda._ptr(ac), rda._ptr(o_), stream.cuda_stream]

        def call(fn=fn, cargs=cargs):
            if getattr(rda.lib(), fn)(*cargs) != 0:
                raise RuntimeError(f"{fn} failed")
        sec = timed(call, reps, flush)
        S.copy_(S_copy)         # in-place modes advanced the states: restore them
        res[name] = {"us_per_call": sec * 1e6, "GBps": nbytes / sec / 1e9,
                     "frac_of_peak": nbytes / sec / 1e9 / PEAK_HBM_GBPS, "bytes": nbytes,
                     "roofline": hbm_roofline(nbytes, sec)}
    if "verify_commit_in_place" in res:
        # counted HBM bytes of the one-pass call (profiles/hbm_traffic.txt)
        res["verify_commit_in_place"]["traffic"] = read_traffic("rda_decode_tokens")
        res["verify_commit_in_place"]["roofline"]["traffic"] = read_traffic("rda_decode_tokens")
    if "decode" in out:
        res["three_decode_steps_us"] = 3 * out["decode"]["us_per_step"]
    # parity of the one-pass call on 32 sampled (sequence, head) states
    if not args.no_cpu:
        import oracle
        torch.cuda.synchronize()
        rda.rda_decode_tokens(qd, kd, vd, ad, bd, S, S_out=S, accept=acc, o=od, stream=stream)
        torch.cuda.synchronize()
        rng = np.random.default_rng(9)
        pick = rng.choice(B * H, size=32, replace=False)
        sb, sh = pick // H, pick % H
        sel = lambda arr: np.ascontiguousarray(arr[sb, :, sh][:, :, None])
        ro, rS = oracle.decode_tokens(sel(x.q), sel(x.k), sel(x.v), sel(x.a), sel(x.b),
                                      S0[sb, sh][:, None], x.accept[sb])
        og = od.cpu().numpy()[sb, :, sh].astype(np.float64)
        Sg = S.cpu().numpy()[sb, sh].astype(np.float64)
        res["parity_sampled"] = {
            "o_rel_l2": float(np.linalg.norm(og - ro[:, :, 0]) / np.linalg.norm(ro)),
            "S_rel_l2": float(np.linalg.norm(Sg - rS[:, 0]) / np.linalg.norm(rS))}
        if "diag_verify_commit_in_place" in res:
            S.copy_(S_copy)
            rda.rda_decode_tokens_diag(qd, kd, vd, ald, bd, S, S_out=S, accept=acc, o=od,
                                       stream=stream)
            torch.cuda.synchronize()
            ro, rS = oracle.decode_tokens_diag(sel(x.q), sel(x.k), sel(x.v), sel(alpha),
                                               sel(x.b), S0[sb, sh][:, None], x.accept[sb])
            og = od.cpu().numpy()[sb, :, sh].astype(np.float64)
            Sg = S.cpu().numpy()[sb, sh].astype(np.float64)
            res["diag_verify_commit_in_place"]["parity_sampled"] = {
                "o_rel_l2": float(np.linalg.norm(og - ro[:, :, 0]) / np.linalg.norm(ro)),
                "S_rel_l2": float(np.linalg.norm(Sg - rS[:, 0]) / np.linalg.norm(rS))}
    return res


if __name__ == "__main__":
    main()
