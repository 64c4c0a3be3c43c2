"""Throughput of the fused denoising step on one MI355X.

One "step" is one pass of the whole hot path (vocabulary projection,
temperature, entropy, Gumbel-max sampling, entropy-bounded commit and
re-noise) over one batch of canvases.  Inputs are seeded synthetic tensors
resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gemma_vocab]
                    [--no-cpu-baseline] [--profile-only] [--lm-head-tail] [--sc-topk K]
                    [--power-seconds S]
    python bench.py --oracle-timing      # the CPU oracle on every workload, no GPU

``--lm-head-tail`` adds the model's output norm before the projection and the
logit softcap (c = 30) after it; ``--sc-topk K`` adds the self-conditioning
top-K of every position (and its embedding sum) to each step.

The timed steps run through the library's own step loop (dgd_run_steps), so
no Python runs between steps.  Before them: the measured HBM and MFMA
ceilings, then one instrumented pass of the whole generation with HIP events
around every kernel of every step (the projection's average launch for
``roofline``, and the per-step split), then the W warmup steps.

After them, ``power`` runs the step for ``--power-seconds`` more while
sampling the socket power and graphics clocks with amd-smi (outside the timed
region).

Prints ONE JSON line.  ``roofline`` is for the dominant kernel (the fused
projection); ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same workload.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("denoising steps/s and logit-elems/s (canvas·V) at canvas 256, V 262144; "
          "% roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counters
    (profiles/<kernel>_gemma_vocab_traffic.json), or None when the library
    sources have changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_gemma_vocab_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]


def measured_ceilings(dgd, torch, table, dev):
    """What this GPU sustains on the projection's two resources: a streaming
    read of the table the step reads (HBM), and independent bf16 MFMAs on
    operands taken from it (one wave per SIMD).  Best of 5 runs each."""
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    nbytes = table.numel() * table.element_size()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dgd.dgd_ceiling_hbm_read(table, nbytes, sink)
    best = float("inf")
    for _ in range(5):
        e0.record()
        dgd.dgd_ceiling_hbm_read(table, nbytes, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    hbm = nbytes / best / 1e9
    wgs, rounds = 256, 3000
    fsink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    dgd.dgd_ceiling_mfma_bf16(table, min(nbytes, 1 << 26), rounds, wgs, fsink)
    best = float("inf")
    for _ in range(5):
        e0.record()
        dgd.dgd_ceiling_mfma_bf16(table, min(nbytes, 1 << 26), rounds, wgs, fsink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    mfma = wgs * 4 * rounds * 64 * 32768.0 / best / 1e12
    return {"hbm_read_GBs": hbm, "mfma_bf16_TFLOPs": mfma,
            "how": "streaming 16-byte reads of the step's table (best of 5); "
                   "v_mfma_f32_32x32x16_bf16 on operands from the table, one wave per SIMD (best of 5)"}


def power_leg(run_steps, torch, seconds, start):
    """Sustained step rate with the socket power and graphics clocks sampled
    meanwhile (outside the timed region).  The board holds its socket power at
    a cap by lowering the clocks, so at the cap the step's energy sets its
    time."""
    from uniform_state_discrete_step_amd.power_trace import Sampler, power_cap

    smp = Sampler(0.5)
    smp.start()
    i, batch = start, 48
    run_steps(batch, start=i)     # let the sampler and the clocks settle
    torch.cuda.synchronize()
    i += batch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        run_steps(batch, start=i)
        torch.cuda.synchronize()
        i += batch
        n += batch
    t1 = time.perf_counter()
    r = smp.between(t0, t1)
    smp.stop.set()
    smp.join()
    rate = n / (t1 - t0)
    cap = power_cap()
    r.update({"steps_per_s": rate, "power_cap_W": float(cap) if cap else None,
              "mJ_per_step": (r["socket_power_W"] / rate * 1e3) if r["socket_power_W"] else None,
              "how": f"{n} steps back to back over {t1 - t0:.1f} s after the timed loop; "
                     "amd-smi metric --power --clock every 0.5 s (median; first sample skipped)"})
    return r


def cpu_model_name():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return ""


def time_oracle(wl, W, Hs, steps, threads, tail=None, sc_topk=0):
    """Seconds the oracle (as it stands) takes for the first `steps` steps of
    every canvas of block 0, with its BLAS limited to `threads` threads (the
    rest of the oracle is single-threaded numpy)."""
    from threadpoolctl import threadpool_limits

    from oracle import dgd_oracle as O
    P = O.Params(N=wl.N, t_min=wl.t_min, t_max=wl.t_max, confidence=wl.confidence,
                 stability_threshold=wl.stability_threshold, freeze=wl.freeze,
                 final_emit=wl.final_emit)
    W64 = O.bf16_to_f64(W)              # the oracle's own widening, once per table
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        for c in range(wl.B):
            st = O.init_block(O.new_state(wl.G, wl.L), 0, wl.L, wl.V, wl.seeds[c])
            for s in range(steps):
                st, info = O.step(st, Hs[0, s, c], W, 0, s, P, wl.seeds[c], wl.bounds[c],
                                  W64=W64, tail=None if tail is None else O.Tail(**tail))
                if sc_topk:
                    prob, ids, _ = O.sc_topk(info["z"], info["T"], sc_topk)
                    O.sc_embed(prob, ids, W, math.sqrt(wl.d))
        return time.perf_counter() - t0


def cpu_baseline(wl, W, Hs, tail=None, sc_topk=0):
    """Time the oracle (as it stands) on a few full steps of the workload,
    BLAS on every core this process may run on."""
    cores = len(os.sched_getaffinity(0))
    steps = 2 if sc_topk else 3
    dt = time_oracle(wl, W, Hs, steps, cores, tail, sc_topk)
    return {
        "value": steps / dt,
        "unit": "steps/s",
        "cores": int(cores),
        "cpu_model": cpu_model_name(),
        "kind": "oracle",
        "sample": f"{steps} denoising step(s) of {wl.name} ({wl.B}x{wl.L} positions x V={wl.V}, "
                  f"d={wl.d}); oracle float64 numpy, projection via BLAS on {cores} threads, "
                  f"the rest of the step single-threaded",
        "seconds": dt,
    }


def oracle_timing_all():
    """Oracle wall time per step on every workload (BLAS on all cores of the
    affinity set), and single-threaded on the two small ones.  One JSON line."""
    from uniform_state_discrete_step_amd.inputs import WORKLOADS, make_workload_arrays
    cores = len(os.sched_getaffinity(0))
    plan = [("tiny", 8, True), ("small_vocab", 4, True), ("gemma_vocab", 2, False),
            ("batched", 1, False), ("multi_block", 2, False)]
    out = {"kind": "oracle timing", "cores": cores, "cpu_model": cpu_model_name(), "workloads": {}}
    for name, steps, single in plan:
        wl = WORKLOADS[name]
        W, Hs = make_workload_arrays(wl, threads=min(16, cores))
        rec = {"steps_timed": steps, "canvases": wl.B,
               "s_per_step": time_oracle(wl, W, Hs, steps, cores) / steps}
        if single:
            rec["s_per_step_1thread"] = time_oracle(wl, W, Hs, steps, 1) / steps
        rec["s_per_run"] = rec["s_per_step"] * wl.N * wl.blocks
        out["workloads"][name] = rec
        log(f"[bench] oracle {name}: {rec}")
        del W, Hs
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--workload", default="gemma_vocab")
    ap.add_argument("--layout", choices=["packed", "rows", "q4"], default="packed",
                    help="vocabulary table layout: packed once before timing (default), row-major, "
                         "or a 4-bit table (the synthetic table quantized in groups of 32)")
    ap.add_argument("--lm-head-tail", action="store_true",
                    help="output RMSNorm (eps 1e-6) before the projection and a logit softcap "
                         "(c = 30) after it")
    ap.add_argument("--sc-topk", type=int, default=0,
                    help="self-conditioning top-K per position (0 = off), plus the embedding sum")
    ap.add_argument("--label-read", type=int, default=0,
                    help="also time the sparse label read (dgd_label_probs) of this many labels "
                         "over the workload's positions")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power-seconds", type=float, default=3.0,
                    help="after the timed loop, run the step this long while sampling socket "
                         "power and graphics clocks (amd-smi); 0 skips it")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the timed loop (for rocprofv3 runs)")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the CPU oracle on every workload (no GPU), print one JSON line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the timed loop, run one device-to-device copy of this many MiB "
                         "(a known-size kernel against which HBM byte counters are scaled)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the denoising step of "
              "this library is a single-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.oracle_timing:
        oracle_timing_all()
        return

    import torch

    from uniform_state_discrete_step_amd import dgd
    from uniform_state_discrete_step_amd.inputs import (WORKLOADS, make_norm_weight,
                                                        make_workload_arrays, quantize_q4)

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    W, Hs = make_workload_arrays(wl, threads=16)
    log(f"[bench] generated {wl.name} inputs in {time.perf_counter() - t0:.1f}s")
    Wd = torch.from_numpy(W.view(np.int16)).to(dev)
    W_rows = Wd
    layout = {"packed": dgd.DGD_VOCAB_PACKED, "rows": dgd.DGD_VOCAB_ROWS,
              "q4": dgd.DGD_VOCAB_Q4}[args.layout]
    if layout == dgd.DGD_VOCAB_PACKED:
        # one-time rewrite of the table into the projection's streaming order
        Wd = dgd.pack_vocab(Wd, wl.V, wl.d)
        torch.cuda.synchronize()
    elif layout == dgd.DGD_VOCAB_Q4:
        codes, sc, mn = quantize_q4(W)
        Wd = dgd.pack_vocab_q4(torch.from_numpy(codes.reshape(-1)).to(dev),
                               torch.from_numpy(sc.reshape(-1).view(np.int16)).to(dev),
                               torch.from_numpy(mn.reshape(-1).view(np.int16)).to(dev), wl.V, wl.d)
        torch.cuda.synchronize()
        log(f"[bench] quantized the table to 4 bits: {Wd.numel() / 1e9:.3f} GB")
    if not args.sc_topk:
        W_rows = None    # the row-major copy only serves the self-conditioning gather
    Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
    tail, tkw = None, {}
    if args.lm_head_tail:
        tail = {"norm_weight": make_norm_weight(wl.d, wl.cfg_seed), "norm_eps": 1e-6,
                "softcap": 30.0}
        tkw = {"norm_weight": torch.from_numpy(tail["norm_weight"].view(np.int16)).to(dev),
               "norm_eps": tail["norm_eps"], "softcap": tail["softcap"]}
    ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, outputs=False,
                      vocab_layout=layout, sc_topk=args.sc_topk, **tkw)
    sc_out = (torch.empty(wl.B * wl.L * wl.d, dtype=torch.int16, device=dev)
              if args.sc_topk else None)
    params = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence, wl.stability_threshold,
                             wl.freeze, wl.final_emit)
    canvas = torch.zeros(wl.B * wl.G, dtype=torch.int32, device=dev)
    committed = torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    blocks, N = wl.blocks, wl.N
    total = blocks * N
    use_c_loop = sc_out is None

    def run_steps(k, start=0):
        """Enqueue k consecutive denoising steps (block starts included),
        cycling through the generation."""
        if use_c_loop:
            # the library's own loop: no per-step Python
            i = start % total
            while k > 0:
                n = min(k, total - i)
                dgd.dgd_run_steps(Hd.reshape(-1), Wd, canvas, committed, i, n, params, wl.seeds,
                                  ctx)
                k -= n
                i = 0
            return
        for i in range(start, start + k):
            b, s = divmod(i % total, N)
            if s == 0:
                dgd.dgd_init_block(canvas, committed, b, params, wl.seeds, ctx)
            dgd.dgd_step(Hd[b, s].reshape(-1), Wd, canvas, committed, b, s, params, wl.seeds, ctx)
            # the gather reads whole table rows: the row-major copy serves it
            # (16 contiguous bytes per row per thread; the packed table would
            # scatter them over 64-byte lines)
            dgd.dgd_sc_embed(ctx.sc_prob, ctx.sc_id, wl.B * wl.L, args.sc_topk, W_rows,
                             dgd.DGD_VOCAB_ROWS, wl.V, wl.d, math.sqrt(wl.d), sc_out)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    if not args.profile_only:
        # measured ceilings, then an instrumented pass (HIP events around every
        # kernel of every step, on the library's stream) -- both before the
        # timed loop, so they also bring the GPU to its working clocks
        ceil = measured_ceilings(dgd, torch, Wd, dev)
        log(f"[bench] measured ceilings: HBM read {ceil['hbm_read_GBs']:.0f} GB/s, "
            f"MFMA bf16 {ceil['mfma_bf16_TFLOPs']:.0f} TFLOP/s")
        ctx.time_k1 = True
        dgd.dgd_run(Hd.reshape(-1), Wd, canvas, committed, params, wl.seeds, ctx)
        k1_ms, k1_n = ctx.k1_time()
        tail_ms = ctx.tail_time()
        ctx.time_k1 = False
        torch.cuda.synchronize()

    log(f"[bench] warmup {args.warmup} steps")
    run_steps(args.warmup)
    torch.cuda.synchronize()
    # the library enqueues on torch's current stream, where the events are
    # recorded; the K timed steps are split into 5 segments for a spread
    n_seg = 5 if args.steps >= 5 else 1
    bounds = [args.steps * i // n_seg for i in range(n_seg + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_seg + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record()
    for i in range(n_seg):
        run_steps(bounds[i + 1] - bounds[i], start=args.warmup + bounds[i])
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = evs[0].elapsed_time(evs[-1])
    seg_ms_per_step = sorted(evs[i].elapsed_time(evs[i + 1]) / (bounds[i + 1] - bounds[i])
                             for i in range(n_seg))
    log(f"[bench] timed {args.steps} steps: {ms:.2f} ms (wall {wall * 1e3:.2f} ms)")
    if args.profile_only:
        return

    k1_avg_s = k1_ms / max(k1_n, 1) * 1e-3
    tail_avg_s = tail_ms / max(k1_n, 1) * 1e-3
    M = wl.B * wl.L
    table_bytes = (dgd.dgd_q4_vocab_bytes(wl.V, wl.d) if layout == dgd.DGD_VOCAB_Q4
                   else wl.V * wl.d * 2)
    alg_bytes = table_bytes + M * wl.d * 2
    flops = 2.0 * M * wl.V * wl.d
    gbs = alg_bytes / k1_avg_s / 1e9
    tflops = flops / k1_avg_s / 1e12
    hbm_frac = gbs / HBM_PEAK_GBS
    mfma_frac = tflops / MFMA_BF16_PEAK_TFLOPS
    bound = "hbm" if alg_bytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    roof = ({"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": hbm_frac} if bound == "hbm" else
            {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": mfma_frac})
    kname = "k_project" if layout == dgd.DGD_VOCAB_ROWS else "k_project_packed"
    traffic = (measured_traffic(kname)
               if wl.name == "gemma_vocab" and not args.lm_head_tail and not args.sc_topk
               and layout == dgd.DGD_VOCAB_PACKED else None)
    roof.update({"traffic": traffic,
                 "kernel": kname, "kernel_avg_us": k1_avg_s * 1e6,
                 "kernel_launches": k1_n, "algorithmic_bytes_per_launch": alg_bytes,
                 "flops_per_launch": flops,
                 "other": {"hbm_GBs": gbs, "hbm_frac": hbm_frac, "mfma_TFLOPs": tflops,
                           "mfma_frac": mfma_frac},
                 "measured_ceilings": ceil,
                 "frac_of_measured_ceiling": {
                     "hbm": gbs / ceil["hbm_read_GBs"],
                     "mfma": tflops / ceil["mfma_bf16_TFLOPs"]}})

    steps_per_s = args.steps / (ms * 1e-3)
    out = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "canvases": wl.B, "canvas_len": wl.L, "vocab": wl.V,
                   "hidden": wl.d, "gen_length": wl.G, "num_inference_steps": wl.N,
                   "vocab_layout": args.layout,
                   "lm_head_tail": ({"norm_eps": 1e-6, "softcap": 30.0} if args.lm_head_tail
                                    else None),
                   "sc_topk": args.sc_topk},
        "logit_elems_per_s": steps_per_s * M * wl.V,
        "ms_per_step_segments": {"n": n_seg, "median": seg_ms_per_step[n_seg // 2],
                                 "min": seg_ms_per_step[0], "max": seg_ms_per_step[-1]},
        "step_frac_of_hbm_floor": (steps_per_s * alg_bytes) / (HBM_PEAK_GBS * 1e9),
        "step_split_us": {
            "how": "HIP events on the library's stream around every kernel of each step of one "
                   "instrumented dgd_run pass before the timed loop; other = timed ms/step minus both",
            "projection": k1_avg_s * 1e6,
            "merge_commit": tail_avg_s * 1e6,
            "other": ms / args.steps * 1e3 - (k1_avg_s + tail_avg_s) * 1e6},
        "roofline": roof,
    }
    if args.power_seconds > 0:
        out["power"] = power_leg(run_steps, torch, args.power_seconds, args.warmup + args.steps)
    if args.label_read:
        n = args.label_read
        labels = [int(v) for v in np.linspace(0, wl.V - 1, n).astype(np.int64)]
        M = wl.B * wl.L
        probs = torch.empty(M * n, dtype=torch.float32, device=dev)
        H0 = Hd[0, 0].reshape(-1)
        dgd.dgd_label_probs(H0, M, Wd, layout, wl.V, wl.d, labels, 1.0, 0.0, None, probs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 200
        e0.record()
        for _ in range(reps):
            dgd.dgd_label_probs(H0, M, Wd, layout, wl.V, wl.d, labels, 1.0, 0.0, None, probs)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        out["label_read"] = {"n_labels": n, "positions": M, "us_per_call": us,
                             "table_bytes_read": n * wl.d * 2, "vocab_layout": args.layout}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a few steps")
        W_cpu = W
        if layout == dgd.DGD_VOCAB_Q4:
            # the oracle steps on the bf16 table the 4-bit one stands for
            # (dequantized once, outside the timing, as the GPU packs once)
            from oracle import dgd_oracle as O
            W_cpu = O.dequant_q4(codes, sc, mn)
        out["cpu_baseline"] = cpu_baseline(wl, W_cpu, Hs, tail, args.sc_topk)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
