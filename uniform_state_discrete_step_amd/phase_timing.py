"""Where the packed projection's time goes: per-tile phase times.

Runs a workload's denoising steps on the measurement build of the library
(libdgd_phase.so, built by ``__graft_entry__.build()`` or
``python -m uniform_state_discrete_step_amd.build --phase-timing``), whose
packed projection records the wall clock of every wave at the start of each
vocabulary tile, at the end of its K loop and at the end of its epilogue.  The
kernel's instruction stream is the same as the product build's apart from
those clock reads and stores.

Usage: ``python -m uniform_state_discrete_step_amd.phase_timing
[--workload gemma_vocab] [--layout packed|q4] [--warmup 12] [--samples 3]``.
Prints, per sampled step, the launch's span, its HIP-event time and shader
clock, and per tile slot the mean start offset, K-loop time and epilogue time
over all waves (5th and 95th percentiles in brackets), then one JSON line.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

TICK_US = 0.01   # the wall clock runs at 100 MHz


def summarize(prev: np.ndarray, cur: np.ndarray) -> dict:
    """Statistics of the launch that wrote `cur` (entries that changed since
    `prev`, the previous launch's)."""
    ran = cur[:, :, 0] != prev[:, :, 0]                 # (workgroup, wave) of this launch
    t = cur.astype(np.int64)
    t0 = t[:, :, 0][ran].min()
    start = (t[:, :, 0][ran] - t0) * TICK_US
    end = (t[:, :, 14][ran] - t0) * TICK_US
    wall_s = (t[:, :, 14] - t[:, :, 0])[ran] * TICK_US * 1e-6
    clock_ghz = float(np.median((t[:, :, 15] - t[:, :, 1])[ran] / wall_s) / 1e9)
    out = {"waves": int(ran.sum()), "span_us": float(end.max()),
           "start_spread_us": float(start.max()), "end_first_us": float(end.min()),
           "shader_clock_ghz": clock_ghz, "tiles": []}
    pct = lambda a: [float(np.percentile(a, 5)), float(np.percentile(a, 95))]
    for k in range(4):
        s0, s1, s2 = 2 + 3 * k, 3 + 3 * k, 4 + 3 * k
        fresh = ran & (cur[:, :, s0] != prev[:, :, s0]) & (cur[:, :, s2] != prev[:, :, s2])
        if not fresh.any():
            break
        ts, tk, te = t[:, :, s0][fresh], t[:, :, s1][fresh], t[:, :, s2][fresh]
        kl, ep = (tk - ts) * TICK_US, (te - tk) * TICK_US
        st = (ts - t0) * TICK_US
        out["tiles"].append({"start_us": float(st.mean()), "start_sd_us": float(st.std()),
                             "k_loop_us": float(kl.mean()), "k_loop_p5_p95": pct(kl),
                             "epilogue_us": float(ep.mean()), "epilogue_p5_p95": pct(ep)})
    out["prologue_us"] = float(((t[:, :, 2] - t[:, :, 0])[ran] * TICK_US).mean())
    out["final_merge_us"] = float(((t[:, :, 14] - t[:, :, 13])[ran] * TICK_US).mean())
    return out


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="gemma_vocab")
    ap.add_argument("--layout", choices=("packed", "q4"), default="packed",
                    help="the bf16 packed table, or the 4-bit table (the synthetic table quantized "
                         "in groups of 32)")
    ap.add_argument("--warmup", type=int, default=12, help="steps before the sampled ones")
    ap.add_argument("--samples", type=int, default=3, help="sampled steps")
    args = ap.parse_args(argv)

    import torch

    from uniform_state_discrete_step_amd import dgd
    from uniform_state_discrete_step_amd.inputs import WORKLOADS, make_workload_arrays, quantize_q4

    dgd.load_library(dgd.LIB_PHASE_PATH)   # before anything loads the product build
    wl = WORKLOADS[args.workload]
    if args.warmup + args.samples > wl.N:
        sys.exit(f"--warmup + --samples must not exceed the {wl.N} steps of a block")
    dev = torch.device("cuda:0")
    W, Hs = make_workload_arrays(wl, threads=16)
    if args.layout == "q4":
        codes, sc, mn = quantize_q4(W)
        Wd = dgd.pack_vocab_q4(torch.from_numpy(codes.reshape(-1)).to(dev),
                               torch.from_numpy(sc.reshape(-1).view(np.int16)).to(dev),
                               torch.from_numpy(mn.reshape(-1).view(np.int16)).to(dev), wl.V, wl.d)
        layout = dgd.DGD_VOCAB_Q4
    else:
        Wd = dgd.pack_vocab(torch.from_numpy(W.view(np.int16)).to(dev), wl.V, wl.d)
        layout = dgd.DGD_VOCAB_PACKED
    Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
    ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, outputs=False,
                      vocab_layout=layout)
    params = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence, wl.stability_threshold,
                             wl.freeze, wl.final_emit)
    canvas = torch.zeros(wl.B * wl.G, dtype=torch.int32, device=dev)
    committed = torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=dev)
    dgd.dgd_init_block(canvas, committed, 0, params, wl.seeds, ctx)
    for s in range(args.warmup):
        dgd.dgd_step(Hd[0, s].reshape(-1), Wd, canvas, committed, 0, s, params, wl.seeds, ctx)
    torch.cuda.synchronize()
    prev = dgd.dgd_phase_times()
    results = []
    ctx.time_k1 = True
    for s in range(args.warmup, args.warmup + args.samples):
        dgd.dgd_step(Hd[0, s].reshape(-1), Wd, canvas, committed, 0, s, params, wl.seeds, ctx)
        torch.cuda.synchronize()
        cur = dgd.dgd_phase_times()
        k1_ms, k1_n = ctx.k1_time()
        r = summarize(prev, cur)
        r["step"] = s
        r["event_us"] = 1e3 * k1_ms / max(k1_n, 1)
        results.append(r)
        prev = cur
        print(f"step {s}: span {r['span_us']:.1f} us (HIP events {r['event_us']:.1f} us), "
              f"{r['waves']} waves, starts within {r['start_spread_us']:.1f} us, ends "
              f"{r['end_first_us']:.1f}..{r['span_us']:.1f} us, shader clock "
              f"{r['shader_clock_ghz']:.2f} GHz", flush=True)
        for k, tl in enumerate(r["tiles"]):
            print(f"  tile {k}: start {tl['start_us']:6.1f} (sd {tl['start_sd_us']:4.1f})  "
                  f"K loop {tl['k_loop_us']:5.1f} [{tl['k_loop_p5_p95'][0]:5.1f}, "
                  f"{tl['k_loop_p5_p95'][1]:5.1f}]  epilogue {tl['epilogue_us']:5.1f} "
                  f"[{tl['epilogue_p5_p95'][0]:5.1f}, {tl['epilogue_p5_p95'][1]:5.1f}]", flush=True)
        print(f"  prologue {r['prologue_us']:.1f} us, final merge {r['final_merge_us']:.1f} us",
              flush=True)
    print(json.dumps({"workload": wl.name, "layout": args.layout, "samples": results}))


if __name__ == "__main__":
    main()
