"""Socket power and graphics clocks while the denoising step runs, beside the
two measured ceilings (a streaming read of the table and a bf16 MFMA loop).

Each part runs back to back for ``--seconds`` while a sampler thread reads
``amd-smi metric --power --clock`` every ``--interval`` seconds.  Per part the
script prints the achieved rate, the median socket power and the median
graphics clock over the samples taken while it ran, then one JSON line.
Reading these counters changes no setting of the GPU.

Usage: ``python -m uniform_state_discrete_step_amd.power_trace [--workload gemma_vocab]
[--seconds 6] [--interval 0.5] [--q4]`` (``--q4`` adds the step on the 4-bit table).
"""
from __future__ import annotations

import argparse
import json
import re
import statistics
import subprocess
import threading
import time

import numpy as np


def parse_smi(out: str) -> tuple[float | None, list[float]]:
    """(socket power in W, graphics clock of each XCD in MHz) from the JSON
    text of ``amd-smi metric --power --clock --json`` (first GPU)."""
    p = re.search(r'"socket_power":\s*\{\s*"value":\s*([0-9.]+)', out)
    clks = re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*([0-9.]+)', out)
    return (float(p.group(1)) if p else None), [float(c) for c in clks]


def read_smi() -> tuple[float | None, list[float]]:
    """(socket power in W, graphics clock of each XCD in MHz) of GPU 0."""
    try:
        out = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"],
                             capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.TimeoutExpired):
        return None, []
    return parse_smi(out)


def power_cap() -> str | None:
    """The board's power cap as rocm-smi reports it (None if unavailable)."""
    try:
        out = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True,
                             timeout=20).stdout
    except (OSError, subprocess.TimeoutExpired):
        return None
    m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", out)
    return m.group(1) if m else None


class Sampler(threading.Thread):
    def __init__(self, interval: float):
        super().__init__(daemon=True)
        self.interval, self.samples, self.stop = interval, [], threading.Event()

    def run(self):
        while not self.stop.is_set():
            t = time.perf_counter()
            p, clks = read_smi()
            self.samples.append((t, p, clks))
            self.stop.wait(max(0.0, self.interval - (time.perf_counter() - t)))

    def between(self, t0: float, t1: float) -> dict:
        # skip the first sample of a part: the counters average over a window
        sel = [s for s in self.samples if t0 + self.interval <= s[0] <= t1]
        pw = [s[1] for s in sel if s[1] is not None]
        ck = [statistics.mean(s[2]) for s in sel if s[2]]
        return {"samples": len(sel),
                "socket_power_W": statistics.median(pw) if pw else None,
                "socket_power_max_W": max(pw) if pw else None,
                "gfx_clock_MHz": statistics.median(ck) if ck else None}


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="gemma_vocab")
    ap.add_argument("--seconds", type=float, default=6.0, help="run time of each part")
    ap.add_argument("--interval", type=float, default=0.5, help="sampling interval (s)")
    ap.add_argument("--q4", action="store_true",
                    help="also run the step on the 4-bit table (the synthetic table quantized in "
                         "groups of 32)")
    args = ap.parse_args(argv)

    import torch

    from uniform_state_discrete_step_amd import dgd
    from uniform_state_discrete_step_amd.inputs import WORKLOADS, make_workload_arrays, quantize_q4

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    W, Hs = make_workload_arrays(wl, threads=16)
    Wd = dgd.pack_vocab(torch.from_numpy(W.view(np.int16)).to(dev), wl.V, wl.d)
    Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
    ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, outputs=False,
                      vocab_layout=dgd.DGD_VOCAB_PACKED)
    if args.q4:
        codes, sc, mn = quantize_q4(W)
        Wq = dgd.pack_vocab_q4(torch.from_numpy(codes.reshape(-1)).to(dev),
                               torch.from_numpy(sc.reshape(-1).view(np.int16)).to(dev),
                               torch.from_numpy(mn.reshape(-1).view(np.int16)).to(dev), wl.V, wl.d)
        ctx_q4 = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, outputs=False,
                             vocab_layout=dgd.DGD_VOCAB_Q4)
    params = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence, wl.stability_threshold,
                             wl.freeze, wl.final_emit)
    canvas = torch.zeros(wl.B * wl.G, dtype=torch.int32, device=dev)
    committed = torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=dev)
    total = wl.blocks * wl.N
    nbytes = Wd.numel() * Wd.element_size()
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    wgs, rounds = 256, 3000
    fsink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    mfma_bytes = min(nbytes, 1 << 26)

    def steps(n, table=Wd, c=ctx):
        dgd.dgd_run_steps(Hd.reshape(-1), table, canvas, committed, 0, min(n, total), params,
                          wl.seeds, c)
        return min(n, total)

    parts = {
        # name: (one batch of work -> units done, unit, units per batch)
        "hbm_read": (lambda: [dgd.dgd_ceiling_hbm_read(Wd, nbytes, sink) for _ in range(20)],
                     "GB/s", 20 * nbytes / 1e9),
        "mfma_bf16": (lambda: [dgd.dgd_ceiling_mfma_bf16(Wd, mfma_bytes, rounds, wgs, fsink)
                               for _ in range(2)],
                      "TFLOP/s", 2 * wgs * 4 * rounds * 64 * 32768.0 / 1e12),
        "denoising_step": (lambda: steps(total), "steps/s", float(total)),
    }
    if args.q4:
        parts["denoising_step_q4"] = (lambda: steps(total, Wq, ctx_q4), "steps/s", float(total))
    for fn, _, _ in parts.values():   # warm up (and load) every kernel once
        fn()
    torch.cuda.synchronize()

    sampler = Sampler(args.interval)
    sampler.start()
    time.sleep(2 * args.interval)
    results = {"power_cap_W": power_cap()}
    t0 = time.perf_counter()
    time.sleep(max(2.0, 4 * args.interval))
    results["idle"] = sampler.between(t0, time.perf_counter())
    for name, (fn, unit, per_batch) in parts.items():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        batches = 0
        while time.perf_counter() - t0 < args.seconds:
            fn()
            batches += 1
            torch.cuda.synchronize()
        t1 = time.perf_counter()
        r = sampler.between(t0, t1)
        r["rate"] = batches * per_batch / (t1 - t0)
        r["unit"] = unit
        results[name] = r
        print(f"{name}: {r['rate']:.1f} {unit}, socket power {r['socket_power_W']} W "
              f"(max {r['socket_power_max_W']}), gfx clock {r['gfx_clock_MHz']} MHz, "
              f"{r['samples']} samples", flush=True)
    sampler.stop.set()
    sampler.join()
    print(f"idle: socket power {results['idle']['socket_power_W']} W, gfx clock "
          f"{results['idle']['gfx_clock_MHz']} MHz; power cap {results['power_cap_W']} W", flush=True)
    print(json.dumps({"workload": wl.name, **results}))


if __name__ == "__main__":
    main()
