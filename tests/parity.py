"""Lockstep comparison of the HIP step with the CPU oracle, with tie bands.

Sticky commits cascade (one flipped decision changes every later step), so
the GPU is compared in lockstep: before every step it receives the oracle's
state (canvas, committed mask, previous argmax, stability count, done flag)
and that single step's outputs are compared.

Agreement criteria (float tolerances are those the method's specification
fixes for bf16 inputs with fp32 accumulation):
* entropies within 1e-3 nats at every position;
* argmax equal unless the oracle's top two tempered logits are within 1e-5;
* sampled tokens equal unless the oracle's top two Gumbel-perturbed logits
  are within 1e-4;
* commit decisions equal unless the position is in the commit band: its
  entropy is within 1e-5 nats of the last accepted or first rejected
  entropy, or it is one of those two ranks and the running sum before it is
  within 1e-5 of the bound;
* the early-stop decision equal unless |mean entropy - confidence| < 1e-5,
  or the oracle's own rule, given the GPU's argmax canvas (whose every
  difference is a validated argmax band event), reaches the GPU's decision;
* re-noised and initial tokens bit-exact (pure integer functions);
* self-conditioning top-K: the same ids unless an id's oracle tempered logit
  is within 1e-4 of the K-th one (the sample band: both rest on the same fp32
  logits), listed best first up to that band, probabilities within 1e-3
  relative (the entropy bar: an error of e nats in x - lse moves p by e) or
  1e-30 absolute (float32 probabilities flush below its normal range).
* an excused mismatch must itself be a valid choice: the oracle's tempered
  logit at the GPU's argmax within 1e-5 of the maximum, the oracle's
  perturbed logit at the GPU's sample within 1e-4 of the largest;
* the GPU's gap output (top-two Gumbel gap, nats) within 2e-3 nats of the
  oracle's (two perturbed values, each held to the 1e-3 nats bar of a
  per-position float output) plus fp32 rounding at their magnitude;
* band events at most max(3, 0.5%) of the compared position-steps (the
  expected rates are ~1e-4 per position-step: the top-two spacing of the
  perturbed values is exponential with mean ~1 nat, that of the tempered
  logits ~0.02-0.05 nats on the flattest rows).
Band events are counted, never hidden.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import dgd_oracle as O
from uniform_state_discrete_step_amd.inputs import quantize_q4

TOL_ENTROPY = 1e-3
BAND_ARGMAX = 1e-5
BAND_SAMPLE = 1e-4
BAND_COMMIT = 1e-5
BAND_CONV = 1e-5
TOL_LOGIT_REL = 2e-2
BAND_SC = 1e-4
TOL_SC_PROB_REL = 1e-3
TOL_SC_PROB_ABS = 1e-30
TOL_GAP = 2 * TOL_ENTROPY
BAND_CAP_FRAC = 0.005
BAND_CAP_MIN = 3
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@dataclasses.dataclass
class Report:
    steps: int = 0
    positions: int = 0
    stat_rows: int = 0          # position-steps whose statistics were compared with the oracle's
    max_entropy_err: float = 0.0
    max_gap_err: float = 0.0
    argmax_band: int = 0
    sample_band: int = 0
    commit_band: int = 0
    conv_band: int = 0
    renoised: int = 0
    accepted: int = 0
    norm_rows: int = 0
    norm_inexact: int = 0
    sc_rows: int = 0
    sc_band: int = 0
    sc_recomputed: int = 0
    free_steps: int = 0         # free-running steps before the first divergence
    divergence: tuple = None    # (block, step, canvas) of the first divergence of a free run
    resyncs: int = 0
    failures: list = dataclasses.field(default_factory=list)

    def fail(self, msg):
        if len(self.failures) < 50:
            self.failures.append(msg)

    @property
    def band_events(self) -> int:
        return self.argmax_band + self.sample_band + self.commit_band + self.conv_band

    def check_band_rate(self):
        """Band events may not exceed max(BAND_CAP_MIN, BAND_CAP_FRAC) of the
        compared position-steps: a systematic error cannot hide in the bands."""
        n = max(self.stat_rows, 1)
        cap = max(BAND_CAP_MIN, BAND_CAP_FRAC * n)
        if self.band_events > cap:
            self.fail(f"{self.band_events} band events over {n} compared position-steps "
                      f"(cap {cap:.1f})")

    def summary(self) -> str:
        return (f"steps={self.steps} positions={self.positions} compared={self.stat_rows} "
                f"max|dH|={self.max_entropy_err:.2e} max|dgap|={self.max_gap_err:.2e} "
                f"bands: argmax={self.argmax_band} sample={self.sample_band} "
                f"commit={self.commit_band} convergence={self.conv_band} "
                f"accepted={self.accepted} renoised={self.renoised}"
                + (f" free steps={self.free_steps} first divergence={self.divergence} "
                   f"resyncs={self.resyncs}" if self.free_steps or self.divergence else "")
                + (f" norm rows={self.norm_rows} (1-step diffs {self.norm_inexact})"
                   if self.norm_rows else "")
                + (f" sc rows={self.sc_rows} band={self.sc_band} recomputed parts="
                   f"{self.sc_recomputed}" if self.sc_rows else ""))


def oracle_stats(z, T, seed, p_abs, gstep, threads=None):
    """O.position_stats over chunks of rows in threads.  Rows are independent
    in every quantity it returns, so the result is the same as one call."""
    threads = THREADS if threads is None else threads
    rows = z.shape[0]
    p_abs = np.asarray(p_abs)
    if threads <= 1 or rows < 2 * threads:
        return O.position_stats(z, T, seed, p_abs, gstep)
    chunks = [c for c in np.array_split(np.arange(rows), threads) if c.size]
    with ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: O.position_stats(z[c], T, seed, p_abs[c], gstep), chunks))
    return {k: np.concatenate([pt[k] for pt in parts]) for k in parts[0]}


def oracle_step(state, H_bits, W_bits, block, step_idx, P, seed, bound, W64=None, tail=None):
    """O.step, with the per-position statistics taken by oracle_stats."""
    if state.done:
        return state.copy(), {"skipped": True}
    L, V = H_bits.shape[0], W_bits.shape[0]
    T = O.temperature(step_idx, P.N, P.t_min, P.t_max)
    z = O.logits(H_bits, W_bits, tail, W64=W64)
    stats = oracle_stats(z, T, seed, block * L + np.arange(L), block * P.N + step_idx)
    new, info = O.step_from_stats(state, stats, block, step_idx, L, V, P, seed, bound)
    info["T"] = T
    info["z"] = z
    return new, info


def q4_device_table(W, V, d, device):
    """The packed 4-bit form of a bf16 table (quantized on the host)."""
    import torch
    from uniform_state_discrete_step_amd import dgd
    codes, sc, mn = quantize_q4(W)
    return dgd.pack_vocab_q4(torch.from_numpy(codes.reshape(-1)).to(device),
                             torch.from_numpy(sc.reshape(-1).view(np.int16)).to(device),
                             torch.from_numpy(mn.reshape(-1).view(np.int16)).to(device), V, d)


def ordered_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns -> integers in the order of the values (adjacent
    values differ by 1; +0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def commit_band_positions(info, bound) -> set:
    """Positions whose commit decision may legitimately differ (see module doc)."""
    order = info.get("order")
    if not order:
        return set()
    h = info["stats"]["entropy"].astype(np.float64)
    sums = info["sums"]
    acc = info["accepted"]
    k = int(sum(1 for p in order if acc[p]))          # accepted ranks 0..k-1
    edges = [r for r in (k - 1, k) if 0 <= r < len(order)]
    band = set()
    for r, p in enumerate(order):
        if any(abs(h[p] - h[order[e]]) <= BAND_COMMIT for e in edges):
            band.add(p)
        if r in edges and abs(sums[r] - bound) <= BAND_COMMIT:
            band.add(p)
    return band


def compare_stats(rep: Report, tag: str, st: dict, gpu: dict, z, T: float, seed: int, p_abs,
                  gstep: int, rows=None):
    """Entropy / argmax / sample / gap agreement for the rows of an oracle
    stats dict.  gpu: the GPU's "entropy", "argmax", "token" and (optional)
    "gap" of the same rows; z, T: the oracle's logits of those rows and the
    temperature; seed, p_abs, gstep: the rows' noise coordinates.  Returns the
    sets of rows whose argmax / sample differ (every one a validated band
    event, or a recorded failure)."""
    H_gpu, A_gpu, T_gpu = gpu["entropy"], gpu["argmax"], gpu["token"]
    H_o, A_o, T_o = st["entropy"], st["argmax"], st["token"]
    n, V = z.shape
    p_abs = np.asarray(p_abs).reshape(-1)
    rep.stat_rows += n
    err = float(np.max(np.abs(H_gpu.astype(np.float64) - H_o.astype(np.float64))))
    rep.max_entropy_err = max(rep.max_entropy_err, err)
    if err > TOL_ENTROPY:
        rep.fail(f"{tag}: entropy error {err:.3e} > {TOL_ENTROPY}")

    def where(i):
        return i if rows is None else rows[i]

    am = np.nonzero(A_gpu != A_o)[0]
    for i in am:
        a = int(A_gpu[i])
        x = z[i] / T
        ok = st["argmax_gap"][i] < BAND_ARGMAX and 0 <= a < V and x[a] >= x.max() - BAND_ARGMAX
        if ok:
            rep.argmax_band += 1
        else:
            rep.fail(f"{tag}: argmax differs at row {where(i)} (gpu {a}, oracle {A_o[i]}, "
                     f"gap {st['argmax_gap'][i]:.3e}"
                     + (f", oracle x at gpu id {x[a]:.7g} vs max {x.max():.7g})" if 0 <= a < V
                        else ")"))
    tm = np.nonzero(T_gpu != T_o)[0]
    for i in tm:
        t = int(T_gpu[i])
        y = (z[i, t] / T + float(O.gumbel_at(seed, p_abs[i], gstep, t))) if 0 <= t < V else -np.inf
        if st["gap"][i] < BAND_SAMPLE and y >= st["y1"][i] - BAND_SAMPLE:
            rep.sample_band += 1
        else:
            rep.fail(f"{tag}: token differs at row {where(i)} (gpu {t}, oracle {T_o[i]}, "
                     f"gap {st['gap'][i]:.3e}, oracle y at gpu id {y:.7g} vs y1 {st['y1'][i]:.7g})")
    if gpu.get("gap") is not None:
        g_o = st["gap"]
        fin = np.isfinite(g_o)
        if np.any(fin):
            dg = np.abs(gpu["gap"].astype(np.float64)[fin] - g_o[fin])
            tol = TOL_GAP + 2.0 ** -20 * (np.abs(st["y1"][fin]) + np.abs(st["y2"][fin]))
            rep.max_gap_err = max(rep.max_gap_err, float(dg.max()))
            bad = np.nonzero(dg > tol)[0]
            if bad.size:
                i = np.nonzero(fin)[0][bad[0]]
                rep.fail(f"{tag}: gap differs at row {where(i)} (gpu {gpu['gap'][i]:.7g}, "
                         f"oracle {g_o[i]:.7g})")
    return set(am.tolist()), set(tm.tolist())


def compare_sc(rep: Report, tag: str, z, T: float, K: int, prob_gpu, id_gpu, status_gpu=None,
               rows=None):
    """Self-conditioning top-K of the GPU against the oracle's, row by row."""
    prob_o, ids_o, x = O.sc_topk(z, T, K)
    for r in range(z.shape[0]):
        rt = r if rows is None else rows[r]
        rep.sc_rows += 1
        if status_gpu is not None:
            if status_gpu[r] < 0:
                rep.fail(f"{tag} row {rt}: self-conditioning recomputation budget ran out")
            rep.sc_recomputed += int(max(status_gpu[r], 0))
        g, o = [int(v) for v in id_gpu[r]], [int(v) for v in ids_o[r]]
        if any(v < 0 or v >= x.shape[1] for v in g):
            rep.fail(f"{tag} row {rt}: invalid self-conditioning id in {g}")
            continue
        xk = x[r, o[-1]]
        diff = set(g) ^ set(o)
        for v in diff:
            if abs(x[r, v] - xk) <= BAND_SC:
                rep.sc_band += 1
            else:
                rep.fail(f"{tag} row {rt}: top-{K} id {v} differs (x {x[r, v]:.6f}, K-th {xk:.6f})")
        xs = x[r, g]
        if np.any(xs[1:] > xs[:-1] + BAND_SC):
            rep.fail(f"{tag} row {rt}: top-{K} not in descending order")
        po = dict(zip(o, prob_o[r]))
        for j, v in enumerate(g):
            if v in po and abs(prob_gpu[r, j] - po[v]) > TOL_SC_PROB_REL * po[v] + TOL_SC_PROB_ABS:
                rep.fail(f"{tag} row {rt}: probability of id {v}: gpu {prob_gpu[r, j]:.6e}, "
                         f"oracle {po[v]:.6e}")


def compare_step(rep: Report, tag: str, before: O.CanvasState, after: O.CanvasState, info: dict,
                 gpu: dict, L: int, V: int, block: int, step: int, params: O.Params, seed: int,
                 bound: float):
    """Compare one canvas' step.  ``gpu`` holds the GPU's outputs and new state."""
    base = block * L
    blk = slice(base, base + L)
    if info.get("skipped"):
        if not (np.array_equal(gpu["canvas"], before.canvas)
                and np.array_equal(gpu["committed"], before.committed)):
            rep.fail(f"{tag}: a done canvas was modified")
        return
    rep.steps += 1
    rep.positions += L
    st = info["stats"]
    gstep = block * params.N + step
    am_set, tok_set = compare_stats(rep, tag, st, gpu, info["z"], info["T"], seed,
                                    base + np.arange(L), gstep)
    if not np.array_equal(gpu["prev_argmax"], gpu["argmax"]):
        rep.fail(f"{tag}: state prev_argmax is not this step's argmax")
    # untouched regions
    if not np.array_equal(np.delete(gpu["canvas"], np.arange(base, base + L)),
                          np.delete(before.canvas, np.arange(base, base + L))):
        rep.fail(f"{tag}: positions outside the block changed")

    gpu_final = bool(gpu["done"])
    if gpu_final != info["final"]:
        conf = float(np.float32(params.confidence))
        near = abs(info["mean_H"] - conf) < BAND_CONV
        # the oracle's rule on the GPU's argmax canvas (its differences are
        # validated argmax band events, or have failed above)
        stable_g = bool(np.all(gpu["argmax"] == before.prev_argmax))
        count_g = before.stable_count + 1 if stable_g else 0
        final_g = ((info["mean_H"] < conf and count_g >= params.stability_threshold)
                   or step == params.N - 1)
        if near or (am_set and final_g == gpu_final):
            rep.conv_band += 1
        else:
            rep.fail(f"{tag}: final-step decision differs (gpu {gpu_final}, oracle "
                     f"{info['final']}, mean H {info['mean_H']:.6g})")
        return
    if int(gpu["steps_used"]) != step + 1:
        rep.fail(f"{tag}: steps_used {gpu['steps_used']} != {step + 1}")

    g_can, g_com = gpu["canvas"][blk], gpu["committed"][blk]
    o_can, o_com = after.canvas[blk], after.committed[blk]
    b_can, b_com = before.canvas[blk], before.committed[blk]
    if info["final"]:
        if not np.all(g_com == 1):
            rep.fail(f"{tag}: final step left positions open")
        for p in range(L):
            if g_can[p] != o_can[p]:
                band = (p in am_set) if params.final_emit else (p in tok_set)
                if not band:
                    rep.fail(f"{tag}: final token differs at {p} (gpu {g_can[p]}, oracle {o_can[p]})")
        return

    band = commit_band_positions(info, bound)
    p_abs = base + np.arange(L)
    renoise = O.renoise_token(seed, p_abs, gstep, V)
    for p in range(L):
        if g_com[p] != o_com[p]:
            if p in band:
                rep.commit_band += 1
            else:
                rep.fail(f"{tag}: commit decision differs at {p} (gpu {g_com[p]}, oracle {o_com[p]},"
                         f" H {st['entropy'][p]:.6g})")
            continue
        eligible = params.freeze == 0 or b_com[p] == 0
        if not eligible:
            if g_can[p] != b_can[p]:
                rep.fail(f"{tag}: frozen position {p} changed")
            continue
        if g_com[p] == 1:
            rep.accepted += 1
            if g_can[p] != gpu["token"][p]:
                rep.fail(f"{tag}: accepted position {p} does not hold its sample")
            if g_can[p] != o_can[p] and p not in tok_set:
                rep.fail(f"{tag}: accepted token differs at {p}")
        else:
            rep.renoised += 1
            if g_can[p] != renoise[p] or o_can[p] != renoise[p]:
                rep.fail(f"{tag}: re-noised token differs at {p} (gpu {g_can[p]}, "
                         f"oracle {o_can[p]}, expected {renoise[p]})")


class Lockstep:
    """Drive the HIP library and the oracle side by side on one workload."""

    def __init__(self, wl, W, Hs, device, logits=False, layout=0, tail: O.Tail = None, sc_topk=0):
        import torch
        from uniform_state_discrete_step_amd import dgd
        self.dgd, self.torch = dgd, torch
        self.wl, self.W, self.Hs, self.dev = wl, W, Hs, device
        self.tail = tail
        if layout == dgd.DGD_VOCAB_Q4:
            # a 4-bit table: the GPU streams its packed form, the oracle
            # steps on the bf16 table it stands for
            self.Wd = q4_device_table(W, wl.V, wl.d, device)
            self.W = W = O.dequant_q4(*quantize_q4(W))
        else:
            self.Wd = torch.from_numpy(W.view(np.int16)).to(device)
            if layout == dgd.DGD_VOCAB_PACKED:
                self.Wd = dgd.pack_vocab(self.Wd, wl.V, wl.d)
        self.Hd = torch.from_numpy(Hs.view(np.int16)).to(device)
        tkw = {}
        if tail is not None:
            if tail.norm_weight is not None:
                tkw["norm_weight"] = torch.from_numpy(
                    np.ascontiguousarray(tail.norm_weight).view(np.int16)).to(device)
                tkw["norm_eps"] = tail.norm_eps
            tkw["softcap"] = tail.softcap
        self.sc_topk = sc_topk
        self.ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=device,
                               logits=logits, vocab_layout=layout, sc_topk=sc_topk,
                               sc_status=sc_topk > 0, **tkw)
        self.params = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence,
                                      wl.stability_threshold, wl.freeze, wl.final_emit)
        self.P = O.Params(N=wl.N, t_min=wl.t_min, t_max=wl.t_max, confidence=wl.confidence,
                          stability_threshold=wl.stability_threshold, freeze=wl.freeze,
                          final_emit=wl.final_emit)
        self.canvas = torch.zeros(wl.B * wl.G, dtype=torch.int32, device=device)
        self.committed = torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=device)
        self.W64 = O.bf16_to_f64(W)
        self.states = [O.new_state(wl.G, wl.L) for _ in range(wl.B)]

    def push_state(self):
        """Copy the oracle's state of every canvas into the GPU buffers."""
        torch, wl = self.torch, self.wl
        can = np.concatenate([s.canvas for s in self.states]).astype(np.int32)
        com = np.concatenate([s.committed for s in self.states]).astype(np.uint8)
        self.canvas.copy_(torch.from_numpy(can))
        self.committed.copy_(torch.from_numpy(com))
        sv = self.ctx.state_views()
        sv["prev_argmax"].copy_(torch.from_numpy(
            np.concatenate([s.prev_argmax for s in self.states]).astype(np.int32)))
        sv["stable_count"].copy_(torch.tensor([s.stable_count for s in self.states], dtype=torch.int32))
        sv["done"].copy_(torch.tensor([int(s.done) for s in self.states], dtype=torch.int32))
        sv["steps_used"].copy_(torch.tensor([s.steps_used for s in self.states], dtype=torch.int32))

    def pull(self, c):
        wl = self.wl
        sl = slice(c * wl.L, (c + 1) * wl.L)
        sv = self.ctx.state_views()
        return {
            "entropy": self.ctx.entropy[sl].cpu().numpy(),
            "argmax": self.ctx.argmax[sl].cpu().numpy().astype(np.int64),
            "token": self.ctx.token[sl].cpu().numpy().astype(np.int64),
            "gap": self.ctx.gap[sl].cpu().numpy(),
            "canvas": self.canvas[c * wl.G:(c + 1) * wl.G].cpu().numpy().astype(np.int64),
            "committed": self.committed[c * wl.G:(c + 1) * wl.G].cpu().numpy(),
            "prev_argmax": sv["prev_argmax"][sl].cpu().numpy().astype(np.int64),
            "done": int(sv["done"][c]),
            "steps_used": int(sv["steps_used"][c]),
        }

    def check_norm(self, rep: Report, b: int, s_idx: int):
        """The normalised rows the GPU wrote: within one bfloat16 step of the
        oracle's (both round once from a float64 value; only the order of the
        norm's sum differs)."""
        wl = self.wl
        g = self.ctx.norm_h.cpu().numpy().view(np.uint16).reshape(wl.B * wl.L, wl.d)
        o = O.rms_norm(self.Hs[b, s_idx].reshape(wl.B * wl.L, wl.d), self.tail.norm_weight,
                       self.tail.norm_eps)
        ulp = np.abs(ordered_bf16(g) - ordered_bf16(o))
        rep.norm_rows += g.shape[0]
        rep.norm_inexact += int(np.count_nonzero(ulp))
        if ulp.max() > 1:
            r, k = np.unravel_index(int(np.argmax(ulp)), ulp.shape)
            rep.fail(f"block {b} step {s_idx}: normalised row {r} element {k} differs by "
                     f"{int(ulp.max())} bf16 steps (gpu {g[r, k]:#06x}, oracle {o[r, k]:#06x})")

    def gpu_state(self, c) -> O.CanvasState:
        """The GPU's canvas, mask and state of canvas c, as an oracle state."""
        wl = self.wl
        sv = self.ctx.state_views()
        return O.CanvasState(
            self.canvas[c * wl.G:(c + 1) * wl.G].cpu().numpy().astype(np.int64),
            self.committed[c * wl.G:(c + 1) * wl.G].cpu().numpy().copy(),
            sv["prev_argmax"][c * wl.L:(c + 1) * wl.L].cpu().numpy().astype(np.int64),
            int(sv["stable_count"][c]), bool(int(sv["done"][c])), int(sv["steps_used"][c]))

    def run(self, blocks=None, steps=None, rep: Report = None, progress=None,
            free=False) -> Report:
        """Step both sides and compare every step.

        free=False (lockstep): before every step the GPU receives the
        oracle's state.  free=True: the GPU runs on its own state; after each
        step its state must equal the oracle's.  At the first step where they
        part, both had started from the same state, so that step has already
        been compared as a lockstep step: it must show a counted band event
        (else it fails).  The oracle's state is then pushed to the GPU
        (resync) and the run goes on, so every step is still compared."""
        torch, wl, dgd = self.torch, self.wl, self.dgd
        rep = rep or Report()
        if free:
            assert steps is None, "a free run takes every step"
        for b in (range(wl.blocks) if blocks is None else blocks):
            self.states = [O.init_block(s, b, wl.L, wl.V, wl.seeds[c])
                           for c, s in enumerate(self.states)]
            dgd.dgd_init_block(self.canvas, self.committed, b, self.params, wl.seeds, self.ctx)
            torch.cuda.synchronize()
            can = self.canvas.cpu().numpy()
            for c, s in enumerate(self.states):
                if not np.array_equal(can[c * wl.G:(c + 1) * wl.G], s.canvas):
                    rep.fail(f"block {b} canvas {c}: initial tokens differ")
            synced = free
            for s_idx in (range(wl.N) if steps is None else steps):
                if not synced:
                    self.push_state()
                    synced = free
                dgd.dgd_step(self.Hd[b, s_idx].reshape(-1), self.Wd, self.canvas, self.committed,
                             b, s_idx, self.params, wl.seeds, self.ctx)
                torch.cuda.synchronize()
                if self.tail is not None and self.tail.norm_weight is not None:
                    self.check_norm(rep, b, s_idx)
                for c in range(wl.B):
                    before = self.states[c]
                    after, info = oracle_step(before, self.Hs[b, s_idx, c], self.W, b, s_idx,
                                              self.P, wl.seeds[c], wl.bounds[c], W64=self.W64,
                                              tail=self.tail)
                    tag = f"block {b} step {s_idx} canvas {c}"
                    n_bands = rep.band_events
                    compare_step(rep, tag, before, after, info, self.pull(c), wl.L, wl.V, b, s_idx,
                                 self.P, wl.seeds[c], float(np.float32(wl.bounds[c])))
                    if self.sc_topk and not info.get("skipped"):
                        K, sl = self.sc_topk, slice(c * wl.L, (c + 1) * wl.L)
                        compare_sc(rep, tag, info["z"], info["T"], K,
                                   self.ctx.sc_prob.cpu().numpy().reshape(-1, K)[sl],
                                   self.ctx.sc_id.cpu().numpy().reshape(-1, K)[sl],
                                   self.ctx.sc_status.cpu().numpy()[sl])
                    if free and synced:
                        g = self.gpu_state(c)
                        same = (np.array_equal(g.canvas, after.canvas)
                                and np.array_equal(g.committed, after.committed)
                                and np.array_equal(g.prev_argmax, after.prev_argmax)
                                and (g.stable_count, g.done, g.steps_used)
                                == (after.stable_count, after.done, after.steps_used))
                        if not same:
                            # both sides started this step from the same state
                            if rep.band_events == n_bands:
                                rep.fail(f"free run: {tag} parts from the oracle without a "
                                         f"band event")
                            if rep.divergence is None:
                                rep.divergence = (b, s_idx, c)
                            rep.resyncs += 1
                            synced = False
                    self.states[c] = after
                if free and rep.divergence is None:
                    rep.free_steps += 1
                if progress:
                    progress(b, s_idx, rep)
                if all(s.done for s in self.states):
                    break
        rep.check_band_rate()
        return rep


def free_running(ls: Lockstep, rep: Report = None):
    """A whole generation with each side on its own state (see Lockstep.run,
    free=True).  Returns (rep, first divergence or None)."""
    rep = ls.run(rep=rep, free=True)
    return rep, rep.divergence
