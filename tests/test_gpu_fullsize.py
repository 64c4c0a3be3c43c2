"""GPU parity at the full workload sizes (V = 262144, d = 2816), in the launch
configuration the benchmark times (packed vocabulary table), and on the
row-major table.

* The headline workload (256 positions) on the packed table is compared
  position by position at every step: a free run (the GPU on its own state)
  with a lockstep comparison of every step, resynchronised from the oracle
  after a band event (tests/parity.py, Lockstep.run with free=True).  Its
  logits are checked on one row of every 32-position MFMA block.
* The other full-size runs compare per-position statistics (entropy,
  argmax, sample, gap) on one row of every 32-position block of every canvas
  at sampled steps, and on every position of every canvas at every fourth
  step of every block (the batched and multi-block workloads) or at two
  steps (the variants of the headline run), recomputed by the oracle for
  those rows, and the whole
  step's decision logic (early stop, sort, entropy bound, sample write,
  re-noise) at EVERY step: the oracle's step rule applied to the GPU's own
  per-position statistics must reproduce the GPU's new canvas, committed
  mask and state bit for bit (same inputs, so no tie band).
* Invariants that hold at any size (entropy range), batch invariance (a
  canvas in the batched run equals the same canvas run alone) and run-to-run
  determinism.
Long tests append progress lines to the file DGD_PROGRESS_LOG names, if set.
"""
import numpy as np
import pytest

from oracle import dgd_oracle as O
from tests.parity import (BAND_CONV, BAND_SAMPLE, TOL_LOGIT_REL, Lockstep, Report,
                          commit_band_positions, compare_sc, compare_stats, oracle_stats,
                          q4_device_table)
from uniform_state_discrete_step_amd.inputs import (WORKLOADS, make_workload_arrays, quantize_q4,
                                                    shrink)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def block_rows(L, rng):
    """One random row in every 32-position block (the MFMA's position blocks)."""
    return np.array([b0 + int(rng.integers(min(32, L - b0))) for b0 in range(0, L, 32)])


def progress(msg):
    """A progress line for long runs, appended to the file DGD_PROGRESS_LOG
    names (outside pytest's capture), if it is set."""
    import os
    path = os.environ.get("DGD_PROGRESS_LOG")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(msg + "\n")


class FullRun:
    """Step a workload on the GPU with dgd_step and check every step."""

    def __init__(self, wl, dev, W=None, Hs=None, layout=1, Wd=None, tail: O.Tail = None,
                 sc_topk=0):
        import torch
        from uniform_state_discrete_step_amd import dgd
        self.torch, self.dgd, self.wl, self.dev = torch, dgd, wl, dev
        if W is None:
            W, Hs = make_workload_arrays(wl, threads=16)
        self.W, self.Hs = W, Hs
        if layout == dgd.DGD_VOCAB_Q4 and Wd is None:
            # the GPU streams the 4-bit form; the oracle uses the table it stands for
            Wd = q4_device_table(W, wl.V, wl.d, dev)
            self.W = W = O.dequant_q4(*quantize_q4(W))
        if Wd is None:
            Wd = torch.from_numpy(W.view(np.int16)).to(dev)
            if layout == dgd.DGD_VOCAB_PACKED:
                Wd = dgd.pack_vocab(Wd, wl.V, wl.d)
        self.Wd = Wd
        self.Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
        self.tail = tail
        tkw = {}
        if tail is not None:
            if tail.norm_weight is not None:
                tkw["norm_weight"] = torch.from_numpy(tail.norm_weight.view(np.int16)).to(dev)
                tkw["norm_eps"] = tail.norm_eps
            tkw["softcap"] = tail.softcap
        self.sc_topk = sc_topk
        self.ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev,
                               vocab_layout=layout, sc_topk=sc_topk, sc_status=sc_topk > 0,
                               **tkw)
        self.params = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence,
                                      wl.stability_threshold, wl.freeze, wl.final_emit)
        self.P = O.Params(N=wl.N, t_min=wl.t_min, t_max=wl.t_max, confidence=wl.confidence,
                          stability_threshold=wl.stability_threshold, freeze=wl.freeze,
                          final_emit=wl.final_emit)
        self.canvas = torch.zeros(wl.B * wl.G, dtype=torch.int32, device=dev)
        self.committed = torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=dev)
        self.W64 = None

    def gpu_state(self, c):
        wl = self.wl
        sv = self.ctx.state_views()
        return O.CanvasState(
            self.canvas[c * wl.G:(c + 1) * wl.G].cpu().numpy().astype(np.int64),
            self.committed[c * wl.G:(c + 1) * wl.G].cpu().numpy().copy(),
            sv["prev_argmax"][c * wl.L:(c + 1) * wl.L].cpu().numpy().astype(np.int64),
            int(sv["stable_count"][c]), bool(int(sv["done"][c])), int(sv["steps_used"][c]))

    def sampled_rows(self, rep, b, s, every_row=False):
        """Statistics of one row in every 32-position block of every canvas
        (of every row, with every_row)."""
        wl = self.wl
        if self.W64 is None:
            self.W64 = O.bf16_to_f64(self.W)
        T = O.temperature(s, wl.N, wl.t_min, wl.t_max)
        rng = np.random.default_rng([b, s])
        H = self.ctx.entropy.cpu().numpy()
        A = self.ctx.argmax.cpu().numpy().astype(np.int64)
        Tk = self.ctx.token.cpu().numpy().astype(np.int64)
        gap = self.ctx.gap.cpu().numpy()
        for c in range(wl.B):
            rows = np.arange(wl.L) if every_row else block_rows(wl.L, rng)
            z = O.logits(self.Hs[b, s, c][rows], self.W, self.tail, W64=self.W64)
            p_abs, gstep = b * wl.L + rows, b * wl.N + s
            st = oracle_stats(z, T, wl.seeds[c], p_abs, gstep)
            sl = slice(c * wl.L, (c + 1) * wl.L)
            if self.sc_topk:
                K = self.sc_topk
                compare_sc(rep, f"block {b} step {s} canvas {c}", z, T, K,
                           self.ctx.sc_prob.cpu().numpy().reshape(-1, K)[sl][rows],
                           self.ctx.sc_id.cpu().numpy().reshape(-1, K)[sl][rows],
                           self.ctx.sc_status.cpu().numpy()[sl][rows], rows=rows)
            gpu = {"entropy": H[sl][rows], "argmax": A[sl][rows], "token": Tk[sl][rows],
                   "gap": gap[sl][rows]}
            compare_stats(rep, f"block {b} step {s} canvas {c}", st, gpu, z, T, wl.seeds[c],
                          p_abs, gstep, rows=rows)

    def check_band_counters(self, rep, tag, c, info, gap):
        """The state's tie counts of the step against the same counts taken
        by the step rule on the GPU's own statistics (equal numbers, so equal
        counts; the convergence flag may differ only when the float64 mean,
        summed in another order, lies on the band's edge)."""
        sv = self.ctx.state_views()
        if int(sv["status"][c]) != 0:
            rep.fail(f"{tag}: status {int(sv['status'][c])} on finite inputs")
        n_sample = int(np.count_nonzero(gap.astype(np.float64) < BAND_SAMPLE))
        n_commit = len(commit_band_positions(info, float(np.float32(self.wl.bounds[c]))))
        if (int(sv["band_sample"][c]), int(sv["band_commit"][c])) != (n_sample, n_commit):
            rep.fail(f"{tag}: band counters (sample, commit) = ({int(sv['band_sample'][c])}, "
                     f"{int(sv['band_commit'][c])}), expected ({n_sample}, {n_commit})")
        dconf = abs(info["mean_H"] - float(np.float32(self.wl.confidence)))
        if int(sv["band_conv"][c]) != int(dconf < BAND_CONV) and abs(dconf - BAND_CONV) > 1e-12:
            rep.fail(f"{tag}: convergence band flag {int(sv['band_conv'][c])} "
                     f"(|mean - confidence| = {dconf:.3e})")

    def run(self, sample_every=8, blocks=None, full_steps=()):
        torch, wl, dgd = self.torch, self.wl, self.dgd
        rep = Report()
        for b in (range(wl.blocks) if blocks is None else blocks):
            dgd.dgd_init_block(self.canvas, self.committed, b, self.params, wl.seeds, self.ctx)
            torch.cuda.synchronize()
            for c in range(wl.B):
                p_abs = b * wl.L + np.arange(wl.L)
                init = self.canvas[c * wl.G + b * wl.L:c * wl.G + (b + 1) * wl.L].cpu().numpy()
                if not np.array_equal(init, O.init_token(wl.seeds[c], p_abs, b, wl.V)):
                    rep.fail(f"block {b} canvas {c}: initial tokens differ")
            for s in range(wl.N):
                before = [self.gpu_state(c) for c in range(wl.B)]
                dgd.dgd_step(self.Hd[b, s].reshape(-1), self.Wd, self.canvas, self.committed, b, s,
                             self.params, wl.seeds, self.ctx)
                torch.cuda.synchronize()
                H = self.ctx.entropy.cpu().numpy()
                A = self.ctx.argmax.cpu().numpy().astype(np.int64)
                T = self.ctx.token.cpu().numpy().astype(np.int64)
                gap = self.ctx.gap.cpu().numpy()
                for c in range(wl.B):
                    sl = slice(c * wl.L, (c + 1) * wl.L)
                    stats = {"entropy": H[sl], "argmax": A[sl], "token": T[sl]}
                    expect, info = O.step_from_stats(before[c], stats, b, s, wl.L, wl.V, self.P,
                                                     wl.seeds[c], float(np.float32(wl.bounds[c])))
                    got = self.gpu_state(c)
                    tag = f"block {b} step {s} canvas {c}"
                    if not np.array_equal(got.canvas, expect.canvas):
                        rep.fail(f"{tag}: canvas differs from the step rule on the GPU's statistics")
                    if not np.array_equal(got.committed, expect.committed):
                        rep.fail(f"{tag}: committed mask differs from the step rule")
                    if (got.stable_count, got.done, got.steps_used) != (
                            expect.stable_count, expect.done, expect.steps_used):
                        rep.fail(f"{tag}: state differs from the step rule")
                    if not np.all((H[sl] >= 0) & (H[sl] <= np.log(wl.V) + 1e-3)):
                        rep.fail(f"{tag}: entropy out of [0, ln V]")
                    if not info.get("skipped"):
                        self.check_band_counters(rep, tag, c, info, gap[sl])
                    rep.steps += 1
                    rep.positions += wl.L
                if s in full_steps:
                    self.sampled_rows(rep, b, s, every_row=True)
                    progress(f"{wl.name} block {b} step {s} (every position): {rep.summary()}")
                elif s % sample_every == 0 or s == wl.N - 1:
                    self.sampled_rows(rep, b, s)
                    progress(f"{wl.name} block {b} step {s}: {rep.summary()}")
                if all(self.gpu_state(c).done for c in range(wl.B)):
                    break
        rep.check_band_rate()
        return rep


def _check(rep, name):
    print(f"\n[{name}] {rep.summary()}", flush=True)
    assert not rep.failures, "\n".join(rep.failures)


def test_gemma_vocab_every_position_every_step(dev):
    """The benchmarked configuration (packed table, 256 positions: one
    256 x 256 tile per workgroup, four tiles per vocabulary group) against
    the oracle at every position of every step: a free run, each step also
    compared in lockstep, resynchronised after a band event."""
    import time
    wl = WORKLOADS["gemma_vocab"]
    W, Hs = make_workload_arrays(wl, threads=16)
    ls = Lockstep(wl, W, Hs, dev, layout=1)
    t0 = time.perf_counter()

    def prog(b, s, rep):
        progress(f"{wl.name} free run step {s} ({time.perf_counter() - t0:.0f}s): {rep.summary()}")

    rep = ls.run(free=True, progress=prog)
    print(f"\n[{wl.name} packed, every position] {rep.summary()}", flush=True)
    assert not rep.failures, "\n".join(rep.failures)
    assert rep.steps == wl.N and rep.stat_rows == wl.N * wl.L


def test_gemma_vocab_logits_on_sampled_rows(dev):
    """Full-size logits (packed table) on one row of every 32-position block,
    at two steps, within the 2e-2 relative bar."""
    import torch
    wl = WORKLOADS["gemma_vocab"]
    W, Hs = make_workload_arrays(wl, threads=16)
    ls = Lockstep(wl, W, Hs, dev, logits=True, layout=1)
    W64 = ls.W64
    worst = 0.0
    for s in (0, 29):
        ls.states = [O.init_block(O.new_state(wl.G, wl.L), 0, wl.L, wl.V, wl.seeds[0])]
        ls.push_state()
        ls.dgd.dgd_step(ls.Hd[0, s].reshape(-1), ls.Wd, ls.canvas, ls.committed, 0, s, ls.params,
                        wl.seeds, ls.ctx)
        torch.cuda.synchronize()
        rows = block_rows(wl.L, np.random.default_rng([7, s]))
        zg = ls.ctx.logits.view(wl.L, wl.V)[torch.from_numpy(rows).to(dev)].cpu().numpy()
        z = O.projection(Hs[0, s, 0][rows], W, W64=W64)
        scale = np.maximum(np.abs(z), np.sqrt(np.mean(z * z, axis=1, keepdims=True)))
        rel = np.abs(zg.astype(np.float64) - z) / np.maximum(scale, 1e-30)
        worst = max(worst, float(rel.max()))
        print(f"\n[{wl.name} step {s} rows {rows.tolist()}] logits: max rel err {rel.max():.3e}, "
              f"max abs err {np.abs(zg - z).max():.3e}", flush=True)
    assert worst <= TOL_LOGIT_REL


def test_gemma_vocab_full_run_rows(dev):
    """The row-major table at the full size."""
    wl = WORKLOADS["gemma_vocab"]
    _check(FullRun(wl, dev, layout=0).run(sample_every=6), f"{wl.name} layout=0")


def test_batched_full_run_and_batch_invariance(dev):
    import torch
    wl = WORKLOADS["batched"]
    run = FullRun(wl, dev)
    _check(run.run(sample_every=6, full_steps=range(0, wl.N, 4)), wl.name)
    # canvas 5 of the batch, run alone, must be bitwise identical
    c = 5
    alone = shrink(wl, name="batched_c5", B=1, seeds=(wl.seeds[c],), bounds=(wl.bounds[c],))
    Hs1 = np.ascontiguousarray(run.Hs[:, :, c:c + 1])
    solo = FullRun(alone, dev, W=run.W, Hs=Hs1, Wd=run.Wd)
    solo.W64 = run.W64
    _check(solo.run(sample_every=1000), alone.name)
    torch.cuda.synchronize()
    assert np.array_equal(solo.canvas.cpu().numpy(),
                          run.canvas[c * wl.G:(c + 1) * wl.G].cpu().numpy())
    assert np.array_equal(solo.committed.cpu().numpy(),
                          run.committed[c * wl.G:(c + 1) * wl.G].cpu().numpy())


def test_gemma_vocab_full_run_with_lm_head_tail(dev):
    """Output norm + projection + softcap (c = 30) at the full size, packed table."""
    from uniform_state_discrete_step_amd.inputs import make_norm_weight
    wl = WORKLOADS["gemma_vocab"]
    tail = O.Tail(norm_weight=make_norm_weight(wl.d, wl.cfg_seed), norm_eps=1e-6, softcap=30.0)
    _check(FullRun(wl, dev, tail=tail).run(sample_every=6, full_steps=(0, 24)),
           f"{wl.name} with output norm and softcap")


def test_gemma_vocab_full_run_q4_table(dev):
    """The 4-bit table stream at the full size."""
    wl = WORKLOADS["gemma_vocab"]
    _check(FullRun(wl, dev, layout=2).run(sample_every=6, full_steps=(0, 24)),
           f"{wl.name} 4-bit table")


def test_gemma_vocab_full_run_with_self_conditioning(dev):
    """Top-32 per position at the full size, with the output norm and softcap."""
    from uniform_state_discrete_step_amd.inputs import make_norm_weight
    wl = WORKLOADS["gemma_vocab"]
    tail = O.Tail(norm_weight=make_norm_weight(wl.d, wl.cfg_seed), norm_eps=1e-6, softcap=30.0)
    run = FullRun(wl, dev, tail=tail, sc_topk=32)
    rep = run.run(sample_every=8, full_steps=(0,))
    st = run.ctx.sc_status.cpu().numpy()
    print(f"\nrecomputed parts in the last step: {int(st.sum())}, rows budget-exhausted "
          f"{int((st < 0).sum())}", flush=True)
    _check(rep, f"{wl.name} with self-conditioning top-32")


@pytest.mark.parametrize("layout", [1, 0], ids=["packed", "rows"])
def test_multi_block_full_run(dev, layout):
    wl = WORKLOADS["multi_block"]
    full = range(0, wl.N, 4) if layout == 1 else ()
    _check(FullRun(wl, dev, layout=layout).run(sample_every=8, full_steps=full),
           f"{wl.name} layout={layout}")


def test_dgd_run_matches_stepping_and_is_deterministic(dev):
    """dgd_run (the benchmarked entry point) equals step-by-step driving, twice."""
    import torch
    wl = WORKLOADS["gemma_vocab"]
    run = FullRun(wl, dev)
    rep = run.run(sample_every=1000)
    _check(rep, wl.name + " stepped")
    outs = []
    # twice with per-step outputs, once without (the benchmark's configuration)
    quiet = run.dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, outputs=False,
                            vocab_layout=1)
    for ctx in (run.ctx, run.ctx, quiet):
        can = torch.zeros_like(run.canvas)
        com = torch.zeros_like(run.committed)
        run.dgd.dgd_run(run.Hd.reshape(-1), run.Wd, can, com, run.params, wl.seeds, ctx)
        torch.cuda.synchronize()
        outs.append((can.cpu().numpy(), com.cpu().numpy()))
    assert np.array_equal(outs[2][0], outs[0][0]) and np.array_equal(outs[2][1], outs[0][1])
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][0], run.canvas.cpu().numpy())
    assert np.array_equal(outs[0][1], run.committed.cpu().numpy())
