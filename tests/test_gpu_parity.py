"""GPU parity of the HIP step (through the C ABI) with the CPU oracle.

Lockstep comparisons at sizes the oracle finishes in seconds, spanning
several vocabulary tiles, several 64-element hidden chunks and ragged tails,
plus the degenerate cases of the method.  Criteria: see tests/parity.py.
"""
import dataclasses
import math

import numpy as np
import pytest

from oracle import dgd_oracle as O
from tests.parity import TOL_LOGIT_REL, Lockstep
from uniform_state_discrete_step_amd.inputs import (WORKLOADS, f32_to_bf16_bits,
                                                    make_norm_weight, make_workload_arrays,
                                                    shrink)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


# every lockstep case runs on both vocabulary layouts: 0 = row-major table,
# 1 = the packed table of dgd_pack_vocab
@pytest.fixture(params=[0, 1], ids=["rows", "packed"])
def layout(request):
    return request.param


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def run_lockstep(wl, dev, W=None, Hs=None, logits=False, layout=0, tail=None, sc_topk=0, **kw):
    if W is None:
        W, Hs = make_workload_arrays(wl, threads=8)
    ls = Lockstep(wl, W, Hs, dev, logits=logits, layout=layout, tail=tail, sc_topk=sc_topk)
    rep = ls.run(**kw)
    tag = "" if tail is None else (f" norm={tail.norm_weight is not None} eps={tail.norm_eps}"
                                   f" softcap={tail.softcap}")
    tag += f" sc_topk={sc_topk}" if sc_topk else ""
    print(f"\n[{wl.name} layout={layout} B={wl.B} L={wl.L} G={wl.G} V={wl.V} d={wl.d} N={wl.N} "
          f"freeze={wl.freeze} final_emit={wl.final_emit}{tag}] {rep.summary()}", flush=True)
    assert not rep.failures, "\n".join(rep.failures)
    return ls, rep


# ----------------------------------------------------------------------------
def test_gumbel_transform_every_cell(dev):
    """The fused step's noise on all 2^23 uniform cells, against float64."""
    import torch
    from uniform_state_discrete_step_amd import dgd
    k = np.arange(1 << 23, dtype=np.uint32)
    words = (k << np.uint32(9)) | np.uint32(0x155)
    wd = torch.from_numpy(words.view(np.int32)).to(dev)
    out = torch.empty(words.shape[0], dtype=torch.float32, device=dev)
    dgd.dgd_debug_gumbel(wd, out)
    g_gpu = out.cpu().numpy().astype(np.float64) * math.log(2) - math.log(math.log(2))
    g_ref = O.gumbel_from_word(words)
    err = np.abs(g_gpu - g_ref)
    worst = int(np.argmax(err))
    print(f"\nmax |g_gpu - g| = {err[worst]:.3e} at cell {worst} (g = {g_ref[worst]:.6f}); "
          f"mean {err.mean():.3e}", flush=True)
    assert err.max() <= 2e-5


@pytest.mark.parametrize("keyed", [True, False], ids=["per_call_keys", "uniform_key"])
def test_philox_words_match_the_oracle(dev, keyed):
    """The GPU generator against the oracle's separate implementation, bit
    for bit, on 2^25 calls (1.3e8 words) with varied counters and keys."""
    import torch
    from uniform_state_discrete_step_amd import dgd
    n = 1 << 25
    rng = np.random.default_rng(20)
    i = np.arange(n, dtype=np.uint64)
    ctr = np.empty((n, 4), dtype=np.uint32)
    ctr[:, 0] = i                                                    # every value of c0's range start
    ctr[:, 1] = rng.integers(0, 1 << 32, n, dtype=np.uint64)
    ctr[:, 2] = (i * 2654435761) >> 7
    ctr[:, 3] = rng.integers(0, 4, n)                               # tags 0..3
    key = rng.integers(0, 1 << 32, (n, 2), dtype=np.uint64).astype(np.uint32)
    ukey = 0xFEEDFACE_0BADF00D
    out = torch.empty(n * 4, dtype=torch.int32, device=dev)
    dgd.dgd_debug_philox(torch.from_numpy(ctr.view(np.int32).reshape(-1)).to(dev),
                         torch.from_numpy(key.view(np.int32).reshape(-1)).to(dev) if keyed else None,
                         ukey, out)
    torch.cuda.synchronize()
    g = out.cpu().numpy().view(np.uint32).reshape(n, 4)
    k0 = key[:, 0] if keyed else np.uint32(ukey & 0xFFFFFFFF)
    k1 = key[:, 1] if keyed else np.uint32(ukey >> 32)
    for a in range(0, n, 1 << 23):                                   # in slices: host memory
        sl = slice(a, a + (1 << 23))
        o = O.philox4x32_10(ctr[sl, 0], ctr[sl, 1], ctr[sl, 2], ctr[sl, 3],
                            k0[sl] if keyed else k0, k1[sl] if keyed else k1)
        for w in range(4):
            bad = np.nonzero(g[sl, w] != o[w])[0]
            assert bad.size == 0, f"word {w} differs at call {a + int(bad[0])}"


@pytest.mark.parametrize("name,shape", [
    ("tiny", {}),
    ("tiny", dict(B=3, G=32, seeds=(0, 1, 2**63 + 5), bounds=(0.1, 0.0, 1.0))),
    ("tiny", dict(V=1001, d=72, L=37, B=3, G=74, N=5, seeds=(4, 5, 6), bounds=(0.1, 0.3, 0.05))),
    ("small_vocab", {}),
    ("tiny", dict(V=65536, d=128, L=256, G=256, N=6, cfg_seed=23)),
], ids=["tiny", "tiny_batched", "ragged", "small_vocab", "full_tile"])
def test_free_running_generation_matches_the_oracle(dev, name, shape):
    """End to end: whole generations on both sides from their own state."""
    from tests.parity import free_running
    wl = shrink(WORKLOADS[name], **shape) if shape else WORKLOADS[name]
    W, Hs = make_workload_arrays(wl, threads=8)
    ls = Lockstep(wl, W, Hs, dev, layout=1)
    rep, div = free_running(ls)
    print(f"\n[free run {name}] {rep.summary()} first divergence: {div}", flush=True)
    assert not rep.failures, "\n".join(rep.failures)
    assert rep.steps > 0


def test_tiny_lockstep(dev, layout):
    run_lockstep(WORKLOADS["tiny"], dev, layout=layout)


@pytest.mark.parametrize("variant", [
    dict(B=3, G=32, seeds=(0, 1, 2**63 + 5), bounds=(0.1, 0.0, 1.0)),
    dict(freeze=0),
    dict(final_emit=1),
    dict(stability_threshold=0, confidence=1.0),
    dict(N=1),
    dict(N=3, t_min=0.0, t_max=1.0),
    # near-greedy temperature on a ragged vocabulary: tempered logits ~1e3x
    # the raw ones, masked ids far below them, one-hot distributions
    dict(V=1001, N=2, t_min=0.001, t_max=0.001),
])
def test_tiny_variants(dev, variant, layout):
    run_lockstep(shrink(WORKLOADS["tiny"], **variant), dev, layout=layout)


@pytest.mark.parametrize("shape", [
    dict(V=1001, d=72, L=37, B=3, G=74, N=5),     # ragged vocabulary, hidden and rows; 2 blocks
    dict(V=129, d=8, L=1, B=2, G=3, N=4),          # one-position canvases, 3 blocks
    dict(V=1, d=16, L=5, B=1, G=5, N=3),           # one-token vocabulary
    dict(V=4096, d=136, L=70, B=2, G=70, N=6),     # rows straddle 32-row blocks of one tile
    dict(V=1024, d=64, L=600, B=1, G=600, N=4),    # canvas over 512: sorting network path
    dict(V=2048, d=128, L=512, B=2, G=512, N=3),   # largest canvas of the counting-rank path
    # 256 positions: the benchmark's 256 x 256 tile (eight 32-position blocks
    # per wave), one tile per vocabulary group ...
    dict(V=65536, d=128, L=256, B=1, G=256, N=4),
    # ... and two or three tiles per group, a ragged last tile (100 rows) and
    # a hidden size of three chunks (the two-chunk ring runs one padding chunk)
    dict(V=131172, d=192, L=256, B=1, G=256, N=3),
])
def test_ragged_shapes(dev, shape, layout):
    B = shape["B"]
    wl = shrink(WORKLOADS["tiny"], name="ragged", cfg_seed=7, seeds=tuple(range(B)),
                bounds=tuple((0.1, 0.3, 0.05)[c % 3] for c in range(B)), **shape)
    run_lockstep(wl, dev, layout=layout)


def test_small_vocab_lockstep(dev, layout):
    run_lockstep(WORKLOADS["small_vocab"], dev, layout=layout)


# ----------------------------------------------------------------------------
# the lm-head tail: output RMSNorm before the projection, softcap after it
# ----------------------------------------------------------------------------
def _tail(wl, norm=True, eps=1e-6, softcap=30.0, wscale=(0.5, 8.0)):
    return O.Tail(norm_weight=make_norm_weight(wl.d, wl.cfg_seed, wscale) if norm else None,
                  norm_eps=eps, softcap=softcap)


@pytest.mark.parametrize("tail", [
    dict(norm=True, softcap=0.0),
    dict(norm=False, softcap=30.0),
    dict(norm=True, softcap=30.0),
    dict(norm=True, softcap=5.0, eps=0.0),           # a cap that bites on most logits
    dict(norm=True, softcap=30.0, wscale=(0.05, 0.5)),  # small weights: high entropies
], ids=["norm", "cap30", "norm_cap30", "norm_cap5", "norm_small_w"])
def test_tail_lockstep(dev, tail, layout):
    wl = WORKLOADS["tiny"]
    run_lockstep(wl, dev, layout=layout, tail=_tail(wl, **tail))


@pytest.mark.parametrize("shape", [
    dict(V=1001, d=72, L=37, B=3, G=74, N=5),
    dict(V=4096, d=136, L=70, B=2, G=70, N=6),
    dict(V=777, d=4104, L=33, B=1, G=33, N=3),     # three hidden-row passes, ragged
], ids=["ragged", "straddle", "wide_hidden"])
def test_tail_ragged_shapes(dev, shape, layout):
    B = shape["B"]
    wl = shrink(WORKLOADS["tiny"], name="ragged_tail", cfg_seed=9, seeds=tuple(range(B)),
                bounds=tuple((0.1, 0.3, 0.05)[c % 3] for c in range(B)), **shape)
    run_lockstep(wl, dev, layout=layout, tail=_tail(wl))


def test_tail_small_vocab_lockstep(dev, layout):
    wl = WORKLOADS["small_vocab"]
    run_lockstep(wl, dev, layout=layout, tail=_tail(wl), steps=range(0, 48, 6))


def test_norm_of_special_rows(dev):
    """Zero rows, rows of one nonzero value, tiny and huge rows, negative
    zeros: the normalised rows against the oracle, within one bf16 step."""
    wl = shrink(WORKLOADS["tiny"], L=8, G=8, N=1, d=64)
    W, Hs = make_workload_arrays(wl, threads=1)
    x = O.bf16_to_f64(Hs[0, 0, 0]).copy()
    x[0] = 0.0
    x[1] = 0.0
    x[1, 5] = -3.0
    x[2] *= 2.0 ** -100                 # tiny rows (every input stays a normal bf16)
    x[3] *= 2.0 ** 100
    x[4, ::2] = 0.0
    x[5] = 0.0                          # one huge value: the others normalise below 2^-126
    x[5, 0], x[5, 1], x[5, 2], x[5, 3] = 2.0 ** 60, 2.0 ** -70, -(2.0 ** -72), 3 * 2.0 ** -75
    Hs = Hs.copy()
    Hs[0, 0, 0] = bf16(x)
    Hs[0, 0, 0, 0, ::3] = 0x8000        # negative zeros in the zero row
    tail = _tail(wl, eps=1e-6, softcap=0.0)
    ls = Lockstep(wl, W, Hs, dev, tail=tail)
    rep = ls.run()
    print(f"\n[special rows] {rep.summary()}", flush=True)
    assert not rep.failures, "\n".join(rep.failures)
    g = ls.ctx.norm_h.cpu().numpy().view(np.uint16).reshape(wl.L, wl.d)
    assert not (g[0] & 0x7FFF).any()                  # a zero row stays zero (eps > 0)


def test_tail_logits_are_the_projection_of_the_normalised_rows(dev, layout):
    wl = WORKLOADS["tiny"]
    W, Hs = make_workload_arrays(wl, threads=1)
    tail = _tail(wl, softcap=5.0)
    z_gpu, z = _logit_check(wl, dev, W, Hs, steps=[0, 1], layout=layout, tail=tail)
    # ctx->logits holds the projection before the cap: some logits exceed it
    assert np.abs(z_gpu).max() > 6.0


# ----------------------------------------------------------------------------
# self-conditioning: top-K per position and the embedding sum
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("K", [32, 5, 1])
def test_sc_topk_lockstep(dev, K):
    run_lockstep(WORKLOADS["tiny"], dev, layout=1, sc_topk=K)


@pytest.mark.parametrize("shape,K", [
    (dict(V=1001, d=72, L=37, B=3, G=74, N=5), 32),
    (dict(V=4096, d=136, L=70, B=2, G=70, N=4), 32),
    (dict(V=129, d=8, L=1, B=2, G=3, N=4), 32),
    (dict(V=40, d=64, L=16, B=1, G=16, N=3), 32),      # lists cannot hold K: parts recomputed
    (dict(V=1, d=16, L=5, B=1, G=5, N=3), 1),
    (dict(V=70000, d=96, L=48, B=1, G=48, N=3), 32),   # 274 tiles: groups of 2 tiles
], ids=["ragged", "straddle", "one_position", "v40", "v1", "two_tile_groups"])
def test_sc_topk_ragged(dev, shape, K):
    B = shape["B"]
    wl = shrink(WORKLOADS["tiny"], name="ragged_sc", cfg_seed=13, seeds=tuple(range(B)),
                bounds=tuple((0.1, 0.3, 0.05)[c % 3] for c in range(B)), **shape)
    ls, rep = run_lockstep(wl, dev, layout=1, sc_topk=K)
    if wl.V == 40:
        assert rep.sc_recomputed > 0


def test_sc_topk_with_tail_and_small_vocab(dev):
    wl = WORKLOADS["small_vocab"]
    run_lockstep(wl, dev, layout=1, tail=_tail(wl, softcap=30.0), sc_topk=32,
                 steps=range(0, 48, 12))


def _clustered_table(wl, seed=21):
    """A table whose highest logits for every position sit together: rows
    0..39 (one band of tile 0) and rows 256+{0,1,2,3,8} (one lane's ids in
    tile 1) copy a row aligned with every position's hidden state, so the
    band list and a lane list both overflow and must be recomputed."""
    W, Hs = make_workload_arrays(wl, threads=1)
    W = W.copy()
    Hf = O.bf16_to_f64(Hs).reshape(-1, wl.d)
    u = Hf.sum(axis=0)
    u /= np.linalg.norm(u)
    rng = np.random.default_rng(seed)
    for v in range(40):
        W[v] = bf16(u * 8.0 + rng.standard_normal(wl.d) * 1e-2)
    for v in (256, 257, 258, 259, 264):
        W[v] = bf16(u * 8.0 + rng.standard_normal(wl.d) * 1e-2)
    return W, Hs, u


def test_sc_topk_recomputes_overflowing_lists(dev):
    wl = shrink(WORKLOADS["tiny"], name="clustered", L=16, G=16, N=4,
                scale=(5.0, 10.0))
    W, Hs, _ = _clustered_table(wl)
    ls, rep = run_lockstep(wl, dev, W=W, Hs=Hs, layout=1, sc_topk=32)
    assert rep.sc_recomputed > 0


def test_sc_topk_exact_ties(dev):
    """Identical table rows give identical logits: the lower id goes first.
    Six copies of one dominant row lead every position's top K."""
    wl = shrink(WORKLOADS["tiny"], name="ties", N=3, scale=(5.0, 10.0))
    W, Hs, u = _clustered_table(wl)
    W = make_workload_arrays(wl, threads=1)[0].copy()
    for v in (3, 70, 300, 301, 500, 900):
        W[v] = bf16(u * 8.0)
    run_lockstep(wl, dev, W=W, Hs=Hs, layout=1, sc_topk=32)


@pytest.mark.parametrize("layout", [0, 1], ids=["rows", "packed"])
def test_sc_embed_matches_the_oracle(dev, layout):
    import torch
    from uniform_state_discrete_step_amd import dgd
    wl = shrink(WORKLOADS["tiny"], V=3000, d=200, L=48, B=2, G=48, N=2, seeds=(4, 5),
                bounds=(0.1, 0.2))
    W, Hs = make_workload_arrays(wl, threads=1)
    K = 32
    ls = Lockstep(wl, W, Hs, dev, layout=1, sc_topk=K)
    ls.run(steps=[0])
    torch.cuda.synchronize()
    rows = wl.B * wl.L
    Wt = torch.from_numpy(W.view(np.int16)).to(dev)
    if layout == 1:
        Wt = dgd.pack_vocab(Wt, wl.V, wl.d)
    out = torch.empty(rows * wl.d, dtype=torch.int16, device=dev)
    scale = math.sqrt(wl.d)
    dgd.dgd_sc_embed(ls.ctx.sc_prob, ls.ctx.sc_id, rows, K, Wt, layout, wl.V, wl.d, scale, out)
    torch.cuda.synchronize()
    g = out.cpu().numpy().view(np.uint16).reshape(rows, wl.d)
    p = ls.ctx.sc_prob.cpu().numpy().reshape(rows, K).astype(np.float64)
    ids = ls.ctx.sc_id.cpu().numpy().reshape(rows, K)
    o = O.sc_embed(p, ids, W, scale)
    from tests.parity import ordered_bf16
    ulp = np.abs(ordered_bf16(g) - ordered_bf16(o))
    print(f"\n[sc_embed layout={layout}] max bf16 steps {ulp.max()}, "
          f"inexact {np.count_nonzero(ulp)} of {ulp.size}", flush=True)
    assert ulp.max() <= 1


# ----------------------------------------------------------------------------
# 4-bit table
# ----------------------------------------------------------------------------
def test_q4_projection_is_exact_on_small_integers(dev):
    """Scale 1 and minimum -8 give table values -8..7; with small-integer H
    every fp32 partial sum is exact, so the logits must equal the integer
    dot products bit for bit (catches any slip in the code, scale or
    fragment layout of the 4-bit stream)."""
    import torch
    from uniform_state_discrete_step_amd import dgd
    wl = shrink(WORKLOADS["tiny"], V=300, d=160, L=40, B=1, G=40, N=2)
    rng = np.random.default_rng(17)
    q = rng.integers(0, 16, size=(wl.V, wl.d)).astype(np.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sc = np.full((wl.V, wl.d // 32), 0x3F80, dtype=np.uint16)            # 1.0
    mn = np.full((wl.V, wl.d // 32), 0xC100, dtype=np.uint16)            # -8.0
    Hi = rng.integers(-2, 3, size=(wl.L, wl.d))
    Hs = bf16(Hi).reshape(1, 1, 1, wl.L, wl.d).repeat(wl.N, axis=1)
    Wq = dgd.pack_vocab_q4(torch.from_numpy(codes.reshape(-1)).to(dev),
                           torch.from_numpy(sc.reshape(-1).view(np.int16)).to(dev),
                           torch.from_numpy(mn.reshape(-1).view(np.int16)).to(dev), wl.V, wl.d)
    ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, logits=True,
                      vocab_layout=dgd.DGD_VOCAB_Q4)
    params = dgd.make_params(wl.N)
    canvas = torch.zeros(wl.G, dtype=torch.int32, device=dev)
    committed = torch.zeros(wl.G, dtype=torch.uint8, device=dev)
    dgd.dgd_init_block(canvas, committed, 0, params, wl.seeds, ctx)
    Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
    dgd.dgd_step(Hd[0, 0].reshape(-1), Wq, canvas, committed, 0, 0, params, wl.seeds, ctx)
    torch.cuda.synchronize()
    z = ctx.logits.cpu().numpy().reshape(wl.L, wl.V).astype(np.float64)
    ref = (Hi @ (q.astype(np.int64) - 8).T).astype(np.float64)
    assert np.array_equal(z, ref)
    # and the oracle's dequantized table is that integer table
    assert np.array_equal(O.bf16_to_f64(O.dequant_q4(codes, sc, mn)), q.astype(np.float64) - 8)


@pytest.mark.parametrize("shape", [
    dict(),                                               # tiny: V 1024, d 64
    dict(V=1001, d=96, L=37, B=3, G=74, N=5),             # ragged rows, vocabulary, two blocks
    dict(V=4096, d=160, L=70, B=2, G=70, N=4),            # a half-filled last chunk
    dict(V=129, d=32, L=1, B=2, G=3, N=4),                # one group, one-position canvases
], ids=["tiny", "ragged", "half_chunk", "one_group"])
def test_q4_lockstep(dev, shape):
    B = shape.get("B", 1)
    wl = shrink(WORKLOADS["tiny"], name="q4", cfg_seed=19, seeds=tuple(range(B)),
                bounds=tuple((0.1, 0.3, 0.05)[c % 3] for c in range(B)), **shape)
    run_lockstep(wl, dev, layout=2)


def test_q4_lockstep_with_tail_small_vocab(dev):
    wl = WORKLOADS["small_vocab"]
    run_lockstep(wl, dev, layout=2, tail=_tail(wl, softcap=30.0), steps=range(0, 48, 12))


# ----------------------------------------------------------------------------
# sparse label read
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("case", [
    dict(V=1024, d=64, rows=16, labels=[3, 17], T=1.0, cap=0.0),
    dict(V=1001, d=72, rows=37, labels=[1000, 0, 500, 500, 7], T=0.45, cap=0.0),
    dict(V=32768, d=1024, rows=256, labels=list(range(0, 32768, 64)), T=0.8, cap=30.0),
    dict(V=4096, d=4104, rows=3, labels=[4095, 1, 2, 3], T=0.6, cap=5.0),
    dict(V=262144, d=2816, rows=64, labels=[11, 262143, 130000, 5, 77777, 250000], T=1.0, cap=0.0),
], ids=["two", "ragged_repeats", "512_labels_capped", "wide_hidden", "gemma_vocab"])
@pytest.mark.parametrize("layout", [0, 1], ids=["rows", "packed"])
def test_label_probs_match_the_oracle(dev, case, layout):
    import torch
    from uniform_state_discrete_step_amd import dgd
    from uniform_state_discrete_step_amd.inputs import make_h, make_w
    V, d, rows, labels = case["V"], case["d"], case["rows"], case["labels"]
    if V > 65536:                      # only the label rows matter: zero the rest
        W = np.zeros((V, d), dtype=np.uint16)
        W[labels] = make_w(len(labels), d, 31)
    else:
        W = make_w(V, d, 31)
    H = make_h(rows, d, 31, 0, 0)
    Wt = torch.from_numpy(W.view(np.int16)).to(dev)
    if layout == 1:
        Wt = dgd.pack_vocab(Wt, V, d)
    Hd = torch.from_numpy(H.view(np.int16)).to(dev)
    n = len(labels)
    logits = torch.empty(rows * n, dtype=torch.float32, device=dev)
    probs = torch.empty(rows * n, dtype=torch.float32, device=dev)
    dgd.dgd_label_probs(Hd, rows, Wt, layout, V, d, labels, case["T"], case["cap"], logits, probs)
    torch.cuda.synchronize()
    zg = logits.cpu().numpy().reshape(rows, n).astype(np.float64)
    pg = probs.cpu().numpy().reshape(rows, n).astype(np.float64)
    zo, po = O.label_probs(H, W, labels, case["T"], case["cap"])
    scale = np.maximum(np.abs(zo), np.sqrt(np.mean(zo * zo, axis=1, keepdims=True)))
    zerr = (np.abs(zg - zo) / np.maximum(scale, 1e-30)).max()
    perr = (np.abs(pg - po) / np.maximum(po, 1e-30)).max()
    print(f"\n[labels n={n} V={V} d={d} layout={layout}] logit rel err {zerr:.2e}, "
          f"prob rel err {perr:.2e}", flush=True)
    assert zerr <= TOL_LOGIT_REL
    assert np.all(np.abs(pg - po) <= 1e-3 * po + 1e-30)
    assert np.allclose(pg.sum(axis=1), 1.0, atol=1e-5)


# ----------------------------------------------------------------------------
def _logit_check(wl, dev, W, Hs, steps, layout, tail=None):
    import torch
    ls = Lockstep(wl, W, Hs, dev, logits=True, layout=layout, tail=tail)
    ls.run(steps=steps)
    torch.cuda.synchronize()
    z_gpu = ls.ctx.logits.cpu().numpy().reshape(wl.B * wl.L, wl.V).astype(np.float64)
    b, s = wl.blocks - 1, steps[-1]
    H_rows = Hs[b, s].reshape(wl.B * wl.L, wl.d)
    if tail is not None and tail.norm_weight is not None:
        H_rows = O.rms_norm(H_rows, tail.norm_weight, tail.norm_eps)
    z = O.projection(H_rows, W)
    scale = np.maximum(np.abs(z), np.sqrt(np.mean(z * z, axis=1, keepdims=True)))
    rel = np.abs(z_gpu - z) / np.maximum(scale, 1e-30)
    print(f"\n[{wl.name}] logits: max rel err {rel.max():.3e}, max abs err "
          f"{np.abs(z_gpu - z).max():.3e}", flush=True)
    assert rel.max() <= TOL_LOGIT_REL
    return z_gpu, z


def test_logits_tiny(dev, layout):
    wl = WORKLOADS["tiny"]
    W, Hs = make_workload_arrays(wl, threads=1)
    _logit_check(wl, dev, W, Hs, steps=[0, 1, 2], layout=layout)


def test_logits_small_vocab(dev, layout):
    wl = WORKLOADS["small_vocab"]
    W, Hs = make_workload_arrays(wl, threads=8)
    _logit_check(wl, dev, W, Hs, steps=[0], layout=layout)


def test_projection_is_exact_on_small_integers(dev, layout):
    """Small-integer bf16 H and W: every fp32 partial sum is exact, so the
    logits must equal the exact integer dot products bit for bit (a wrong
    operand layout, transposition or hidden-chunk mapping cannot pass)."""
    wl = shrink(WORKLOADS["tiny"], V=300, d=200, L=40, B=1, G=40, N=2)
    rng = np.random.default_rng(11)
    W = bf16(rng.integers(-2, 3, size=(wl.V, wl.d)))
    Hs = bf16(rng.integers(-2, 3, size=(1, wl.N, 1, wl.L, wl.d)))
    z_gpu, z = _logit_check(wl, dev, W, Hs, steps=[0], layout=layout)
    assert np.array_equal(z_gpu, z)


# ----------------------------------------------------------------------------
def test_first_step_from_uniform_logits(dev, layout):
    """H = 0 gives uniform logits: entropy ln V everywhere, every argmax the
    first id (ties go to the lowest id, across lanes, waves, tiles and
    vocabulary groups) and one commit, at position 0."""
    wl = shrink(WORKLOADS["tiny"], V=2048, d=64, L=64, G=64, N=4)
    W, _ = make_workload_arrays(wl, threads=1)
    Hs = np.zeros((1, wl.N, 1, wl.L, wl.d), dtype=np.uint16)
    ls, rep = run_lockstep(wl, dev, W=W, Hs=Hs, steps=[0], layout=layout)
    H = ls.ctx.entropy.cpu().numpy()
    assert np.all(np.abs(H - math.log(wl.V)) < 1e-5)
    assert np.all(ls.ctx.argmax.cpu().numpy() == 0)
    com = ls.committed.cpu().numpy()
    assert com.tolist() == [1] + [0] * (wl.L - 1)


def test_convergence_on_stable_peaked_inputs(dev, layout):
    """Identical one-hot logits every step: the canvas converges at step 1."""
    V = d = 64
    L = 32
    wl = shrink(WORKLOADS["tiny"], V=V, d=d, L=L, G=L, N=8)
    W = bf16(np.eye(V))
    toks = (np.arange(L) * 7 + 3) % V
    h = np.zeros((L, d), dtype=np.float32)
    h[np.arange(L), toks] = 60.0
    Hs = np.broadcast_to(bf16(h), (1, wl.N, 1, L, d)).copy()
    ls, rep = run_lockstep(wl, dev, W=W, Hs=Hs, layout=layout)
    sv = ls.ctx.state_views()
    assert int(sv["steps_used"][0]) == 2 and int(sv["converged"][0]) == 1
    assert np.array_equal(ls.canvas.cpu().numpy(), toks)


# ----------------------------------------------------------------------------
@pytest.mark.parametrize("V,d", [(1001, 72), (64, 64), (300, 200), (1, 8)])
def test_pack_vocab_layout(dev, V, d):
    """dgd_pack_vocab against the layout include/dgd.h documents, bit for bit:
    element j of lane l of fragment f, step s, chunk c, row group rg holds
    W[64 rg + 32 f + l % 32][64 c + 32 (l // 32) + 8 s + j], zeros past V, d."""
    import torch
    from uniform_state_discrete_step_amd import dgd
    rng = np.random.default_rng(V * 1000 + d)
    W = rng.integers(0, 1 << 16, size=(V, d), dtype=np.uint16)
    Wd = torch.from_numpy(W.view(np.int16)).to(dev)
    got = dgd.pack_vocab(Wd, V, d).cpu().numpy().view(np.uint16)
    n_rg, nk = -(-V // 64), -(-d // 64)
    Wpad = np.zeros((n_rg * 64, nk * 64), dtype=np.uint16)
    Wpad[:V, :d] = W
    rg, c, s, f, l, j = np.meshgrid(np.arange(n_rg), np.arange(nk), np.arange(4), np.arange(2),
                                    np.arange(64), np.arange(8), indexing="ij")
    expect = Wpad[64 * rg + 32 * f + l % 32, 64 * c + 32 * (l // 32) + 8 * s + j]
    assert got.shape[0] == dgd.dgd_packed_vocab_bytes(V, d) // 2 == expect.size
    assert np.array_equal(got, expect.reshape(-1))


# ----------------------------------------------------------------------------
def test_resume_from_saved_state(dev, layout):
    """Stopping after a step, saving canvas, mask and state to the host and
    resuming in a fresh context gives the uninterrupted run, bit for bit."""
    import torch
    from uniform_state_discrete_step_amd import dgd
    wl = shrink(WORKLOADS["tiny"], B=2, G=48, L=16, N=6, seeds=(4, 9), bounds=(0.1, 0.3))
    W, Hs = make_workload_arrays(wl, threads=1)
    Wd = torch.from_numpy(W.view(np.int16)).to(dev)
    if layout == dgd.DGD_VOCAB_PACKED:
        Wd = dgd.pack_vocab(Wd, wl.V, wl.d)
    Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
    prm = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence, wl.stability_threshold,
                          wl.freeze, wl.final_emit)

    def ctx():
        return dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev, vocab_layout=layout)

    def fresh():
        return (torch.zeros(wl.B * wl.G, dtype=torch.int32, device=dev),
                torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=dev))

    can_a, com_a = fresh()
    dgd.dgd_run(Hd.reshape(-1), Wd, can_a, com_a, prm, wl.seeds, ctx())
    torch.cuda.synchronize()

    def steps(c, can, com, todo):
        for b, s in todo:
            if s == 0:
                dgd.dgd_init_block(can, com, b, prm, wl.seeds, c)
            dgd.dgd_step(Hd[b, s].reshape(-1), Wd, can, com, b, s, prm, wl.seeds, c)

    order = [(b, s) for b in range(wl.blocks) for s in range(wl.N)]
    cut = wl.N + 2                      # inside the second block
    c1 = ctx()
    can_b, com_b = fresh()
    steps(c1, can_b, com_b, order[:cut])
    torch.cuda.synchronize()
    saved = (can_b.cpu(), com_b.cpu(), c1.state.cpu())
    c2 = ctx()
    can_c, com_c = fresh()
    can_c.copy_(saved[0]); com_c.copy_(saved[1]); c2.state.copy_(saved[2])
    steps(c2, can_c, com_c, order[cut:])
    torch.cuda.synchronize()
    assert np.array_equal(can_c.cpu().numpy(), can_a.cpu().numpy())
    assert np.array_equal(com_c.cpu().numpy(), com_a.cpu().numpy())


# ----------------------------------------------------------------------------
# non-finite logits: the canvas stops with a status, untouched
# ----------------------------------------------------------------------------
def test_nonfinite_logits_stop_the_canvas(dev, layout):
    """A NaN in a row of H (canvas 1, step 2) and a row of the largest finite
    bf16 value, whose fp32 projection overflows (canvas 0, step 4): at that
    step the canvas keeps its tokens, mask and argmax reference, its status
    becomes DGD_STATUS_NONFINITE and it is done; the offending position's
    entropy and gap are NaN and its ids -1; the other canvas goes on as the
    oracle does (lockstep), and later steps leave the stopped canvas alone."""
    import torch
    from tests.parity import Report, compare_step, oracle_step
    from uniform_state_discrete_step_amd import dgd
    wl = shrink(WORKLOADS["tiny"], B=2, G=16, seeds=(0, 1), bounds=(0.1, 0.2))
    W, Hs = make_workload_arrays(wl, threads=1)
    Hs = Hs.copy()
    bad = {(2, 1): 5, (4, 0): 9}                     # (step, canvas) -> position
    Hs[0, 2, 1, 5, 7] = 0x7FC0                        # NaN
    Hs[0, 4, 0, 9, :] = 0x7F7F                        # 3.39e38 everywhere
    ls = Lockstep(wl, W, Hs, dev, layout=layout)
    ls.states = [O.init_block(st, 0, wl.L, wl.V, wl.seeds[c]) for c, st in enumerate(ls.states)]
    dgd.dgd_init_block(ls.canvas, ls.committed, 0, ls.params, wl.seeds, ls.ctx)
    rep = Report()
    stopped = set()
    for s_idx in range(6):
        ls.push_state()
        dgd.dgd_step(ls.Hd[0, s_idx].reshape(-1), ls.Wd, ls.canvas, ls.committed, 0, s_idx,
                     ls.params, wl.seeds, ls.ctx)
        torch.cuda.synchronize()
        sv = ls.ctx.state_views()
        for c in range(wl.B):
            before = ls.states[c]
            g = ls.pull(c)
            if (s_idx, c) in bad or c in stopped:
                p = bad.get((s_idx, c))
                assert np.array_equal(g["canvas"], before.canvas)
                assert np.array_equal(g["committed"], before.committed)
                assert np.array_equal(g["prev_argmax"], before.prev_argmax)
                assert int(sv["status"][c]) == dgd.DGD_STATUS_NONFINITE
                assert int(sv["done"][c]) == 1 and int(sv["converged"][c]) == 0
                if p is not None:
                    assert int(sv["steps_used"][c]) == s_idx + 1
                    assert np.isnan(g["entropy"][p]) and np.isnan(g["gap"][p])
                    assert g["argmax"][p] == -1 and g["token"][p] == -1
                    ls.states[c] = dataclasses.replace(before, done=True, steps_used=s_idx + 1)
                    stopped.add(c)
                continue
            after, info = oracle_step(before, Hs[0, s_idx, c], W, 0, s_idx, ls.P, wl.seeds[c],
                                      wl.bounds[c], W64=ls.W64)
            compare_step(rep, f"step {s_idx} canvas {c}", before, after, info, g, wl.L, wl.V, 0,
                         s_idx, ls.P, wl.seeds[c], float(np.float32(wl.bounds[c])))
            if not info.get("skipped"):
                assert int(sv["status"][c]) == dgd.DGD_STATUS_OK
            ls.states[c] = after
    print(f"\n[non-finite rows] {rep.summary()} stopped canvases {sorted(stopped)}", flush=True)
    assert not rep.failures, "\n".join(rep.failures)
    assert stopped == {0, 1}
