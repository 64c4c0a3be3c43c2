"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one function of ``oracle/dgd_oracle.py`` against a published
known-answer vector, a figure the pages print, a closed form, a brute-force
enumeration or a statistical law, chosen so that a dropped term, a wrong sign,
a wrong index or a transposed operand fails at least one of them.
"""
import math
import os
from itertools import combinations

import numpy as np
import pytest

from oracle import dgd_oracle as O
from tests.conftest import read_page_figures
from uniform_state_discrete_step_amd.inputs import f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def identity_w(V):
    """W = I (V x V): the logits are then the hidden row itself."""
    return bf16(np.eye(V, dtype=np.float32))


# ----------------------------------------------------------------------------
# random numbers
# ----------------------------------------------------------------------------
def test_philox_known_answers(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([int(t, 16) for t in line.split()])
    assert len(rows) == 3
    for r in rows:
        out = O.philox4x32_10(*r[:6])
        assert [int(w) for w in out] == r[6:]


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(4, 64), dtype=np.uint64)
    k = rng.integers(0, 2**32, size=2, dtype=np.uint64)
    vec = O.philox4x32_10(c[0], c[1], c[2], c[3], k[0], k[1])
    for i in range(64):
        one = O.philox4x32_10(int(c[0, i]), int(c[1, i]), int(c[2, i]), int(c[3, i]),
                              int(k[0]), int(k[1]))
        assert [int(w[i]) for w in vec] == [int(w) for w in one]


def test_seed_key_split():
    assert O.seed_key(0x0123456789ABCDEF) == (0x89ABCDEF, 0x01234567)
    assert O.seed_key(7) == (7, 0)


def test_uniform_cells_are_symmetric_and_open():
    w = np.array([0, 1, 511, 512, 2**31, 2**32 - 1], dtype=np.uint32)
    u = O.uniform_from_word(w)
    assert u[0] == 2.0 ** -24 and u[-1] == 1 - 2.0 ** -24
    assert u[1] == u[0] and u[2] == u[0] and u[3] == 3 * 2.0 ** -24
    rng = np.random.default_rng(0)
    ws = rng.integers(0, 2**32, size=1000, dtype=np.uint64).astype(np.uint32)
    # the cell of w and the cell of its complement mirror each other around 1/2
    assert np.all(O.uniform_from_word(ws) + O.uniform_from_word(~ws) == 1.0)


def test_gumbel_extremes_bound_the_noise():
    g_lo, g_hi = O.gumbel_extremes()
    # -ln(-ln u) is increasing in u: the extreme cells give the extreme values
    assert -3.0 < g_lo < -2.8 and 16.6 < g_hi < 16.7
    rng = np.random.default_rng(1)
    ws = rng.integers(0, 2**32, size=100000, dtype=np.uint64).astype(np.uint32)
    g = O.gumbel_from_word(ws)
    assert g.min() >= g_lo and g.max() <= g_hi
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    assert abs(g.mean() - 0.5772156649) < 0.02
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05


def _chi2_pvalue(obs, expected):
    from scipy.stats import chisquare
    return chisquare(obs, expected).pvalue


def test_gumbel_max_samples_the_tempered_softmax():
    """Token frequencies follow softmax(z / T) (Gumbel-max theorem)."""
    V, n, T = 8, 120000, 0.5
    z = np.array([0.3, -0.2, 0.9, 0.0, -1.0, 0.5, 0.1, -0.4])
    rows = np.tile(z, (n, 1))
    st = O.position_stats(rows, T, seed=123, p_abs=np.arange(n), gstep=7)
    counts = np.bincount(st["token"], minlength=V)
    p = np.exp(z / T) / np.exp(z / T).sum()
    assert _chi2_pvalue(counts, p * n) > 1e-4
    # the same draw at T = 1 must NOT match softmax(z / 0.5): temperature is applied
    st1 = O.position_stats(rows, 1.0, seed=123, p_abs=np.arange(n), gstep=7)
    c1 = np.bincount(st1["token"], minlength=V)
    assert _chi2_pvalue(c1, p * n) < 1e-6


def test_gumbel_words_layout():
    """Word (row, v) is word v & 3 of the counter (v >> 2, p_abs, gstep, 0)."""
    seed, gstep, V = 0xDEADBEEF12345678, 11, 10
    words = O.gumbel_words(seed, np.array([3, 9]), gstep, V)
    k0, k1 = O.seed_key(seed)
    for r, p in enumerate([3, 9]):
        for v in range(V):
            w = O.philox4x32_10(v // 4, p, gstep, 0, k0, k1)[v % 4]
            assert int(words[r, v]) == int(w)


def test_uniform_tokens():
    # power-of-two V: the token is the top log2(V) bits of the word
    rng = np.random.default_rng(2)
    ws = rng.integers(0, 2**32, size=5000, dtype=np.uint64)
    for logv in (1, 10, 18):
        assert np.array_equal(O.uniform_token(ws, 2 ** logv), (ws >> (32 - logv)).astype(np.int64))
    # any V: tokens are in range and uniform
    n = 200000
    for V in (10, 1000):
        t = O.renoise_token(99, np.arange(n), 5, V)
        assert t.min() >= 0 and t.max() < V
        counts = np.bincount(t, minlength=V)
        assert _chi2_pvalue(counts, np.full(V, n / V)) > 1e-4
        t0 = O.init_token(99, np.arange(n), 0, V)
        assert _chi2_pvalue(np.bincount(t0, minlength=V), np.full(V, n / V)) > 1e-4
    # adjacent positions and steps are not correlated
    a = O.renoise_token(5, np.arange(n), 3, 1 << 16).astype(np.float64)
    b = O.renoise_token(5, np.arange(n), 4, 1 << 16).astype(np.float64)
    assert abs(np.corrcoef(a[:-1], a[1:])[0, 1]) < 0.01
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.01
    # the three streams (Gumbel, renoise, init) differ for the same position
    assert not np.array_equal(O.renoise_token(5, np.arange(64), 0, 1 << 16),
                              O.init_token(5, np.arange(64), 0, 1 << 16))


# ----------------------------------------------------------------------------
# temperature schedule
# ----------------------------------------------------------------------------
def test_schedule_matches_both_pages(golden_dir):
    fig = read_page_figures(os.path.join(golden_dir, "page_figures.txt"))
    N, t_min, t_max = fig["num_inference_steps"], fig["t_min"], fig["t_max"]
    Ts = [O.temperature(i, N, t_min, t_max) for i in range(N)]
    # node page form: T = t_min + (t_max - t_min) * t, t = (N - i) / N
    for i, T in enumerate(Ts):
        t = (N - i) / N
        assert abs(T - (t_min + (t_max - t_min) * t)) < 1e-15
    assert Ts[0] == t_max
    # the schedule position bottoms out at 1/N: t_min itself is never applied
    assert abs((Ts[-1] - t_min) / (t_max - t_min) - fig["schedule_position_last"]) < 1e-15
    assert abs(Ts[-1] - 0.4083333333333333) < 1e-15
    assert min(Ts) > t_min
    diffs = np.diff(Ts)
    assert np.allclose(diffs, (t_min - t_max) / N, rtol=0, atol=1e-15)
    assert abs(O.temperature(7, 8, 0.4, 0.8) - 0.45) < 1e-15


# ----------------------------------------------------------------------------
# projection
# ----------------------------------------------------------------------------
def test_projection_is_exact_on_small_integers():
    rng = np.random.default_rng(3)
    rows, V, d = 5, 7, 48
    Hi = rng.integers(-4, 5, size=(rows, d))
    Wi = rng.integers(-4, 5, size=(V, d))
    z = O.projection(bf16(Hi), bf16(Wi))
    for r in range(rows):
        for v in range(V):
            assert z[r, v] == sum(int(Hi[r, k]) * int(Wi[v, k]) for k in range(d))


def test_projection_chunking_is_invisible():
    rng = np.random.default_rng(4)
    H = bf16(rng.standard_normal((3, 32)))
    W = bf16(rng.standard_normal((50, 32)))
    assert np.array_equal(O.projection(H, W, v_chunk=7), O.projection(H, W, v_chunk=64))


# ----------------------------------------------------------------------------
# the lm-head tail: bfloat16 rounding, output RMSNorm, softcap
# ----------------------------------------------------------------------------
def test_round_bf16_agrees_with_the_float32_rounding():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.ldexp(rng.integers(1, 1 << 24, 200).astype(np.float64), -149)])
    x32 = x.astype(np.float32)                      # values that float32 holds exactly
    assert np.array_equal(O.round_bf16(x32.astype(np.float64)), f32_to_bf16_bits(x32))


def test_the_two_bf16_roundings_agree_on_float32_values():
    rng = np.random.default_rng(18)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)   # exact halves
    for v in (x, ties, -ties):
        assert np.array_equal(O.round_bf16_f32(v), O.round_bf16(v.astype(np.float64)))


def test_round_bf16_ties_to_even_and_rounds_once():
    one = 0x3F80
    assert O.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == one           # tie -> even (down)
    assert O.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == one + 2   # tie -> even (up)
    assert O.round_bf16(np.array([-(1.0 + 2.0 ** -8)]))[0] == 0x8000 | one
    # just above the tie: one rounding from float64 goes up; a detour through
    # float32 would land on the tie and then go down to even
    assert O.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == one + 1
    assert O.round_bf16(np.array([2.0 ** -130, 0.0]))[1] == 0
    assert O.round_bf16(np.array([2.0 ** -130]))[0] == 1 << 3               # subnormal


def _norm_inputs(seed, rows=6, d=96):
    rng = np.random.default_rng(seed)
    H = bf16(rng.standard_normal((rows, d)) * 3.0)
    w = bf16(np.exp(rng.uniform(np.log(0.5), np.log(8.0), d)))
    return H, w


def bf16_f64(b):
    return O.bf16_to_f64(b)


def test_rms_norm_hand_example():
    # x = (3, 4): ||x|| = 5, sqrt(d) = sqrt(2); unit weights
    out = bf16_f64(O.rms_norm(bf16([[3.0, 4.0]]), bf16([1.0, 1.0]), 0.0))[0]
    assert np.allclose(out, [0.6 * math.sqrt(2), 0.8 * math.sqrt(2)], rtol=2 ** -8)
    # twice the weights: twice the output, bit for bit
    out2 = bf16_f64(O.rms_norm(bf16([[3.0, 4.0]]), bf16([2.0, 2.0]), 0.0))[0]
    assert np.array_equal(out2, 2 * out)


def test_rms_norm_gives_unit_rms_along_the_row():
    H, _ = _norm_inputs(1)
    d = H.shape[1]
    out = bf16_f64(O.rms_norm(H, bf16(np.ones(d)), 0.0))
    assert np.allclose(np.sqrt((out ** 2).mean(axis=1)), 1.0, rtol=2 ** -8)
    x = bf16_f64(H)
    assert np.allclose(out * np.linalg.norm(x, axis=1, keepdims=True) / math.sqrt(d), x,
                       rtol=2 ** -8, atol=0)       # same direction as the input


def test_rms_norm_scale_and_sign_invariance():
    H, w = _norm_inputs(2)
    base = O.rms_norm(H, w, 0.0)
    for k in (-6, -1, 3, 9):                        # powers of two scale exactly
        Hs = bf16(bf16_f64(H) * 2.0 ** k)
        assert np.array_equal(O.rms_norm(Hs, w, 0.0), base)
    assert np.array_equal(O.rms_norm(H ^ np.uint16(0x8000), w, 0.0), base ^ np.uint16(0x8000))


def test_rms_norm_epsilon_is_added_to_the_norm():
    H, w = _norm_inputs(3, rows=4)
    x = bf16_f64(H)
    n = np.linalg.norm(x, axis=1)
    for r in range(H.shape[0]):
        # eps equal to the row's norm halves the output exactly
        half = bf16_f64(O.rms_norm(H[r:r + 1], w, float(n[r])))
        full = bf16_f64(O.rms_norm(H[r:r + 1], w, 0.0))
        assert np.array_equal(half, full / 2)
    # a zero row with eps > 0 stays zero
    assert not bf16_f64(O.rms_norm(bf16(np.zeros((1, 8))), bf16(np.ones(8)), 1e-6)).any()


def test_softcap_closed_forms():
    c = 30.0
    z = np.linspace(-500, 500, 2001)
    y = O.softcap(z, c)
    assert np.all(np.abs(y) < c) and np.all(np.diff(y) > 0)
    assert np.array_equal(O.softcap(-z, c), -y)
    assert abs(O.softcap(np.array([c * math.atanh(0.5)]), c)[0] - c / 2) < 1e-12
    small = np.array([1e-3, -2e-3])
    assert np.allclose(O.softcap(small, c), small - small ** 3 / (3 * c * c), rtol=1e-15)
    assert np.array_equal(O.softcap(z, 0.0), z)


def test_tail_logits_are_invariant_to_the_hidden_scale():
    rng = np.random.default_rng(5)
    H, w = _norm_inputs(4, rows=3, d=64)
    W = bf16(rng.standard_normal((40, 64)))
    tail = O.Tail(norm_weight=w, norm_eps=0.0, softcap=15.0)
    z = O.logits(H, W, tail)
    assert np.array_equal(O.logits(bf16(bf16_f64(H) * 16.0), W, tail), z)
    assert np.all(np.abs(z) < 15.0)
    plain = O.logits(H, W, None)
    assert np.array_equal(plain, O.projection(H, W))
    # a cap far above every logit pulls it in by z^3 / (3 c^2) to leading order
    c = 1e6
    big = O.logits(H, W, O.Tail(softcap=c))
    lead = plain ** 3 / (3 * c * c)
    assert np.all(np.abs((plain - big) - lead) <= 1e-3 * np.abs(lead) + 1e-12 * np.abs(plain))


def test_step_with_softcap_keeps_the_argmax():
    rng = np.random.default_rng(6)
    L, V, d = 8, 48, 32
    H = bf16(rng.standard_normal((L, d)))
    W = bf16(rng.standard_normal((V, d)))
    P = O.Params(N=4, t_min=0.4, t_max=0.8)
    st0 = O.init_block(O.new_state(L, L), 0, L, V, 7)
    _, a = O.step(st0, H, W, 0, 1, P, 7, 0.5)
    _, b = O.step(st0, H, W, 0, 1, P, 7, 0.5, tail=O.Tail(softcap=2.0))
    sa, sb = a["stats"], b["stats"]
    assert np.array_equal(sa["argmax"], sb["argmax"])          # the cap is monotone
    # a cap of 2 squeezes these logits into (-2, 2): every row is flatter
    assert np.all(sb["entropy64"] >= sa["entropy64"] - 1e-12)
    assert np.any(sb["entropy64"] > sa["entropy64"] + 1e-3)


# ----------------------------------------------------------------------------
# self-conditioning: top-K and the embedding sum
# ----------------------------------------------------------------------------
def test_sc_topk_two_level_closed_form():
    # k ids at logit a, the rest at b: the k high ids come first (by id), then
    # the lowest low ids; probabilities e^a / (k e^a + (V - k) e^b)
    V, k, a, b, T = 50, 3, 2.0, -1.0, 0.5
    z = np.full((1, V), b)
    hi = [7, 31, 44]
    z[0, hi] = a
    prob, ids, _ = O.sc_topk(z, T, 5)
    assert ids[0].tolist() == hi + [0, 1]
    den = k * math.exp(a / T) + (V - k) * math.exp(b / T)
    assert np.allclose(prob[0, :3], math.exp(a / T) / den, rtol=1e-14)
    assert np.allclose(prob[0, 3:], math.exp(b / T) / den, rtol=1e-14)


def test_sc_topk_uniform_row_and_full_k():
    V = 40
    prob, ids, _ = O.sc_topk(np.zeros((2, V)), 0.7, V)
    assert np.array_equal(ids, np.tile(np.arange(V), (2, 1)))     # all tied: by id
    assert np.allclose(prob, 1.0 / V, rtol=1e-15)
    rng = np.random.default_rng(8)
    z = rng.standard_normal((4, V)) * 3
    prob, ids, _ = O.sc_topk(z, 0.4, V)
    assert np.allclose(prob.sum(axis=1), 1.0, rtol=1e-13)          # K = V: the whole law
    assert np.all(np.diff(prob, axis=1) <= 0)
    for r in range(4):
        assert sorted(ids[r].tolist()) == list(range(V))


def test_sc_topk_follows_a_permutation_and_ignores_shifts():
    rng = np.random.default_rng(9)
    V, K = 300, 32
    z = rng.standard_normal((3, V)) * 4
    prob, ids, _ = O.sc_topk(z, 0.6, K)
    perm = rng.permutation(V)                    # new id of old id v is perm[v]
    zp = np.empty_like(z)
    zp[:, perm] = z
    prob_p, ids_p, _ = O.sc_topk(zp + 17.0, 0.6, K)
    assert np.array_equal(ids_p, perm[ids])      # continuous logits: no ties
    assert np.allclose(prob_p, prob, rtol=1e-12)
    # the top-K probabilities are the largest K of softmax, so they bound the rest
    p_all = np.exp(z / 0.6 - (z / 0.6).max(axis=1, keepdims=True))
    p_all /= p_all.sum(axis=1, keepdims=True)
    for r in range(3):
        rest = np.delete(p_all[r], ids[r])
        assert rest.max() <= prob[r, -1]


def test_sc_embed_one_hot_and_identity_table():
    rng = np.random.default_rng(10)
    V, d = 16, 16
    W = bf16(rng.standard_normal((V, d)))
    # K = 1 with probability 1: the scaled embedding row itself
    out = O.sc_embed(np.array([[1.0], [1.0]]), np.array([[3], [12]]), W, 4.0)
    assert np.array_equal(out, bf16(O.bf16_to_f64(W[[3, 12]]) * 4.0))
    # identity table: row r reads back scale * bf16(p) at each id
    I = bf16(np.eye(V))
    p = np.array([[0.5, 0.3, 0.15, 0.05]])
    idx = np.array([[9, 2, 14, 0]])
    out = O.bf16_to_f64(O.sc_embed(p, idx, I, 2.0))[0]
    expect = np.zeros(V)
    expect[idx[0]] = 2.0 * O.bf16_to_f64(bf16(p[0]))
    assert np.array_equal(out, O.bf16_to_f64(bf16(expect)))


def test_sc_embed_is_exact_on_dyadic_inputs():
    # dyadic probabilities and small-integer embeddings: every product and sum
    # is exact, so the result is the integer combination itself
    rng = np.random.default_rng(12)
    V, d, K = 64, 24, 4
    Wi = rng.integers(-3, 4, size=(V, d))
    W = bf16(Wi)
    p = np.array([[0.5, 0.25, 0.125, 0.0625]] * 2)
    idx = np.array([[5, 17, 33, 60], [0, 1, 2, 3]])
    out = O.bf16_to_f64(O.sc_embed(p, idx, W, 8.0))
    for r in range(2):
        ref = 8.0 * sum(p[r, j] * Wi[idx[r, j]] for j in range(K))
        assert np.array_equal(out[r], ref)


# ----------------------------------------------------------------------------
# sparse label read
# ----------------------------------------------------------------------------
def test_label_probs_closed_forms():
    rng = np.random.default_rng(14)
    d, V = 16, 40
    W = bf16(rng.standard_normal((V, d)))
    H = bf16(rng.standard_normal((3, d)))
    # identical label rows: equal probabilities
    Weq = W.copy()
    Weq[[5, 9, 30]] = W[2]
    _, p = O.label_probs(H, Weq, [2, 5, 9, 30], 0.7)
    assert np.allclose(p, 0.25, rtol=1e-15)
    # two labels: the logistic function of the tempered difference
    z, p = O.label_probs(H, W, [3, 17], 0.5)
    zz = O.projection(H, W)
    assert np.array_equal(z, zz[:, [3, 17]])
    assert np.allclose(p[:, 0], 1.0 / (1.0 + np.exp(-(zz[:, 3] - zz[:, 17]) / 0.5)), rtol=1e-14)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-15)


def test_label_probs_are_exact_integer_logits():
    rng = np.random.default_rng(15)
    Hi = rng.integers(-3, 4, size=(2, 40))
    Wi = rng.integers(-3, 4, size=(30, 40))
    labels = [29, 0, 7]
    z, _ = O.label_probs(bf16(Hi), bf16(Wi), labels, 1.0)
    assert np.array_equal(z, (Hi @ Wi[labels].T).astype(np.float64))


def test_label_probs_on_the_top_k_agree_with_the_top_k_probabilities():
    # labels = a position's top K: the label law is the top-K law renormalised
    rng = np.random.default_rng(16)
    V, d, T, K = 300, 24, 0.6, 12
    W = bf16(rng.standard_normal((V, d)))
    H = bf16(rng.standard_normal((1, d)) * 3)
    z = O.projection(H, W)
    prob, ids, _ = O.sc_topk(z, T, K)
    zl, p = O.label_probs(H, W, ids[0], T)
    assert np.allclose(p[0], prob[0] / prob[0].sum(), rtol=1e-12)
    # and the softcap applies to the logits before the temperature
    zc, pc = O.label_probs(H, W, ids[0], T, softcap_c=2.0)
    assert np.allclose(zc, 2.0 * np.tanh(zl / 2.0), rtol=1e-15)
    assert np.all(np.abs(zc) < 2.0)


# ----------------------------------------------------------------------------
# 4-bit table
# ----------------------------------------------------------------------------
def test_dequant_q4_by_hand():
    # one row of 32 elements: codes 0..15 then 15..0; scale 0.5, min -2
    q = np.array(list(range(16)) + list(range(15, -1, -1)), dtype=np.uint8)
    codes = (q[0::2] | (q[1::2] << 4))[None, :]
    w = O.bf16_to_f64(O.dequant_q4(codes, bf16([[0.5]]), bf16([[-2.0]])))[0]
    assert np.array_equal(w, 0.5 * q - 2.0)           # every value exact in bf16
    # element order: low nibble first
    c = np.zeros((1, 16), dtype=np.uint8)
    c[0, 0] = 0x31                                     # element 0 -> 1, element 1 -> 3
    w = O.bf16_to_f64(O.dequant_q4(c, bf16([[1.0]]), bf16([[0.0]])))[0]
    assert w[0] == 1.0 and w[1] == 3.0 and not w[2:].any()


def test_dequant_q4_rounds_once_to_nearest_even():
    # s q + m = 1 + k 2^-8 lands halfway between bf16 neighbours for odd k
    c = np.zeros((1, 16), dtype=np.uint8)
    c[0, 0] = 0x31                                     # q = 1, 3
    w = O.dequant_q4(c, bf16([[2.0 ** -8]]), bf16([[1.0]]))[0]
    assert w[0] == 0x3F80                              # 1 + 2^-8 -> 1 (even)
    assert w[1] == 0x3F82                              # 1 + 3 2^-8 -> 1 + 2^-6 (even)
    assert np.all(w[2:] == 0x3F80)                     # q = 0: the minimum itself


def test_quantized_table_is_close_to_the_original():
    from uniform_state_discrete_step_amd.inputs import make_w, quantize_q4
    W = make_w(64, 96, 3)
    codes, sc, mn = quantize_q4(W)
    Wq = O.bf16_to_f64(O.dequant_q4(codes, sc, mn))
    W0 = O.bf16_to_f64(W)
    step = np.repeat(O.bf16_to_f64(sc), 32, axis=1)
    # within half a step (plus the bf16 roundings of scale, minimum and value)
    assert np.all(np.abs(Wq - W0) <= 0.5 * step + 0.02 * np.abs(W0) + 1e-3)


# ----------------------------------------------------------------------------
# entropy and argmax
# ----------------------------------------------------------------------------
def test_entropy_of_uniform_row_is_log_v(golden_dir):
    fig = read_page_figures(os.path.join(golden_dir, "page_figures.txt"))
    bits = fig["uniform_melt_bits"]
    V = 2 ** bits
    z = O.projection(bf16(np.zeros((1, 8))), bf16(np.ones((V, 8)) * 0.5))
    st = O.position_stats(z, 0.8, 0, [0], 0)
    assert abs(st["entropy64"][0] - bits * math.log(2)) < 1e-9
    assert round(float(st["entropy"][0]), 2) == fig["uniform_melt_nats"]
    assert st["argmax"][0] == 0                    # all tied: first index
    st2 = O.position_stats(np.zeros((1, 1024)), 0.45, 0, [0], 0)
    assert abs(st2["entropy64"][0] - math.log(1024)) < 1e-12


def test_entropy_of_one_hot_row_is_zero():
    V = 64
    z = np.zeros((1, V))
    z[0, 37] = 90.0                                 # 90 / 0.4 = 225 nats ahead
    st = O.position_stats(z, 0.4, 0, [0], 0)
    assert st["entropy64"][0] < 1e-90 and st["entropy"][0] == 0.0
    assert st["argmax"][0] == 37 and st["token"][0] == 37


def test_entropy_of_k_hot_rows_is_log_k():
    V = 128
    for k in (1, 2, 3, 7, 100):
        h = np.full(V, -40.0, dtype=np.float32)
        top = np.sort(np.random.default_rng(k).choice(V, size=k, replace=False))
        h[top] = 8.0
        z = O.projection(bf16(h[None, :]), identity_w(V))
        st = O.position_stats(z, 0.5, 0, [0], 0)
        assert abs(st["entropy64"][0] - math.log(k)) < 1e-12
        assert st["argmax"][0] == top[0]
        assert st["token"][0] in set(top.tolist())


def test_entropy_two_level_closed_form():
    V, T = 300, 0.6
    for k, a, b in [(1, 2.0, 0.0), (5, 1.5, -0.5), (150, 0.25, 0.0), (299, 0.0, 3.0)]:
        h = np.full(V, b, dtype=np.float32)
        h[:k] = a
        z = O.projection(bf16(h[None, :]), identity_w(V))
        st = O.position_stats(z, T, 0, [0], 0)
        ea, eb = math.exp(a / T), math.exp(b / T)
        Z = k * ea + (V - k) * eb
        p1, p2 = ea / Z, eb / Z
        closed = -k * p1 * math.log(p1) - (V - k) * p2 * math.log(p2)
        assert abs(st["entropy64"][0] - closed) < 1e-12
        assert st["argmax"][0] == (0 if a > b else k)


def test_entropy_of_gaussian_logits():
    """Random-energy-model law: H ~ ln V - sigma^2 / 2 for tempered N(0, sigma^2) logits."""
    V, sigma = 1 << 16, 1.0
    rng = np.random.default_rng(6)
    z = rng.standard_normal((16, V)) * sigma * 0.7
    st = O.position_stats(z, 0.7, 0, np.arange(16), 0)
    assert abs(st["entropy64"].mean() - (math.log(V) - sigma ** 2 / 2)) < 0.02


def test_entropy_is_nonnegative_and_at_most_log_v():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((64, 500)) * rng.uniform(0.01, 50, size=(64, 1))
    st = O.position_stats(z, 0.4, 1, np.arange(64), 2)
    assert np.all(st["entropy64"] >= 0) and np.all(st["entropy64"] <= math.log(500) + 1e-12)
    assert np.all(st["gap"] >= 0) and np.all(st["argmax_gap"] >= 0)


# ----------------------------------------------------------------------------
# the top-two gaps that decide the tie bands (argmax_gap on the tempered
# logits, gap on the Gumbel-perturbed ones)
# ----------------------------------------------------------------------------
def _kat_zero_words(golden_dir):
    """The published Philox4x32-10 output for counter (0,0,0,0) and key (0,0):
    the Gumbel words of ids 0..3 at seed 0, position 0, global step 0."""
    with open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            r = [int(t, 16) for t in line.split()]
            if r[:6] == [0] * 6:
                return r[6:]
    raise AssertionError("no all-zero known-answer row")


def _gumbel_of_word(w):
    """g = -ln(-ln u), u the midpoint of cell w >> 9 of 2^23 (scalar floats)."""
    u = ((w >> 9) + 0.5) * 2.0 ** -23
    return -math.log(-math.log(u))


def test_argmax_gap_closed_forms():
    """argmax_gap = (largest - second largest) / T of the logits; 0 on an exact tie."""
    z = np.array([[5.0, 1.0, 3.0, 2.0],
                  [1.0, 5.0, 3.0, 2.0],
                  [4.0, 4.0, 1.0, 0.0],
                  [-1.0, -7.0, -1.5, -30.0],
                  [0.0, 0.0, 0.0, 0.0],
                  [2.0, 9.0, 9.0 - 2.0 ** -20, -3.0]])
    T = 0.5
    st = O.position_stats(z, T, 0, np.arange(z.shape[0]), 0)
    expect = np.array([2.0, 2.0, 0.0, 0.5, 0.0, 2.0 ** -20]) / T
    assert np.array_equal(st["argmax_gap"], expect)
    assert st["argmax"].tolist() == [0, 1, 0, 0, 0, 1]


def test_gumbel_gap_on_separated_logits(golden_dir):
    """Logits 100 apart cannot be reordered by the noise (|g| < 17), so the
    sample and its runner-up are fixed: y1 = x_top + g_top, y2 = x_next + g_next,
    with the four g from the published known-answer words (ids 0..3 at seed 0,
    position 0, global step 0 use exactly that Philox counter and key)."""
    g = [_gumbel_of_word(w) for w in _kat_zero_words(golden_dir)]
    for z, T in (([200.0, 0.0, 300.0, 100.0], 1.0), ([0.0, 300.0, 100.0, 200.0], 0.5),
                 ([300.0, 200.0, 100.0, 0.0], 2.0)):
        x = np.array(z) / T
        top, nxt = int(np.argmax(x)), int(np.argsort(x)[-2])
        st = O.position_stats(np.array([z]), T, 0, [0], 0)
        assert st["token"][0] == top
        assert abs(st["y1"][0] - (x[top] + g[top])) < 1e-9
        assert abs(st["y2"][0] - (x[nxt] + g[nxt])) < 1e-9
        assert abs(st["gap"][0] - (x[top] - x[nxt] + g[top] - g[nxt])) < 1e-9


def test_gumbel_gap_with_one_dominant_logit(golden_dir):
    """One logit far ahead: the runner-up is the largest noise among the others."""
    g = [_gumbel_of_word(w) for w in _kat_zero_words(golden_dir)]
    for k in range(4):
        z = np.zeros((1, 4))
        z[0, k] = 1000.0
        st = O.position_stats(z, 1.0, 0, [0], 0)
        rest = max(g[v] for v in range(4) if v != k)
        assert st["token"][0] == k
        assert abs(st["gap"][0] - (1000.0 + g[k] - rest)) < 1e-9


def test_gumbel_gap_on_two_token_rows(golden_dir):
    """V = 2: y_v = x_v + g_v with the first two known-answer words; the
    sample is the larger (id 0 on a tie) and the gap |y_0 - y_1|, across the
    crossover where the noise decides."""
    g0, g1 = (_gumbel_of_word(w) for w in _kat_zero_words(golden_dir)[:2])
    cross = g1 - g0                       # x_0 - x_1 at which y_0 = y_1
    for delta in (-3.0, -0.5, -1e-3, 1e-3, 0.5, 3.0):
        a = cross + delta
        z = np.array([[a, 0.0]])
        st = O.position_stats(z, 1.0, 0, [0], 0)
        y0, y1 = a + g0, g1
        assert st["token"][0] == (0 if y0 >= y1 else 1)
        assert abs(st["gap"][0] - abs(y0 - y1)) < 1e-9
        assert abs(st["gap"][0] - abs(delta)) < 1e-9


def test_gumbel_at_is_the_noise_of_the_row(golden_dir):
    """gumbel_at picks the same word as gumbel_words, and the known answers."""
    g = [_gumbel_of_word(w) for w in _kat_zero_words(golden_dir)]
    assert np.allclose(O.gumbel_at(0, 0, 0, np.arange(4)), g, rtol=0, atol=1e-12)
    seed, gstep, V = 0x0123456789ABCDEF, 29, 37
    p = np.array([[0], [5], [1000]])
    v = np.arange(V)[None, :]
    assert np.array_equal(O.gumbel_at(seed, p, gstep, v),
                          O.gumbel_from_word(O.gumbel_words(seed, p[:, 0], gstep, V)))


# ----------------------------------------------------------------------------
# commit rule
# ----------------------------------------------------------------------------
def brute_force_commit(h, eligible, bound):
    """Largest subset S of the eligible set with sum(S) - max(S) <= bound;
    among those, the one with the smallest total (unique for distinct h)."""
    elig = [p for p in range(len(h)) if eligible[p]]
    best = None
    for size in range(len(elig), 0, -1):
        feas = [S for S in combinations(elig, size)
                if sum(float(h[p]) for p in S) - max(float(h[p]) for p in S) <= bound]
        if feas:
            best = min(feas, key=lambda S: sum(float(h[p]) for p in S))
            break
    out = np.zeros(len(h), dtype=bool)
    if best is not None:
        out[list(best)] = True
    return out


def test_commit_rule_brute_force():
    rng = np.random.default_rng(8)
    grid = np.arange(0, 64) / 64.0                 # dyadic: every sum is exact
    for trial in range(400):
        n = int(rng.integers(1, 11))
        h = rng.choice(grid, size=n, replace=False).astype(np.float32)
        eligible = rng.random(n) < 0.8
        bound = float(rng.choice([0.0, 1 / 64, 0.1, 0.25, 0.5, 1.0, 3.0]))
        acc, order, sums = O.commit_rule(h, eligible, bound)
        assert np.array_equal(acc, brute_force_commit(h, eligible, bound)), (h, eligible, bound)
        if eligible.any():
            assert acc.sum() >= 1                   # the first ranked position always commits
        assert not np.any(acc & ~eligible)


def test_commit_rule_ties_and_special_cases():
    # all-equal entropies above the bound: only the lowest eligible index commits
    h = np.full(10, math.log(1024), dtype=np.float32)
    elig = np.ones(10, dtype=bool)
    elig[0] = False
    acc, _, _ = O.commit_rule(h, elig, 0.1)
    assert acc.tolist() == [False, True] + [False] * 8
    # all-zero entropies: everything eligible commits
    acc, _, _ = O.commit_rule(np.zeros(6, dtype=np.float32), np.ones(6, dtype=bool), 0.1)
    assert acc.all()
    # bound 0: rank one plus every following zero-entropy rank
    h = np.array([0.3, 0.0, 0.2, 0.0, 0.5], dtype=np.float32)
    acc, order, _ = O.commit_rule(h, np.ones(5, dtype=bool), 0.0)
    assert order == [1, 3, 2, 0, 4]
    assert acc.tolist() == [False, True, True, True, False]
    # the cut is inclusive: a running sum equal to the bound still admits its rank
    h = np.array([0.25, 0.5, 0.125, 0.75], dtype=np.float32)
    acc, _, sums = O.commit_rule(h, np.ones(4, dtype=bool), 0.375)
    assert sums == [0.0, 0.125, 0.375, 0.875]          # ranks: positions 2, 0, 1, 3
    assert acc.tolist() == [True, True, True, False]
    acc, _, _ = O.commit_rule(h, np.ones(4, dtype=bool), float(np.nextafter(0.375, 0)))
    assert acc.tolist() == [True, False, True, False]
    # nothing eligible: nothing commits
    acc, order, _ = O.commit_rule(h, np.zeros(4, dtype=bool), 1.0)
    assert not acc.any() and order == []


def test_commit_rule_monotone_in_bound_and_downward_closed():
    rng = np.random.default_rng(9)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        h = (rng.exponential(0.05, size=n) * (rng.random(n) < 0.7)).astype(np.float32)
        elig = rng.random(n) < 0.9
        b1, b2 = sorted(rng.uniform(0, 0.5, size=2))
        a1, order, _ = O.commit_rule(h, elig, b1)
        a2, _, _ = O.commit_rule(h, elig, b2)
        assert not np.any(a1 & ~a2)
        ranks = [a1[p] for p in order]              # accepted set is a prefix of the ranking
        assert ranks == sorted(ranks, reverse=True)


# ----------------------------------------------------------------------------
# whole steps
# ----------------------------------------------------------------------------
def peaked_rows(L, V, tokens, margin=60.0):
    """Hidden rows that, with W = I, give each position one dominant token."""
    h = np.zeros((L, V), dtype=np.float32)
    h[np.arange(L), tokens] = margin
    return bf16(h)


def test_first_step_from_uniform_logits_commits_one_position():
    """The walkthrough's first iteration ranks uniform logits: one position commits."""
    L, V = 12, 16
    P = O.Params(N=8)
    st = O.init_block(O.new_state(L, L), 0, L, V, seed=4)
    new, info = O.step(st, bf16(np.zeros((L, V))), identity_w(V), 0, 0, P, 4, 0.1)
    assert info["accepted"].tolist() == [True] + [False] * (L - 1)
    assert new.committed.tolist() == [1] + [0] * (L - 1)
    assert np.all(info["stats"]["entropy"] == np.float32(math.log(V)))
    # everything else is re-noised with the step's renoise stream
    exp = O.renoise_token(4, np.arange(1, L), 0, V)
    assert np.array_equal(new.canvas[1:], exp)


def test_convergence_on_constructed_stable_inputs():
    L, V = 8, 16
    P = O.Params(N=8)
    toks = np.array([3, 5, 1, 7, 2, 2, 9, 4])
    st = O.init_block(O.new_state(L, L), 0, L, V, seed=1)
    H = peaked_rows(L, V, toks)
    s1, i1 = O.step(st, H, identity_w(V), 0, 0, P, 1, 0.1)
    assert not i1["converged"] and i1["mean_H"] < P.confidence  # argmax moved off the zero start
    s2, i2 = O.step(s1, H, identity_w(V), 0, 1, P, 1, 0.1)
    assert i2["converged"] and i2["final"] and s2.done and s2.steps_used == 2
    assert s2.committed.all() and np.array_equal(s2.canvas, toks)
    # a done canvas is left alone
    s3, i3 = O.step(s2, bf16(np.zeros((L, V))), identity_w(V), 0, 2, P, 1, 0.1)
    assert i3["skipped"] and np.array_equal(s3.canvas, s2.canvas)
    # argmax all zero from the start: stable at the first step, converges at once
    s0, i0 = O.step(st, peaked_rows(L, V, np.zeros(L, dtype=int)), identity_w(V), 0, 0, P, 1, 0.1)
    assert i0["converged"] and s0.steps_used == 1 and np.all(s0.canvas == 0)
    # stability threshold 2 needs two unchanged steps
    P2 = O.Params(N=8, stability_threshold=2)
    t1, _ = O.step(st, H, identity_w(V), 0, 0, P2, 1, 0.1)
    t2, j2 = O.step(t1, H, identity_w(V), 0, 1, P2, 1, 0.1)
    t3, j3 = O.step(t2, H, identity_w(V), 0, 2, P2, 1, 0.1)
    assert not j2["converged"] and j3["converged"] and t3.steps_used == 3


def test_convergence_needs_mean_entropy_strictly_below_confidence():
    L, V = 4, 4
    st = O.init_block(O.new_state(L, L), 0, L, V, seed=2)
    H = bf16(np.zeros((L, V)))                     # mean entropy = ln 4
    P = O.Params(N=8, confidence=float(np.float32(math.log(4))))
    s1, i1 = O.step(st, H, identity_w(V), 0, 0, P, 2, 0.1)   # argmax all 0: stable at once
    assert i1["mean_H"] >= P.confidence and not i1["converged"]
    P_hi = O.Params(N=8, confidence=1.0 * np.nextafter(np.float32(math.log(4)), np.float32(2)))
    _, i2 = O.step(st, H, identity_w(V), 0, 0, P_hi, 2, 0.1)
    assert i2["converged"]


def test_last_step_commits_everything_and_final_emit():
    L, V = 6, 32
    rng = np.random.default_rng(10)
    P = O.Params(N=3)
    st = O.init_block(O.new_state(L, L), 0, L, V, seed=3)
    H = bf16(rng.standard_normal((L, V)) * 0.3)
    s, info = O.step(st, H, identity_w(V), 0, 2, P, 3, 0.1)
    assert info["final"] and s.committed.all() and s.done and s.steps_used == 3
    assert np.array_equal(s.canvas, info["stats"]["token"])
    Pa = O.Params(N=3, final_emit=1)
    sa, ia = O.step(st, H, identity_w(V), 0, 2, Pa, 3, 0.1)
    assert np.array_equal(sa.canvas, ia["stats"]["argmax"])


def _run_tiny(freeze, seed=0, B=2, blocks=2):
    from uniform_state_discrete_step_amd.inputs import WORKLOADS, make_workload_arrays, shrink
    wl = shrink(WORKLOADS["tiny"], B=B, G=16 * blocks, freeze=freeze,
                seeds=tuple(range(seed, seed + B)), bounds=(0.1, 0.3)[:B])
    W, Hs = make_workload_arrays(wl, threads=1)
    P = O.Params(N=wl.N, freeze=freeze)
    log = []
    O.run(Hs, W, wl.G, P, wl.seeds, wl.bounds,
          on_step=lambda b, s, c, before, after, info: log.append((b, s, c, before, after, info)))
    return wl, log


def test_sticky_run_invariants():
    wl, log = _run_tiny(freeze=1)
    L = wl.L
    for b, s, c, before, after, info in log:
        if info.get("skipped"):
            continue
        blk = slice(b * L, (b + 1) * L)
        # earlier blocks never change
        assert np.array_equal(before.canvas[:b * L], after.canvas[:b * L])
        assert np.all(after.committed[:b * L] == 1)
        # committed positions are monotone and keep their tokens
        was = before.committed[blk] == 1
        assert np.all(after.committed[blk][was] == 1)
        assert np.array_equal(after.canvas[blk][was], before.canvas[blk][was])
        assert np.all((after.canvas[blk] >= 0) & (after.canvas[blk] < wl.V))
        if info["final"]:
            assert after.done and after.committed[blk].all()
        else:
            newly = (after.committed[blk] == 1) & ~was
            assert newly.sum() >= 1 or was.all()
            # newly committed positions hold their sampled tokens
            assert np.array_equal(after.canvas[blk][newly], info["stats"]["token"][newly])
            # the accepted set is downward closed in (entropy, position) order
            ranks = [info["accepted"][p] for p in info["order"]]
            assert ranks == sorted(ranks, reverse=True)
    # every block ran all its steps (the random stand-in never converges)
    finals = [(b, c) for b, s, c, _, _, info in log if info.get("final")]
    assert sorted(finals) == [(b, c) for b in range(wl.blocks) for c in range(wl.B)]


def test_stateless_mode_reranks_every_position():
    wl, log = _run_tiny(freeze=0, B=1, blocks=1)
    saw_reopen = False
    for b, s, c, before, after, info in log:
        if info["final"]:
            assert after.committed.all()
            assert np.array_equal(after.canvas, info["stats"]["token"])
            continue
        assert np.array_equal(after.committed == 1, info["accepted"])
        saw_reopen |= bool(np.any((before.committed == 1) & (after.committed == 0)))
    assert saw_reopen


def test_schedule_restarts_per_block_and_blocks_start_uniform():
    wl, log = _run_tiny(freeze=1, B=1, blocks=2)
    Ts = {(b, s): info["T"] for b, s, c, _, _, info in log}
    assert Ts[(0, 0)] == Ts[(1, 0)] == 0.8
    b1_first = [before for b, s, c, before, _, _ in log if (b, s) == (1, 0)][0]
    p_abs = np.arange(wl.L, 2 * wl.L)
    assert np.array_equal(b1_first.canvas[p_abs], O.init_token(wl.seeds[0], p_abs, 1, wl.V))
    assert np.all(b1_first.committed[p_abs] == 0)


def test_step_is_deterministic_and_resumable():
    wl, log = _run_tiny(freeze=1, B=1, blocks=1)
    from uniform_state_discrete_step_amd.inputs import make_workload_arrays
    W, Hs = make_workload_arrays(wl, threads=1)
    P = O.Params(N=wl.N)
    # resume from the saved state after step 3 and replay the rest
    st = log[3][4]
    for s in range(4, wl.N):
        st, _ = O.step(st, Hs[0, s, 0], W, 0, s, P, wl.seeds[0], wl.bounds[0])
    final = log[-1][4]
    assert np.array_equal(st.canvas, final.canvas) and st.steps_used == final.steps_used


@pytest.mark.parametrize("bound", [0.0, 0.1, 1.0])
def test_more_budget_commits_faster(bound):
    """A larger bound never leaves more positions open after the same first step."""
    L, V = 32, 64
    rng = np.random.default_rng(11)
    H = bf16(rng.standard_normal((L, V)) * rng.uniform(0.1, 8, size=(L, 1)))
    st = O.init_block(O.new_state(L, L), 0, L, V, seed=5)
    P = O.Params(N=8)
    s_lo, _ = O.step(st, H, identity_w(V), 0, 0, P, 5, bound)
    s_hi, _ = O.step(st, H, identity_w(V), 0, 0, P, 5, bound + 0.5)
    assert s_hi.committed.sum() >= s_lo.committed.sum()
