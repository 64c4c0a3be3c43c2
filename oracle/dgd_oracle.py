"""Plain CPU oracle of the uniform-state discrete diffusion denoising step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library; both sides receive the
same seeded inputs and are compared output by output.

What one step computes, for every canvas independently (sources are the four
pages this work follows; citations give page and section):

1. Temperature.  The annotated DiffusionGemma walkthrough ("Sampling", "Apply
   temperature") anneals linearly, t_i = t_max + (i/N)(t_min - t_max) for
   i = 0..N-1, and divides the logits by t_i.  The ComfyUI node page ("Inputs",
   t_min / t_max rows) writes the same schedule as T = t_min + (t_max - t_min) t
   with t = (N - i)/N, so t_min itself is never applied.
2. Logits.  z = H W_vocab^T with the tied embedding table as unembedding
   (walkthrough, "Complete DiffusionGemma model"; TensorSharp doc, "2. Forward
   graph": tied lm-head).  Computed here in float64 from the bf16 inputs.
   Optionally the model's tail around it: the output RMSNorm
   h = w x sqrt(d) / (||x|| + eps), rounded to bfloat16, before the
   projection, and the softcap c tanh(z / c) after it (walkthrough, "RMSNorm"
   and "Logit Softcapping").
3. Entropy in nats, H(p) = -sum_v p_v log p_v (walkthrough, "Compute entropy";
   node page, entropy_bound row: natural-log entropy).  float64, then rounded
   to float32: that float32 value is the position's entropy in every later
   decision.
4. Argmax of the tempered logits (walkthrough, "Check for early stopping");
   the first index wins ties.
5. Sampling.  The pages draw from the tempered categorical; this oracle draws
   by Gumbel-max: y_v = x_v + g_v, g = -ln(-ln u), token = first argmax of y.
   u comes from a Philox4x32-10 word (Salmon, Moraes, Dror, Shaw, "Parallel
   Random Numbers: As Easy as 1, 2, 3", SC'11) with key = the 64-bit seed and
   counter (v >> 2, p_abs, gstep, 0); word v & 3 is used and
   u = ((w >> 9) + 0.5) * 2^-23.
6. Early stop (walkthrough, "Check for early stopping"; TensorSharp doc,
   "3. Sampler contract"): the canvas has converged when its mean per-position
   entropy is below confidence_threshold AND the argmax canvas has been
   unchanged for stability_threshold consecutive steps (the argmax before the
   first step is all zeros, the argmax of the walkthrough's uniform starting
   logits).  A block ends on convergence or after N steps, and then every
   position still open takes its sample (or its argmax, when asked).
7. Commit (walkthrough, "Keep a low-entropy prefix and renoise the rest"):
   sort the eligible positions by entropy (ties by position), accept rank r
   when the exclusive running sum of the entropies before it is <= the bound,
   i.e. the largest prefix ending at k with sum_{j<k} H_(j) <= entropy_bound.
   Accepted positions take their sample; every other eligible position is
   re-noised to a uniform token (Philox word 0 of counter (0, p_abs, gstep, 1),
   token = (w * V) >> 32).  In the default sticky mode (freeze=1) committed
   positions stay frozen and leave the ranking, as the ComfyUI pack describes
   ("What it is": the most certain positions freeze into place, the rest are
   re-noised); freeze=0 re-ranks every position each step as the walkthrough's
   loop does.
8. A new block starts from uniform tokens (Philox word 0 of counter
   (0, p_abs, block, 2)); earlier blocks are never touched; the schedule
   restarts for each block (node page, gen_length row).
11. A 4-bit table (the pages run quantized checkpoints: INT4 W4A16 and
   GGUF K-quant files, ComfyUI pack "What works today" and "Downloads"):
   groups of 32 hidden elements of a row share a bf16 scale s and minimum m,
   each element keeps a 4-bit code q, and the step uses the table
   w = bf16(fp32(s) * q + fp32(m)) (one float32 rounding, then nearest-even
   to bf16).  Everything after the table is unchanged.
10. Typed decisions (TensorSharp doc, "1. Origin and intent": label
   probabilities read from a canvas in one denoising step through a sparse
   output projection): logits of a given list of label ids only, and their
   probabilities normalised over that list.
9. Self-conditioning input for the next forward (walkthrough, "Complete
   DiffusionGemma model" and "Denoise, stage, commit, and generate": the
   decoder receives the previous step's tempered probabilities P and forms
   (P @ W_embed) * sqrt(hidden), with P cast to the model dtype; TensorSharp
   doc, self-conditioning top-K cutoff, default 32): the K most probable
   tokens of each position (ties by lower id) with their exact probabilities
   (not renormalised), and the embedding sum over those K only.

All functions below are deliberately direct: one pass per definition, no
blocking, fusion or streaming.  Every function is pinned by the CPU tests.

Parity unpinned: three readings cannot be pinned to the pages because the
pages disagree; the tests pin the oracle to the readings, not the readings to
the pages.  They are the sticky freeze of committed positions (point 7; the
walkthrough's loop re-ranks every position), what `confidence` measures
(point 6; the node page calls it a probability, the TensorSharp doc a mean
entropy), and the end of a block (point 6; the walkthrough returns a sample on
convergence and has no exit after N steps).
"""
from __future__ import annotations

import dataclasses

import numpy as np

MASK32 = 0xFFFFFFFF

# Philox4x32 constants from Salmon et al. (SC'11): round multipliers and the
# Weyl-sequence key increments.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10

TAG_GUMBEL = 0
TAG_RENOISE = 1
TAG_INIT = 2


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# 1. temperature
# ----------------------------------------------------------------------------
def temperature(step: int, N: int, t_min: float, t_max: float) -> float:
    """t_step = t_max + (step / N) (t_min - t_max), in float64."""
    return float(t_max) + (float(step) / float(N)) * (float(t_min) - float(t_max))


# ----------------------------------------------------------------------------
# 2. logits
# ----------------------------------------------------------------------------
def projection(H_bits: np.ndarray, W_bits: np.ndarray, v_chunk: int = 16384,
               W64: np.ndarray = None) -> np.ndarray:
    """z[r, v] = sum_k H[r, k] W[v, k] in float64 (products of bf16 are exact).

    ``W64`` may carry W already widened to float64 (same values) to avoid
    re-widening the table on every call.
    """
    H = bf16_to_f64(H_bits)
    rows, V = H.shape[0], W_bits.shape[0]
    z = np.empty((rows, V), dtype=np.float64)
    for v0 in range(0, V, v_chunk):
        v1 = min(V, v0 + v_chunk)
        Wc = W64[v0:v1] if W64 is not None else bf16_to_f64(W_bits[v0:v1])
        z[:, v0:v1] = H @ Wc.T
    return z


# ----------------------------------------------------------------------------
# 2b. the lm-head tail: output norm before the projection, logit softcap after
#     (walkthrough, "RMSNorm", "Logit Softcapping" and the end of the model's
#     forward: rms(x, model_norm), then x @ W_embed^T, then the tanh cap;
#     TensorSharp doc, "2. Forward graph": output norm -> tied lm-head ->
#     final logit softcap)
# ----------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, rounded once to nearest, ties to even.

    Each value is rounded at the spacing of bfloat16 in its binade (8
    significant bits; the subnormal spacing 2^-133 below 2^-126): dividing by
    a power of two is exact and numpy's rint rounds half to even.  Finite
    inputs inside the bfloat16 range only.
    """
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)                                  # |x| = f 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, -126)                         # exponent of the binade
    spacing = np.ldexp(1.0, e - 7)
    q = np.rint(x / spacing) * spacing                  # exactly a bfloat16 value
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rms_norm(H_bits: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """h = w * x * sqrt(d) / (||x||_2 + eps) per row, in float64, rounded to
    bfloat16 (the model casts the normalized state back to its dtype before
    the projection).  H_bits [rows, d], w_bits [d]: bf16 bits."""
    x = bf16_to_f64(H_bits)
    w = bf16_to_f64(w_bits)
    d = x.shape[-1]
    norm = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return round_bf16(w * x * np.sqrt(float(d)) / (norm + float(eps)))


def softcap(z: np.ndarray, c: float) -> np.ndarray:
    """c * tanh(z / c); c = 0 means no cap."""
    z = np.asarray(z, dtype=np.float64)
    return z if c == 0 else float(c) * np.tanh(z / float(c))


# ----------------------------------------------------------------------------
# random numbers
# ----------------------------------------------------------------------------
def seed_key(seed: int):
    """64-bit seed -> Philox key (low word, high word)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on (broadcastable) uint32 counter words.

    One round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 as 64-bit products;
    the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).  The key is
    advanced by the Weyl increments between rounds.
    """
    u64 = np.uint64
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = np.asarray(k0, dtype=np.uint64)
    k1 = np.asarray(k1, dtype=np.uint64)
    m32 = u64(MASK32)
    for r in range(PHILOX_ROUNDS):
        if r > 0:
            k0 = (k0 + u64(PHILOX_W0)) & m32
            k1 = (k1 + u64(PHILOX_W1)) & m32
        p0 = u64(PHILOX_M0) * c0
        p1 = u64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> u64(32), p0 & m32
        hi1, lo1 = p1 >> u64(32), p1 & m32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def uniform_from_word(w) -> np.ndarray:
    """u = ((w >> 9) + 1/2) 2^-23, the midpoint of one of 2^23 equal cells of (0, 1)."""
    k = np.asarray(w, dtype=np.uint32) >> np.uint32(9)
    return (k.astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_from_word(w) -> np.ndarray:
    """Standard Gumbel variate g = -ln(-ln u) in float64."""
    return -np.log(-np.log(uniform_from_word(w)))


def uniform_token(w, V: int) -> np.ndarray:
    """Map a 32-bit word onto {0..V-1} by the high half of w * V."""
    return ((np.asarray(w, dtype=np.uint64) * np.uint64(V)) >> np.uint64(32)).astype(np.int64)


def gumbel_words(seed: int, p_abs: np.ndarray, gstep: int, V: int) -> np.ndarray:
    """Word for (row, v): Philox(key, (v >> 2, p_abs, gstep, 0))[v & 3]; [rows, V]."""
    k0, k1 = seed_key(seed)
    p_abs = np.asarray(p_abs, dtype=np.uint64).reshape(-1, 1)
    groups = (V + 3) // 4
    c0 = np.arange(groups, dtype=np.uint64).reshape(1, -1)
    w = philox4x32_10(c0, p_abs, np.uint64(gstep), np.uint64(TAG_GUMBEL), k0, k1)
    words = np.stack(w, axis=-1).reshape(p_abs.shape[0], groups * 4)
    return words[:, :V]


def gumbel_at(seed: int, p_abs, gstep: int, v) -> np.ndarray:
    """The Gumbel noise g of given (row, id) pairs: word v & 3 of
    Philox(key, (v >> 2, p_abs, gstep, 0)), as in gumbel_words, for arrays
    p_abs and v of one shape (broadcast)."""
    k0, k1 = seed_key(seed)
    p_abs, v = np.broadcast_arrays(np.asarray(p_abs, dtype=np.uint64), np.asarray(v, dtype=np.uint64))
    w = np.stack(philox4x32_10(v >> np.uint64(2), p_abs, np.uint64(gstep), np.uint64(TAG_GUMBEL),
                               k0, k1), axis=-1)
    word = np.take_along_axis(w, (v & np.uint64(3)).astype(np.int64)[..., None], axis=-1)[..., 0]
    return gumbel_from_word(word)


def renoise_token(seed: int, p_abs, gstep: int, V: int) -> np.ndarray:
    k0, k1 = seed_key(seed)
    w = philox4x32_10(np.uint64(0), np.asarray(p_abs, dtype=np.uint64), np.uint64(gstep),
                      np.uint64(TAG_RENOISE), k0, k1)[0]
    return uniform_token(w, V)


def init_token(seed: int, p_abs, block: int, V: int) -> np.ndarray:
    k0, k1 = seed_key(seed)
    w = philox4x32_10(np.uint64(0), np.asarray(p_abs, dtype=np.uint64), np.uint64(block),
                      np.uint64(TAG_INIT), k0, k1)[0]
    return uniform_token(w, V)


# ----------------------------------------------------------------------------
# 3-5. per-position statistics of one step
# ----------------------------------------------------------------------------
def position_stats(z: np.ndarray, T: float, seed: int, p_abs, gstep: int) -> dict:
    """Everything one step derives from the logits of a set of positions.

    z: float64 logits [rows, V]; T: the step's temperature; p_abs: absolute
    position of each row.  Returns float32 entropies, argmax, sampled token,
    the top two Gumbel-perturbed values and the top-two logit gap.
    """
    z = np.asarray(z, dtype=np.float64)
    rows, V = z.shape
    x = z / T                                            # tempered logits

    argmax = np.argmax(x, axis=1)                        # first maximum
    xs = np.sort(x, axis=1)
    x_gap = xs[:, -1] - xs[:, -2] if V > 1 else np.full(rows, np.inf)

    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    S = e.sum(axis=1, keepdims=True)
    lse = m + np.log(S)
    p = e / S
    H = -(p * (x - lse)).sum(axis=1)                     # nats, float64
    H32 = H.astype(np.float32)

    g = gumbel_from_word(gumbel_words(seed, p_abs, gstep, V))
    y = x + g
    tok = np.argmax(y, axis=1)
    r_idx = np.arange(rows)
    y1 = y[r_idx, tok]
    if V > 1:
        y_rest = y.copy()
        y_rest[r_idx, tok] = -np.inf
        y2 = y_rest.max(axis=1)
    else:
        y2 = np.full(rows, -np.inf)
    return {
        "entropy64": H,
        "entropy": H32,
        "argmax": argmax.astype(np.int64),
        "argmax_gap": x_gap,
        "token": tok.astype(np.int64),
        "y1": y1,
        "y2": y2,
        "gap": y1 - y2,
    }


# ----------------------------------------------------------------------------
# 9. self-conditioning: top-K of the tempered distribution, and its embedding
# ----------------------------------------------------------------------------
def sc_topk(z: np.ndarray, T: float, K: int):
    """The K most probable tokens of softmax(z / T) per row.

    Order: probability descending, then id ascending (equal logits give equal
    probabilities; the lower id comes first).  Returns (prob float64 [rows, K],
    ids int64 [rows, K], x float64 [rows, V] the tempered logits, for bands).
    """
    x = np.asarray(z, dtype=np.float64) / T
    rows, V = x.shape
    ids = np.empty((rows, K), dtype=np.int64)
    for r in range(rows):
        order = np.lexsort((np.arange(V), -x[r]))       # last key is primary
        ids[r] = order[:K]
    m = x.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(x - m).sum(axis=1, keepdims=True))
    prob = np.exp(np.take_along_axis(x, ids, axis=1) - lse)
    return prob, ids, x


def sc_embed(prob: np.ndarray, ids: np.ndarray, W_bits: np.ndarray, scale: float) -> np.ndarray:
    """scale * sum_j bf16(prob_j) * E[id_j] per row, float64, rounded once to
    bfloat16.  prob [rows, K] (float32 or float64), ids [rows, K], W_bits the
    tied table [V, d] as bf16 bits; returns bf16 bits [rows, d]."""
    p16 = bf16_to_f64(round_bf16(np.asarray(prob, dtype=np.float64)))
    E = bf16_to_f64(W_bits[np.asarray(ids, dtype=np.int64)])     # [rows, K, d]
    return round_bf16(float(scale) * (p16[:, :, None] * E).sum(axis=1))


# ----------------------------------------------------------------------------
# 11. 4-bit table: dequantization
# ----------------------------------------------------------------------------
Q4_GROUP = 32


def dequant_q4(codes: np.ndarray, scales: np.ndarray, mins: np.ndarray) -> np.ndarray:
    """The bf16 table a 4-bit table stands for.

    codes uint8 [V, d/2]: element 2i in the low nibble of byte i, element
    2i + 1 in the high nibble; scales, mins bf16 bits [V, d/32].  Each value
    is s * q + m in float32 (the product of a bf16 and a 4-bit integer is
    exact in float32, so one rounding), then rounded to bf16.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    V, half = codes.shape
    d = 2 * half
    q = np.empty((V, d), dtype=np.float32)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    s = np.repeat(bf16_to_f64(scales).astype(np.float32), Q4_GROUP, axis=1)
    m = np.repeat(bf16_to_f64(mins).astype(np.float32), Q4_GROUP, axis=1)
    w32 = s * q + m                               # float32: exact product, one rounding
    return round_bf16_f32(w32)


def round_bf16_f32(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, nearest with ties to even, on the bit
    pattern: add 0x7FFF plus the lowest kept bit, drop the low 16 bits (finite
    inputs).  The same rounding as round_bf16 for values float32 holds."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)       # finite: the sum stays below 2^32
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# 10. sparse label read
# ----------------------------------------------------------------------------
def label_probs(H_bits: np.ndarray, W_bits: np.ndarray, labels, T: float, softcap_c: float = 0.0):
    """Logits of the label ids only, z[r, l] = H[r] . W[labels[l]] (then the
    softcap c tanh(z / c) when c > 0), and p[r, l] = softmax over the labels
    of z / T.  Returns (z float64 [rows, n], p float64 [rows, n])."""
    labels = np.asarray(labels, dtype=np.int64)
    z = softcap(projection(H_bits, W_bits[labels]), softcap_c)
    x = z / float(T)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return z, e / e.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# 7. commit rule
# ----------------------------------------------------------------------------
def commit_rule(entropy32: np.ndarray, eligible: np.ndarray, bound: float):
    """Accepted subset of the eligible positions under the entropy budget.

    Eligible positions are ranked by (entropy, position); rank r is accepted
    when the float64 sum of the entropies ranked before it is <= bound.
    Returns (accepted mask, ranked positions, exclusive sums).
    """
    h = np.asarray(entropy32, dtype=np.float32)
    n = h.shape[0]
    candidates = [p for p in range(n) if eligible[p]]
    order = sorted(candidates, key=lambda p: (float(h[p]), p))
    accepted = np.zeros(n, dtype=bool)
    sums = []
    running = 0.0
    for p in order:
        sums.append(running)
        if running <= float(bound):
            accepted[p] = True
        running += float(h[p])
    return accepted, order, sums


# ----------------------------------------------------------------------------
# 6-8. one step of one canvas, blocks, whole runs
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Params:
    N: int = 48
    t_min: float = 0.4
    t_max: float = 0.8
    confidence: float = 0.005
    stability_threshold: int = 1
    freeze: int = 1
    final_emit: int = 0


@dataclasses.dataclass
class CanvasState:
    canvas: np.ndarray        # int64 [G]
    committed: np.ndarray     # uint8 [G]
    prev_argmax: np.ndarray   # int64 [L]
    stable_count: int = 0
    done: bool = False
    steps_used: int = 0

    def copy(self) -> "CanvasState":
        return CanvasState(self.canvas.copy(), self.committed.copy(), self.prev_argmax.copy(),
                           self.stable_count, self.done, self.steps_used)


def new_state(G: int, L: int) -> CanvasState:
    return CanvasState(np.zeros(G, dtype=np.int64), np.zeros(G, dtype=np.uint8),
                       np.zeros(L, dtype=np.int64))


def init_block(state: CanvasState, block: int, L: int, V: int, seed: int) -> CanvasState:
    """Uniform tokens over block ``block``; its positions open; fresh step state."""
    s = state.copy()
    p_abs = block * L + np.arange(L)
    s.canvas[p_abs] = init_token(seed, p_abs, block, V)
    s.committed[p_abs] = 0
    s.prev_argmax[:] = 0
    s.stable_count = 0
    s.done = False
    s.steps_used = 0
    return s


def step_from_stats(state: CanvasState, stats: dict, block: int, step: int, L: int, V: int,
                    params: Params, seed: int, bound: float):
    """Convergence, commit, sampling write and re-noise, given a step's statistics."""
    s = state.copy()
    info = {"stats": stats, "skipped": state.done}
    if state.done:
        return s, info
    base = block * L
    p_abs = base + np.arange(L)
    gstep = block * params.N + step
    H = stats["entropy"]
    a = stats["argmax"]

    mean_H = sum(float(h) for h in H) / L
    stable = bool(np.all(a == state.prev_argmax))
    s.stable_count = state.stable_count + 1 if stable else 0
    converged = (mean_H < float(np.float32(params.confidence))
                 and s.stable_count >= params.stability_threshold)
    final = converged or step == params.N - 1
    info.update(mean_H=mean_H, converged=converged, final=final)

    open_ = state.committed[p_abs] == 0
    emit = a if params.final_emit else stats["token"]
    if final:
        take = np.ones(L, dtype=bool) if params.freeze == 0 else open_
        s.canvas[p_abs[take]] = emit[take]
        s.committed[p_abs] = 1
        s.done = True
        s.steps_used = step + 1
        info.update(accepted=take, order=None, sums=None, renoised=np.zeros(L, dtype=bool))
    else:
        eligible = open_ if params.freeze else np.ones(L, dtype=bool)
        accepted, order, sums = commit_rule(H, eligible, float(np.float32(bound)))
        renoised = eligible & ~accepted
        s.canvas[p_abs[accepted]] = stats["token"][accepted]
        s.committed[p_abs[accepted]] = 1
        s.canvas[p_abs[renoised]] = renoise_token(seed, p_abs[renoised], gstep, V)
        s.committed[p_abs[renoised]] = 0
        s.steps_used = step + 1
        info.update(accepted=accepted, order=order, sums=sums, renoised=renoised)
    s.prev_argmax = a.astype(np.int64).copy()
    return s, info


@dataclasses.dataclass
class Tail:
    """The optional lm-head tail: output-norm weights (bf16 bits [d], None =
    no norm), its epsilon, and the softcap c (0 = no cap)."""
    norm_weight: np.ndarray = None
    norm_eps: float = 0.0
    softcap: float = 0.0


def logits(H_bits: np.ndarray, W_bits: np.ndarray, tail: Tail = None, W64=None) -> np.ndarray:
    """The step's logits: [output norm ->] projection [-> softcap]."""
    if tail is not None and tail.norm_weight is not None:
        H_bits = rms_norm(H_bits, tail.norm_weight, tail.norm_eps)
    z = projection(H_bits, W_bits, W64=W64)
    if tail is not None and tail.softcap:
        z = softcap(z, tail.softcap)
    return z


def step(state: CanvasState, H_bits: np.ndarray, W_bits: np.ndarray, block: int, step_idx: int,
         params: Params, seed: int, bound: float, W64: np.ndarray = None, tail: Tail = None):
    """One denoising step of one canvas: H_bits [L, d] bf16 bits, W_bits [V, d]."""
    L = H_bits.shape[0]
    V = W_bits.shape[0]
    if state.done:
        return state.copy(), {"skipped": True}
    T = temperature(step_idx, params.N, params.t_min, params.t_max)
    z = logits(H_bits, W_bits, tail, W64=W64)
    stats = position_stats(z, T, seed, block * L + np.arange(L), block * params.N + step_idx)
    new, info = step_from_stats(state, stats, block, step_idx, L, V, params, seed, bound)
    info["T"] = T
    info["z"] = z
    return new, info


def run(H_steps: np.ndarray, W_bits: np.ndarray, G: int, params: Params, seeds, bounds,
        on_step=None, tail: Tail = None):
    """Whole generation for every canvas.  H_steps: [G/L, N, B, L, d] bf16 bits."""
    n_blocks, N, B, L, _ = H_steps.shape
    V = W_bits.shape[0]
    assert N == params.N and n_blocks * L == G
    states = [new_state(G, L) for _ in range(B)]
    for b in range(n_blocks):
        for c in range(B):
            states[c] = init_block(states[c], b, L, V, seeds[c])
        for s_idx in range(N):
            for c in range(B):
                before = states[c]
                states[c], info = step(before, H_steps[b, s_idx, c], W_bits, b, s_idx, params,
                                       seeds[c], bounds[c], tail=tail)
                if on_step is not None:
                    on_step(b, s_idx, c, before, states[c], info)
            if all(st.done for st in states):
                break
    return states


def gumbel_extremes():
    """(G_MIN, G_MAX): the Gumbel values of the smallest and largest possible u."""
    lo = float(gumbel_from_word(np.uint32(0)))
    hi = float(gumbel_from_word(np.uint32(MASK32)))
    return lo, hi


__all__ = [
    "Params", "CanvasState", "new_state", "init_block", "step", "step_from_stats", "run",
    "temperature", "projection", "position_stats", "commit_rule", "philox4x32_10",
    "seed_key", "uniform_from_word", "gumbel_from_word", "uniform_token", "gumbel_words",
    "renoise_token", "init_token", "bf16_to_f64", "gumbel_extremes",
]

