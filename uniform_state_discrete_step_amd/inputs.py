"""Seeded synthetic workloads for the denoising step.

This module only draws numbers: it holds none of the step's arithmetic (no
projection, temperature, entropy, sampling or commit rule).  Both the CPU
oracle and the HIP path receive the exact bytes produced here, so every
comparison between the two starts from identical inputs.

Recipe (the transformer that would produce the canvas hidden states is
replaced by seeded Gaussian rows, following the annotated DiffusionGemma
walkthrough, section "Setup + Load Model", where the unembedding matrix is the
tied [V x d] embedding table):

* W_vocab [V, d]: standard normal scaled by 1/sqrt(d) in float32, rounded to
  bfloat16 (round-to-nearest-even).  Rows are drawn in chunks of
  ``W_CHUNK_ROWS``; chunk ``j`` uses ``numpy.random.default_rng([cfg_seed, 0,
  j])`` so the matrix can be generated in parallel and still be bit-identical.
* H for (canvas c, block b, step s) [L, d]: generator
  ``default_rng([cfg_seed, 1, c, b*N + s])``; first L log-uniform row scales
  ``r = exp(U(ln lo, ln hi))``, then an [L, d] float32 standard normal; the row
  is ``r * z`` rounded to bfloat16.
* A 4-bit table (for runs of the quantized stream): the bf16 table above,
  quantized group by group (32 hidden elements): scale = bf16((max - min)/15)
  (1 if the group is constant), min = bf16(min), codes = the nearest of
  0..15 to (w - min) / scale.  Only a way to obtain realistic codes.
* Output-norm weights [d] (only for runs with the lm-head tail): generator
  ``default_rng([cfg_seed, 2])``, log-uniform per channel in [lo, hi] (default
  [0.5, 8]), rounded to bfloat16.  The walkthrough prints no trained values.

bfloat16 values are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

W_CHUNK_ROWS = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the step (shapes, knobs and seeds)."""

    name: str
    B: int                 # canvases denoised together
    L: int                 # canvas (block) length
    G: int                 # generated length per canvas (a multiple of L)
    V: int                 # vocabulary size
    d: int                 # hidden size
    N: int                 # num_inference_steps per block
    cfg_seed: int          # seeds the W / H draws
    seeds: tuple           # per-canvas sampler seed (uint64)
    bounds: tuple          # per-canvas entropy_bound, nats
    scale: tuple = (0.1, 10.0)   # log-uniform row-scale range of H
    t_min: float = 0.4
    t_max: float = 0.8
    confidence: float = 0.005
    stability_threshold: int = 1
    freeze: int = 1
    final_emit: int = 0

    @property
    def blocks(self) -> int:
        return self.G // self.L

    @property
    def rows(self) -> int:
        return self.B * self.L


def _batched_bounds(B: int) -> tuple:
    choices = (0.05, 0.1, 0.2)
    return tuple(choices[c % 3] for c in range(B))


WORKLOADS = {
    "tiny": Workload("tiny", B=1, L=16, G=16, V=1024, d=64, N=8, cfg_seed=0,
                     seeds=(0,), bounds=(0.1,)),
    "small_vocab": Workload("small_vocab", B=1, L=256, G=256, V=32768, d=1024, N=48,
                            cfg_seed=1, seeds=(1,), bounds=(0.1,)),
    "gemma_vocab": Workload("gemma_vocab", B=1, L=256, G=256, V=262144, d=2816, N=48,
                            cfg_seed=2, seeds=(2,), bounds=(0.1,)),
    "batched": Workload("batched", B=8, L=256, G=256, V=262144, d=2816, N=48,
                        cfg_seed=10, seeds=tuple(range(10, 18)), bounds=_batched_bounds(8)),
    "multi_block": Workload("multi_block", B=1, L=256, G=2048, V=262144, d=2816, N=48,
                            cfg_seed=3, seeds=(3,), bounds=(0.1,), scale=(1.0, 30.0)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs only: u + 0x7FFF + lsb cannot wrap below 2^32
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_w(V: int, d: int, cfg_seed: int, threads: int = 8) -> np.ndarray:
    """W_vocab [V, d] as bfloat16 bits (see module docstring)."""
    out = np.empty((V, d), dtype=np.uint16)
    inv = np.float32(1.0 / math.sqrt(d))

    def chunk(j: int) -> None:
        r0 = j * W_CHUNK_ROWS
        r1 = min(V, r0 + W_CHUNK_ROWS)
        rng = np.random.default_rng([cfg_seed, 0, j])
        z = rng.standard_normal((r1 - r0, d), dtype=np.float32)
        out[r0:r1] = f32_to_bf16_bits(z * inv)

    n_chunks = (V + W_CHUNK_ROWS - 1) // W_CHUNK_ROWS
    if n_chunks == 1 or threads <= 1:
        for j in range(n_chunks):
            chunk(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(chunk, range(n_chunks)))
    return out


def make_h(L: int, d: int, cfg_seed: int, canvas: int, gstep: int,
           scale=(0.1, 10.0)) -> np.ndarray:
    """Hidden states of one canvas at global step ``gstep`` as bf16 bits [L, d]."""
    rng = np.random.default_rng([cfg_seed, 1, canvas, gstep])
    lo, hi = scale
    log_r = rng.uniform(math.log(lo), math.log(hi), size=L)
    z = rng.standard_normal((L, d), dtype=np.float32)
    r = np.exp(log_r).astype(np.float32)
    return f32_to_bf16_bits(z * r[:, None])


def make_h_steps(wl: Workload, threads: int = 8) -> np.ndarray:
    """All hidden states of a run, [G/L, N, B, L, d] bf16 bits, contiguous."""
    out = np.empty((wl.blocks, wl.N, wl.B, wl.L, wl.d), dtype=np.uint16)
    jobs = [(b, s, c) for b in range(wl.blocks) for s in range(wl.N) for c in range(wl.B)]

    def one(job):
        b, s, c = job
        out[b, s, c] = make_h(wl.L, wl.d, wl.cfg_seed, c, b * wl.N + s, wl.scale)

    if threads <= 1 or len(jobs) < 4:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
    return out


def make_workload_arrays(wl: Workload, threads: int = 8):
    """(W [V, d], H_steps [G/L, N, B, L, d]) bf16 bits for a workload."""
    return make_w(wl.V, wl.d, wl.cfg_seed, threads), make_h_steps(wl, threads)


def shrink(wl: Workload, **kw) -> Workload:
    """Copy of a workload with some fields replaced (for edge-case tests)."""
    return dataclasses.replace(wl, **kw)


def make_norm_weight(d: int, cfg_seed: int, scale=(0.5, 8.0)) -> np.ndarray:
    """Output-norm weights [d] as bfloat16 bits (see module docstring)."""
    rng = np.random.default_rng([cfg_seed, 2])
    lo, hi = scale
    w = np.exp(rng.uniform(math.log(lo), math.log(hi), size=d)).astype(np.float32)
    return f32_to_bf16_bits(w)


def quantize_q4(W_bits: np.ndarray):
    """(codes uint8 [V, d/2], scales bf16 bits [V, d/32], mins bf16 bits [V, d/32])
    of a bf16 table (see module docstring); d must be a multiple of 32."""
    V, d = W_bits.shape
    w = bf16_bits_to_f32(W_bits).reshape(V, d // 32, 32)
    lo, hi = w.min(axis=2), w.max(axis=2)
    scale = np.where(hi > lo, (hi - lo) / np.float32(15.0), np.float32(1.0)).astype(np.float32)
    s_bits = f32_to_bf16_bits(scale)
    m_bits = f32_to_bf16_bits(lo)
    s = bf16_bits_to_f32(s_bits)[:, :, None]
    m = bf16_bits_to_f32(m_bits)[:, :, None]
    q = np.clip(np.rint((w - m) / s), 0, 15).astype(np.uint8).reshape(V, d)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s_bits, m_bits
