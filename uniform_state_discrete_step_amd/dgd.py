"""ctypes binding of libdgd.so (the HIP denoising-step library).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  The functions keep the C names of include/dgd.h and take torch
tensors (device memory and streams come from PyTorch); there is no fallback of
any kind, and calling into a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgd.so")
# the measurement build that records the projection's phase times
LIB_PHASE_PATH = os.path.join(_HERE, "libdgd_phase.so")
PHASE_WORKGROUPS, PHASE_SLOTS = 1024, 16

DGD_OK = 0
DGD_EINVAL = -1
DGD_EUNSUPPORTED = -2
DGD_EWORKSPACE = -3
DGD_EHIP = -4
DGD_MAX_CANVASES = 64
DGD_MAX_CANVAS_LEN = 4096

DGD_VOCAB_ROWS = 0
DGD_VOCAB_PACKED = 1
DGD_VOCAB_Q4 = 2
DGD_STATUS_OK = 0
DGD_STATUS_NONFINITE = 1

EXPORTED = ("dgd_state_bytes", "dgd_workspace_bytes", "dgd_init_block", "dgd_step", "dgd_run",
            "dgd_run_steps", "dgd_step_noalloc",
            "dgd_packed_vocab_bytes", "dgd_pack_vocab", "dgd_q4_vocab_bytes", "dgd_pack_vocab_q4",
            "dgd_sc_embed", "dgd_label_probs",
            "dgd_ceiling_hbm_read", "dgd_ceiling_mfma_bf16", "dgd_debug_philox",
            "dgd_debug_gumbel", "dgd_phase_times",
            "dgd_last_error")


class DgdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdgd error {code}: {msg}")
        self.code = code


class DgdParams(ctypes.Structure):
    _fields_ = [
        ("num_inference_steps", ctypes.c_int32),
        ("t_min", ctypes.c_float),
        ("t_max", ctypes.c_float),
        ("confidence", ctypes.c_float),
        ("stability_threshold", ctypes.c_int32),
        ("freeze", ctypes.c_int32),
        ("final_emit", ctypes.c_int32),
    ]


class DgdCtx(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("L", ctypes.c_int32), ("V", ctypes.c_int32),
        ("d", ctypes.c_int32), ("G", ctypes.c_int32),
        ("entropy_bound", ctypes.POINTER(ctypes.c_float)),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("state", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
        ("entropy", ctypes.c_void_p),
        ("argmax", ctypes.c_void_p),
        ("token", ctypes.c_void_p),
        ("gap", ctypes.c_void_p),
        ("logits", ctypes.c_void_p),
        ("commit_step", ctypes.c_void_p),
        ("k1_ms", ctypes.POINTER(ctypes.c_double)),
        ("k1_launches", ctypes.POINTER(ctypes.c_int32)),
        ("vocab_layout", ctypes.c_int32),
        ("norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("norm_h", ctypes.c_void_p),
        ("sc_topk", ctypes.c_int32),
        ("sc_prob", ctypes.c_void_p),
        ("sc_id", ctypes.c_void_p),
        ("sc_status", ctypes.c_void_p),
        ("tail_ms", ctypes.POINTER(ctypes.c_double)),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdgd.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.dgd_state_bytes.restype = ctypes.c_size_t
    lib.dgd_state_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.dgd_workspace_bytes.restype = ctypes.c_size_t
    lib.dgd_workspace_bytes.argtypes = [ctypes.c_int32] * 4
    lib.dgd_last_error.restype = ctypes.c_char_p
    lib.dgd_last_error.argtypes = []
    pp = ctypes.POINTER(DgdParams)
    pc = ctypes.POINTER(DgdCtx)
    pseed = ctypes.POINTER(ctypes.c_uint64)
    lib.dgd_init_block.restype = ctypes.c_int
    lib.dgd_init_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, pp, pseed, pc]
    lib.dgd_step.restype = ctypes.c_int
    lib.dgd_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_int32, ctypes.c_int32, pp, pseed, pc]
    lib.dgd_step_noalloc.restype = ctypes.c_int
    lib.dgd_step_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, pp, pseed, pc]
    lib.dgd_run.restype = ctypes.c_int
    lib.dgd_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                            pp, pseed, pc]
    lib.dgd_run_steps.restype = ctypes.c_int
    lib.dgd_run_steps.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, pp, pseed, pc]
    lib.dgd_packed_vocab_bytes.restype = ctypes.c_size_t
    lib.dgd_packed_vocab_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.dgd_pack_vocab.restype = ctypes.c_int
    lib.dgd_pack_vocab.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p]
    lib.dgd_q4_vocab_bytes.restype = ctypes.c_size_t
    lib.dgd_q4_vocab_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.dgd_pack_vocab_q4.restype = ctypes.c_int
    lib.dgd_pack_vocab_q4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p]
    lib.dgd_sc_embed.restype = ctypes.c_int
    lib.dgd_sc_embed.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    lib.dgd_label_probs.restype = ctypes.c_int
    lib.dgd_label_probs.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                    ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.dgd_ceiling_hbm_read.restype = ctypes.c_int
    lib.dgd_ceiling_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.dgd_ceiling_mfma_bf16.restype = ctypes.c_int
    lib.dgd_ceiling_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.dgd_debug_philox.restype = ctypes.c_int
    lib.dgd_debug_philox.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.dgd_debug_gumbel.restype = ctypes.c_int
    lib.dgd_debug_gumbel.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p]
    lib.dgd_phase_times.restype = ctypes.c_int
    lib.dgd_phase_times.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != DGD_OK:
        raise DgdError(rc, load_library().dgd_last_error().decode())


def make_params(N=48, t_min=0.4, t_max=0.8, confidence=0.005, stability_threshold=1, freeze=1,
                final_emit=0) -> DgdParams:
    return DgdParams(int(N), float(t_min), float(t_max), float(confidence),
                     int(stability_threshold), int(freeze), int(final_emit))


def _seeds(seeds) -> ctypes.Array:
    arr = np.asarray(seeds, dtype=np.uint64).reshape(-1)
    return (ctypes.c_uint64 * len(arr))(*[int(s) for s in arr])


def _ptr(t, dtype_size=None, device=True) -> int:
    if t is None:
        return None
    if device and not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtype_size is not None and t.element_size() != dtype_size:
        raise ValueError(f"expected {dtype_size}-byte elements, got {t.dtype}")
    return t.data_ptr()


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Context:
    """Shapes, per-canvas bounds, caller-owned scratch and state, optional outputs.

    Owns torch device tensors: ``workspace`` (uint8), ``state`` (int32 words, see
    ``state_views``) and the optional per-step outputs.
    """

    def __init__(self, B, L, V, d, G, bounds, device="cuda", outputs=True, logits=False,
                 commit_trace=False, vocab_layout=DGD_VOCAB_ROWS, norm_weight=None,
                 norm_eps=0.0, softcap=0.0, sc_topk=0, sc_status=False):
        """norm_weight: optional device int16[d] (bf16 bits) output-norm weights;
        when given, ``norm_h`` (int16[B*L*d]) receives the normalised rows each
        step.  softcap: the logit cap c (0 = none).  sc_topk: K > 0 allocates
        ``sc_prob`` (float32[B*L*K]) and ``sc_id`` (int32[B*L*K]), and with
        sc_status ``sc_status`` (int32[B*L])."""
        import torch
        lib = load_library()
        self.B, self.L, self.V, self.d, self.G = int(B), int(L), int(V), int(d), int(G)
        b = np.asarray(bounds, dtype=np.float32).reshape(-1)
        if b.shape[0] != self.B:
            raise ValueError("need one entropy bound per canvas")
        self._bounds = (ctypes.c_float * self.B)(*[float(x) for x in b])
        ws = lib.dgd_workspace_bytes(self.B, self.L, self.V, self.d)
        if ws == 0:
            raise ValueError(f"unsupported shape B={B} L={L} V={V} d={d}")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        sb = lib.dgd_state_bytes(self.B, self.L)
        self.state = torch.zeros(sb // 4, dtype=torch.int32, device=device)
        BL = self.B * self.L
        self.entropy = torch.empty(BL, dtype=torch.float32, device=device) if outputs else None
        self.argmax = torch.empty(BL, dtype=torch.int32, device=device) if outputs else None
        self.token = torch.empty(BL, dtype=torch.int32, device=device) if outputs else None
        self.gap = torch.empty(BL, dtype=torch.float32, device=device) if outputs else None
        self.logits = (torch.empty(BL * self.V, dtype=torch.float32, device=device)
                       if logits else None)
        self.commit_step = (torch.full((self.B * self.G,), -1, dtype=torch.int16, device=device)
                            if commit_trace else None)
        self._k1_ms = ctypes.c_double(0.0)
        self._k1_n = ctypes.c_int32(0)
        self._tail_ms = ctypes.c_double(0.0)
        self.time_k1 = False
        self.vocab_layout = int(vocab_layout)
        self.norm_weight = norm_weight
        self.norm_eps = float(norm_eps)
        self.softcap = float(softcap)
        self.norm_h = (torch.empty(BL * self.d, dtype=torch.int16, device=device)
                       if norm_weight is not None else None)
        self.sc_topk = int(sc_topk)
        K = max(self.sc_topk, 0)
        self.sc_prob = torch.zeros(BL * K, dtype=torch.float32, device=device) if K else None
        self.sc_id = torch.zeros(BL * K, dtype=torch.int32, device=device) if K else None
        self.sc_status = (torch.zeros(BL, dtype=torch.int32, device=device)
                          if K and sc_status else None)

    def state_views(self) -> dict:
        B, BL = self.B, self.B * self.L
        s = self.state
        return {
            "prev_argmax": s[:BL],
            "stable_count": s[BL:BL + B],
            "done": s[BL + B:BL + 2 * B],
            "steps_used": s[BL + 2 * B:BL + 3 * B],
            "converged": s[BL + 3 * B:BL + 4 * B],
            "n_committed": s[BL + 4 * B:BL + 5 * B],
            "mean_entropy": s[BL + 5 * B:BL + 6 * B].view(__import__("torch").float32),
            "new_commits": s[BL + 6 * B:BL + 7 * B],
            "status": s[BL + 7 * B:BL + 8 * B],
            "band_sample": s[BL + 8 * B:BL + 9 * B],
            "band_commit": s[BL + 9 * B:BL + 10 * B],
            "band_conv": s[BL + 10 * B:BL + 11 * B],
        }

    def k1_time(self):
        """(summed projection-kernel ms, launches) of the last timed call."""
        return self._k1_ms.value, self._k1_n.value

    def tail_time(self):
        """Summed ms from each projection's end to its step's end, last timed call."""
        return self._tail_ms.value

    def as_ctypes(self, stream=None) -> DgdCtx:
        c = DgdCtx()
        c.B, c.L, c.V, c.d, c.G = self.B, self.L, self.V, self.d, self.G
        c.entropy_bound = self._bounds
        c.workspace = _ptr(self.workspace)
        c.workspace_bytes = self.workspace.numel()
        c.state = _ptr(self.state)
        c.stream = _stream_handle(stream)
        c.entropy = _ptr(self.entropy)
        c.argmax = _ptr(self.argmax)
        c.token = _ptr(self.token)
        c.gap = _ptr(self.gap)
        c.logits = _ptr(self.logits)
        c.commit_step = _ptr(self.commit_step)
        c.vocab_layout = self.vocab_layout
        c.norm_weight = _ptr(self.norm_weight)
        c.norm_eps = self.norm_eps
        c.softcap = self.softcap
        c.norm_h = _ptr(self.norm_h)
        c.sc_topk = self.sc_topk
        c.sc_prob = _ptr(self.sc_prob)
        c.sc_id = _ptr(self.sc_id)
        c.sc_status = _ptr(self.sc_status)
        if self.time_k1:
            c.k1_ms = ctypes.pointer(self._k1_ms)
            c.k1_launches = ctypes.pointer(self._k1_n)
            c.tail_ms = ctypes.pointer(self._tail_ms)
        return c


# ----------------------------------------------------------------------------
# C entry points
# ----------------------------------------------------------------------------
def dgd_state_bytes(B: int, L: int) -> int:
    return int(load_library().dgd_state_bytes(B, L))


def dgd_workspace_bytes(B: int, L: int, V: int, d: int) -> int:
    return int(load_library().dgd_workspace_bytes(B, L, V, d))


def dgd_last_error() -> str:
    return load_library().dgd_last_error().decode()


def dgd_init_block(canvas, committed, block, params: DgdParams, seeds, ctx: Context, stream=None):
    c = ctx.as_ctypes(stream)
    _check(load_library().dgd_init_block(_ptr(canvas, 4), _ptr(committed, 1), int(block),
                                         ctypes.byref(params), _seeds(seeds), ctypes.byref(c)))


def dgd_step(H, W_vocab, canvas, committed, block, step, params: DgdParams, seeds, ctx: Context,
             stream=None):
    c = ctx.as_ctypes(stream)
    # (W_vocab: bf16 words, or the bytes of a 4-bit table: no element size)
    _check(load_library().dgd_step(_ptr(H, 2), _ptr(W_vocab), _ptr(canvas, 4),
                                   _ptr(committed, 1), int(block), int(step),
                                   ctypes.byref(params), _seeds(seeds), ctypes.byref(c)))


def dgd_step_noalloc(H, W_vocab, canvas, committed, block, step, params: DgdParams, seeds,
                     ctx: Context, stream=None):
    """dgd_step with the library's own per-GPU scratch instead of ctx's workspace."""
    c = ctx.as_ctypes(stream)
    _check(load_library().dgd_step_noalloc(_ptr(H, 2), _ptr(W_vocab), _ptr(canvas, 4),
                                           _ptr(committed, 1), int(block), int(step),
                                           ctypes.byref(params), _seeds(seeds), ctypes.byref(c)))


def dgd_run(H_steps, W_vocab, canvas, committed, params: DgdParams, seeds, ctx: Context,
            stream=None):
    c = ctx.as_ctypes(stream)
    _check(load_library().dgd_run(_ptr(H_steps, 2), _ptr(W_vocab), _ptr(canvas, 4),
                                  _ptr(committed, 1), ctypes.byref(params), _seeds(seeds),
                                  ctypes.byref(c)))


def dgd_run_steps(H_steps, W_vocab, canvas, committed, first_step: int, n_steps: int,
                  params: DgdParams, seeds, ctx: Context, stream=None):
    c = ctx.as_ctypes(stream)
    _check(load_library().dgd_run_steps(_ptr(H_steps, 2), _ptr(W_vocab), _ptr(canvas, 4),
                                        _ptr(committed, 1), int(first_step), int(n_steps),
                                        ctypes.byref(params), _seeds(seeds), ctypes.byref(c)))


def dgd_packed_vocab_bytes(V: int, d: int) -> int:
    return int(load_library().dgd_packed_vocab_bytes(V, d))


def dgd_pack_vocab(W_vocab, W_packed, V: int, d: int, stream=None):
    _check(load_library().dgd_pack_vocab(_ptr(W_vocab, 2), _ptr(W_packed, 2), int(V), int(d),
                                         _stream_handle(stream)))


def pack_vocab(W_vocab, V: int, d: int, stream=None):
    """Packed copy of a device bf16 table (a new torch tensor of int16 words)."""
    import torch
    out = torch.empty(dgd_packed_vocab_bytes(V, d) // 2, dtype=torch.int16, device=W_vocab.device)
    dgd_pack_vocab(W_vocab, out, V, d, stream)
    return out


def dgd_q4_vocab_bytes(V: int, d: int) -> int:
    return int(load_library().dgd_q4_vocab_bytes(V, d))


def dgd_pack_vocab_q4(codes, scales, mins, W_q4, V: int, d: int, stream=None):
    _check(load_library().dgd_pack_vocab_q4(_ptr(codes, 1), _ptr(scales, 2), _ptr(mins, 2),
                                            _ptr(W_q4, 1), int(V), int(d), _stream_handle(stream)))


def pack_vocab_q4(codes, scales, mins, V: int, d: int, stream=None):
    """Streaming form of a 4-bit table (a new uint8 device tensor) from device
    tensors: codes uint8 [V*d/2], scales/mins int16 [V*d/32] (bf16 bits)."""
    import torch
    out = torch.empty(dgd_q4_vocab_bytes(V, d), dtype=torch.uint8, device=codes.device)
    dgd_pack_vocab_q4(codes, scales, mins, out, V, d, stream)
    return out


def dgd_sc_embed(sc_prob, sc_id, rows: int, K: int, W_vocab, vocab_layout: int, V: int, d: int,
                 scale: float, out, stream=None):
    _check(load_library().dgd_sc_embed(_ptr(sc_prob, 4), _ptr(sc_id, 4), int(rows), int(K),
                                       _ptr(W_vocab, 2), int(vocab_layout), int(V), int(d),
                                       float(scale), _ptr(out, 2), _stream_handle(stream)))


def dgd_label_probs(H, rows: int, W_vocab, vocab_layout: int, V: int, d: int, labels,
                    temperature: float, softcap: float, logits, probs, stream=None):
    """labels: host sequence of ints; logits may be None."""
    lab = np.asarray(labels, dtype=np.int32).reshape(-1)
    arr = (ctypes.c_int32 * len(lab))(*[int(x) for x in lab])
    _check(load_library().dgd_label_probs(_ptr(H, 2), int(rows), _ptr(W_vocab, 2),
                                          int(vocab_layout), int(V), int(d), arr, len(lab),
                                          float(temperature), float(softcap), _ptr(logits, 4),
                                          _ptr(probs, 4), _stream_handle(stream)))


def dgd_ceiling_hbm_read(buf, nbytes: int, sink, stream=None):
    _check(load_library().dgd_ceiling_hbm_read(_ptr(buf), int(nbytes), _ptr(sink, 4),
                                               _stream_handle(stream)))


def dgd_ceiling_mfma_bf16(ops, nbytes: int, rounds: int, workgroups: int, sink, stream=None):
    _check(load_library().dgd_ceiling_mfma_bf16(_ptr(ops), int(nbytes), int(rounds),
                                                int(workgroups), _ptr(sink, 4),
                                                _stream_handle(stream)))


def dgd_debug_philox(ctr, key, uniform_key: int, out, stream=None):
    """ctr int32 [n*4], key int32 [n*2] or None, out int32 [n*4] (device)."""
    n = ctr.numel() // 4
    _check(load_library().dgd_debug_philox(_ptr(ctr, 4), _ptr(key, 4), int(uniform_key),
                                           _ptr(out, 4), n, _stream_handle(stream)))


def dgd_debug_gumbel(words, out, stream=None):
    _check(load_library().dgd_debug_gumbel(_ptr(words, 4), _ptr(out, 4), int(words.numel()),
                                           _stream_handle(stream)))


def dgd_phase_times():
    """Phase times of the last packed projection (a library built with
    phase timing only): uint64 array [workgroup, wave, slot]."""
    import numpy as np
    out = np.zeros(PHASE_WORKGROUPS * 4 * PHASE_SLOTS, dtype=np.uint64)
    _check(load_library().dgd_phase_times(out.ctypes.data_as(ctypes.c_void_p), out.size))
    return out.reshape(PHASE_WORKGROUPS, 4, PHASE_SLOTS)
