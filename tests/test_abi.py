"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/dgd.h declares, size
its buffers as documented, and refuse invalid arguments on the host before
any GPU work is enqueued (so these calls never touch a device).
"""
import ctypes
import os
import re

import pytest

from uniform_state_discrete_step_amd import dgd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dgd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dgd_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return dgd.load_library()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(dgd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_state_and_workspace_sizes(lib):
    # prev_argmax per position, then 11 words per canvas (stable count, done,
    # steps used, converged, committed, mean entropy, new commits, status and
    # the three band counters)
    assert dgd.dgd_state_bytes(1, 256) == (256 + 11) * 4
    assert dgd.dgd_state_bytes(8, 256) == (8 * 256 + 88) * 4
    assert dgd.dgd_state_bytes(0, 16) == 0
    # 256 positions x 256 vocabulary groups x (32-byte record + 16 x 8-byte
    # self-conditioning candidates) dominate
    ws = dgd.dgd_workspace_bytes(1, 256, 262144, 2816)
    assert 256 * 256 * (32 + 128) <= ws <= 256 * 256 * (32 + 128) + 16384
    assert dgd.dgd_workspace_bytes(1, 16, 1024, 64) >= 16 * 4 * (32 + 128)   # V=1024: 4 groups
    for bad in [(0, 16, 1024, 64), (65, 16, 1024, 64), (1, 4097, 1024, 64), (1, 16, 0, 64),
                (1, 16, 1024, 60), (1, 16, 1024, 0), (1, 16, (1 << 24) + 1, 64)]:
        assert dgd.dgd_workspace_bytes(*bad) == 0, bad


FAKE = 0x10000  # never dereferenced: every call below is refused on the host


def _ctx(**kw):
    c = dgd.DgdCtx()
    c.B, c.L, c.V, c.d, c.G = kw.get("B", 1), kw.get("L", 16), kw.get("V", 1024), kw.get("d", 64), kw.get("G", 16)
    bounds = kw.get("bounds", [0.1] * c.B)
    c._keep = (ctypes.c_float * len(bounds))(*bounds)
    c.entropy_bound = c._keep if kw.get("with_bounds", True) else None
    c.workspace = kw.get("workspace", FAKE * 16)
    c.workspace_bytes = kw.get("workspace_bytes", 1 << 30)
    c.state = kw.get("state", FAKE)
    c.vocab_layout = kw.get("vocab_layout", 0)
    c.norm_weight = kw.get("norm_weight", None)
    c.norm_eps = kw.get("norm_eps", 0.0)
    c.softcap = kw.get("softcap", 0.0)
    c.norm_h = kw.get("norm_h", None)
    c.sc_topk = kw.get("sc_topk", 0)
    c.sc_prob = kw.get("sc_prob", None)
    c.sc_id = kw.get("sc_id", None)
    c.sc_status = kw.get("sc_status", None)
    return c


def _step(lib, ctx, params=None, seeds=(0,), block=0, step=0, H=FAKE, W=FAKE):
    p = params or dgd.make_params(N=8)
    s = (ctypes.c_uint64 * len(seeds))(*seeds)
    return lib.dgd_step(H, W, FAKE, FAKE, block, step, ctypes.byref(p), s, ctypes.byref(ctx))


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), dgd.DGD_EINVAL),
    (dict(N=1025), dgd.DGD_EINVAL),
    (dict(t_min=float("nan")), dgd.DGD_EINVAL),
    (dict(t_max=1.5), dgd.DGD_EINVAL),
    (dict(t_min=0.0, t_max=0.0), dgd.DGD_EINVAL),
    (dict(t_min=1e-5, t_max=1e-5), dgd.DGD_EINVAL),
    (dict(N=1, t_min=0.0, t_max=5e-5), dgd.DGD_EINVAL),
    (dict(confidence=-0.1), dgd.DGD_EINVAL),
    (dict(stability_threshold=-1), dgd.DGD_EINVAL),
    (dict(freeze=2), dgd.DGD_EINVAL),
    (dict(final_emit=-1), dgd.DGD_EINVAL),
])
def test_invalid_knobs_are_refused(lib, kw, code):
    args = dict(N=8)
    args.update(kw)
    assert _step(lib, _ctx(), params=dgd.make_params(**args)) == code
    assert dgd.dgd_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), dgd.DGD_EUNSUPPORTED),
    (dict(B=65, bounds=[0.1] * 65), dgd.DGD_EUNSUPPORTED),
    (dict(L=0), dgd.DGD_EUNSUPPORTED),
    (dict(L=5000, G=5000), dgd.DGD_EUNSUPPORTED),
    (dict(G=24), dgd.DGD_EINVAL),
    (dict(G=8 * 1024 + 16), dgd.DGD_EINVAL),
    (dict(V=0), dgd.DGD_EUNSUPPORTED),
    (dict(d=60), dgd.DGD_EUNSUPPORTED),
    (dict(bounds=[1.5]), dgd.DGD_EINVAL),
    (dict(bounds=[float("inf")]), dgd.DGD_EINVAL),
    (dict(with_bounds=False), dgd.DGD_EINVAL),
    (dict(state=None), dgd.DGD_EINVAL),
    (dict(workspace=None), dgd.DGD_EINVAL),
    (dict(workspace=FAKE * 16 + 8), dgd.DGD_EINVAL),
    (dict(workspace_bytes=100), dgd.DGD_EWORKSPACE),
    (dict(vocab_layout=3), dgd.DGD_EINVAL),
    (dict(vocab_layout=-1), dgd.DGD_EINVAL),
    (dict(vocab_layout=2, d=72), dgd.DGD_EUNSUPPORTED),        # 4-bit table: d % 32 != 0
    (dict(vocab_layout=2, sc_topk=8, sc_prob=FAKE, sc_id=FAKE), dgd.DGD_EUNSUPPORTED),
])
def test_invalid_shapes_and_buffers_are_refused(lib, kw, code):
    assert _step(lib, _ctx(**kw)) == code


def test_invalid_step_block_and_pointers_are_refused(lib):
    assert _step(lib, _ctx(), step=8) == dgd.DGD_EINVAL
    assert _step(lib, _ctx(), step=-1) == dgd.DGD_EINVAL
    assert _step(lib, _ctx(), block=1) == dgd.DGD_EINVAL
    assert _step(lib, _ctx(), H=None) == dgd.DGD_EINVAL
    assert _step(lib, _ctx(), W=None) == dgd.DGD_EINVAL
    assert _step(lib, _ctx(), H=FAKE + 8) == dgd.DGD_EINVAL          # not 16-byte aligned
    assert _step(lib, _ctx(vocab_layout=1), W=FAKE + 2) == dgd.DGD_EINVAL
    p = dgd.make_params(N=8)
    assert lib.dgd_step(FAKE, FAKE, FAKE, FAKE, 0, 0, ctypes.byref(p), None, ctypes.byref(_ctx())) == dgd.DGD_EINVAL
    assert lib.dgd_step(FAKE, FAKE, FAKE, FAKE, 0, 0, None, None, ctypes.byref(_ctx())) == dgd.DGD_EINVAL
    assert lib.dgd_run(FAKE, FAKE, FAKE, FAKE, ctypes.byref(p), None, None) == dgd.DGD_EINVAL
    s1 = (ctypes.c_uint64 * 1)(0)
    c = _ctx()                                     # G/L = 1 block of N = 8 steps
    for first, n in ((-1, 1), (0, -1), (0, 9), (8, 1), (5, 4)):
        assert lib.dgd_run_steps(FAKE, FAKE, FAKE, FAKE, first, n, ctypes.byref(p), s1,
                                 ctypes.byref(c)) == dgd.DGD_EINVAL, (first, n)
    assert lib.dgd_run_steps(None, FAKE, FAKE, FAKE, 0, 1, ctypes.byref(p), s1,
                             ctypes.byref(c)) == dgd.DGD_EINVAL
    assert lib.dgd_run_steps(FAKE, FAKE, FAKE, FAKE, 0, 1, None, s1,
                             ctypes.byref(c)) == dgd.DGD_EINVAL
    # an empty range is a valid call that enqueues nothing
    assert lib.dgd_run_steps(FAKE, FAKE, FAKE, FAKE, 8, 0, ctypes.byref(p), s1,
                             ctypes.byref(c)) == dgd.DGD_OK
    s = (ctypes.c_uint64 * 1)(0)
    assert lib.dgd_init_block(FAKE, FAKE, 3, ctypes.byref(p), s, ctypes.byref(_ctx())) == dgd.DGD_EINVAL
    assert lib.dgd_init_block(None, FAKE, 0, ctypes.byref(p), s, ctypes.byref(_ctx())) == dgd.DGD_EINVAL
    assert lib.dgd_debug_gumbel(None, FAKE, 4, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_gumbel(FAKE, FAKE, -1, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_gumbel(FAKE, FAKE, 0, None) == dgd.DGD_OK
    assert lib.dgd_debug_philox(None, None, 0, FAKE, 4, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_philox(FAKE, None, 0, None, 4, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_philox(FAKE, None, 0, FAKE, -1, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_philox(FAKE + 4, None, 0, FAKE, 4, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_philox(FAKE, FAKE + 4, 0, FAKE, 4, None) == dgd.DGD_EINVAL
    assert lib.dgd_debug_philox(FAKE, None, 0, FAKE, 0, None) == dgd.DGD_OK
    assert lib.dgd_ceiling_hbm_read(None, 64, FAKE, None) == dgd.DGD_EINVAL
    assert lib.dgd_ceiling_hbm_read(FAKE, 60, FAKE, None) == dgd.DGD_EINVAL
    assert lib.dgd_ceiling_hbm_read(FAKE + 8, 64, FAKE, None) == dgd.DGD_EINVAL
    assert lib.dgd_ceiling_hbm_read(FAKE, 0, FAKE, None) == dgd.DGD_OK
    assert lib.dgd_ceiling_mfma_bf16(FAKE, 128, 1, 1, FAKE, None) == dgd.DGD_EINVAL   # < 256 bytes
    assert lib.dgd_ceiling_mfma_bf16(FAKE, 4096, 0, 1, FAKE, None) == dgd.DGD_EINVAL
    assert lib.dgd_ceiling_mfma_bf16(FAKE, 4096, 1, 0, FAKE, None) == dgd.DGD_EINVAL
    assert lib.dgd_ceiling_mfma_bf16(None, 4096, 1, 1, FAKE, None) == dgd.DGD_EINVAL


@pytest.mark.parametrize("kw", [
    dict(softcap=-1.0),
    dict(softcap=0.001),
    dict(softcap=2e4),
    dict(softcap=float("nan")),
    dict(softcap=float("inf")),
    dict(norm_weight=FAKE * 4),                                   # no norm_h
    dict(norm_weight=FAKE * 4 + 2, norm_h=FAKE * 8),              # misaligned weights
    dict(norm_weight=FAKE * 4, norm_h=FAKE * 8 + 4),              # misaligned norm_h
    dict(norm_weight=FAKE * 4, norm_h=FAKE * 8, norm_eps=-1e-6),
    dict(norm_weight=FAKE * 4, norm_h=FAKE * 8, norm_eps=float("nan")),
    dict(norm_weight=FAKE * 4, norm_h=FAKE * 8, norm_eps=2.0),
    dict(norm_weight=FAKE * 4, norm_h=FAKE),                      # norm_h overlaps H
    dict(norm_weight=FAKE * 4, norm_h=FAKE + 16 * 64 * 2 - 16),   # ... at H's last bytes
])
def test_invalid_tail_is_refused(lib, kw):
    assert _step(lib, _ctx(**kw)) == dgd.DGD_EINVAL
    assert dgd.dgd_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(sc_topk=-1, vocab_layout=1, sc_prob=FAKE, sc_id=FAKE), dgd.DGD_EINVAL),
    (dict(sc_topk=33, vocab_layout=1, sc_prob=FAKE, sc_id=FAKE), dgd.DGD_EINVAL),
    (dict(sc_topk=8, V=7, vocab_layout=1, sc_prob=FAKE, sc_id=FAKE), dgd.DGD_EINVAL),   # K > V
    (dict(sc_topk=8, vocab_layout=1, sc_id=FAKE), dgd.DGD_EINVAL),                   # no sc_prob
    (dict(sc_topk=8, vocab_layout=1, sc_prob=FAKE), dgd.DGD_EINVAL),                 # no sc_id
    (dict(sc_topk=8, vocab_layout=0, sc_prob=FAKE, sc_id=FAKE), dgd.DGD_EUNSUPPORTED),  # rows
])
def test_invalid_self_conditioning_is_refused(lib, kw, code):
    assert _step(lib, _ctx(**kw)) == code
    assert dgd.dgd_last_error()


def test_q4_table_size_and_refusals(lib):
    # 40 bytes per 64 elements: 32 of codes, 8 of scales and minima
    assert dgd.dgd_q4_vocab_bytes(262144, 2816) == 262144 * 2816 // 64 * 40
    assert dgd.dgd_q4_vocab_bytes(100, 96) == 128 * 2 * 64 * 40 // 64
    for bad in [(0, 64), (1 << 25, 64), (64, 48), (64, 0), (64, 16)]:
        assert dgd.dgd_q4_vocab_bytes(*bad) == 0, bad
    f = lib.dgd_pack_vocab_q4
    assert f(None, FAKE, FAKE, FAKE * 64, 64, 64, None) == dgd.DGD_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 64, 64, None) == dgd.DGD_EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE * 64, 64, 48, None) == dgd.DGD_EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE * 64, 0, 64, None) == dgd.DGD_EUNSUPPORTED
    assert f(FAKE + 4, FAKE, FAKE, FAKE * 64, 64, 64, None) == dgd.DGD_EINVAL   # codes misaligned
    assert f(FAKE, FAKE + 1, FAKE, FAKE * 64, 64, 64, None) == dgd.DGD_EINVAL   # scales misaligned
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE, 64, 64, None) == dgd.DGD_EINVAL    # output overlaps codes
    assert dgd.dgd_last_error()


def test_sc_embed_refusals(lib):
    f = lib.dgd_sc_embed
    ok = (FAKE, FAKE, 4, 8, FAKE, 1, 1024, 64, 8.0, FAKE, None)

    def call(**kw):
        names = ["prob", "ids", "rows", "K", "W", "layout", "V", "d", "scale", "out", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])

    assert call(rows=0) == dgd.DGD_OK                      # nothing to do, nothing read
    for kw, code in [(dict(prob=None), dgd.DGD_EINVAL), (dict(ids=None), dgd.DGD_EINVAL),
                     (dict(W=None), dgd.DGD_EINVAL), (dict(out=None), dgd.DGD_EINVAL),
                     (dict(rows=-1), dgd.DGD_EINVAL), (dict(K=0), dgd.DGD_EINVAL),
                     (dict(K=33), dgd.DGD_EINVAL), (dict(V=0), dgd.DGD_EUNSUPPORTED),
                     (dict(d=60), dgd.DGD_EUNSUPPORTED), (dict(layout=2), dgd.DGD_EINVAL),
                     (dict(scale=float("nan")), dgd.DGD_EINVAL),
                     (dict(W=FAKE + 4), dgd.DGD_EINVAL), (dict(out=FAKE + 2), dgd.DGD_EINVAL)]:
        assert call(**kw) == code, kw
        assert dgd.dgd_last_error()


def test_label_probs_refusals(lib):
    f = lib.dgd_label_probs

    def call(labels=(1, 2), **kw):
        arr = (ctypes.c_int32 * max(len(labels), 1))(*labels)
        args = dict(H=FAKE, rows=4, W=FAKE, layout=0, V=1024, d=64, n=len(labels), T=1.0, cap=0.0,
                    logits=None, probs=FAKE, stream=None)
        args.update(kw)
        return f(args["H"], args["rows"], args["W"], args["layout"], args["V"], args["d"],
                 kw.get("labels_ptr", arr), args["n"], args["T"], args["cap"], args["logits"],
                 args["probs"], args["stream"])

    assert call(rows=0) == dgd.DGD_OK                      # nothing to do, nothing read
    cases = [(dict(H=None), dgd.DGD_EINVAL), (dict(W=None), dgd.DGD_EINVAL),
             (dict(probs=None), dgd.DGD_EINVAL), (dict(labels_ptr=None), dgd.DGD_EINVAL),
             (dict(rows=-1), dgd.DGD_EINVAL), (dict(V=0), dgd.DGD_EUNSUPPORTED),
             (dict(d=12), dgd.DGD_EUNSUPPORTED), (dict(layout=3), dgd.DGD_EINVAL),
             (dict(n=0), dgd.DGD_EINVAL), (dict(T=0.0), dgd.DGD_EINVAL),
             (dict(T=float("inf")), dgd.DGD_EINVAL), (dict(cap=-2.0), dgd.DGD_EINVAL),
             (dict(cap=1e5), dgd.DGD_EINVAL), (dict(H=FAKE + 2), dgd.DGD_EINVAL),
             (dict(W=FAKE + 8), dgd.DGD_EINVAL)]
    for kw, code in cases:
        assert call(**kw) == code, kw
        assert dgd.dgd_last_error()
    assert call(labels=(1, 1024)) == dgd.DGD_EINVAL       # id past V
    assert call(labels=(-1,)) == dgd.DGD_EINVAL
    assert call(labels=tuple(range(513))) == dgd.DGD_EINVAL


def test_tail_overlap_is_checked_over_every_step_of_a_run(lib):
    # H_steps spans N steps of B*L*d bf16 values; norm_h just past step 0 still overlaps
    p = dgd.make_params(N=8)
    s = (ctypes.c_uint64 * 1)(0)
    step_bytes = 16 * 64 * 2
    for nh in (FAKE + step_bytes, FAKE + 8 * step_bytes - 16):
        ctx = _ctx(norm_weight=FAKE * 64, norm_h=nh)
        assert lib.dgd_run(FAKE, FAKE * 128, FAKE * 256, FAKE * 512, ctypes.byref(p), s,
                           ctypes.byref(ctx)) == dgd.DGD_EINVAL
        assert "overlaps" in dgd.dgd_last_error()


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError):
        dgd._lib, saved = None, dgd._lib
        try:
            dgd.load_library(str(tmp_path / "missing.so"))
        finally:
            dgd._lib = saved


def test_packed_vocab_size_and_refusals(lib):
    # whole 64-row groups and 64-element hidden chunks, 2 bytes each
    assert dgd.dgd_packed_vocab_bytes(262144, 2816) == 262144 * 2816 * 2
    assert dgd.dgd_packed_vocab_bytes(1001, 72) == 1024 * 128 * 2
    assert dgd.dgd_packed_vocab_bytes(1, 8) == 64 * 64 * 2
    for bad in [(0, 64), (1024, 0), (1024, 60), ((1 << 24) + 1, 64), (1024, 65536 + 8)]:
        assert dgd.dgd_packed_vocab_bytes(*bad) == 0, bad
    assert lib.dgd_pack_vocab(None, FAKE, 64, 64, None) == dgd.DGD_EINVAL
    assert lib.dgd_pack_vocab(FAKE, None, 64, 64, None) == dgd.DGD_EINVAL
    assert lib.dgd_pack_vocab(FAKE, FAKE * 4, 0, 64, None) == dgd.DGD_EUNSUPPORTED
    assert lib.dgd_pack_vocab(FAKE, FAKE * 4, 64, 12, None) == dgd.DGD_EUNSUPPORTED
    assert lib.dgd_pack_vocab(FAKE + 4, FAKE * 4, 64, 64, None) == dgd.DGD_EINVAL
    # destination overlapping the source
    assert lib.dgd_pack_vocab(FAKE, FAKE + 64 * 64, 64, 64, None) == dgd.DGD_EINVAL
    assert dgd.dgd_last_error()


def test_no_alloc_step_refusals(lib):
    """Refusals of the no-allocation step happen on the host, before any HIP
    call: invalid arguments as for dgd_step, a shape whose scratch exceeds the
    library's array, and a timing request (events would be created)."""
    p = dgd.make_params(N=8)
    s = (ctypes.c_uint64 * 8)(*range(8))

    def call(ctx, H=FAKE, step=0):
        return lib.dgd_step_noalloc(H, FAKE, FAKE, FAKE, 0, step, ctypes.byref(p), s,
                                    ctypes.byref(ctx))

    c = _ctx(workspace=None, workspace_bytes=0)
    assert call(c, H=None) == dgd.DGD_EINVAL
    assert call(c, step=8) == dgd.DGD_EINVAL
    assert call(c, H=FAKE + 8) == dgd.DGD_EINVAL
    # 8 x 2048 positions x 256 vocabulary groups x 32 B of records = 128 MiB > 32 MiB
    big = _ctx(B=8, L=2048, G=2048, V=262144, d=2816, workspace=None, workspace_bytes=0)
    assert call(big) == dgd.DGD_EUNSUPPORTED
    assert "scratch" in dgd.dgd_last_error()
    # 2048 positions fit without a top-K, not with one (candidates: 128 B per record)
    sc = _ctx(B=8, L=256, G=256, V=262144, d=2816, workspace=None, workspace_bytes=0,
              sc_topk=32, sc_prob=FAKE * 32, sc_id=FAKE * 64, vocab_layout=1)
    assert call(sc) == dgd.DGD_EUNSUPPORTED
    t = _ctx(workspace=None, workspace_bytes=0)
    ms = ctypes.c_double(0.0)
    t.k1_ms = ctypes.pointer(ms)
    assert call(t) == dgd.DGD_EINVAL
    assert "k1_ms" in dgd.dgd_last_error()


def test_phase_times_refusals(lib):
    # the default build records no phase times and says so; bad arguments
    # are refused first
    buf = (ctypes.c_uint64 * 16)()
    assert lib.dgd_phase_times(None, 16) == dgd.DGD_EINVAL
    assert lib.dgd_phase_times(buf, dgd.PHASE_WORKGROUPS * 4 * dgd.PHASE_SLOTS + 1) == dgd.DGD_EINVAL
    assert lib.dgd_phase_times(buf, 16) == dgd.DGD_EUNSUPPORTED
    assert b"DGD_PHASE_TIMING" in lib.dgd_last_error()


def test_phase_build_exports_the_same_functions():
    if not os.path.exists(dgd.LIB_PHASE_PATH):
        pytest.skip("libdgd_phase.so is not built (__graft_entry__.build() builds it)")
    phase = ctypes.CDLL(dgd.LIB_PHASE_PATH)
    for n in declared_functions():
        assert hasattr(phase, n), n
