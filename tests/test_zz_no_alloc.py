"""The no-allocation step (dgd_step_noalloc) against dgd_step, through the C ABI.

Both run the same kernels on the same inputs, one with a workspace the
caller allocated, the other with the library's per-GPU scratch array and a
NULL ctx->workspace, so every output must be identical bit for bit: canvas,
committed mask, the whole state block, and the per-step outputs (entropy,
argmax, sample, gap, self-conditioning top-K).  Two runs in a row on one
GPU, the second on a smaller shape, so the array's leftovers from the first
must not show in the second.
"""
import ctypes

import numpy as np
import pytest

from uniform_state_discrete_step_amd.inputs import WORKLOADS, make_workload_arrays, shrink

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run_pair(wl, dev, layout, sc_topk):
    import torch
    from uniform_state_discrete_step_amd import dgd
    lib = dgd.load_library()
    W, Hs = make_workload_arrays(wl, threads=8)
    Wd = torch.from_numpy(W.view(np.int16)).to(dev)
    if layout == dgd.DGD_VOCAB_PACKED:
        Wd = dgd.pack_vocab(Wd, wl.V, wl.d)
    Hd = torch.from_numpy(Hs.view(np.int16)).to(dev)
    params = dgd.make_params(wl.N, wl.t_min, wl.t_max, wl.confidence, wl.stability_threshold,
                             wl.freeze, wl.final_emit)
    sides = []
    for _ in range(2):
        ctx = dgd.Context(wl.B, wl.L, wl.V, wl.d, wl.G, wl.bounds, device=dev,
                          vocab_layout=layout, sc_topk=sc_topk, sc_status=sc_topk > 0)
        canvas = torch.zeros(wl.B * wl.G, dtype=torch.int32, device=dev)
        committed = torch.zeros(wl.B * wl.G, dtype=torch.uint8, device=dev)
        sides.append((ctx, canvas, committed))
    seeds = (ctypes.c_uint64 * wl.B)(*wl.seeds)
    steps = 0
    for b in range(wl.blocks):
        for ctx, canvas, committed in sides:
            dgd.dgd_init_block(canvas, committed, b, params, wl.seeds, ctx)
        for s in range(wl.N):
            H = Hd[b, s].reshape(-1)
            ref_ctx, ref_can, ref_com = sides[0]
            dgd.dgd_step(H, Wd, ref_can, ref_com, b, s, params, wl.seeds, ref_ctx)
            ctx, can, com = sides[1]
            c = ctx.as_ctypes()
            c.workspace = None                 # the no-allocation step ignores it
            c.workspace_bytes = 0
            rc = lib.dgd_step_noalloc(H.data_ptr(), Wd.data_ptr(), can.data_ptr(), com.data_ptr(),
                                      b, s, ctypes.byref(params), seeds, ctypes.byref(c))
            assert rc == dgd.DGD_OK, dgd.dgd_last_error()
            torch.cuda.synchronize()
            tag = f"{wl.name} block {b} step {s}"
            for name in ("canvas", "committed"):
                a = (ref_can if name == "canvas" else ref_com).cpu().numpy()
                g = (can if name == "canvas" else com).cpu().numpy()
                assert np.array_equal(a, g), f"{tag}: {name} differs"
            assert np.array_equal(ref_ctx.state.cpu().numpy(), ctx.state.cpu().numpy()), \
                f"{tag}: state differs"
            outs = ["entropy", "argmax", "token", "gap"] + (["sc_prob", "sc_id"] if sc_topk else [])
            for name in outs:
                a = getattr(ref_ctx, name).cpu().numpy()
                g = getattr(ctx, name).cpu().numpy()
                assert np.array_equal(a.view(np.uint32), g.view(np.uint32)), f"{tag}: {name} differs"
            steps += 1
            if int(ref_ctx.state_views()["done"].min()) == 1:
                break
    return steps


def test_no_alloc_step_equals_the_step(dev):
    from uniform_state_discrete_step_amd import dgd
    # first: 512 positions over 257 vocabulary tiles (ragged), packed table,
    # top-32: records and candidates fill 20 MB of the scratch
    big = shrink(WORKLOADS["tiny"], name="noalloc_big", B=2, L=256, G=256, V=65573, d=192, N=4,
                 seeds=(5, 6), bounds=(0.1, 0.2), cfg_seed=41)
    n1 = _run_pair(big, dev, dgd.DGD_VOCAB_PACKED, 32)
    # then a smaller shape on the same scratch: two blocks, row-major table
    small = shrink(WORKLOADS["tiny"], name="noalloc_small", B=1, L=16, G=32, N=3, seeds=(7,),
                   bounds=(0.1,), cfg_seed=42)
    n2 = _run_pair(small, dev, dgd.DGD_VOCAB_ROWS, 0)
    print(f"\n[no-allocation step] {n1} + {n2} steps identical to dgd_step", flush=True)
    assert n1 == big.N and n2 >= 2
