"""The step's device calls replayed from a HIP graph.

Every kernel of the path resets the state it reads (claim cursors, -inf
partial rows, packed copies) inside its own launches and the library makes no
memset, copy or allocation call, so a forward + merge + backward captured once
replays with the plans already on the device.  Each replay follows eager work
that clears the outputs, and must reproduce the eager step bitwise.
"""
import pytest
import torch

from block_sparse_draft_amd import binding as B
from helpers import make_path, to_device
from synthetic import make

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("noalloc", [False, True])
def test_step_replays_from_a_hip_graph(noalloc):
    w = make("c3", seed=91, with_do=True, n_ctx_range=(900, 2100), n_anchor=5, hq=8, hkv=2, chunk=512)
    path = make_path(w, DEV, with_bwd=True, fwd_runs_per_worker=2, fwd_run_imbalance=None)
    q, k, v, do = (to_device(w, n, DEV) for n in ("q", "k", "v", "do"))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # eager step: uploads the plans and gives the reference
    path.forward(q, k, v)
    path.backward(q, k, v, do, dq, dk, dv, noalloc=noalloc)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (path.o, path.lse, dq, dk, dv)]

    p = path.problem
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        B.sparse_attn_partial_fwd(p, path.fwd_plan, q, k, v, path.o_part, path.m_part, path.lse_part, s)
        B.lse_merge_all(p, path.d_part_base, path.o_part, path.m_part, path.lse_part, path.o, path.lse, s)
        if noalloc:
            B.sparse_attn_bwd_noalloc(p, path.bwd_plan, path.dq_plan, q, k, v, path.o, path.lse, do, dq, dk, dv, s)
        else:
            B.sparse_attn_bwd(p, path.bwd_plan, path.dq_plan, q, k, v, path.o, path.lse, do, dq, dk, dv,
                              path.workspace, s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (path.o, path.lse, dq, dk, dv, path.o_part, path.m_part, path.lse_part):
            t.zero_()  # eager work between replays, on the default stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "LSE", "dQ", "dK", "dV"), (path.o, path.lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (rep, name)
