"""The backward without a caller workspace (sparse_attn_bwd_noalloc, whose
workspace is the library's static scratch) against sparse_attn_bwd with a
caller workspace: two no-allocation calls in a row on one GPU, the second on a
smaller problem (so it runs over what the first left in the scratch), each
bitwise equal to the workspace call on the same inputs; the first is also
checked against the oracle's gradients."""
import numpy as np
import pytest
import torch

from block_sparse_draft_amd import binding as B
from helpers import BF16_ABS, BF16_FROB, assert_close, make_path, to_device, to_np64
from synthetic import make

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (config recipe, overrides): the first problem is the larger one
PROBLEMS = [("c3", dict(n_ctx_range=(3000, 9000), n_anchor=24, hq=8, hkv=2, chunk=1024)),
            ("c5", dict(n_ctx=2500, n_anchor=5, hq=4, hkv=4, chunk=512))]


def _setup(cfg, over, seed):
    w = make(cfg, seed=seed, with_do=True, **over)
    path = make_path(w, DEV, with_bwd=True, n_workers=48, fwd_runs_per_worker=2, fwd_run_imbalance=None)
    assert path.problem.bwd_workspace_bytes() <= B.SKV_NOALLOC_SCRATCH_BYTES
    q, k, v, do = (to_device(w, n, DEV) for n in ("q", "k", "v", "do"))
    path.forward(q, k, v)
    return w, path, (q, k, v, do)


def _grads(path, t, noalloc):
    q, k, v, do = t
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    path.backward(q, k, v, do, dq, dk, dv, noalloc=noalloc)
    return dq, dk, dv


def test_noalloc_backward_matches_workspace_backward():
    runs = [_setup(cfg, over, seed) for seed, (cfg, over) in enumerate(PROBLEMS)]
    sizes = [r[1].problem.bwd_workspace_bytes() for r in runs]
    print("workspace bytes", sizes)
    assert sizes[1] < sizes[0]
    ref = [_grads(path, t, noalloc=False) for _, path, t in runs]
    torch.cuda.synchronize()
    got = [_grads(path, t, noalloc=True) for _, path, t in runs]   # two calls in a row, larger first
    torch.cuda.synchronize()
    for i, (r, g) in enumerate(zip(ref, got)):
        for name, a, b in zip(("dQ", "dK", "dV"), r, g):
            assert torch.isfinite(b).all(), f"problem {i} {name}: unwritten or non-finite values"
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"problem {i} {name} differs"
    w, path, _ = runs[0]
    dq, dk, dv = (to_np64(x) for x in got[0])
    rq, rk, rv, _, _ = oracle.bwd_workload(w)
    assert_close("dQ", dq, rq, BF16_ABS, BF16_FROB)
    assert_close("dK", dk, rk, BF16_ABS, BF16_FROB)
    assert_close("dV", dv, rv, BF16_ABS, BF16_FROB)
