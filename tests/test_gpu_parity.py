"""GPU parity: the HIP path, called through the C ABI, against the float64
oracle on identical seeded inputs (bf16 inputs are compared with the oracle
fed the same bf16-rounded values).  Small cases span several tiles, chunks and
a ragged tail; the full configurations are checked on sampled sequences / KV
heads and through invariants that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (BF16_ABS, BF16_FROB, BF16_LSE_REL, F32_ABS, assert_close, assert_lse, make_path, to_device,
                     to_np64)
from synthetic import add_own_block, make, make_custom

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _upload(w):
    return [to_device(w, n, DEV) for n in ("q", "k", "v")]


def _check_partials(path, w, seqs=None, heads=None, abs_tol=BF16_ABS, frob_tol=BF16_FROB, lse_tol=BF16_LSE_REL):
    """Compare every visible partial row, normalised by its own LSE (the
    chunk-local attention output), plus m_c and LSE_c."""
    for s in (range(w.cfg.n_seq) if seqs is None else seqs):
        op, mp, lp = oracle.partials_workload(w, s, heads=heads)
        go, gm, gl = [to_np64(t) for t in path.partial_view(s)]
        hs = list(range(w.cfg.hq)) if heads is None else list(heads)
        op, mp, lp, go, gm, gl = op[:, hs], mp[:, hs], lp[:, hs], go[:, hs], gm[:, hs], gl[:, hs]
        assert_lse(f"seq{s} lse_part", gl, lp, lse_tol)
        assert_lse(f"seq{s} m_part", gm, mp, lse_tol)
        vis = np.isfinite(lp)
        with np.errstate(invalid="ignore", over="ignore"):
            gn = go * np.exp(np.where(vis, gm - gl, 0.0))[..., None]
            on = op * np.exp(np.where(vis, mp - lp, 0.0))[..., None]
        assert_close(f"seq{s} normalised o_part", gn[vis], on[vis], abs_tol, frob_tol)


def _check_merged(path, w, O, L, heads=None, rows=None, abs_tol=BF16_ABS, frob_tol=BF16_FROB, lse_tol=BF16_LSE_REL):
    go, gl = to_np64(path.o), to_np64(path.lse)
    hs = slice(None) if heads is None else list(heads)
    rs = slice(None) if rows is None else rows
    assert_close("O", go[rs][:, hs], O[rs][:, hs], abs_tol, frob_tol)
    assert_lse("LSE", gl[rs][:, hs], L[rs][:, hs], lse_tol)


# ---------------------------------------------------------------------------
# fp32 (tiny config, full)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_c1_fp32_partials_and_merge(seed):
    w = make("c1", seed=seed)
    path = make_path(w, DEV)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    _check_partials(path, w, abs_tol=F32_ABS, frob_tol=None, lse_tol=F32_ABS)
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L, abs_tol=F32_ABS, frob_tol=None, lse_tol=F32_ABS)


@pytest.mark.parametrize("d", [64, 128])
def test_c1_fp32_chunk_runs(d):
    """The fp32 forward over chunk runs (one partial per run): merged output,
    each run's partial against the oracle's merge of its chunks."""
    w = make("c1", seed=5, d=d, n_ctx=2048, n_anchor=8, chunk=128)
    path = make_path(w, DEV, n_workers=4, fwd_runs_per_worker=1, fwd_run_imbalance=None)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L, abs_tol=F32_ABS, frob_tol=None, lse_tol=F32_ABS)
    items, cost = path.fwd_plan.table
    assert (items["n_chunk"] > 1).any()
    op, mp, lp = oracle.partials_workload(w, 0)
    go, gm, gl = [to_np64(t) for t in path.partial_view(0)]
    G, B = w.cfg.hq // w.cfg.hkv, w.cfg.block
    for it, c in zip(items, cost):
        if c == 0:
            continue
        g, c0, n = int(it["kv_head"]), int(it["chunk"]), int(it["n_chunk"])
        rows, hs = slice(int(it["lo"]) * B, int(it["hi"]) * B), slice(g * G, (g + 1) * G)
        ro, rl = oracle.lse_merge(op[c0:c0 + n, hs, rows], mp[c0:c0 + n, hs, rows], lp[c0:c0 + n, hs, rows])
        assert_lse("run lse", gl[c0, hs, rows].T, rl, F32_ABS)
        vis = np.isfinite(rl)
        with np.errstate(invalid="ignore"):
            gn = go[c0, hs, rows] * np.exp(np.where(vis.T, gm[c0, hs, rows] - gl[c0, hs, rows], 0.0))[..., None]
        assert_close("run o", gn.transpose(1, 0, 2)[vis], ro[vis], F32_ABS)
        assert np.all(gl[c0 + 1:c0 + n, hs, rows] == -np.inf)


def test_fp32_head_dim_128_ragged():
    w = make("c1", seed=3, n_ctx=777, d=128, hq=4, hkv=2, chunk=192)
    path = make_path(w, DEV)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L, abs_tol=F32_ABS, frob_tol=None, lse_tol=F32_ABS)


# ---------------------------------------------------------------------------
# bf16 forward
# ---------------------------------------------------------------------------

SMALL_BF16 = {
    # c2 recipe: 3 chunks, ragged tail (3000 = 46 tiles + 56), anchors reach the end
    "c2_small": ("c2", dict(n_ctx=3000, n_anchor=8, hq=8, hkv=2, chunk=1024)),
    # c3 recipe: several sequences of ragged lengths, GQA 4
    "c3_small": ("c3", dict(n_ctx_range=(500, 2500), n_anchor=6, hq=8, hkv=2, chunk=512)),
    # c5 recipe: G = 1, 32-token blocks, anchors clustered late
    "c5_small": ("c5", dict(n_ctx=4100, n_anchor=12, hq=4, hkv=4, chunk=1024)),
    # c4 recipe: many chunks merged
    "c4_small": ("c4", dict(n_ctx=8192, n_anchor=8, hq=4, hkv=1, chunk=256)),
}


@pytest.mark.parametrize("case", sorted(SMALL_BF16))
def test_bf16_forward_small(case):
    cfg, over = SMALL_BF16[case]
    w = make(cfg, seed=7, with_do=False, **over)
    path = make_path(w, DEV, with_bwd=False)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    _check_partials(path, w)
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L)


@pytest.mark.parametrize("case,runs_per_worker", [("c4_small", 1), ("c3_small", 2), ("c5_small", 1),
                                                  ("c2_small", 0.5)])
def test_bf16_forward_chunk_runs(case, runs_per_worker):
    """Forward items that cover runs of consecutive chunks of the same rows
    (one partial per run, in the run's first chunk): the merged O and LSE match
    the oracle, each run's partial is the oracle's merge of its chunks'
    partials, and the run's other chunk rows stay -inf."""
    cfg, over = SMALL_BF16[case]
    w = make(cfg, seed=7, with_do=False, **over)
    path = make_path(w, DEV, with_bwd=False, n_workers=8, fwd_runs_per_worker=runs_per_worker,
                     fwd_run_imbalance=None)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L)
    items, cost = path.fwd_plan.table
    assert (items["n_chunk"] > 1).any()
    G, B = w.cfg.hq // w.cfg.hkv, w.cfg.block
    parts = {s: oracle.partials_workload(w, s) for s in range(w.cfg.n_seq)}
    views = {s: [to_np64(t) for t in path.partial_view(s)] for s in range(w.cfg.n_seq)}
    for it, c in zip(items, cost):
        if c == 0:
            continue
        s, g, c0, n = int(it["seq"]), int(it["kv_head"]), int(it["chunk"]), int(it["n_chunk"])
        rows = slice(int(it["lo"]) * B, int(it["hi"]) * B)
        hs = slice(g * G, (g + 1) * G)
        op, mp, lp = (x[c0:c0 + n, hs, rows] for x in parts[s])
        ro, rl = oracle.lse_merge(op, mp, lp)            # [rows, G, D], [rows, G]
        go, gm, gl = (x[:, hs, rows] for x in views[s])
        assert_lse(f"run s{s} g{g} c{c0}+{n} lse", gl[c0].T, rl, BF16_LSE_REL)
        vis = np.isfinite(rl)
        with np.errstate(invalid="ignore", over="ignore"):
            gn = go[c0] * np.exp(np.where(vis.T, gm[c0] - gl[c0], 0.0))[..., None]
        assert_close(f"run s{s} g{g} c{c0}+{n} o", gn.transpose(1, 0, 2)[vis], ro[vis], BF16_ABS, BF16_FROB)
        assert np.all(gl[c0 + 1:c0 + n] == -np.inf) and np.all(gm[c0 + 1:c0 + n] == -np.inf)


def test_bf16_forward_edge_anchors():
    """Anchors at 0, at N-1 (clipped block), duplicates, and a context whose
    length is not a multiple of the tile."""
    w = make_custom([1000, 130], [[0, 0, 63, 64, 700], [1, 2, 3, 128, 129]], block=16, hq=4, hkv=2, d=128,
                    dtype="bf16", chunk=128, seed=4, with_do=True)
    path = make_path(w, DEV)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    _check_partials(path, w)
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L)


def test_bf16_forward_c2_full():
    w = make("c2", seed=0)
    path = make_path(w, DEV)
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L)
    _check_partials(path, w, heads=[0, 13, 31])


# ---------------------------------------------------------------------------
# bf16 backward
# ---------------------------------------------------------------------------

def _bwd(w, path, q, k, v):
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    path.forward(q, k, v)
    path.backward(q, k, v, do, dq, dk, dv)
    torch.cuda.synchronize()
    return to_np64(dq), to_np64(dk), to_np64(dv)


def _check_grads(w, got, kv_heads=None, seqs=None):
    dq, dk, dv = got
    rq, rk, rv, _, _ = oracle.bwd_workload(w, kv_heads=kv_heads, seqs=seqs)
    G = w.cfg.hq // w.cfg.hkv
    gs = list(range(w.cfg.hkv)) if kv_heads is None else list(kv_heads)
    hs = [h for g in gs for h in range(g * G, (g + 1) * G)]
    ss = list(range(w.cfg.n_seq)) if seqs is None else list(seqs)
    qr = np.concatenate([np.arange(w.q_off[s], w.q_off[s + 1]) for s in ss])
    kr = np.concatenate([np.arange(w.kv_off[s], w.kv_off[s + 1]) for s in ss])
    assert_close("dQ", dq[qr][:, hs], rq[qr][:, hs], BF16_ABS, BF16_FROB)
    assert_close("dK", dk[kr][:, gs], rk[kr][:, gs], BF16_ABS, BF16_FROB)
    assert_close("dV", dv[kr][:, gs], rv[kr][:, gs], BF16_ABS, BF16_FROB)


@pytest.mark.parametrize("case", ["c2_small", "c3_small", "c5_small", "c4_small"])
def test_bf16_backward_small(case):
    cfg, over = SMALL_BF16[case]
    w = make(cfg, seed=11, with_do=True, **over)
    path = make_path(w, DEV, with_bwd=True, bwd_granule=192)
    q, k, v = _upload(w)
    got = _bwd(w, path, q, k, v)
    _check_grads(w, got)


@pytest.mark.parametrize("case,runs_per_worker", [("c4_small", 1), ("c3_small", 2), ("c5_small", 1)])
def test_bf16_backward_chunk_runs(case, runs_per_worker):
    """Forward and query-owner plans over chunk runs (one dQ partial per run,
    summed along the run lengths) give the oracle's gradients."""
    cfg, over = SMALL_BF16[case]
    w = make(cfg, seed=11, with_do=True, **over)
    path = make_path(w, DEV, with_bwd=True, bwd_granule=192, n_workers=8, fwd_runs_per_worker=runs_per_worker,
                     fwd_run_imbalance=None)
    assert (path.dq_plan.table[0]["n_chunk"] > 1).any()
    q, k, v = _upload(w)
    got = _bwd(w, path, q, k, v)
    _check_grads(w, got)


def test_bf16_backward_edge_anchors():
    w = make_custom([1000, 130], [[0, 0, 63, 64, 700], [1, 2, 3, 128, 129]], block=16, hq=4, hkv=2, d=128,
                    dtype="bf16", chunk=128, seed=5, with_do=True)
    path = make_path(w, DEV, with_bwd=True, bwd_granule=64)
    q, k, v = _upload(w)
    got = _bwd(w, path, q, k, v)
    _check_grads(w, got)
    # keys no query sees (716 .. 999 of the first sequence) get exactly zero gradient
    dk, dv = got[1], got[2]
    assert np.all(dk[716:1000] == 0) and np.all(dv[716:1000] == 0)
    assert np.abs(dk[:716]).max() > 0


@pytest.mark.parametrize("cfg,kv_heads,seqs", [("c3", [3], [1]), ("c3", [6], [2]), ("c3", [0], [0]), ("c3", [7], [3]),
                                               ("c4", [2], None), ("c5", [9], None)])
def test_full_size_fwd_bwd_sampled(cfg, kv_heads, seqs):
    """Full configuration on the GPU, compared with the oracle on one KV head
    (and one sequence for the 4-sequence config: every c3 sequence is sampled
    once, each on another KV head)."""
    w = make(cfg, seed=0)
    path = make_path(w, DEV, fwd_runs_per_worker=4)  # the driver's default plan (chunk runs)
    q, k, v = _upload(w)
    got = _bwd(w, path, q, k, v)
    G = w.cfg.hq // w.cfg.hkv
    hs = list(range(kv_heads[0] * G, (kv_heads[0] + 1) * G))
    ss = list(range(w.cfg.n_seq)) if seqs is None else seqs
    O = np.zeros((int(w.q_off[-1]), w.cfg.hq, w.cfg.d))
    L = np.full((int(w.q_off[-1]), w.cfg.hq), -np.inf)
    for s in ss:
        q64 = w.as_f64("q", rows=slice(int(w.q_off[s]), int(w.q_off[s + 1])))
        k64 = w.as_f64("k", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
        v64 = w.as_f64("v", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
        o, l = oracle.attention(q64, k64, v64, w.seq_anchors(s), w.cfg.block, w.sm_scale, heads=hs)
        O[int(w.q_off[s]):int(w.q_off[s + 1])] = o
        L[int(w.q_off[s]):int(w.q_off[s + 1])] = l
    rows = np.concatenate([np.arange(w.q_off[s], w.q_off[s + 1]) for s in ss])
    _check_merged(path, w, O, L, heads=hs, rows=rows)
    _check_grads(w, got, kv_heads=kv_heads, seqs=seqs)


# ---------------------------------------------------------------------------
# invariants at any size
# ---------------------------------------------------------------------------

def test_forward_and_merge_are_bitwise_deterministic_and_plan_independent():
    w = make("c3", seed=2, with_do=False, n_ctx_range=(3000, 9000), n_anchor=16, hq=8, hkv=2, chunk=1024)
    q, k, v = _upload(w)
    a = make_path(w, DEV, with_bwd=False)
    a.forward(q, k, v)
    o1, l1 = a.o.clone(), a.lse.clone()
    a.forward(q, k, v)
    b = make_path(w, DEV, with_bwd=False, policy="static")
    b.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, a.o) and torch.equal(l1, a.lse)
    assert torch.equal(o1, b.o) and torch.equal(l1, b.lse)


def test_poisoned_invisible_tiles_are_never_read():
    """NaN in every key tile that no draft block sees leaves outputs bitwise unchanged."""
    w = make("c2", seed=3, with_do=False, n_ctx=6000, n_anchor=8, hq=8, hkv=2, chunk=1024)
    q, k, v = _upload(w)
    path = make_path(w, DEV, with_bwd=False)
    path.forward(q, k, v)
    o1, l1 = path.o.clone(), path.lse.clone()
    e_max = int(min(w.anchors.max() + w.cfg.block, 6000))
    first_dead_tile = -(-e_max // 64) * 64
    assert first_dead_tile < 6000
    k2, v2 = k.clone(), v.clone()
    k2[first_dead_tile:] = float("nan")
    v2[first_dead_tile:] = float("inf")
    path.forward(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(o1, path.o) and torch.equal(l1, path.lse)


def test_split_matches_single_chunk():
    """Split-then-merge equals the unsplit result (one chunk covering the context)."""
    w = make("c2", seed=4, with_do=False, n_ctx=5000, n_anchor=8, hq=8, hkv=2, chunk=512)
    q, k, v = _upload(w)
    a = make_path(w, DEV, with_bwd=False)
    a.forward(q, k, v)
    import dataclasses
    w1 = dataclasses.replace(w, cfg=dataclasses.replace(w.cfg, chunk=5056))
    b = make_path(w1, DEV, with_bwd=False)
    b.forward(q, k, v)
    torch.cuda.synchronize()
    assert_close("split vs unsplit O", to_np64(a.o), to_np64(b.o), 4e-3, 4e-3)
    assert_lse("split vs unsplit LSE", to_np64(a.lse), to_np64(b.lse), 1e-5)


def test_identical_keys_and_constant_values():
    """Identical keys: O = mean of the visible V rows, dQ = 0.  Constant V: O = v."""
    w = make("c2", seed=5, with_do=True, n_ctx=3000, n_anchor=8, hq=4, hkv=2, chunk=1024)
    w.k[:] = w.k[0:1]
    q, k, v = _upload(w)
    path = make_path(w, DEV, with_bwd=True)
    dq, dk, dv = _bwd(w, path, q, k, v)
    O, _ = oracle.attention_workload(w)
    assert_close("O (identical keys)", to_np64(path.o), O, BF16_ABS, BF16_FROB)
    assert np.abs(dq).max() < 5e-3
    w.v[:] = w.v[5:6]
    q, k, v = _upload(w)
    path.forward(q, k, v)
    torch.cuda.synchronize()
    o = to_np64(path.o)
    for h in range(w.cfg.hq):
        vv = w.as_f64("v", rows=slice(5, 6))[0, h // 2]
        assert np.abs(o[:, h] - vv).max() <= 2 ** -7 * np.abs(vv).max()


def test_backward_bitwise_deterministic_across_plans_and_stealing():
    """The backward has no atomics: dQ, dK, dV are bitwise the same on a rerun,
    under the static plan, with tail stealing off, and on grids of 13 (not a
    multiple of the 8 XCDs, so workgroups map to workers one to one) and 600
    workgroups (more than the compute units); every workgroup reports its busy
    time when asked."""
    w = make("c3", seed=6, with_do=True, n_ctx_range=(2000, 7000), n_anchor=12, hq=8, hkv=2, chunk=1024)
    q, k, v = _upload(w)
    ref = None
    for kw in (dict(), dict(), dict(policy="static"), dict(steal=False, ticks=True),
               dict(policy="static", steal=False, ticks=True), dict(n_workers=13, ticks=True),
               dict(n_workers=600, steal=False)):
        path = make_path(w, DEV, with_bwd=True, bwd_granule=128, **kw)
        do = to_device(w, "do", DEV)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        path.forward(q, k, v)
        path.backward(q, k, v, do, dq, dk, dv)
        torch.cuda.synchronize()
        got = (path.o.clone(), path.lse.clone(), dq, dk, dv)
        if ref is None:
            ref = got
            _check_grads(w, (to_np64(dq), to_np64(dk), to_np64(dv)))
        else:
            for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), ref, got):
                assert torch.equal(a, b), f"{name} differs under {kw}"
        if kw.get("ticks"):
            for plan in (path.fwd_plan, path.bwd_plan, path.dq_plan):
                t = plan.ticks.cpu().numpy()
                busy = np.diff(plan.worker_off) > 0
                assert (t >= 0).all() and (t[busy] > 0).all()


# ---------------------------------------------------------------------------
# own-block mask variant: context prefix [0, a_b) plus the block's own keys
# ---------------------------------------------------------------------------

OWN_CASES = {
    "c3_small": ("c3", dict(n_ctx_range=(500, 2500), n_anchor=6, hq=8, hkv=2, chunk=512)),
    "c5_small": ("c5", dict(n_ctx=4100, n_anchor=12, hq=4, hkv=4, chunk=1024)),   # G = 1, 32-token blocks
    "c4_small": ("c4", dict(n_ctx=8192, n_anchor=8, hq=4, hkv=1, chunk=256)),     # G = 4, many chunks
    # the largest own-block shapes the C ABI accepts: block 64 with G = 1
    # (G * block^2 = 4096) and with G = 2 (8192: the own-block backward's
    # largest LDS footprint)
    "b64_g1": ("c5", dict(n_ctx=3000, n_anchor=6, block=64, hq=4, hkv=4, chunk=512)),
    "b64_g2": ("c3", dict(n_ctx_range=(1500, 3000), n_anchor=5, block=64, hq=4, hkv=2, chunk=512)),
}


def _own_upload(w):
    return to_device(w, "k_own", DEV), to_device(w, "v_own", DEV)


@pytest.mark.parametrize("seed", [0, 1])
def test_c1_fp32_own_block_forward(seed):
    """The fp32 tiny config under the own-block reading of its mask."""
    w = add_own_block(make("c1", seed=seed))
    path = make_path(w, DEV, mask="own_block")
    q, k, v = _upload(w)
    ko, vo = _own_upload(w)
    path.forward(q, k, v, k_own=ko, v_own=vo)
    torch.cuda.synchronize()
    O, L = oracle.attention_own_workload(w)
    assert np.isfinite(to_np64(path.lse)).all()
    _check_merged(path, w, O, L, abs_tol=F32_ABS, frob_tol=None, lse_tol=F32_ABS)
    # the own-block partial of each sequence sits after its chunks
    for s in range(w.cfg.n_seq):
        qs = slice(int(w.q_off[s]), int(w.q_off[s + 1]))
        o, m, lse = oracle.own_partial(w.as_f64("q", rows=qs), w.as_f64("k_own", rows=qs), w.as_f64("v_own", rows=qs),
                                       w.cfg.block, w.sm_scale, w.cfg.hkv)
        go, gm, gl = [to_np64(t)[-1] for t in path.partial_view(s)]
        assert_lse(f"seq{s} own lse", gl, lse, F32_ABS)
        assert_close(f"seq{s} own o", go * np.exp(gm - gl)[..., None], o * np.exp(m - lse)[..., None], F32_ABS)


@pytest.mark.parametrize("case", sorted(OWN_CASES))
def test_bf16_own_block_forward_and_backward(case):
    cfg, over = OWN_CASES[case]
    w = add_own_block(make(cfg, seed=13, with_do=True, **over))
    path = make_path(w, DEV, with_bwd=True, bwd_granule=192, mask="own_block", fwd_runs_per_worker=2,
                     fwd_run_imbalance=None)
    q, k, v = _upload(w)
    ko, vo = _own_upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
    path.forward(q, k, v, k_own=ko, v_own=vo)
    path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
    torch.cuda.synchronize()
    O, L = oracle.attention_own_workload(w)
    _check_merged(path, w, O, L)
    rq, rk, rv, rko, rvo = oracle.bwd_own_workload(w)
    assert_close("dQ", to_np64(dq), rq, BF16_ABS, BF16_FROB)
    assert_close("dK", to_np64(dk), rk, BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv), rv, BF16_ABS, BF16_FROB)
    assert_close("dK_own", to_np64(dko), rko, BF16_ABS, BF16_FROB)
    assert_close("dV_own", to_np64(dvo), rvo, BF16_ABS, BF16_FROB)


def test_bf16_own_block_matches_prefix_mask_when_own_keys_are_context_keys():
    """Own keys copied from the context at [a_b, a_b + B): the own-block path
    reproduces the prefix-mask path's O, LSE and dQ (up to rounding), and its
    dK_own / dV_own scattered back complete the prefix path's dK / dV."""
    w = make_custom([1000, 700], [[0, 40, 41, 500], [3, 64, 300, 684]], block=16, hq=8, hkv=2, d=128,
                    dtype="bf16", chunk=128, seed=21, with_do=True)
    w = add_own_block(w, from_context=True)
    q, k, v = _upload(w)
    ko, vo = _own_upload(w)
    do = to_device(w, "do", DEV)
    res = {}
    for mask in ("prefix", "own_block"):
        path = make_path(w, DEV, with_bwd=True, mask=mask)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
        if mask == "prefix":
            path.forward(q, k, v)
            path.backward(q, k, v, do, dq, dk, dv)
        else:
            path.forward(q, k, v, k_own=ko, v_own=vo)
            path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
        torch.cuda.synchronize()
        res[mask] = [to_np64(t) for t in (path.o, path.lse, dq, dk, dv, dko, dvo)]
    a, b = res["prefix"], res["own_block"]
    assert_close("O", b[0], a[0], BF16_ABS, BF16_FROB)
    assert_lse("LSE", b[1], a[1], BF16_LSE_REL)
    assert_close("dQ", b[2], a[2], BF16_ABS, BF16_FROB)
    dk_sum, dv_sum = b[3].copy(), b[4].copy()
    B = w.cfg.block
    for s in range(w.cfg.n_seq):
        k0, t0 = int(w.kv_off[s]), int(w.q_off[s])
        for bi, an in enumerate(w.seq_anchors(s)):
            rows = slice(t0 + bi * B, t0 + (bi + 1) * B)
            dk_sum[k0 + an:k0 + an + B] += b[5][rows]
            dv_sum[k0 + an:k0 + an + B] += b[6][rows]
    assert_close("dK", dk_sum, a[3], 2 * BF16_ABS, BF16_FROB)
    assert_close("dV", dv_sum, a[4], 2 * BF16_ABS, BF16_FROB)


@pytest.mark.parametrize("cfg,g", [("c3", 1), ("c5", 9)])
def test_full_size_own_block_sampled(cfg, g):
    """Own-block mask at full c3 and c5 sizes in the bench's configuration
    (default chunk runs, 256 workgroups), checked against the oracle on one
    sequence and one KV head (c4's shape is covered under the prefix mask)."""
    w = add_own_block(make(cfg, seed=0))
    path = make_path(w, DEV, mask="own_block", fwd_runs_per_worker=4)
    q, k, v = _upload(w)
    ko, vo = _own_upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
    path.forward(q, k, v, k_own=ko, v_own=vo)
    path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
    torch.cuda.synchronize()
    s = 0
    G = w.cfg.hq // w.cfg.hkv
    hs = list(range(g * G, (g + 1) * G))
    qs = slice(int(w.q_off[s]), int(w.q_off[s + 1]))
    ks = slice(int(w.kv_off[s]), int(w.kv_off[s + 1]))
    f = w.as_f64
    rq, rk, rv, rko, rvo, O, L = oracle.attention_own_bwd(
        f("q", rows=qs), f("k", rows=ks), f("v", rows=ks), f("k_own", rows=qs), f("v_own", rows=qs),
        w.seq_anchors(s), w.cfg.block, w.sm_scale, f("do", rows=qs), kv_heads=[g])
    assert_close("O", to_np64(path.o)[qs][:, hs], O[:, hs], BF16_ABS, BF16_FROB)
    assert_lse("LSE", to_np64(path.lse)[qs][:, hs], L[:, hs], BF16_LSE_REL)
    assert_close("dQ", to_np64(dq)[qs][:, hs], rq[:, hs], BF16_ABS, BF16_FROB)
    assert_close("dK", to_np64(dk)[ks][:, g], rk[:, g], BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv)[ks][:, g], rv[:, g], BF16_ABS, BF16_FROB)
    assert_close("dK_own", to_np64(dko)[qs][:, g], rko[:, g], BF16_ABS, BF16_FROB)
    assert_close("dV_own", to_np64(dvo)[qs][:, g], rvo[:, g], BF16_ABS, BF16_FROB)


@pytest.mark.parametrize("mask", ["prefix", "own_block"])
def test_bf16_edge_sequences_both_masks(mask):
    """An empty context (its rows see nothing under the prefix mask, only their
    own keys under the own-block mask), anchors at 0, duplicated and at N - 1,
    a context shorter than one tile; forward with chunk runs, then backward."""
    w = make_custom([0, 1000, 50], [[0, 0, 0, 0], [0, 0, 500, 999], [0, 10, 20, 49]], block=16, hq=8, hkv=2,
                    d=128, dtype="bf16", chunk=128, seed=31, with_do=True)
    if mask == "own_block":
        add_own_block(w)
    path = make_path(w, DEV, with_bwd=True, mask=mask, n_workers=16, fwd_runs_per_worker=2,
                     fwd_run_imbalance=None)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if mask == "own_block":
        ko, vo = _own_upload(w)
        dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
        path.forward(q, k, v, k_own=ko, v_own=vo)
        path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
        torch.cuda.synchronize()
        O, L = oracle.attention_own_workload(w)
        rq, rk, rv, rko, rvo = oracle.bwd_own_workload(w)
        assert_close("dK_own", to_np64(dko), rko, BF16_ABS, BF16_FROB)
        assert_close("dV_own", to_np64(dvo), rvo, BF16_ABS, BF16_FROB)
    else:
        path.forward(q, k, v)
        path.backward(q, k, v, do, dq, dk, dv)
        torch.cuda.synchronize()
        O, L = oracle.attention_workload(w)
        rq, rk, rv = oracle.bwd_workload(w)[:3]
        assert np.all(to_np64(path.lse)[:64] == -np.inf) and np.all(to_np64(path.o)[:64] == 0)
    _check_merged(path, w, O, L)
    assert_close("dQ", to_np64(dq), rq, BF16_ABS, BF16_FROB)
    assert_close("dK", to_np64(dk), rk, BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv), rv, BF16_ABS, BF16_FROB)


@pytest.mark.parametrize("mask", ["prefix", "own_block"])
def test_bf16_more_than_64_partials_per_row(mask):
    """71 chunks of 128 keys (72 partials per row with the own-block one), one
    partial per chunk: the merge lists a row's nonzero weights 64 partials at a
    time, so late anchors take its second block; the dQ finalize sums as many
    partials.  Forward, both merges and backward against the oracle."""
    w = make("c4", seed=70, with_do=True, n_ctx=9000, n_anchor=8, hq=4, hkv=1, chunk=128)
    # three blocks whose context prefix (under either mask) spans more than 64 chunks
    assert -(-9000 // 128) == 71 and int(np.sum(w.anchors > 64 * 128)) == 3
    if mask == "own_block":
        add_own_block(w)
    path = make_path(w, DEV, with_bwd=True, mask=mask, fwd_runs_per_worker=None)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if mask == "own_block":
        ko, vo = _own_upload(w)
        dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
        path.forward(q, k, v, k_own=ko, v_own=vo)
        o_all, l_all = path.o.clone(), path.lse.clone()
        path.merge_per_sequence()
        path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
        torch.cuda.synchronize()
        O, L = oracle.attention_own_workload(w)
        rq, rk, rv, rko, rvo = oracle.bwd_own_workload(w)
        assert_close("dK_own", to_np64(dko), rko, BF16_ABS, BF16_FROB)
        assert_close("dV_own", to_np64(dvo), rvo, BF16_ABS, BF16_FROB)
    else:
        path.forward(q, k, v)
        o_all, l_all = path.o.clone(), path.lse.clone()
        path.merge_per_sequence()
        path.backward(q, k, v, do, dq, dk, dv)
        torch.cuda.synchronize()
        O, L = oracle.attention_workload(w)
        rq, rk, rv = oracle.bwd_workload(w)[:3]
    assert torch.equal(o_all, path.o) and torch.equal(l_all, path.lse)
    _check_merged(path, w, O, L)
    assert_close("dQ", to_np64(dq), rq, BF16_ABS, BF16_FROB)
    assert_close("dK", to_np64(dk), rk, BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv), rv, BF16_ABS, BF16_FROB)


MAX_KV_HEADS, MAX_D = 4, 128
MAX_N = (2**31 - 1) // (MAX_KV_HEADS * MAX_D * 2)   # 2,097,151 keys: the longest sequence the C ABI accepts


@pytest.mark.parametrize("mask", ["prefix", "own_block"])
def test_bf16_longest_sequence_the_abi_accepts(mask):
    """One sequence whose packed K/V rows span 2^31 - 1024 bytes, the most that
    32-bit buffer offsets address: the last block's window is cut at N (ragged)
    and reaches the last key (the prefix mask; the own-block window stops 11
    keys short of it), a middle block ends near 2^20 keys, in the bench's
    plan (chunk runs).  Forward, backward and every gradient of KV head 3 (the
    highest byte offsets) against the oracle over all N keys.  K/V rows repeat
    with an odd prime period, so no power-of-two addressing error lands on an
    identical row."""
    n = MAX_N
    w = make_custom([n], [[0, 1_048_570, n - 11]], block=16, hq=MAX_KV_HEADS, hkv=MAX_KV_HEADS, d=MAX_D,
                    dtype="bf16", chunk=8192, seed=3, with_do=True, kv_period=16411)
    if mask == "own_block":
        add_own_block(w)
    path = make_path(w, DEV, with_bwd=True, mask=mask, fwd_runs_per_worker=4)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    g = MAX_KV_HEADS - 1
    f = w.as_f64
    q64, do64 = f("q")[:, [g]], f("do")[:, [g]]
    k64, v64 = f("k", head=g)[:, None], f("v", head=g)[:, None]
    if mask == "own_block":
        ko, vo = _own_upload(w)
        dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
        path.forward(q, k, v, k_own=ko, v_own=vo)
        path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
        torch.cuda.synchronize()
        rq, rk, rv, rko, rvo, O, L = oracle.attention_own_bwd(
            q64, k64, v64, f("k_own", head=g)[:, None], f("v_own", head=g)[:, None], w.seq_anchors(0),
            w.cfg.block, w.sm_scale, do64)
        assert_close("dK_own", to_np64(dko[:, g]), rko[:, 0], BF16_ABS, BF16_FROB)
        assert_close("dV_own", to_np64(dvo[:, g]), rvo[:, 0], BF16_ABS, BF16_FROB)
    else:
        path.forward(q, k, v)
        path.backward(q, k, v, do, dq, dk, dv)
        torch.cuda.synchronize()
        rq, rk, rv, O, L = oracle.attention_bwd(q64, k64, v64, w.seq_anchors(0), w.cfg.block, w.sm_scale, do64)
    assert_close("O", to_np64(path.o[:, g]), O[:, 0], BF16_ABS, BF16_FROB)
    assert_lse("LSE", to_np64(path.lse[:, g]), L[:, 0], BF16_LSE_REL)
    assert_close("dQ", to_np64(dq[:, g]), rq[:, 0], BF16_ABS, BF16_FROB)
    del k64, v64
    assert_close("dK", to_np64(dk[:, g]), rk[:, 0], BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv[:, g]), rv[:, 0], BF16_ABS, BF16_FROB)
    # the prefix mask's last window reaches key N - 1; the own-block mask's
    # ends at its anchor, N - 11, and the 11 keys after it get exactly zero
    last = n - 1 if mask == "prefix" else n - 12
    assert np.abs(rk[last, 0]).max() > 0 and np.abs(rv[last, 0]).max() > 0
    if mask == "own_block":
        assert not torch.any(dk[last + 1:]) and not torch.any(dv[last + 1:])


ODD_SHAPES = {
    # (block, hq, hkv): rows per (draft block, KV head) G*B = 16, 15, 1 and 80, so
    # the 32-row query tiles of the backward end in padding rows and the packed
    # row index splits at odd strides
    "gb16": (16, 2, 2),
    "gb15": (5, 6, 2),
    "gb1": (1, 4, 4),
    "gb80": (40, 2, 1),
}


@pytest.mark.parametrize("mask", ["prefix", "own_block"])
@pytest.mark.parametrize("shape", sorted(ODD_SHAPES))
def test_bf16_odd_block_and_group_sizes(shape, mask):
    """Forward, merge and backward at draft-block sizes and GQA groups whose
    row counts are not multiples of the kernels' tiles, two ragged sequences."""
    block, hq, hkv = ODD_SHAPES[shape]
    rng = np.random.default_rng(61)
    anchors = [sorted(rng.integers(0, 1500, size=9).tolist()), sorted(rng.integers(0, 700, size=9).tolist())]
    anchors[0][-1] = 1499  # a block reaching the end of the context
    w = make_custom([1500, 700], anchors, block=block, hq=hq, hkv=hkv, d=128, dtype="bf16", chunk=256, seed=62,
                    with_do=True)
    if mask == "own_block":
        add_own_block(w)
    path = make_path(w, DEV, with_bwd=True, mask=mask, fwd_runs_per_worker=2, fwd_run_imbalance=None)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if mask == "own_block":
        ko, vo = _own_upload(w)
        dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
        path.forward(q, k, v, k_own=ko, v_own=vo)
        path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
        torch.cuda.synchronize()
        O, L = oracle.attention_own_workload(w)
        rq, rk, rv, rko, rvo = oracle.bwd_own_workload(w)
        assert_close("dK_own", to_np64(dko), rko, BF16_ABS, BF16_FROB)
        assert_close("dV_own", to_np64(dvo), rvo, BF16_ABS, BF16_FROB)
    else:
        path.forward(q, k, v)
        path.backward(q, k, v, do, dq, dk, dv)
        torch.cuda.synchronize()
        O, L = oracle.attention_workload(w)
        rq, rk, rv = oracle.bwd_workload(w)[:3]
    _check_merged(path, w, O, L)
    assert_close("dQ", to_np64(dq), rq, BF16_ABS, BF16_FROB)
    assert_close("dK", to_np64(dk), rk, BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv), rv, BF16_ABS, BF16_FROB)


def test_bf16_strided_views_through_the_c_abi():
    """Q, O, dO and dQ as views with a padding head slot; K and V as two halves
    of one packed [N, 2, hkv + 1, d] tensor, dK and dV likewise.  The C ABI
    takes the row and head strides; every output equals the contiguous run
    bitwise, NaN padding in the inputs is never read and the outputs' padding
    is never written."""
    from block_sparse_draft_amd import binding as B
    w = make("c3", seed=71, with_do=True, n_ctx_range=(900, 2100), n_anchor=5, hq=8, hkv=2, chunk=512)
    c = w.cfg
    path = make_path(w, DEV, with_bwd=True, fwd_runs_per_worker=2, fwd_run_imbalance=None)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    path.forward(q, k, v)
    ref_o, ref_l = path.o.clone(), path.lse.clone()
    path.backward(q, k, v, do, dq, dk, dv)
    torch.cuda.synchronize()

    tq, tk, hq, hkv, d = q.shape[0], k.shape[0], c.hq, c.hkv, c.d
    nan, mark = float("nan"), 7.0
    bf = dict(dtype=torch.bfloat16, device=DEV)
    Qb = torch.full((tq, hq + 1, d), nan, **bf); Qb[:, :hq] = q
    DOb = torch.full((tq, hq + 1, d), nan, **bf); DOb[:, :hq] = do
    KVb = torch.full((tk, 2, hkv + 1, d), nan, **bf); KVb[:, 0, :hkv] = k; KVb[:, 1, :hkv] = v
    Ob = torch.full((tq, hq + 1, d), mark, **bf)
    dQb = torch.full((tq, hq + 1, d), mark, **bf)
    dKVb = torch.full((tk, 2, hkv + 1, d), mark, **bf)
    lse = torch.empty((tq, hq), dtype=torch.float32, device=DEV)
    prob = B.Problem(w.q_off, w.kv_off, w.anchors, c.block, hq, hkv, d, c.chunk, B.SKV_BF16, w.sm_scale,
                     q_strides=((hq + 1) * d, d), kv_strides=(2 * (hkv + 1) * d, d), device=DEV)
    prob.check()
    B.sparse_attn_partial_fwd(prob, path.fwd_plan, Qb[:, :hq], KVb[:, 0, :hkv], KVb[:, 1, :hkv], path.o_part,
                              path.m_part, path.lse_part)
    B.lse_merge_all(prob, path.d_part_base, path.o_part, path.m_part, path.lse_part, Ob[:, :hq], lse)
    B.sparse_attn_bwd(prob, path.bwd_plan, path.dq_plan, Qb[:, :hq], KVb[:, 0, :hkv], KVb[:, 1, :hkv], Ob[:, :hq],
                      lse, DOb[:, :hq], dQb[:, :hq], dKVb[:, 0, :hkv], dKVb[:, 1, :hkv], path.workspace)
    torch.cuda.synchronize()
    assert torch.equal(Ob[:, :hq], ref_o) and torch.equal(lse, ref_l)
    assert torch.equal(dQb[:, :hq], dq)
    assert torch.equal(dKVb[:, 0, :hkv], dk) and torch.equal(dKVb[:, 1, :hkv], dv)
    assert bool((Ob[:, hq] == mark).all()) and bool((dQb[:, hq] == mark).all())
    assert bool((dKVb[:, :, hkv] == mark).all())


def test_side_streams_match_the_default_stream():
    """Steps replanned and run on a caller's side streams (forward on one,
    backward on another, one step passing raw stream handles): the plan copy
    goes to the stream of the step's first kernel call, and every result equals
    the default-stream one bitwise."""
    w = make("c3", seed=81, with_do=True, n_ctx_range=(900, 2100), n_anchor=5, hq=8, hkv=2, chunk=512)
    path = make_path(w, DEV, with_bwd=True, fwd_runs_per_worker=2, fwd_run_imbalance=None)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    path.forward(q, k, v)
    ref_o, ref_l = path.o.clone(), path.lse.clone()
    path.backward(q, k, v, do, dq, dk, dv)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for step in range(3):
        path.replan()
        dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        a1, a2 = (s1, s2) if step != 1 else (s1.cuda_stream, s2.cuda_stream)
        s1.wait_stream(torch.cuda.current_stream())
        path.forward(q, k, v, stream=a1)
        s2.wait_stream(s1)
        path.backward(q, k, v, do, dq2, dk2, dv2, stream=a2)
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        assert torch.equal(path.o, ref_o) and torch.equal(path.lse, ref_l), step
        assert torch.equal(dq2, dq) and torch.equal(dk2, dk) and torch.equal(dv2, dv), step


@pytest.mark.parametrize("mask", ["prefix", "own_block"])
def test_bf16_batch_without_queries(mask):
    """No draft blocks at all (zero query rows; empty tensors may have NULL
    data pointers): the forward computes nothing, and the backward still writes
    exact zeros to every dK / dV row."""
    w = make_custom([300, 0, 77], [[], [], []], block=16, hq=4, hkv=2, d=128, dtype="bf16", chunk=128, seed=91,
                    with_do=True)
    if mask == "own_block":
        add_own_block(w)
    path = make_path(w, DEV, with_bwd=True, mask=mask)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    assert q.shape[0] == 0 and k.shape[0] == 377
    dq = torch.empty_like(q)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    if mask == "own_block":
        ko, vo = _own_upload(w)
        o, lse = path.forward(q, k, v, k_own=ko, v_own=vo)
        path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, torch.empty_like(ko), torch.empty_like(vo)))
    else:
        o, lse = path.forward(q, k, v)
        path.backward(q, k, v, do, dq, dk, dv)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and lse.shape[0] == 0
    assert bool((dk == 0).all()) and bool((dv == 0).all())


@pytest.mark.parametrize("mask", ["prefix", "own_block"])
def test_merge_all_equals_per_sequence_merge(mask):
    """The one-launch merge of every sequence gives bitwise the per-sequence
    lse_merge results (sequences of different lengths, rows straddling
    workgroup boundaries, a sequence without context)."""
    w = make_custom([0, 900, 3000], [[0, 5, 9], [3, 300, 880], [10, 1500, 2999]], block=16, hq=8, hkv=2, d=128,
                    dtype="bf16", chunk=256, seed=41, with_do=False)
    kw = {}
    if mask == "own_block":
        add_own_block(w)
    path = make_path(w, DEV, mask=mask)
    q, k, v = _upload(w)
    if mask == "own_block":
        kw = dict(zip(("k_own", "v_own"), _own_upload(w)))
    path.partial_fwd(q, k, v, **kw)
    path.merge()
    torch.cuda.synchronize()
    o1, l1 = path.o.clone(), path.lse.clone()
    path.o.zero_()
    path.lse.zero_()
    path.merge_per_sequence()
    torch.cuda.synchronize()
    assert torch.equal(path.o, o1) and torch.equal(path.lse, l1)
    O, L = oracle.attention_own_workload(w) if mask == "own_block" else oracle.attention_workload(w)
    _check_merged(path, w, O, L)


# ---------------------------------------------------------------------------
# seeded random problems: shapes, masks and plans drawn together
# ---------------------------------------------------------------------------

def _random_problem(seed, dtype="bf16"):
    """One random problem: 1-4 sequences of 0-3000 keys, 1-6 anchors each
    (some past the context end), any draft-block size up to 64, GQA groups of
    1-8, chunks of 64-1024 keys, either mask where its limits allow, and a
    random plan (LPT with or without chunk runs, or static; 1-256 workgroups;
    stealing on or off; backward key ranges of 64-512); fp32 problems also
    draw a head dim of 64 or 128."""
    r = np.random.default_rng([71 if dtype == "bf16" else 72, seed])
    n_seq = int(r.integers(1, 5))
    hkv = int(r.choice([1, 2, 4]))
    group = int(r.choice([1, 2, 3, 4, 8]))
    block = int(r.choice([1, 2, 3, 5, 8, 13, 16, 32, 64]))
    lens = [int(x) for x in r.integers(0, 3001, size=n_seq)]
    if r.random() < 0.2:
        lens[int(r.integers(n_seq))] = 0
    n_anchor = int(r.integers(1, 7))
    anchors = [[int(x) for x in r.integers(0, n + 9, size=n_anchor)] for n in lens]
    own_ok = group * block * block <= 8192
    mask = "own_block" if own_ok and r.random() < 0.5 else "prefix"
    policy = "static" if r.random() < 0.2 else "lpt"
    plan = dict(n_workers=int(r.choice([1, 5, 64, 256])), steal=bool(r.random() < 0.7), policy=policy,
                bwd_granule=int(r.choice([64, 128, 256, 512])),
                fwd_runs_per_worker=[None, 1, 2, 4][int(r.integers(4))], fwd_run_imbalance=None)
    d = 128 if dtype == "bf16" else int(r.choice([64, 128]))
    w = make_custom(lens, anchors, block=block, hq=hkv * group, hkv=hkv, d=d, dtype=dtype,
                    chunk=int(r.choice([64, 128, 256, 512, 1024])), seed=1000 + seed, with_do=dtype == "bf16")
    if mask == "own_block":
        add_own_block(w)
    return w, mask, plan


@pytest.mark.parametrize("seed", range(24))
def test_bf16_random_problems(seed):
    w, mask, plan = _random_problem(seed)
    c = w.cfg
    print(f"seed {seed}: lens {list(w.n_ctx)}, anchors/seq {c.n_anchor}, block {c.block}, hq {c.hq}, "
          f"hkv {c.hkv}, chunk {c.chunk}, mask {mask}, plan {plan}", flush=True)
    path = make_path(w, DEV, with_bwd=True, mask=mask, **plan)
    q, k, v = _upload(w)
    do = to_device(w, "do", DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if mask == "own_block":
        ko, vo = _own_upload(w)
        dko, dvo = torch.empty_like(ko), torch.empty_like(vo)
        path.forward(q, k, v, k_own=ko, v_own=vo)
        path.backward(q, k, v, do, dq, dk, dv, own=(ko, vo, dko, dvo))
        torch.cuda.synchronize()
        O, L = oracle.attention_own_workload(w)
        rq, rk, rv, rko, rvo = oracle.bwd_own_workload(w)
        assert_close("dK_own", to_np64(dko), rko, BF16_ABS, BF16_FROB)
        assert_close("dV_own", to_np64(dvo), rvo, BF16_ABS, BF16_FROB)
    else:
        path.forward(q, k, v)
        path.backward(q, k, v, do, dq, dk, dv)
        torch.cuda.synchronize()
        O, L = oracle.attention_workload(w)
        rq, rk, rv = oracle.bwd_workload(w)[:3]
    _check_merged(path, w, O, L)
    assert_close("dQ", to_np64(dq), rq, BF16_ABS, BF16_FROB)
    assert_close("dK", to_np64(dk), rk, BF16_ABS, BF16_FROB)
    assert_close("dV", to_np64(dv), rv, BF16_ABS, BF16_FROB)


@pytest.mark.parametrize("seed", range(12))
def test_fp32_random_problems_forward(seed):
    """The fp32 forward and merge on random problems drawn as above."""
    w, mask, plan = _random_problem(seed, dtype="f32")
    c = w.cfg
    print(f"seed {seed}: lens {list(w.n_ctx)}, anchors/seq {c.n_anchor}, block {c.block}, hq {c.hq}, "
          f"hkv {c.hkv}, d {c.d}, chunk {c.chunk}, mask {mask}, plan {plan}", flush=True)
    path = make_path(w, DEV, mask=mask, **plan)
    q, k, v = _upload(w)
    if mask == "own_block":
        ko, vo = _own_upload(w)
        path.forward(q, k, v, k_own=ko, v_own=vo)
        torch.cuda.synchronize()
        O, L = oracle.attention_own_workload(w)
    else:
        path.forward(q, k, v)
        torch.cuda.synchronize()
        O, L = oracle.attention_workload(w)
    _check_merged(path, w, O, L, abs_tol=F32_ABS, frob_tol=None, lse_tol=F32_ABS)
