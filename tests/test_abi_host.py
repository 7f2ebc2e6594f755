"""CPU tests of the C ABI: the library loads and exports every declared call,
host planning matches the oracle bit for bit, and invalid arguments are
rejected (before any HIP call, so no GPU is needed)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from block_sparse_draft_amd import binding as B
from synthetic import make

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_call():
    hdr = open(os.path.join(ROOT, "include", "splitkv.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", hdr, flags=re.M))
    assert {"sparse_attn_partial_fwd", "lse_merge", "sparse_attn_bwd", "lpt_plan"} <= names
    lib = C.CDLL(B.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(B.EXPORTED) == names


def _problem_from(w, device=None):
    dt = B.SKV_BF16 if w.is_bf16 else B.SKV_F32
    return B.Problem(w.q_off, w.kv_off, w.anchors, w.cfg.block, w.cfg.hq, w.cfg.hkv, w.cfg.d, w.cfg.chunk, dt,
                     w.sm_scale, device=device)


def _oracle_table(w, kind, granule):
    anchors = [w.seq_anchors(s) for s in range(w.cfg.n_seq)]
    return oracle.item_table(list(w.n_ctx), anchors, w.cfg.block, w.cfg.hq, w.cfg.hkv, w.cfg.chunk, kind, granule)


@pytest.mark.parametrize("cfg,over", [
    ("c1", {}), ("c2", {}), ("c3", {}), ("c5", {}),
    ("c3", {"n_ctx_range": (100, 2000), "chunk": 128}),
])
@pytest.mark.parametrize("kind,granule", [("fwd", 1), ("fwd", 4), ("bwd", 64), ("bwd", 256)])
def test_item_table_matches_oracle(cfg, over, kind, granule):
    w = make(cfg, seed=1, with_do=False, **over) if cfg in ("c1", "c2") else _meta_only(cfg, over)
    p = _problem_from(w)
    items, cost, tok, total = p.item_table(B.SKV_ITEM_FWD if kind == "fwd" else B.SKV_ITEM_BWD, granule)
    desc, ocost, otok, ototal = _oracle_table(w, kind, granule)
    assert np.array_equal(cost, ocost)
    assert np.array_equal(tok, otok) and total == ototal
    assert np.array_equal(np.stack([items["seq"], items["kv_head"], items["chunk"], items["range"]], 1), desc)


def _meta_only(cfg, over):
    """Full-size metadata without drawing the big tensors."""
    from synthetic import workloads as W
    c = W.CONFIGS[cfg]
    import dataclasses
    c = dataclasses.replace(c, **over)
    rl = W._rng(1, c.cid, W.STREAM_LEN)
    if c.n_ctx_range is not None:
        n_ctx = rl.integers(c.n_ctx_range[0], c.n_ctx_range[1], size=c.n_seq, endpoint=True).astype(np.int64)
    else:
        n_ctx = np.full(c.n_seq, c.n_ctx, dtype=np.int64)
    ra = W._rng(1, c.cid, W.STREAM_ANCHOR)
    anchors = np.concatenate([W._draw_anchors(ra, c, int(n)) for n in n_ctx]).astype(np.int32)
    mq = c.n_anchor * c.block
    e = np.empty((0,), np.uint16)
    return W.Workload(c, n_ctx, anchors, np.arange(c.n_seq + 1, dtype=np.int64) * mq,
                      np.concatenate([[0], np.cumsum(n_ctx)]).astype(np.int64), e, e, e, None, c.d ** -0.5, 1)


@pytest.mark.parametrize("seed", range(25))
def test_lpt_bit_exact_with_oracle_under_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 300))
    W = int(rng.integers(1, 40))
    cost = rng.integers(0, 6, size=n) * int(rng.integers(1, 4))   # many ties, zeros
    a1, o1, f1, l1 = B.lpt_plan(cost, W)
    a2, o2, f2, l2 = oracle.lpt(cost, W)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2) and np.array_equal(f1, f2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("n_workers,shift", [(1, 54), (37, 55), (300, 54), (256, 30)])
def test_lpt_bit_exact_with_oracle_at_large_costs(n_workers, shift):
    """Totals past 2^(62 - bits(W - 1)) no longer fit the packed (load, worker)
    heap key and take the general heap ((37, 55) and (300, 54)); costs that
    span several bytes take several radix passes.  Totals stay below 2^62."""
    rng = np.random.default_rng(shift * 1000 + n_workers)
    n = 64
    big = rng.integers(0, 4, size=n) * (np.int64(1) << shift)
    small = rng.integers(0, 1 << 20, size=n)
    cost = np.where(rng.random(n) < 0.5, big, small).astype(np.int64)
    assert int(cost.sum()) < 1 << 62
    a1, o1, f1, l1 = B.lpt_plan(cost, n_workers)
    a2, o2, f2, l2 = oracle.lpt(cost, n_workers)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2) and np.array_equal(f1, f2) and np.array_equal(l1, l2)


def test_lpt_worked_example_and_degenerate_inputs():
    a, o, f, l = B.lpt_plan([3, 3, 2, 2, 2], 2)
    assert list(a) == [0, 1, 0, 1, 0] and list(l) == [7, 5]
    a, o, f, l = B.lpt_plan(np.zeros(0, np.int64), 3)
    assert len(a) == 0 and list(f) == [0, 0, 0, 0] and list(l) == [0, 0, 0]
    a, o, f, l = B.lpt_plan([5, 5], 7)
    assert list(a) == [0, 1] and list(l) == [5, 5, 0, 0, 0, 0, 0]
    with pytest.raises(B.SkvError) as e:
        B.lpt_plan([1, 2], 0)
    assert e.value.code == B.SKV_EINVAL
    with pytest.raises(B.SkvError):
        B.lpt_plan([1, -2], 2)


@pytest.mark.parametrize("cfg", ["c3", "c5"])
def test_lpt_and_static_on_full_size_items_match_oracle(cfg):
    w = _meta_only(cfg, {})
    p = _problem_from(w)
    G = w.cfg.hq // w.cfg.hkv
    items, cost, tok, total = p.item_table(B.SKV_ITEM_FWD, max(1, 256 // (G * w.cfg.block)))
    a1, o1, f1, l1 = B.lpt_plan(cost, 256)
    a2, o2, f2, l2 = oracle.lpt(cost, 256)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2) and np.array_equal(l1, l2)
    s1, so1, sf1 = B.skv_static_plan(tok, total, 256)
    s2 = oracle.static_assign(tok, total, 256)
    so2, sf2 = oracle.csr_from_assign(s2, 256)
    assert np.array_equal(s1, s2) and np.array_equal(so1, so2) and np.array_equal(sf1, sf2)
    g = B.skv_gather_items(items, o1)
    assert np.array_equal(g, items[o1])


def test_partial_layout():
    w = _meta_only("c3", {})
    p = _problem_from(w)
    base, nchunk = p.partial_layout()
    C_s = -(-w.n_ctx // w.cfg.chunk)
    assert list(nchunk) == list(C_s)
    mq = w.cfg.n_anchor * w.cfg.block
    assert list(np.diff(base)) == list(C_s * w.cfg.hq * mq)


def _bad(w, **kw):
    p = _problem_from(w)
    for k, v in kw.items():
        setattr(p.c, k, v)
    return p


def test_problem_validation_codes():
    w = make("c1", seed=0)
    assert B.lib.skv_check_problem(C.byref(_problem_from(w).c)) == B.SKV_OK
    cases = [({"hq": 3, "hkv": 2}, B.SKV_ESHAPE), ({"chunk": 100}, B.SKV_ESHAPE), ({"chunk": 0}, B.SKV_ESHAPE),
             ({"d": 96}, B.SKV_ESHAPE), ({"dtype": 7}, B.SKV_EDTYPE), ({"block": 0}, B.SKV_EINVAL),
             ({"sm_scale": float("nan")}, B.SKV_EINVAL), ({"h_anchor": None}, B.SKV_EINVAL),
             ({"q_stride_tok": 3}, B.SKV_ESHAPE), ({"n_seq": -1}, B.SKV_EINVAL),
             ({"q_stride_tok": 32}, B.SKV_ESHAPE), ({"kv_stride_tok": 32}, B.SKV_ESHAPE)]
    for kw, code in cases:
        p = _bad(w, **kw)
        assert B.lib.skv_check_problem(C.byref(p.c)) == code, kw
        assert B.last_error() != "no error"
    # bf16 supports head_dim 128 only
    p = _bad(w, dtype=B.SKV_BF16)
    assert B.lib.skv_check_problem(C.byref(p.c)) == B.SKV_ESHAPE
    # bf16 K/V rows of one sequence must span at most 2^31 bytes (32-bit buffer offsets)
    wb = make("c2", seed=0, n_ctx=1024, n_anchor=2)
    pb = _problem_from(wb)
    assert B.lib.skv_check_problem(C.byref(pb.c)) == B.SKV_OK
    pb.c.kv_stride_tok = (1 << 30) // 1024 + 8          # 1024 rows * stride * 2 bytes > 2^31
    pb.c.kv_stride_head = 128
    assert B.lib.skv_check_problem(C.byref(pb.c)) == B.SKV_ESHAPE and "2^31" in B.last_error()
    # packed [N, 4, 128] bf16 K/V: 2,097,151 keys (2^31 - 1024 bytes) pass, one key more does not
    for n, code in ((2097151, B.SKV_OK), (2097152, B.SKV_ESHAPE)):
        pm = B.Problem([0, 48], [0, n], [0, 1_048_570, n - 11], 16, 4, 4, 128, 8192, B.SKV_BF16, 0.125)
        assert B.lib.skv_check_problem(C.byref(pm.c)) == code, n
    # anchors past the context are allowed (they see all of it) up to 2^31 - 1 - block
    for a_last, code in ((5000, B.SKV_OK), (2**31 - 1 - 16, B.SKV_OK), (2**31 - 16, B.SKV_EINVAL)):
        pa = B.Problem([0, 32], [0, 1024], [3, a_last], 16, 4, 4, 128, 256, B.SKV_BF16, 0.125)
        assert B.lib.skv_check_problem(C.byref(pa.c)) == code, a_last
    # query rows start at row 0 (kernels that walk the whole batch index rows from 0)
    for q_off, code in (([0, 48], B.SKV_OK), ([16, 48], B.SKV_EINVAL)):
        pq = B.Problem(q_off, [0, 1024], [3, 5, 7][:q_off[1] // 16], 16, 4, 4, 128, 256,
                       B.SKV_BF16, 0.125)
        assert B.lib.skv_check_problem(C.byref(pq.c)) == code, q_off
    assert "q_off[0]" in B.last_error()
    # unsorted anchors
    p = _problem_from(w)
    p.h_anchor[:] = p.h_anchor[::-1].copy()
    assert B.lib.skv_check_problem(C.byref(p.c)) == B.SKV_EINVAL
    assert "sorted" in B.last_error()


def test_device_calls_reject_bad_arguments_before_touching_the_gpu():
    w = make("c1", seed=0)
    p = _problem_from(w)           # host-only: device arrays NULL
    plan = B.skv_plan(B.SKV_ITEM_FWD, 4, 1, 16, 16, 16)
    fake = C.c_void_p(4096)
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(plan), fake, fake, fake, fake, fake, fake, None)
    assert rc == B.SKV_EINVAL and "device" in B.last_error()
    # wrong plan kind
    p.c.d_q_off = p.c.d_kv_off = p.c.d_anchor = 4096
    bplan = B.skv_plan(B.SKV_ITEM_BWD, 4, 1, 16, 16, 16)
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(bplan), fake, fake, fake, fake, fake, fake, None)
    assert rc == B.SKV_EPLAN
    zplan = B.skv_plan(B.SKV_ITEM_FWD, 0, 1, 16, 16, 16)
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(zplan), fake, fake, fake, fake, fake, fake, None)
    assert rc == B.SKV_EPLAN
    nclaim = B.skv_plan(B.SKV_ITEM_FWD, 4, 1, 16, 16, None)   # claim cursors are required
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(nclaim), fake, fake, fake, fake, fake, fake, None)
    assert rc == B.SKV_EPLAN
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(plan), None, fake, fake, fake, fake, fake, None)
    assert rc == B.SKV_EINVAL
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(plan), C.c_void_p(4098), fake, fake, fake, fake, fake,
                                       None)
    assert rc == B.SKV_ESHAPE
    # bwd: fp32 problems are rejected, workspace is checked
    rc = B.lib.sparse_attn_bwd(C.byref(p.c), C.byref(bplan), C.byref(plan), *([fake] * 10), 1 << 30, None, None)
    assert rc == B.SKV_EDTYPE
    wb = make("c2", seed=0, n_ctx=256, n_anchor=2)
    pb = _problem_from(wb)
    pb.c.d_q_off = pb.c.d_kv_off = pb.c.d_anchor = 4096
    need = B.lib.skv_bwd_workspace_bytes(C.byref(pb.c))
    # dQ partials: 1 chunk (256 keys, chunk 1024) x 32 heads x 32 rows x 128 fp32, and their
    # run lengths (int32 each); packed Q and dO (1024 rows x 128 bf16 each); packed LSE, Delta,
    # prefix end (1024 x 4 bytes each); 2 offsets
    assert need == 32 * 32 * 128 * 4 + 1024 * 4 + 2 * 1024 * 128 * 2 + 3 * 1024 * 4 + 256
    qplan = B.skv_plan(B.SKV_ITEM_FWD, 4, 1, 16, 16, 32)
    rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(bplan), C.byref(qplan), *([fake] * 10), need - 1, None, None)
    assert rc == B.SKV_EWORKSPACE
    rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(bplan), C.byref(bplan), *([fake] * 10), need, None, None)
    assert rc == B.SKV_EPLAN                       # second plan must be a forward plan
    rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(bplan), C.byref(plan), *([fake] * 10), need, None, None)
    assert rc == B.SKV_EPLAN                       # shared claim cursors are rejected
    tk = B.skv_plan(B.SKV_ITEM_BWD, 4, 1, 16, 16, 48, 0, 0, 64)
    tq = B.skv_plan(B.SKV_ITEM_FWD, 4, 1, 16, 16, 32, 0, 0, 64)
    rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(tk), C.byref(tq), *([fake] * 10), need, None, None)
    assert rc == B.SKV_EPLAN and "ticks" in B.last_error()   # shared ticks arrays are rejected
    kp2 = B.skv_plan(B.SKV_ITEM_BWD, 4, 1, 16, 16, 48)
    for i in (7, 8):                               # dk, dv written with 16-byte stores
        args = [fake] * 10
        args[i] = C.c_void_p(4098)
        rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(kp2), C.byref(qplan), *args, need, None, None)
        assert rc == B.SKV_ESHAPE and "aligned" in B.last_error()
    # the no-allocation backward: the same checks, and problems whose workspace
    # exceeds the static scratch are rejected before any device work
    rc = B.lib.sparse_attn_bwd_noalloc(C.byref(pb.c), C.byref(bplan), C.byref(plan), *([fake] * 9), None, None)
    assert rc == B.SKV_EPLAN
    wbig = _meta_only("c3", {})
    pbig = _problem_from(wbig)
    pbig.c.d_q_off = pbig.c.d_kv_off = pbig.c.d_anchor = 4096
    assert B.lib.skv_bwd_workspace_bytes(C.byref(pbig.c)) > B.SKV_NOALLOC_SCRATCH_BYTES
    rc = B.lib.sparse_attn_bwd_noalloc(C.byref(pbig.c), C.byref(bplan), C.byref(qplan), *([fake] * 9), None, None)
    assert rc == B.SKV_EWORKSPACE and "static scratch" in B.last_error()
    badflags = B.skv_plan(B.SKV_ITEM_FWD, 4, 1, 16, 16, 16, 2, 0, None)
    rc = B.lib.sparse_attn_partial_fwd(C.byref(p.c), C.byref(badflags), fake, fake, fake, fake, fake, fake, None)
    assert rc == B.SKV_EPLAN and "flags" in B.last_error()
    # merge
    rc = B.lib.lse_merge(4, 2, 64, 96, fake, fake, fake, fake, 128, 64, B.SKV_F32, fake, 2, None)
    assert rc == B.SKV_ESHAPE
    rc = B.lib.lse_merge(-1, 2, 64, 64, fake, fake, fake, fake, 128, 64, B.SKV_F32, fake, 2, None)
    assert rc == B.SKV_EINVAL
    rc = B.lib.lse_merge(4, 2, 64, 64, fake, fake, fake, fake, 128, 64, 5, fake, 2, None)
    assert rc == B.SKV_EDTYPE
    assert B.lib.lse_merge(4, 2, 0, 64, None, None, None, None, 128, 64, B.SKV_F32, None, 2, None) == B.SKV_OK


def test_null_anchor_array_only_without_draft_blocks():
    """A batch without draft blocks may pass NULL anchors; one with blocks may not."""
    empty = B.Problem(np.array([0, 0, 0], np.int64), np.array([0, 300, 377], np.int64), np.zeros(0, np.int32),
                      16, 4, 2, 128, 128, B.SKV_BF16, 0.088)
    empty.c.h_anchor = None
    empty.check()
    w = make("c2", seed=0, n_ctx=4096, n_anchor=4, with_do=False)
    p = _problem_from(w)
    p.c.h_anchor = None
    with pytest.raises(B.SkvError) as e:
        p.check()
    assert e.value.code == B.SKV_EINVAL


def test_timing_api_without_launches():
    """Timing switches on and off and collects an empty tally without any GPU work."""
    B.timing_enable(True)
    assert B.timing_collect() == {}
    B.timing_enable(False)
    assert B.timing_collect() == {}
    n = C.c_int32(-1)
    assert B.lib.skv_timing_collect(None, 0, C.byref(n)) == B.SKV_OK and n.value == 0
    assert B.lib.skv_timing_collect(None, 3, C.byref(n)) == B.SKV_EINVAL


def test_plan_struct_layout():
    """skv_plan as the header lays it out on LP64: 56 bytes, d_ticks last."""
    assert C.sizeof(B.skv_plan) == 56
    assert B.skv_plan.flags.offset == 40 and B.skv_plan.d_ticks.offset == 48


def test_drop_zero_cost_matches_filtering():
    """skv_drop_zero_cost keeps each worker's nonzero-cost items in order."""
    rng = np.random.default_rng(7)
    for W in (1, 3, 16):
        cost = rng.integers(0, 4, size=200).astype(np.int64) * rng.integers(0, 2, size=200)
        _, order, off, _ = B.lpt_plan(cost, W)
        o2, w2 = B.skv_drop_zero_cost(cost, order, off)
        assert w2[0] == 0 and w2[-1] == len(o2) == int((cost != 0).sum())
        for w in range(W):
            lst = order[off[w]:off[w + 1]]
            assert np.array_equal(o2[w2[w]:w2[w + 1]], lst[cost[lst] != 0])
    # a c5-shaped forward table: LPT alone gives one worker every zero-cost item
    w = _meta_only("c5", {})
    p = _problem_from(w)
    items, cost, tok, total = p.item_table(B.SKV_ITEM_FWD, 8)
    _, order, off, _ = B.lpt_plan(cost, 256)
    counts = np.diff(off)
    assert counts.max() > 1000
    o2, w2 = B.skv_drop_zero_cost(cost, order, off)
    assert np.diff(w2).max() < 100
    bad = off.copy(); bad[-1] += 1
    with pytest.raises(B.SkvError):
        B.skv_drop_zero_cost(cost, order, bad)


@pytest.mark.parametrize("cfg,granule", [("c3", 4), ("c4", 4), ("c5", 8)])
@pytest.mark.parametrize("target", [1, 97, 2000, 1 << 40])
def test_coarsen_fwd_items_matches_oracle(cfg, granule, target):
    """skv_coarsen_fwd_items forms exactly the oracle's runs (bit-exact)."""
    w = _meta_only(cfg, {})
    p = _problem_from(w)
    items, cost, _, _ = p.item_table(B.SKV_ITEM_FWD, granule)
    assert np.all(items["n_chunk"] == 1)
    it2, c2 = B.skv_coarsen_fwd_items(items, cost, target)
    desc, ocost, _, _ = _oracle_table(w, "fwd", granule)
    first, length, rcost = oracle.coarsen_runs(desc, ocost, target)
    assert np.array_equal(c2, rcost)
    assert np.array_equal(it2["n_chunk"], length)
    ref = items[first]
    for f in ("seq", "kv_head", "chunk", "range", "part_base", "lo", "hi"):
        assert np.array_equal(it2[f], ref[f]), f


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_coarsen_fwd_items_any_input_order(seed):
    """Items in a random order (the grouping sort must not rely on the item
    table's order): runs, costs and output order still equal the oracle's on the
    same permuted table."""
    w = _meta_only("c3", {})
    p = _problem_from(w)
    items, cost, _, _ = p.item_table(B.SKV_ITEM_FWD, 4)
    desc, ocost, _, _ = _oracle_table(w, "fwd", 4)
    perm = np.random.default_rng(seed).permutation(len(cost))
    items, cost, desc, ocost = items[perm], cost[perm], desc[perm], ocost[perm]
    target = int(cost.sum() // 700) + 1
    it2, c2 = B.skv_coarsen_fwd_items(items, cost, target)
    first, length, rcost = oracle.coarsen_runs(desc, ocost, target)
    assert np.array_equal(c2, rcost) and np.array_equal(it2["n_chunk"], length)
    ref = items[first]
    for f in ("seq", "kv_head", "chunk", "range", "part_base", "lo", "hi"):
        assert np.array_equal(it2[f], ref[f]), f
    assert (length > 1).any()


@pytest.mark.parametrize("wide", [False, True])
def test_coarsen_fwd_items_wide_fields(wide):
    """Grouping keys of every width: the same constant added to a field of
    every item changes neither the groups nor chunk adjacency, so the runs stay
    the oracle's.  Wide offsets make the fields need 113 bits together (the
    grouping sort then goes field by field); narrow ones 31 bits (four
    passes of the composite-key sort, one more than without the offset)."""
    w = _meta_only("c3", {})
    p = _problem_from(w)
    items, cost, _, _ = p.item_table(B.SKV_ITEM_FWD, 4)
    desc, ocost, _, _ = _oracle_table(w, "fwd", 4)
    perm = np.random.default_rng(5).permutation(len(cost))
    items, cost, desc, ocost = items[perm].copy(), cost[perm], desc[perm], ocost[perm]
    shift = {"seq": 20, "kv_head": 21, "lo": 22, "hi": 22, "chunk": 23} if wide else {"chunk": 12}
    for f, b in shift.items():
        items[f] += np.int32(1 << b)
    target = int(cost.sum() // 700) + 1
    it2, c2 = B.skv_coarsen_fwd_items(items, cost, target)
    first, length, rcost = oracle.coarsen_runs(desc, ocost, target)
    assert np.array_equal(c2, rcost) and np.array_equal(it2["n_chunk"], length)
    for f in ("seq", "kv_head", "chunk", "range", "part_base", "lo", "hi"):
        assert np.array_equal(it2[f], items[first][f]), f
    assert (length > 1).any()


def _oracle_run_search(desc, cost, n_workers, start, stop, tol):
    """The run-length search restated on the oracle: double the runs per worker
    until LPT over the oracle's runs balances them to within tol."""
    rpw = float(start)
    total = int(np.asarray(cost, dtype=np.int64).sum())
    while True:
        target = max(1, int(np.ceil(total / (n_workers * rpw))))
        first, length, rcost = oracle.coarsen_runs(desc, cost, target)
        _, order, off, load = oracle.lpt(rcost, n_workers)
        mean = total / n_workers
        if rpw >= stop or mean == 0 or load.max() / mean - 1.0 <= tol:
            return first, length, rcost, order, off, load, rpw
        rpw = min(2 * rpw, stop)


@pytest.mark.parametrize("cfg,n_workers,start,stop,tol", [
    ("c3", 256, 4, 64, 0.02), ("c5", 256, 4, 64, 0.02), ("c4", 256, 4, 64, 0.02),
    ("c3", 13, 1, 64, 0.0), ("c5", 64, 2, 2, 0.02), ("c3", 256, 4, 64, 1e9), ("c2", 256, 0.5, 0.5, 0.02),
    ("c2", 256, 4, 64, 0.02),
    ("c5", 100, 3, 40, 0.001)])
def test_plan_fwd_runs_matches_oracle_search(cfg, n_workers, start, stop, tol):
    """skv_plan_fwd_runs picks the same run length as the search over the
    oracle's runs and LPT, and returns the same runs and plan (bit-exact)."""
    w = _meta_only(cfg, {})
    p = _problem_from(w)
    granule = max(1, 256 // ((w.cfg.hq // w.cfg.hkv) * w.cfg.block))
    items, cost, _, _ = p.item_table(B.SKV_ITEM_FWD, granule)
    it2, c2, order, off, load, rpw = B.skv_plan_fwd_runs(items, cost, n_workers, start, stop, tol)
    desc, ocost, _, _ = _oracle_table(w, "fwd", granule)
    first, length, rcost, oorder, ooff, oload, orpw = _oracle_run_search(desc, ocost, n_workers, start, stop, tol)
    assert rpw == orpw
    assert np.array_equal(c2, rcost) and np.array_equal(it2["n_chunk"], length)
    for f in ("seq", "kv_head", "chunk", "lo", "hi", "part_base"):
        assert np.array_equal(it2[f], items[first][f]), f
    assert np.array_equal(order, oorder) and np.array_equal(off, ooff) and np.array_equal(load, oload)


def test_plan_fwd_runs_rejects_bad_input():
    w = make("c2", seed=0, n_ctx=4096, n_anchor=4, with_do=False)
    p = _problem_from(w)
    items, cost, _, _ = p.item_table(B.SKV_ITEM_FWD, 1)
    for args in ((0, 4, 0.02), (4, 2, 0.02), (4, 8, -1.0), (4, 8, float("nan")), (4, float("inf"), 0.02)):
        with pytest.raises(B.SkvError):
            B.skv_plan_fwd_runs(items, cost, 8, *args)
    with pytest.raises(B.SkvError):
        B.skv_plan_fwd_runs(items, cost, 0, 4, 8, 0.02)
    it2, c2, order, off, load, rpw = B.skv_plan_fwd_runs(items[:0], cost[:0], 8, 4, 8, 0.02)
    assert len(c2) == 0 and rpw == 4 and off[-1] == 0


def test_coarsen_fwd_items_rejects_bad_input():
    w = make("c2", seed=0, n_ctx=4096, n_anchor=4, with_do=False)
    p = _problem_from(w)
    items, cost, _, _ = p.item_table(B.SKV_ITEM_FWD, 1)
    with pytest.raises(B.SkvError):
        B.skv_coarsen_fwd_items(items, cost, 0)          # target below 1
    it2, c2 = B.skv_coarsen_fwd_items(items, cost, 1 << 40)
    if (it2["n_chunk"] > 1).any():
        with pytest.raises(B.SkvError):
            B.skv_coarsen_fwd_items(it2, c2, 10)         # already coarsened
    bad = cost.copy(); bad[0] = -1
    with pytest.raises(B.SkvError):
        B.skv_coarsen_fwd_items(items, bad, 10)
    assert B.skv_coarsen_fwd_items(items[:0], cost[:0], 5)[0].shape == (0,)


def test_own_block_mask_host_side():
    """Own-block mask: the context prefix ends at the anchor (the prefix mask's
    cost with anchors moved back by B), one more partial per sequence, and the
    own-block calls reject bad shapes and missing tensors before any launch."""
    w = make("c2", seed=0, n_ctx=3000, n_anchor=8, hq=8, hkv=2, chunk=1024, with_do=False)
    p = B.Problem(w.q_off, w.kv_off, w.anchors, w.cfg.block, w.cfg.hq, w.cfg.hkv, w.cfg.d, w.cfg.chunk, B.SKV_BF16,
                  w.sm_scale, mask=B.SKV_MASK_OWN_BLOCK)
    p.check()
    items, cost, tok, total = p.item_table(B.SKV_ITEM_FWD, 1)
    anchors = [w.seq_anchors(s).astype(np.int64) - w.cfg.block for s in range(w.cfg.n_seq)]
    desc, ocost, _, _ = oracle.item_table(list(w.n_ctx), anchors, w.cfg.block, w.cfg.hq, w.cfg.hkv, w.cfg.chunk,
                                          "fwd", 1)
    assert np.array_equal(cost, ocost)
    base, nchunk = p.partial_layout()
    assert nchunk.tolist() == [3 + 1]
    assert base[-1] == 4 * w.cfg.hq * int(w.q_off[-1])
    assert np.array_equal(items["part_base"][items["chunk"] == 2], np.full((items["chunk"] == 2).sum(),
                                                                           2 * w.cfg.hq * int(w.q_off[-1])))
    fake = C.c_void_p(4096)
    pd = _problem_from(w)
    pd.c.d_q_off = pd.c.d_kv_off = pd.c.d_anchor = 4096
    # prefix-mask problem: the own-block forward is refused
    assert B.lib.sparse_attn_own_fwd(C.byref(pd.c), fake, fake, fake, 256, 128, fake, fake, fake, None) == B.SKV_EINVAL
    pd.c.mask = B.SKV_MASK_OWN_BLOCK
    assert B.lib.sparse_attn_own_fwd(C.byref(pd.c), fake, fake, fake, 100, 128, fake, fake, fake, None) == B.SKV_ESHAPE
    assert B.lib.sparse_attn_own_fwd(C.byref(pd.c), fake, None, fake, 256, 128, fake, fake, fake, None) == B.SKV_EINVAL
    pd.c.mask = 7
    assert B.lib.skv_check_problem(C.byref(pd.c)) == B.SKV_EINVAL
    pd.c.mask = B.SKV_MASK_OWN_BLOCK
    pd.c.block, pd.c.hq = 64, 8     # (hq/hkv) * block^2 = 4 * 4096 > 8192
    assert B.lib.sparse_attn_own_fwd(C.byref(pd.c), fake, fake, fake, 256, 128, fake, fake, fake, None) in (
        B.SKV_ESHAPE, B.SKV_EINVAL)
    # backward: the own-block mask needs its tensors
    pb = _problem_from(w)
    pb.c.d_q_off = pb.c.d_kv_off = pb.c.d_anchor = 4096
    pb.c.mask = B.SKV_MASK_OWN_BLOCK
    need = B.lib.skv_bwd_workspace_bytes(C.byref(pb.c))
    bplan = B.skv_plan(B.SKV_ITEM_BWD, 4, 1, 16, 16, 48)
    qplan = B.skv_plan(B.SKV_ITEM_FWD, 4, 1, 16, 16, 32)
    rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(bplan), C.byref(qplan), *([fake] * 10), need, None, None)
    assert rc == B.SKV_EINVAL
    own = B.skv_own_block(4096, 4096, 4096, 4096, 256, 128)
    pb.c.mask = B.SKV_MASK_PREFIX
    need2 = B.lib.skv_bwd_workspace_bytes(C.byref(pb.c))
    assert need2 < need                                       # one partial fewer per sequence
    rc = B.lib.sparse_attn_bwd(C.byref(pb.c), C.byref(bplan), C.byref(qplan), *([fake] * 10), need, C.byref(own), None)
    assert rc == B.SKV_EINVAL                                 # own-block tensors with the prefix mask
