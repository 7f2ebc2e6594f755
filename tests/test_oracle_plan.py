"""Pins for the planning oracle: LPT against the brute-force optimum and the
Graham bound, a printed tight instance, the cost model against brute-force
enumeration of a dense mask, and the static plan's defining properties."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_graham_tight_instance():
    g = json.load(open(os.path.join(GOLDEN, "lpt_graham_tight.json")))
    assign, order, off, load = oracle.lpt(g["cost"], g["n_workers"])
    assert list(assign) == g["assign"]
    assert list(load) == g["load"]
    assert oracle.brute_force_makespan(g["cost"], g["n_workers"]) == g["optimum"]
    assert max(load) / g["optimum"] == pytest.approx(oracle.graham_bound(2))


@pytest.mark.parametrize("seed", range(40))
def test_lpt_within_graham_bound_of_optimum(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 4))
    n = int(rng.integers(0, 10))
    cost = rng.integers(0, 20, size=n)
    _, _, _, load = oracle.lpt(cost, m)
    opt = oracle.brute_force_makespan(cost, m)
    mk = int(load.max()) if n else 0
    assert mk >= opt
    assert mk <= oracle.graham_bound(m) * opt + 1e-9


def test_lpt_rule_step_by_step():
    """Each item in (cost desc, id asc) order goes to the least-loaded worker,
    lowest id on ties; worker lists keep assignment order."""
    cost = np.array([5, 1, 5, 3, 0, 3, 2, 2])
    assign, order, off, load = oracle.lpt(cost, 3)
    # order of visit: 0(5),2(5),3(3),5(3),6(2),7(2),1(1),4(0)
    # w0<-0 (5), w1<-2 (5), w2<-3 (3), w2<-5 (6), w0<-6 (7), w1<-7 (7), w2<-1? loads (7,7,6) -> w2 (7), w0<-4 (7,7,7 -> w0)
    assert list(assign) == [0, 2, 1, 2, 0, 2, 0, 1]
    assert list(load) == [7, 7, 7]
    assert list(off) == [0, 3, 5, 8]
    assert list(order) == [0, 6, 4, 2, 7, 3, 5, 1]


def test_lpt_degenerate_inputs():
    a, o, off, load = oracle.lpt([], 4)
    assert len(a) == 0 and list(off) == [0] * 5 and list(load) == [0] * 4
    a, o, off, load = oracle.lpt([7, 7, 7], 8)       # more workers than items
    assert list(a) == [0, 1, 2] and list(load) == [7, 7, 7, 0, 0, 0, 0, 0]
    a, o, off, load = oracle.lpt([0, 0, 0, 0], 2)    # zero costs are planned too:
    assert list(a) == [0, 0, 0, 0]                   # load ties -> lowest worker id
    with pytest.raises(ValueError):
        oracle.lpt([1], 0)


def _brute_costs(n_ctx, anchors, B, hq, hkv, L, kind, granule, T=64):
    """Count (block, 64-key tile) pairs with >= 1 visible element from the dense
    mask, per item, times the query heads per KV head."""
    G = hq // hkv
    out = []
    for N, anc in zip(n_ctx, anchors):
        mask = oracle.visible_mask(anc, B, N)               # [A*B, N]
        A = len(anc)
        C = -(-N // L)
        for g in range(hkv):
            for c in range(C):
                lo, hi = c * L, min((c + 1) * L, N)
                if kind == "fwd":
                    for r in range(-(-A // granule)):
                        tot = 0
                        for b in range(r * granule, min((r + 1) * granule, A)):
                            for t0 in range(lo, hi, T):
                                tot += bool(mask[b * B:(b + 1) * B, t0:min(t0 + T, hi)].any())
                        out.append(G * tot)
                else:
                    for klo in range(lo, hi, granule):
                        khi = min(klo + granule, hi)
                        tot = 0
                        for b in range(A):
                            for t0 in range(klo, khi, T):
                                tot += bool(mask[b * B:(b + 1) * B, t0:min(t0 + T, khi)].any())
                        out.append(G * tot)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("kind,granule", [("fwd", 1), ("fwd", 3), ("bwd", 64), ("bwd", 192)])
def test_cost_model_matches_dense_mask_enumeration(kind, granule):
    rng = np.random.default_rng(3)
    n_ctx = [1000, 257, 640]
    B = 16
    anchors = [np.sort(rng.integers(0, n, size=5)) for n in n_ctx]
    anchors[1][-1] = 256  # block clipped at the end of the context
    desc, cost, tok, total = oracle.item_table(n_ctx, anchors, B, 4, 2, 256, kind, granule)
    assert np.array_equal(cost, _brute_costs(n_ctx, anchors, B, 4, 2, 256, kind, granule))
    assert total == 2 * sum(n_ctx)
    # descriptors enumerate (s, g, c, r) row-major
    assert np.all(np.diff(desc[:, 0]) >= 0)


def test_static_plan_properties():
    # equal chunks: worker = floor(i * W / n)
    n_ctx, B, hq, hkv, L = [4096], 32, 2, 2, 512
    anchors = [np.arange(0, 4096, 512)]
    desc, cost, tok, total = oracle.item_table(n_ctx, anchors, B, hq, hkv, L, "fwd", 100)
    units = len(desc)   # one block range per unit here
    a = oracle.static_assign(tok, total, 4)
    assert list(a) == [i * 4 // units for i in range(units)]
    # contiguous and monotone in enumeration order, every worker gets tokens
    desc, cost, tok, total = oracle.item_table([1000, 3000], [[5, 900], [10, 2000]], 16, 4, 2, 256, "bwd", 64)
    a = oracle.static_assign(tok, total, 7)
    assert np.all(np.diff(a) >= 0) and a.min() == 0 and a.max() == 6


def test_lpt_beats_static_under_skewed_anchors():
    """Anchors clustered late (Beta(5,1)) load the static plan's last workers."""
    rng = np.random.default_rng(0)
    N, A, B = 65536, 64, 32
    anc = [np.sort(np.floor(N * rng.beta(5, 1, size=A)).astype(np.int64))]
    desc, cost, tok, total = oracle.item_table([N], anc, B, 4, 4, 4096, "fwd", 8)
    W = 32
    _, _, _, lpt_load = oracle.lpt(cost, W)
    st_load = oracle.loads_from_assign(cost, oracle.static_assign(tok, total, W), W)
    assert oracle.imbalance(lpt_load) < 0.05 < oracle.imbalance(st_load)
    order, off = oracle.csr_from_assign(oracle.static_assign(tok, total, W), W)
    assert sorted(order.tolist()) == list(range(len(cost))) and off[-1] == len(cost)


# ---- local merge of consecutive chunks (runs) ----

def test_coarsen_runs_worked_example():
    # Two row ranges (r = 0, 1) of one (s, g), chunks 0..3, numbered row-major
    # (c, r): ids 0..7.  Costs fall with the chunk as prefixes end.
    desc = [(0, 0, c, r) for c in range(4) for r in range(2)]
    cost = [5, 7, 4, 7, 3, 0, 0, 0]
    first, length, rcost = oracle.coarsen_runs(desc, cost, 8)
    # r = 0: chunks 0+1 (5 + 4 = 9 reaches 8, closes), chunk 2 (3) alone (group ends
    #        with chunk 3 of cost 0, which stays alone);
    # r = 1: chunks 0+1 (7 < 8, then 14), chunk 2 (0) alone, chunk 3 (0) alone.
    assert first.tolist() == [0, 1, 4, 5, 6, 7]
    assert length.tolist() == [2, 2, 1, 1, 1, 1]
    assert rcost.tolist() == [9, 14, 3, 0, 0, 0]
    # target 1: no run grows past one chunk
    f1, l1, c1 = oracle.coarsen_runs(desc, cost, 1)
    assert f1.tolist() == list(range(8)) and l1.tolist() == [1] * 8 and c1.tolist() == cost


def _run_members(desc, first, length):
    idx = {tuple(int(x) for x in d): i for i, d in enumerate(desc)}
    out = []
    for f, n in zip(first, length):
        s, g, c, r = (int(x) for x in desc[f])
        out.append([idx[(s, g, c + k, r)] for k in range(int(n))])
    return out


@pytest.mark.parametrize("target", [1, 40, 500, 10 ** 12])
def test_coarsen_runs_properties(target):
    rng = np.random.default_rng(11)
    n_ctx = [5000, 1500, 9000]
    anchors = [np.sort(rng.integers(0, n, size=12)) for n in n_ctx]
    desc, cost, _, _ = oracle.item_table(n_ctx, anchors, 16, 4, 2, 256, "fwd", 3)
    first, length, rcost = oracle.coarsen_runs(desc, cost, target)
    members = _run_members(desc, first, length)
    # a partition of the items into runs of consecutive chunks, costs preserved
    flat = sorted(i for m in members for i in m)
    assert flat == list(range(len(cost)))
    for m, c in zip(members, rcost):
        assert c == cost[m].sum()
        assert m[0] == min(m)
    assert np.all(np.diff(first) > 0)
    # zero-cost items stand alone; a run is cut below the target only where its
    # group's next chunk is missing or costs nothing
    nxt = {}
    for i, d in enumerate(desc):
        nxt[(int(d[0]), int(d[1]), int(d[2]) - 1, int(d[3]))] = i
    for m, c in zip(members, rcost):
        if any(cost[i] == 0 for i in m):
            assert len(m) == 1
            continue
        s, g, cl, r = (int(x) for x in desc[m[-1]])
        j = nxt.get((s, g, cl, r))
        if j is not None and cost[j] > 0:
            assert c >= target
        # no run keeps growing once it has reached the target
        assert c - cost[m[-1]] < target
    if target == 1:
        assert len(first) == len(cost)
    if target == 10 ** 12:
        # one run per (s, g, r) over its nonzero chunks (they start at chunk 0)
        n_groups = len({(int(d[0]), int(d[1]), int(d[3])) for d, c in zip(desc, cost) if c > 0})
        assert len(first) == n_groups + int((cost == 0).sum())
