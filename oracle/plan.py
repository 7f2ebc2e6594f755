"""Cost model, LPT and static token-count plans for Split-KV work items.

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the pages:
  * Anchor sampling makes each sample touch a different context range, so the
    attention cost varies with the sample and a static, token-count partition
    of the context is easily unbalanced ([P1] "The Query-Context Asymmetry";
    [P1] "LPT Scheduling").
  * LPT sorts tasks from longest to shortest processing time and gives each in
    turn to the least-loaded machine; Split-KV's processing time is the
    realized attention cost of each context KV chunk, observable through the
    global query view ([P1] "LPT Scheduling" and its sidebar; [P3] Abstract).
  * LPT's makespan is within 4/3 of optimal ([P1] "LPT Scheduling" sidebar);
    the tests check Graham's sharper (4/3 - 1/(3m)) form, which implies it.

Readings of what the pages leave open:
  * Work item (fwd): (sequence s, KV head g with its G query heads, KV chunk c,
    range r of ``granule`` consecutive draft blocks).  Work item (bwd):
    (s, g, c, range r of ``granule`` keys inside chunk c).  Items are numbered
    row-major in that tuple order.
  * Realized cost of an item: G times the number of (draft block, 64-key tile)
    pairs of the item in which the block sees at least one key of the tile.
    Block b sees tile t iff t*64 < e_b.
  * Tie-break: items in order of (cost descending, item id ascending); each goes
    to the worker with the smallest (load, worker id).  Zero-cost items are
    planned like any other.
  * Static plan: the (s, g, c) units are laid end to end by token count; an
    item starting at token offset x of that stream goes to worker
    floor(x * W / total).  All block ranges of one unit share its start.
  * Imbalance: max worker load / mean worker load - 1.
  * Local merge before the exchange: the pages' ranks each aggregate the
    attention results of the KV they hold before the query-sized exchange
    ([P1] "Split-KV's Core Mechanism").  Here forward items of the same rows
    (s, g, r) and consecutive chunks are merged into runs, each with one
    partial.  Rule: per (s, g, r) in ascending chunk order, a zero-cost item
    stays alone; an item joins the open run iff its chunk follows the run's
    last chunk and the run's cost is still below the target; runs are listed
    in the order of their first item.
"""
from __future__ import annotations

import itertools
from typing import Sequence

import numpy as np

TILE = 64


def item_table(n_ctx: Sequence[int], anchors: Sequence[Sequence[int]], block: int, hq: int, hkv: int,
               chunk: int, kind: str, granule: int, tile: int = TILE):
    """Enumerate work items with their realized cost and static token start.

    Returns (desc int32 [n, 4] = (s, g, c, r), cost int64 [n], tok_start int64 [n],
    total_tok int).  ``kind`` is "fwd" (granule = draft blocks per item) or
    "bwd" (granule = keys per item, a multiple of ``tile``).
    """
    if chunk % tile or (kind == "bwd" and granule % tile):
        raise ValueError("chunk and bwd granule must be multiples of the tile")
    G = hq // hkv
    desc, cost, tok = [], [], []
    unit_start = 0
    for s, (N, anc) in enumerate(zip(n_ctx, anchors)):
        N = int(N)
        e = np.minimum(np.asarray(anc, dtype=np.int64) + block, N)
        # number of tiles whose first key lies below e_b, per block
        tiles_seen = -(-e // tile)
        C = -(-N // chunk)
        A = len(anc)
        for g in range(hkv):
            for c in range(C):
                lo, hi = c * chunk, min((c + 1) * chunk, N)
                if kind == "fwd":
                    t0, t1 = lo // tile, -(-hi // tile)
                    per_block = np.clip(tiles_seen, t0, t1) - t0
                    for r in range(-(-A // granule)):
                        desc.append((s, g, c, r))
                        cost.append(G * int(per_block[r * granule:(r + 1) * granule].sum()))
                        tok.append(unit_start)
                elif kind == "bwd":
                    for r in range(-(-(hi - lo) // granule)):
                        klo, khi = lo + r * granule, min(lo + (r + 1) * granule, hi)
                        t0, t1 = klo // tile, -(-khi // tile)
                        desc.append((s, g, c, r))
                        cost.append(G * int((np.clip(tiles_seen, t0, t1) - t0).sum()))
                        tok.append(unit_start + (klo - lo))
                else:
                    raise ValueError(kind)
                unit_start += hi - lo
    return (np.asarray(desc, dtype=np.int32).reshape(-1, 4), np.asarray(cost, dtype=np.int64),
            np.asarray(tok, dtype=np.int64), unit_start)


def lpt(cost, n_workers: int):
    """Longest-processing-time-first list scheduling.

    Returns assign int32 [n] (worker of each item), order int64 [n] (item ids
    grouped by worker, each worker's items in the order they were assigned),
    worker_off int64 [W + 1] and load int64 [W].
    """
    cost = np.asarray(cost, dtype=np.int64)
    n = len(cost)
    if n_workers <= 0:
        raise ValueError("need at least one worker")
    seq = sorted(range(n), key=lambda i: (-int(cost[i]), i))
    load = np.zeros(n_workers, dtype=np.int64)
    assign = np.empty(n, dtype=np.int32)
    lists = [[] for _ in range(n_workers)]
    for i in seq:
        w = int(np.argmin(load))          # first minimum: smallest worker id among equal loads
        assign[i] = w
        lists[w].append(i)
        load[w] += cost[i]
    order, off = _csr(lists)
    return assign, order, off, load


def static_assign(tok_start, total_tok: int, n_workers: int):
    """Static token-count plan: worker = floor(tok_start * W / total_tok)."""
    t = np.asarray(tok_start, dtype=np.int64)
    if total_tok <= 0:
        return np.zeros(len(t), dtype=np.int32)
    return ((t * n_workers) // int(total_tok)).astype(np.int32)


def csr_from_assign(assign, n_workers: int):
    """Group item ids by worker, each worker's items in ascending id order."""
    lists = [[] for _ in range(n_workers)]
    for i, w in enumerate(np.asarray(assign)):
        lists[int(w)].append(i)
    return _csr(lists)


def _csr(lists):
    off = np.zeros(len(lists) + 1, dtype=np.int64)
    off[1:] = np.cumsum([len(x) for x in lists])
    order = np.asarray([i for x in lists for i in x], dtype=np.int64)
    return order, off


def loads_from_assign(cost, assign, n_workers: int):
    load = np.zeros(n_workers, dtype=np.int64)
    for c, w in zip(np.asarray(cost, dtype=np.int64), np.asarray(assign)):
        load[int(w)] += c
    return load


def imbalance(load) -> float:
    load = np.asarray(load, dtype=np.float64)
    mean = load.mean() if len(load) else 0.0
    return float(load.max() / mean - 1.0) if mean > 0 else 0.0


def brute_force_makespan(cost, n_workers: int) -> int:
    """Optimal makespan by trying every assignment (tiny instances only)."""
    cost = [int(c) for c in cost]
    best = None
    for assign in itertools.product(range(n_workers), repeat=len(cost)):
        load = [0] * n_workers
        for c, w in zip(cost, assign):
            load[w] += c
        m = max(load) if load else 0
        best = m if best is None else min(best, m)
    return 0 if best is None else best


def graham_bound(n_workers: int) -> float:
    """Graham's worst-case ratio of LPT to the optimum on m machines."""
    return 4.0 / 3.0 - 1.0 / (3.0 * n_workers)


def coarsen_runs(desc, cost, target: int):
    """Merge forward items into runs of consecutive chunks of the same rows.

    ``desc`` rows are (s, g, c, r) as ``item_table`` returns them.  Returns
    (first int64 [m] = item id of each run's first chunk, length int64 [m],
    cost int64 [m]), runs in ascending order of ``first``.
    """
    if target < 1:
        raise ValueError("target must be >= 1")
    desc = np.asarray(desc)
    cost = np.asarray(cost, dtype=np.int64)
    groups = {}
    for i in range(len(cost)):
        s, g, c, r = (int(x) for x in desc[i])
        groups.setdefault((s, g, r), []).append((c, i))
    runs = []  # [first, length, cost, last chunk]
    for key in groups:
        open_run = None
        for c, i in sorted(groups[key]):
            w = int(cost[i])
            if w > 0 and open_run is not None and c == open_run[3] + 1 and open_run[2] < target:
                open_run[1] += 1
                open_run[2] += w
                open_run[3] = c
                continue
            run = [i, 1, w, c]
            runs.append(run)
            open_run = run if w > 0 else None
    runs.sort(key=lambda x: x[0])
    return (np.asarray([x[0] for x in runs], dtype=np.int64), np.asarray([x[1] for x in runs], dtype=np.int64),
            np.asarray([x[2] for x in runs], dtype=np.int64))
