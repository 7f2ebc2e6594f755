"""The Split-KV hot path on one GPU: plan, partial forward, merge, backward.

A thin driver over the C ABI (binding.py).  It owns the device buffers (torch
allocations) and the two plans; every arithmetic step runs in libsplitkv's
kernels.  On one GPU the pages' context-parallel shards become KV chunks and
the ranks become persistent workgroups (Split-KV article, "Split-KV's Core
Mechanism" and "LPT Scheduling").
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding as B


def default_workers(device) -> int:
    import torch
    return torch.cuda.get_device_properties(device).multi_processor_count


RUN_IMBALANCE = 0.02        # LPT cost imbalance accepted for chunk runs
MAX_RUNS_PER_WORKER = 64


def _align256(n: int) -> int:
    return (n + 255) & ~255


class _Staging:
    """Two pinned-host / device buffer pairs shared by the step's plans.  A
    step's plans are packed into one pair on the host (``stage``); the copy to
    the device is issued by the step's first kernel call, on that call's stream
    (``flush``), so the kernels that read the plans are ordered after it on
    whatever stream the caller uses.  Each kernel call records on its stream
    that the pair is in use (``used_on``), and the next copy into the pair
    waits for it, while the previous step's kernels may still read the other
    pair."""

    def __init__(self, nbytes: int, device):
        import torch
        self.slots = [{"h": torch.empty(max(nbytes, 256), dtype=torch.uint8, pin_memory=True),
                       "d": torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device),
                       "copied": torch.cuda.Event(), "done": torch.cuda.Event(), "used": False}
                      for _ in range(2)]
        self.next = 0
        self.cur = None       # the slot of the current step
        self.pending = 0      # bytes staged on the host, not yet copied

    def stage(self, parts):
        """Pack the numpy arrays ``parts`` (256-byte aligned, in order) into the
        next slot's pinned buffer; returns their device addresses."""
        slot = self.slots[self.next]
        self.next ^= 1
        if slot["used"]:
            slot["copied"].synchronize()   # its previous copy has left the pinned buffer
        h = slot["h"].numpy()
        pos, ptrs = 0, []
        for a in parts:
            b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
            h[pos:pos + len(b)] = b
            ptrs.append(slot["d"].data_ptr() + pos)
            pos = _align256(pos + len(b))
        self.cur, self.pending = slot, pos
        return ptrs

    def flush(self, stream):
        """Issue the staged copy on ``stream`` (a torch stream) if not done yet."""
        import torch
        slot = self.cur
        if slot is None or not self.pending:
            return
        if slot["used"]:
            stream.wait_event(slot["done"])  # kernels of two steps ago read this device buffer
        with torch.cuda.stream(stream):
            slot["d"][:self.pending].copy_(slot["h"][:self.pending], non_blocking=True)
        slot["copied"].record(stream)
        slot["used"] = True
        self.pending = 0

    def used_on(self, stream):
        """Kernels reading the current slot were launched on ``stream``."""
        if self.cur is not None:
            self.cur["done"].record(stream)


class _PlanSlots:
    """One kind of plan: its items, claim cursors and optional busy-time
    counters; the host arrays it builds each step go to the device through the
    step's shared staging buffer (_Staging)."""

    def __init__(self, problem: B.Problem, kind: int, granule: int, n_workers: int, policy: str,
                 steal: bool = True, ticks: bool = False, runs_per_worker: Optional[float] = None,
                 run_imbalance: Optional[float] = RUN_IMBALANCE):
        import torch
        self.problem, self.kind, self.granule, self.n_workers, self.policy = problem, kind, granule, n_workers, policy
        # forward only: chunks of the same rows merged into runs of about
        # total cost / (n_workers * runs_per_worker) (None: one chunk per item)
        self.runs_per_worker = runs_per_worker
        self.run_imbalance = run_imbalance  # None: keep runs_per_worker as given
        self.runs_used = None
        self.flags = 0 if steal else B.SKV_PLAN_NO_STEAL
        n = len(problem.item_table(kind, granule)[1])
        dev = problem.device
        self.n_items = n
        # staging bytes this plan needs at most: items, then worker offsets
        self.stage_bytes = _align256(max(n, 1) * B.ITEM_DTYPE.itemsize) + _align256((n_workers + 1) * 8)
        # per-worker claim cursors and the claimed-items count, reset by the library per call
        self.claim = torch.zeros(n_workers + 1, dtype=torch.int32, device=dev)
        # per-workgroup busy time (100 MHz ticks) of the last call, when asked for
        self.ticks = torch.zeros(n_workers, dtype=torch.int64, device=dev) if ticks else None
        self.plan_s = 0.0
        self.c = None
        self.load = self.cost = None
        self.table = None
        self.worker_off = None

    def build(self):
        """Realized costs -> LPT (or static) plan.  Returns the host arrays to
        upload (items in plan order, worker offsets); ``plan_s`` receives the
        host planning time (cost model, plan, gather)."""
        import time
        t0 = time.perf_counter()
        items, cost, tok, total = self.problem.item_table(self.kind, self.granule)
        if self.runs_per_worker and self.kind == B.SKV_ITEM_FWD:
            if self.policy != "lpt":
                raise ValueError("chunk runs are planned with LPT only")
            # Longer runs mean fewer partials but coarser items: the library
            # doubles the runs per worker until LPT balances the runs to within
            # run_imbalance (or MAX_RUNS_PER_WORKER is reached).
            start = float(self.runs_per_worker)
            if self.run_imbalance is None:   # keep runs_per_worker as given
                stop, tol = start, 0.0
            else:
                stop, tol = max(start, MAX_RUNS_PER_WORKER), self.run_imbalance
            items, cost, order, off, load, self.runs_used = B.skv_plan_fwd_runs(
                items, cost, self.n_workers, start, stop, tol)
        self.table = (items, cost)  # the items planned (chunk runs when asked for)
        if self.policy == "lpt":
            if not (self.runs_per_worker and self.kind == B.SKV_ITEM_FWD):
                _, order, off, load = B.lpt_plan(cost, self.n_workers)
        elif self.policy == "static":
            assign, order, off = B.skv_static_plan(tok, total, self.n_workers)
            load = np.bincount(assign, weights=cost, minlength=self.n_workers).astype(np.int64)
        else:
            raise ValueError(self.policy)
        if self.kind == B.SKV_ITEM_FWD:
            # empty forward items only mark rows -inf, which the forward call does for all rows
            order, off = B.skv_drop_zero_cost(cost, order, off)
        gathered = B.skv_gather_items(items, order)
        self.plan_s = time.perf_counter() - t0
        self.cost, self.load = cost, load
        self.n_planned = len(order)
        self.worker_off = off
        return [gathered, np.asarray(off, dtype=np.int64)]

    def follow(self, other: "_PlanSlots"):
        """Take the host results of an identical plan (same problem, kind,
        granule, policy and runs), whose uploaded arrays this plan then binds
        as well; only the claim cursors and busy-time counters stay separate."""
        self.table, self.cost, self.load = other.table, other.cost, other.load
        self.runs_used, self.n_planned, self.worker_off = other.runs_used, other.n_planned, other.worker_off
        self.plan_s = 0.0

    def bind(self, d_items: int, d_off: int):
        """The skv_plan of the arrays uploaded to d_items / d_off."""
        self.c = B.skv_plan(self.kind, self.n_workers, self.n_planned, d_items, d_off, self.claim.data_ptr(),
                            self.flags, 0, None if self.ticks is None else self.ticks.data_ptr())
        return self.c

    @property
    def imbalance(self) -> float:
        mean = self.load.mean()
        return float(self.load.max() / mean - 1.0) if mean > 0 else 0.0


class SplitKVAttention:
    """Block-sparse draft attention of a packed batch, Split-KV style.

    Host metadata: q_off, kv_off (int64 [n_seq+1]) and anchors (int32, sorted
    per sequence).  Device tensors q [sum Mq, hq, d], k, v [sum N, hkv, d] in
    ``dtype`` (torch.bfloat16 or torch.float32).
    """

    def __init__(self, q_off, kv_off, anchors, block: int, hq: int, hkv: int, d: int, chunk: int,
                 sm_scale: float, dtype, device, n_workers: Optional[int] = None,
                 fwd_granule: Optional[int] = None, bwd_granule: int = 256, policy: str = "lpt",
                 with_bwd: bool = True, steal: bool = True, ticks: bool = False,
                 fwd_runs_per_worker: Optional[float] = 4.0, mask: str = "prefix",
                 fwd_run_imbalance: Optional[float] = RUN_IMBALANCE):
        import torch
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dtype = dtype
        self.skv_dtype = B.SKV_BF16 if dtype == torch.bfloat16 else B.SKV_F32
        if mask not in ("prefix", "own_block"):
            raise ValueError(mask)
        # "own_block": each draft block also sees its own tokens' keys (k_own,
        # v_own [sum Mq, hkv, d]), one more partial per row; the context prefix
        # then ends at the anchor
        self.mask = mask
        self.problem = B.Problem(q_off, kv_off, anchors, block, hq, hkv, d, chunk, self.skv_dtype, sm_scale,
                                 device=self.device,
                                 mask=B.SKV_MASK_OWN_BLOCK if mask == "own_block" else B.SKV_MASK_PREFIX)
        self.problem.check()
        self.n_workers = n_workers or default_workers(self.device)
        G = hq // hkv
        self.fwd_granule = fwd_granule or max(1, 256 // (G * block))
        self.bwd_granule = bwd_granule
        kw = dict(steal=steal, ticks=ticks)
        # Forward items cover runs of consecutive chunks of the same rows, about
        # fwd_runs_per_worker per workgroup (more when LPT cannot balance the
        # runs to within fwd_run_imbalance), each with one partial (LPT plans
        # only; None or a static plan: one chunk per item, one partial per chunk).
        self.fwd_runs_per_worker = fwd_runs_per_worker if policy == "lpt" else None
        self.fwd_plan = _PlanSlots(self.problem, B.SKV_ITEM_FWD, self.fwd_granule, self.n_workers, policy, **kw,
                                   runs_per_worker=self.fwd_runs_per_worker, run_imbalance=fwd_run_imbalance)
        self.bwd_plan = (_PlanSlots(self.problem, B.SKV_ITEM_BWD, self.bwd_granule, self.n_workers, policy, **kw)
                         if with_bwd else None)
        # dQ runs over the forward's plan (the same uploaded arrays); its own
        # slots give it separate claim cursors
        self.dq_plan = (_PlanSlots(self.problem, B.SKV_ITEM_FWD, self.fwd_granule, self.n_workers, policy, **kw,
                                   runs_per_worker=self.fwd_runs_per_worker, run_imbalance=fwd_run_imbalance)
                        if with_bwd else None)
        self.staging = _Staging(sum(p.stage_bytes for p in (self.fwd_plan, self.bwd_plan) if p is not None),
                                self.device)
        self.replan()
        self.part_base, self.n_chunk = self.problem.partial_layout()
        self.d_part_base = torch.from_numpy(self.part_base).to(self.device)
        rows = int(self.part_base[-1])
        tq = self.problem.total_q
        self.o_part = torch.empty((max(rows, 1), d), dtype=torch.float32, device=self.device)
        self.m_part = torch.empty(max(rows, 1), dtype=torch.float32, device=self.device)
        self.lse_part = torch.empty(max(rows, 1), dtype=torch.float32, device=self.device)
        self.o = torch.empty((tq, hq, d), dtype=dtype, device=self.device)
        self.lse = torch.empty((tq, hq), dtype=torch.float32, device=self.device)
        self.workspace = None
        if with_bwd:
            nbytes = self.problem.bwd_workspace_bytes()
            self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)

    # -- steps -------------------------------------------------------------
    def replan(self):
        """Mask descriptor -> realized cost per item -> LPT plans, staged for
        one copy to the device that the next kernel call issues on its stream."""
        plans = [self.fwd_plan] + ([self.bwd_plan] if self.bwd_plan is not None else [])
        parts = []
        for p in plans:
            parts += p.build()
        ptrs = self.staging.stage(parts)
        for i, p in enumerate(plans):
            p.bind(ptrs[2 * i], ptrs[2 * i + 1])
        if self.dq_plan is not None:
            self.dq_plan.follow(self.fwd_plan)
            self.dq_plan.bind(ptrs[0], ptrs[1])
        self.plan_s = sum(p.plan_s for p in plans)

    def _check(self, **tensors):
        """The problem uses contiguous [rows, heads, d] strides for every tensor."""
        p = self.problem
        shapes = {"q": (p.total_q, p.hq, p.d), "dout": (p.total_q, p.hq, p.d), "dq": (p.total_q, p.hq, p.d),
                  "k": (p.total_kv, p.hkv, p.d), "v": (p.total_kv, p.hkv, p.d), "dk": (p.total_kv, p.hkv, p.d),
                  "dv": (p.total_kv, p.hkv, p.d)}
        for name, t in tensors.items():
            if t is None:
                continue
            want = shapes.get(name, (p.total_q, p.hkv, p.d))  # own-block tensors
            if tuple(t.shape) != want or not t.is_contiguous() or t.dtype != self.dtype or t.device != self.device:
                raise ValueError(f"{name}: need a contiguous {self.dtype} tensor of shape {want} on {self.device}, "
                                 f"got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _stream(self, stream):
        """The torch stream of a call (None: the current stream of the device;
        an int: a raw hipStream_t)."""
        import torch
        if stream is None:
            return torch.cuda.current_stream(self.device)
        if isinstance(stream, int):
            return torch.cuda.ExternalStream(stream, device=self.device)
        return stream

    def partial_fwd(self, q, k, v, stream=None, k_own=None, v_own=None):
        self._check(q=q, k=k, v=v, k_own=k_own, v_own=v_own)
        if self.mask == "own_block" and (k_own is None or v_own is None):
            raise ValueError("the own-block mask needs k_own and v_own")
        ts = self._stream(stream)
        self.staging.flush(ts)
        B.sparse_attn_partial_fwd(self.problem, self.fwd_plan, q, k, v, self.o_part, self.m_part, self.lse_part, ts)
        if self.mask == "own_block":
            B.sparse_attn_own_fwd(self.problem, q, k_own, v_own, self.o_part, self.m_part, self.lse_part, ts)
        self.staging.used_on(ts)

    def merge(self, stream=None):
        """The exact merge of every sequence's partials, in one launch."""
        B.lse_merge_all(self.problem, self.d_part_base, self.o_part, self.m_part, self.lse_part, self.o, self.lse,
                        stream)

    def merge_per_sequence(self, stream=None):
        """The same merge, one lse_merge call per sequence."""
        p = self.problem
        out_dtype = self.skv_dtype
        for s in range(p.n_seq):
            q0 = int(p.h_q_off[s])
            mq = int(p.h_q_off[s + 1]) - q0
            B.lse_merge(int(self.n_chunk[s]), p.hq, mq, p.d, self.o_part, self.m_part, self.lse_part, self.o,
                        p.hq * p.d, p.d, out_dtype, self.lse, p.hq, stream,
                        part_offset=int(self.part_base[s]), out_offset=q0, lse_offset=q0 * p.hq)

    def forward(self, q, k, v, stream=None, k_own=None, v_own=None):
        """Partials of every KV chunk (and of the own block), then their exact merge.  Returns (O, LSE)."""
        self.partial_fwd(q, k, v, stream, k_own, v_own)
        self.merge(stream)
        return self.o, self.lse

    def backward(self, q, k, v, dout, dq, dk, dv, stream=None, own=None, noalloc: bool = False):
        """dQ, dK, dV from the merged O and LSE of the last forward.  Under the
        own-block mask ``own`` = (k_own, v_own, dk_own, dv_own).  ``noalloc``:
        the library's static scratch instead of this object's workspace
        (sparse_attn_bwd_noalloc)."""
        if (self.mask == "own_block") != (own is not None):
            raise ValueError("own-block tensors go with the own-block mask")
        self._check(q=q, k=k, v=v, dout=dout, dq=dq, dk=dk, dv=dv,
                    **(dict(zip(("k_own", "v_own", "dk_own", "dv_own"), own)) if own is not None else {}))
        ts = self._stream(stream)
        self.staging.flush(ts)
        if noalloc:
            B.sparse_attn_bwd_noalloc(self.problem, self.bwd_plan, self.dq_plan, q, k, v, self.o, self.lse, dout, dq,
                                      dk, dv, ts, own=own)
        else:
            B.sparse_attn_bwd(self.problem, self.bwd_plan, self.dq_plan, q, k, v, self.o, self.lse, dout, dq, dk, dv,
                              self.workspace, ts, own=own)
        self.staging.used_on(ts)
        return dq, dk, dv

    # -- views ---------------------------------------------------------------
    def partial_view(self, s: int):
        """(o_part [C, hq, Mq, d], m_part [C, hq, Mq], lse_part [C, hq, Mq]) of sequence s."""
        p = self.problem
        mq = int(p.h_q_off[s + 1] - p.h_q_off[s])
        c = int(self.n_chunk[s])
        b = int(self.part_base[s])
        n = c * p.hq * mq
        return (self.o_part[b:b + n].view(c, p.hq, mq, p.d), self.m_part[b:b + n].view(c, p.hq, mq),
                self.lse_part[b:b + n].view(c, p.hq, mq))


def unmasked_pairs(q_off, kv_off, anchors, block: int, hq: int, mask: str = "prefix") -> int:
    """Token-exact number of visible (query head, query row, key) triples
    (under the own-block mask: the context prefix [0, min(a_b, N)) plus the
    block's own keys)."""
    total = 0
    shift = block if mask == "prefix" else 0
    for s in range(len(q_off) - 1):
        n = int(kv_off[s + 1] - kv_off[s])
        b0, b1 = int(q_off[s]) // block, int(q_off[s + 1]) // block
        e = np.minimum(np.asarray(anchors[b0:b1], dtype=np.int64) + shift, n)
        if mask != "prefix":
            e = e + block
        total += int(e.sum()) * block
    return total * hq
