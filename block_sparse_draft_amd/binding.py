"""ctypes binding of libsplitkv (include/splitkv.h).

Argument marshalling only: every step of the attention path runs in the HIP
library; this module turns numpy arrays and torch tensors into the pointers,
sizes and structs the C ABI takes.  PyTorch is used for device memory and the
current HIP stream, nothing else.  The library must be built
(``python -m block_sparse_draft_amd.build``); importing this module without it
raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsplitkv.so")

SKV_OK, SKV_EINVAL, SKV_EDTYPE, SKV_ESHAPE, SKV_EHIP, SKV_EWORKSPACE, SKV_EPLAN = 0, -1, -2, -3, -4, -5, -6
SKV_F32, SKV_BF16 = 0, 1
SKV_MASK_PREFIX, SKV_MASK_OWN_BLOCK = 0, 1
SKV_ITEM_FWD, SKV_ITEM_BWD = 0, 1
SKV_TILE = 64
SKV_PLAN_NO_STEAL = 1
SKV_NOALLOC_SCRATCH_BYTES = 64 << 20
_STATUS = {0: "SKV_OK", -1: "SKV_EINVAL", -2: "SKV_EDTYPE", -3: "SKV_ESHAPE", -4: "SKV_EHIP",
           -5: "SKV_EWORKSPACE", -6: "SKV_EPLAN"}


class SkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


class skv_problem(C.Structure):
    _fields_ = [("n_seq", C.c_int32), ("block", C.c_int32), ("hq", C.c_int32), ("hkv", C.c_int32),
                ("d", C.c_int32), ("chunk", C.c_int32), ("dtype", C.c_int32), ("sm_scale", C.c_float),
                ("mask", C.c_int32), ("reserved", C.c_int32),
                ("h_q_off", C.c_void_p), ("d_q_off", C.c_void_p), ("h_kv_off", C.c_void_p), ("d_kv_off", C.c_void_p),
                ("h_anchor", C.c_void_p), ("d_anchor", C.c_void_p),
                ("q_stride_tok", C.c_int64), ("q_stride_head", C.c_int64),
                ("kv_stride_tok", C.c_int64), ("kv_stride_head", C.c_int64)]


class skv_own_block(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("dk", C.c_void_p), ("dv", C.c_void_p),
                ("stride_tok", C.c_int64), ("stride_head", C.c_int64)]


class skv_item(C.Structure):
    _fields_ = [("seq", C.c_int32), ("kv_head", C.c_int32), ("chunk", C.c_int32), ("range", C.c_int32),
                ("part_base", C.c_int64), ("lo", C.c_int32), ("hi", C.c_int32),
                ("n_chunk", C.c_int32), ("reserved", C.c_int32)]


ITEM_DTYPE = np.dtype([("seq", "<i4"), ("kv_head", "<i4"), ("chunk", "<i4"), ("range", "<i4"),
                       ("part_base", "<i8"), ("lo", "<i4"), ("hi", "<i4"), ("n_chunk", "<i4"), ("reserved", "<i4")])
assert ITEM_DTYPE.itemsize == C.sizeof(skv_item) == 40


class skv_plan(C.Structure):
    _fields_ = [("kind", C.c_int32), ("n_workers", C.c_int32), ("n_items", C.c_int64),
                ("d_items", C.c_void_p), ("d_worker_off", C.c_void_p), ("d_claim", C.c_void_p),
                ("flags", C.c_int32), ("reserved", C.c_int32), ("d_ticks", C.c_void_p)]


class skv_kernel_time(C.Structure):
    _fields_ = [("name", C.c_char_p), ("launches", C.c_int64), ("total_ms", C.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python block_sparse_draft_amd/build.py`")
    # torch ships its own HIP runtime.  Load it first so that libsplitkv binds
    # to that same runtime (its libamdhip64 dependency resolves to the copy
    # already in the process); two runtimes in one process do not share
    # devices, streams or allocations.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    P, VP, I32, I64, F = C.POINTER, C.c_void_p, C.c_int32, C.c_int64, C.c_float
    sig = {
        "skv_last_error": (C.c_char_p, []),
        "skv_check_problem": (C.c_int, [P(skv_problem)]),
        "skv_partial_layout": (C.c_int, [P(skv_problem), VP, VP]),
        "skv_item_table": (C.c_int, [P(skv_problem), I32, I32, VP, VP, VP, P(I64), P(I64)]),
        "lpt_plan": (C.c_int, [VP, I64, I32, VP, VP, VP, VP]),
        "skv_static_plan": (C.c_int, [VP, I64, I64, I32, VP, VP, VP]),
        "skv_gather_items": (C.c_int, [VP, I64, VP, I64, VP]),
        "skv_drop_zero_cost": (C.c_int, [VP, I64, I32, VP, VP, VP, VP, P(I64)]),
        "skv_coarsen_fwd_items": (C.c_int, [VP, VP, I64, I64, VP, VP, P(I64)]),
        "skv_plan_fwd_runs": (C.c_int, [VP, VP, I64, I32, C.c_double, C.c_double, C.c_double, VP, VP, P(I64), VP,
                                        VP, VP, P(C.c_double)]),
        "sparse_attn_partial_fwd": (C.c_int, [P(skv_problem), P(skv_plan), VP, VP, VP, VP, VP, VP, VP]),
        "lse_merge": (C.c_int, [I32, I32, I64, I32, VP, VP, VP, VP, I64, I64, I32, VP, I64, VP]),
        "skv_bwd_workspace_bytes": (C.c_size_t, [P(skv_problem)]),
        "sparse_attn_bwd": (C.c_int, [P(skv_problem), P(skv_plan), P(skv_plan)] + [VP] * 10 +
                            [C.c_size_t, P(skv_own_block), VP]),
        "sparse_attn_bwd_noalloc": (C.c_int, [P(skv_problem), P(skv_plan), P(skv_plan)] + [VP] * 9 +
                                    [P(skv_own_block), VP]),
        "sparse_attn_own_fwd": (C.c_int, [P(skv_problem), VP, VP, VP, I64, I64, VP, VP, VP, VP]),
        "lse_merge_all": (C.c_int, [P(skv_problem), VP, VP, VP, VP, VP, VP, VP]),
        "skv_timing_enable": (C.c_int, [I32]),
        "skv_timing_collect": (C.c_int, [P(skv_kernel_time), I32, P(I32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()
EXPORTED = ("skv_last_error", "skv_check_problem", "skv_partial_layout", "skv_item_table", "lpt_plan",
            "skv_static_plan", "skv_gather_items", "skv_drop_zero_cost", "skv_coarsen_fwd_items",
            "skv_plan_fwd_runs",
            "sparse_attn_partial_fwd", "lse_merge", "lse_merge_all",
            "skv_bwd_workspace_bytes", "sparse_attn_bwd", "sparse_attn_bwd_noalloc", "sparse_attn_own_fwd",
            "skv_timing_enable",
            "skv_timing_collect")


def last_error() -> str:
    return lib.skv_last_error().decode()


def _check(rc: int):
    if rc != SKV_OK:
        raise SkvError(rc, last_error())


def _ptr(a) -> Optional[int]:
    """Address of a numpy array or torch tensor (None stays NULL)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags.c_contiguous:
            raise ValueError("numpy arrays passed to libsplitkv must be C-contiguous")
        return a.ctypes.data
    return a.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# Host calls
# ---------------------------------------------------------------------------

def timing_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events on its stream."""
    _check(lib.skv_timing_enable(1 if on else 0))


def timing_collect() -> dict:
    """{kernel name: (launches, total ms)} since the last collect (waits for the events)."""
    n = C.c_int32(0)
    buf = (skv_kernel_time * 16)()  # more entries than the library has kernels
    _check(lib.skv_timing_collect(buf, len(buf), C.byref(n)))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n.value, len(buf)))}


def lpt_plan(cost, n_workers: int):
    """LPT planning (host).  Returns (assign int32, order int64, worker_off int64, load int64)."""
    cost = np.ascontiguousarray(cost, dtype=np.int64)
    n = len(cost)
    assign = np.empty(n, np.int32)
    order = np.empty(n, np.int64)
    off = np.empty(n_workers + 1 if n_workers > 0 else 1, np.int64)
    load = np.empty(max(n_workers, 1), np.int64)
    _check(lib.lpt_plan(_ptr(cost), n, n_workers, _ptr(assign), _ptr(order), _ptr(off), _ptr(load)))
    return assign, order, off, load


def skv_static_plan(tok_start, total_tok: int, n_workers: int):
    """Static token-count plan (host).  Returns (assign, order, worker_off)."""
    t = np.ascontiguousarray(tok_start, dtype=np.int64)
    n = len(t)
    assign = np.empty(n, np.int32)
    order = np.empty(n, np.int64)
    off = np.empty(n_workers + 1 if n_workers > 0 else 1, np.int64)
    _check(lib.skv_static_plan(_ptr(t), n, int(total_tok), n_workers, _ptr(assign), _ptr(order), _ptr(off)))
    return assign, order, off


def skv_gather_items(items: np.ndarray, order: np.ndarray) -> np.ndarray:
    items = np.ascontiguousarray(items, dtype=ITEM_DTYPE)
    order = np.ascontiguousarray(order, dtype=np.int64)
    out = np.empty(len(order), ITEM_DTYPE)
    _check(lib.skv_gather_items(_ptr(items), len(items), _ptr(order), len(order), _ptr(out)))
    return out


def skv_drop_zero_cost(cost, order, worker_off):
    """Plan lists without zero-cost items.  Returns (order, worker_off)."""
    cost = np.ascontiguousarray(cost, dtype=np.int64)
    order = np.ascontiguousarray(order, dtype=np.int64)
    worker_off = np.ascontiguousarray(worker_off, dtype=np.int64)
    nw = len(worker_off) - 1
    o2 = np.empty(max(len(order), 1), np.int64)
    w2 = np.empty(nw + 1, np.int64)
    n = C.c_int64(0)
    _check(lib.skv_drop_zero_cost(_ptr(cost), len(cost), nw, _ptr(order), _ptr(worker_off), _ptr(o2), _ptr(w2),
                                  C.byref(n)))
    return o2[:n.value].copy(), w2


def skv_coarsen_fwd_items(items, cost, target: int):
    """Runs of consecutive chunks of the same rows as single forward items.
    Returns (items ITEM_DTYPE, cost int64)."""
    items = np.ascontiguousarray(items, dtype=ITEM_DTYPE)
    cost = np.ascontiguousarray(cost, dtype=np.int64)
    n = len(cost)
    it2 = np.empty(max(n, 1), ITEM_DTYPE)
    c2 = np.empty(max(n, 1), np.int64)
    m = C.c_int64(0)
    _check(lib.skv_coarsen_fwd_items(_ptr(items), _ptr(cost), n, int(target), _ptr(it2), _ptr(c2), C.byref(m)))
    return it2[:m.value].copy(), c2[:m.value].copy()


def skv_plan_fwd_runs(items, cost, n_workers: int, runs_per_worker: float, max_runs_per_worker: float,
                      max_imbalance: float):
    """Chunk runs and their LPT plan, with the run length chosen by the
    library's search.  Returns (items, cost, order, worker_off, load, rpw_used)."""
    items = np.ascontiguousarray(items, dtype=ITEM_DTYPE)
    cost = np.ascontiguousarray(cost, dtype=np.int64)
    n = len(cost)
    it2 = np.empty(max(n, 1), ITEM_DTYPE)
    c2 = np.empty(max(n, 1), np.int64)
    order = np.empty(max(n, 1), np.int64)
    off = np.empty(n_workers + 1 if n_workers > 0 else 1, np.int64)
    load = np.empty(max(n_workers, 1), np.int64)
    m = C.c_int64(0)
    rpw = C.c_double(0)
    _check(lib.skv_plan_fwd_runs(_ptr(items), _ptr(cost), n, n_workers, float(runs_per_worker),
                                 float(max_runs_per_worker), float(max_imbalance), _ptr(it2), _ptr(c2), C.byref(m),
                                 _ptr(order), _ptr(off), _ptr(load), C.byref(rpw)))
    k = m.value
    return it2[:k].copy(), c2[:k].copy(), order[:k].copy(), off, load, rpw.value


class Problem:
    """A skv_problem plus the host and device arrays it points to.

    q_off, kv_off (int64 [n_seq+1]) and anchors (int32, sorted per sequence)
    are host numpy arrays; their device copies are made with torch when a
    device is given (``device=None`` gives a host-only problem for planning).
    """

    def __init__(self, q_off, kv_off, anchors, block: int, hq: int, hkv: int, d: int, chunk: int,
                 dtype: int, sm_scale: float, q_strides=None, kv_strides=None, device=None, mask: int = 0):
        self.h_q_off = np.ascontiguousarray(q_off, dtype=np.int64)
        self.h_kv_off = np.ascontiguousarray(kv_off, dtype=np.int64)
        self.h_anchor = np.ascontiguousarray(anchors, dtype=np.int32)
        self.n_seq = len(self.h_q_off) - 1
        self.block, self.hq, self.hkv, self.d, self.chunk = block, hq, hkv, d, chunk
        self.dtype, self.sm_scale, self.mask = dtype, sm_scale, mask
        self.q_strides = q_strides or (hq * d, d)
        self.kv_strides = kv_strides or (hkv * d, d)
        self.device = device
        self.d_q_off = self.d_kv_off = self.d_anchor = None
        if device is not None:
            import torch
            self.d_q_off = torch.from_numpy(self.h_q_off).to(device)
            self.d_kv_off = torch.from_numpy(self.h_kv_off).to(device)
            self.d_anchor = torch.from_numpy(self.h_anchor).to(device)
        self.c = skv_problem(self.n_seq, block, hq, hkv, d, chunk, dtype, sm_scale, mask, 0,
                             _ptr(self.h_q_off), _ptr(self.d_q_off), _ptr(self.h_kv_off), _ptr(self.d_kv_off),
                             _ptr(self.h_anchor), _ptr(self.d_anchor),
                             self.q_strides[0], self.q_strides[1], self.kv_strides[0], self.kv_strides[1])

    @property
    def total_q(self) -> int:
        return int(self.h_q_off[-1])

    @property
    def total_kv(self) -> int:
        return int(self.h_kv_off[-1])

    def check(self):
        _check(lib.skv_check_problem(C.byref(self.c)))

    def partial_layout(self):
        base = np.empty(self.n_seq + 1, np.int64)
        nchunk = np.empty(max(self.n_seq, 1), np.int32)
        _check(lib.skv_partial_layout(C.byref(self.c), _ptr(base), _ptr(nchunk)))
        return base, nchunk[:self.n_seq]

    def item_table(self, kind: int, granule: int):
        """(items structured array, cost int64, tok_start int64, total_tok)."""
        n = C.c_int64(0)
        tot = C.c_int64(0)
        _check(lib.skv_item_table(C.byref(self.c), kind, granule, None, None, None, C.byref(n), C.byref(tot)))
        items = np.empty(n.value, ITEM_DTYPE)
        cost = np.empty(n.value, np.int64)
        tok = np.empty(n.value, np.int64)
        _check(lib.skv_item_table(C.byref(self.c), kind, granule, _ptr(items), _ptr(cost), _ptr(tok),
                                  C.byref(n), C.byref(tot)))
        return items, cost, tok, tot.value

    def bwd_workspace_bytes(self) -> int:
        return int(lib.skv_bwd_workspace_bytes(C.byref(self.c)))


# ---------------------------------------------------------------------------
# Device calls (asynchronous on the given / current stream)
# ---------------------------------------------------------------------------

def sparse_attn_partial_fwd(problem: Problem, plan, q, k, v, o_part, m_part, lse_part, stream=None):
    _check(lib.sparse_attn_partial_fwd(C.byref(problem.c), C.byref(plan.c), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(o_part), _ptr(m_part), _ptr(lse_part), _stream(stream)))


def lse_merge(n_part: int, hq: int, mq: int, d: int, o_part, m_part, lse_part, o_out, o_stride_tok: int,
              o_stride_head: int, out_dtype: int, lse_out, lse_stride_tok: int, stream=None,
              part_offset: int = 0, out_offset: int = 0, lse_offset: int = 0):
    """Merge n_part partials of one sequence.  ``*_offset`` are element offsets
    added to the given tensors' base addresses (partial rows start at
    ``part_offset`` rows; the output at token ``out_offset``)."""
    ob = o_out.element_size()
    _check(lib.lse_merge(n_part, hq, mq, d,
                         _ptr(o_part) + part_offset * d * 4, _ptr(m_part) + part_offset * 4,
                         _ptr(lse_part) + part_offset * 4,
                         _ptr(o_out) + out_offset * o_stride_tok * ob, o_stride_tok, o_stride_head, out_dtype,
                         _ptr(lse_out) + lse_offset * 4, lse_stride_tok, _stream(stream)))


def lse_merge_all(problem: Problem, d_part_base, o_part, m_part, lse_part, o_out, lse_out, stream=None):
    """Merge every sequence's partials in one launch (d_part_base: device part_base)."""
    _check(lib.lse_merge_all(C.byref(problem.c), _ptr(d_part_base), _ptr(o_part), _ptr(m_part), _ptr(lse_part),
                             _ptr(o_out), _ptr(lse_out), _stream(stream)))


def _own_strides(t):
    return (t.stride(0), t.stride(1)) if hasattr(t, "stride") and callable(t.stride) else (
        t.strides[0] // t.itemsize, t.strides[1] // t.itemsize)


def sparse_attn_own_fwd(problem: Problem, q, k_own, v_own, o_part, m_part, lse_part, stream=None):
    """Own-block partial of every row (own-block mask), after sparse_attn_partial_fwd."""
    st, sh = _own_strides(k_own)
    if _own_strides(v_own) != (st, sh):
        raise ValueError("k_own and v_own need the same strides")
    _check(lib.sparse_attn_own_fwd(C.byref(problem.c), _ptr(q), _ptr(k_own), _ptr(v_own), st, sh, _ptr(o_part),
                                   _ptr(m_part), _ptr(lse_part), _stream(stream)))


def _own_block_arg(own):
    if own is None:
        return None
    ko, vo, dko, dvo = own
    st, sh = _own_strides(ko)
    if any(_own_strides(t) != (st, sh) for t in (vo, dko, dvo)):
        raise ValueError("own-block tensors need the same strides")
    return C.byref(skv_own_block(_ptr(ko), _ptr(vo), _ptr(dko), _ptr(dvo), st, sh))


def sparse_attn_bwd_noalloc(problem: Problem, plan_kv, plan_q, q, k, v, o, lse, dout, dq, dk, dv, stream=None,
                            own=None):
    """sparse_attn_bwd with the library's static scratch in place of a workspace."""
    _check(lib.sparse_attn_bwd_noalloc(C.byref(problem.c), C.byref(plan_kv.c), C.byref(plan_q.c), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                       _own_block_arg(own), _stream(stream)))


def sparse_attn_bwd(problem: Problem, plan_kv, plan_q, q, k, v, o, lse, dout, dq, dk, dv, workspace, stream=None,
                    own=None):
    """plan_kv: BWD plan (key ranges); plan_q: FWD plan (forward items, for dQ).
    own = (k_own, v_own, dk_own, dv_own) under the own-block mask, else None."""
    nbytes = workspace.numel() * workspace.element_size()
    ob = _own_block_arg(own)
    _check(lib.sparse_attn_bwd(C.byref(problem.c), C.byref(plan_kv.c), C.byref(plan_q.c), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                               ob, _stream(stream)))
