"""Seeded synthetic workloads shaped like the anchor-sampled draft attention the
Split-KV pages describe (short draft-query blocks over a much longer context).

The pages name no dataset for this path; these inputs stand in for the unnamed
training workload: Q, K, V and dO are drawn N(0, 1), anchors are drawn per
sequence (uniform or Beta(5,1)-skewed) and sorted, and each anchor owns one
draft block of ``block`` query rows.

Layouts (token-major, head, then head_dim contiguous):
  q, do : [sum_s Mq_s, hq, d]     with Mq_s = n_anchor * block
  k, v  : [sum_s N_s, hkv, d]
  q_off : int64 [n_seq + 1]  first query row of each sequence
  kv_off: int64 [n_seq + 1]  first context token of each sequence
  anchors: int32 [sum_s n_anchor]  sorted ascending within each sequence

For bf16 workloads the tensors are stored as uint16 bf16 bit patterns
(round-to-nearest-even from float32 draws); for f32 workloads as float32.

Every random stream is keyed by SeedSequence([seed, config id, stream id]) so
that lengths, anchors, Q, K, V and dO are independent and reproducible.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

STREAM_LEN, STREAM_ANCHOR, STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_K_OWN, STREAM_V_OWN = range(8)
_SLAB = 1 << 24  # values drawn per call, keeps peak host memory bounded


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cid: int
    n_seq: int
    n_ctx: Optional[int]              # fixed context length, or None
    n_ctx_range: Optional[tuple]      # inclusive (lo, hi) when lengths vary
    n_anchor: int
    anchor_dist: str                  # "uniform" or "beta51"
    anchor_lo: int                    # lower bound for "uniform"
    block: int                        # draft tokens per anchor (B)
    hq: int
    hkv: int
    d: int
    dtype: str                        # "f32" or "bf16"
    chunk: int                        # KV chunk length (L)
    bwd: bool
    note: str = ""


CONFIGS = {
    "c1": Config("c1", 1, 1, 1024, None, 4, "uniform", 64, 16, 2, 2, 64, "f32", 256, False,
                 "tiny fp32, forward only"),
    "c2": Config("c2", 2, 1, 16384, None, 32, "uniform", 256, 16, 32, 8, 128, "bf16", 1024, False,
                 "bf16 forward, 16K context"),
    "c3": Config("c3", 3, 4, None, (16384, 65536), 64, "uniform", 256, 16, 32, 8, 128, "bf16", 2048, True,
                 "bf16 fwd+bwd, 4 sequences of 16K-64K context"),
    "c4": Config("c4", 4, 1, 524288, None, 64, "uniform", 0, 16, 16, 4, 128, "bf16", 8192, True,
                 "64 KV shards of 8192 on one GPU, 512K context"),
    "c5": Config("c5", 5, 1, 262144, None, 128, "beta51", 0, 32, 16, 16, 128, "bf16", 4096, True,
                 "skewed anchors (Beta(5,1)), 256K context"),
}


@dataclasses.dataclass
class Workload:
    cfg: Config
    n_ctx: np.ndarray        # int64 [n_seq]
    anchors: np.ndarray      # int32 [n_seq * n_anchor]
    q_off: np.ndarray        # int64 [n_seq + 1]
    kv_off: np.ndarray       # int64 [n_seq + 1]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    sm_scale: float
    seed: int
    # own-block keys and values, [sum Mq, Hkv, D] (row t holds draft token t's
    # key): present only for the own-block mask variant, see add_own_block
    k_own: Optional[np.ndarray] = None
    v_own: Optional[np.ndarray] = None

    @property
    def is_bf16(self) -> bool:
        return self.cfg.dtype == "bf16"

    def seq_anchors(self, s: int) -> np.ndarray:
        a = self.cfg.n_anchor
        return self.anchors[s * a:(s + 1) * a]

    def as_f64(self, name: str, rows: Optional[slice] = None, head: Optional[int] = None) -> np.ndarray:
        """Exact float64 view of an input (bf16 bits widened exactly)."""
        x = getattr(self, name)
        if rows is not None:
            x = x[rows]
        if head is not None:
            x = x[:, head]
        if self.is_bf16:
            return f64_from_bf16_bits(x)
        return x.astype(np.float64)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, cid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cid, stream]))


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        for lo in range(0, n, _SLAB):
            hi = min(n, lo + _SLAB)
            out[lo:hi] = bf16_bits_from_f32(rng.standard_normal(hi - lo, dtype=np.float32))
    else:
        out = np.empty(n, dtype=np.float32)
        for lo in range(0, n, _SLAB):
            hi = min(n, lo + _SLAB)
            out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
    return out.reshape(shape)


def _draw_anchors(rng: np.random.Generator, cfg: Config, n_ctx: int) -> np.ndarray:
    if cfg.anchor_dist == "uniform":
        lo = min(cfg.anchor_lo, n_ctx - 1)
        a = rng.integers(lo, n_ctx, size=cfg.n_anchor)
    elif cfg.anchor_dist == "beta51":
        x = rng.beta(5.0, 1.0, size=cfg.n_anchor)
        a = np.clip(np.floor(n_ctx * x).astype(np.int64), 0, n_ctx - 1)
    else:
        raise ValueError(f"unknown anchor distribution {cfg.anchor_dist!r}")
    return np.sort(a).astype(np.int32)


def make(cfg, seed: int = 0, with_do: Optional[bool] = None, **overrides) -> Workload:
    """Build a seeded workload for a named config ("c1".."c5") or a Config.

    ``overrides`` replace Config fields (e.g. n_ctx=4096, n_anchor=8, hq=4)
    so that tests can use the same recipe at sizes the oracle finishes quickly.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    if with_do is None:
        with_do = cfg.bwd
    rl = _rng(seed, cfg.cid, STREAM_LEN)
    if cfg.n_ctx_range is not None:
        lo, hi = cfg.n_ctx_range
        n_ctx = rl.integers(lo, hi, size=cfg.n_seq, endpoint=True).astype(np.int64)
    else:
        n_ctx = np.full(cfg.n_seq, int(cfg.n_ctx), dtype=np.int64)
    ra = _rng(seed, cfg.cid, STREAM_ANCHOR)
    anchors = np.concatenate([_draw_anchors(ra, cfg, int(n)) for n in n_ctx]).astype(np.int32)
    return _assemble(cfg, n_ctx, anchors, seed, with_do)


def make_custom(n_ctx: Sequence[int], anchors: Sequence[Sequence[int]], block: int, hq: int, hkv: int,
                d: int, dtype: str = "bf16", chunk: int = 64, seed: int = 0, with_do: bool = True,
                name: str = "custom", kv_period: Optional[int] = None) -> Workload:
    """Workload with explicit lengths and anchors (anchors are sorted here).

    ``kv_period``: K and V rows repeat with this period (row r holds the
    values of row r mod period of one seeded draw), so that contexts of
    millions of keys are generated in seconds.  An odd prime period keeps
    rows that differ by a power of two distinct.
    """
    n_anchor = len(anchors[0])
    if any(len(a) != n_anchor for a in anchors):
        raise ValueError("every sequence needs the same number of anchors")
    cfg = Config(name, 99, len(n_ctx), None, None, n_anchor, "explicit", 0, block, hq, hkv, d, dtype, chunk, with_do)
    n_ctx = np.asarray(n_ctx, dtype=np.int64)
    anc = np.concatenate([np.sort(np.asarray(a, dtype=np.int64)) for a in anchors]).astype(np.int32)
    return _assemble(cfg, n_ctx, anc, seed, with_do, kv_period)


def _kv_rows(rng: np.random.Generator, tk: int, cfg: Config, period: Optional[int]) -> np.ndarray:
    if period is None or period >= tk:
        return _normal(rng, (tk, cfg.hkv, cfg.d), cfg.dtype)
    base = _normal(rng, (period, cfg.hkv, cfg.d), cfg.dtype)
    return np.tile(base, (-(-tk // period), 1, 1))[:tk]


def _assemble(cfg: Config, n_ctx: np.ndarray, anchors: np.ndarray, seed: int, with_do: bool,
              kv_period: Optional[int] = None) -> Workload:
    mq = cfg.n_anchor * cfg.block
    q_off = np.arange(cfg.n_seq + 1, dtype=np.int64) * mq
    kv_off = np.concatenate([[0], np.cumsum(n_ctx)]).astype(np.int64)
    tq, tk = int(q_off[-1]), int(kv_off[-1])
    q = _normal(_rng(seed, cfg.cid, STREAM_Q), (tq, cfg.hq, cfg.d), cfg.dtype)
    k = _kv_rows(_rng(seed, cfg.cid, STREAM_K), tk, cfg, kv_period)
    v = _kv_rows(_rng(seed, cfg.cid, STREAM_V), tk, cfg, kv_period)
    do = _normal(_rng(seed, cfg.cid, STREAM_DO), (tq, cfg.hq, cfg.d), cfg.dtype) if with_do else None
    return Workload(cfg, n_ctx, anchors, q_off, kv_off, q, k, v, do, 1.0 / math.sqrt(cfg.d), seed)


def add_own_block(w: Workload, from_context: bool = False) -> Workload:
    """Attach own-block keys and values [sum Mq, Hkv, D] to a workload.

    Default: seeded N(0, 1) draws (own streams, bf16-rounded for bf16).  With
    ``from_context`` the rows of draft block b are copies of the context rows
    [a_b, a_b + B) of its sequence (every anchor must satisfy a_b + B <= N_s),
    the case in which the own-block mask reproduces the prefix mask.
    """
    c = w.cfg
    tq = int(w.q_off[-1])
    if not from_context:
        w.k_own = _normal(_rng(w.seed, c.cid, STREAM_K_OWN), (tq, c.hkv, c.d), c.dtype)
        w.v_own = _normal(_rng(w.seed, c.cid, STREAM_V_OWN), (tq, c.hkv, c.d), c.dtype)
        return w
    k_own = np.empty((tq, c.hkv, c.d), dtype=w.k.dtype)
    v_own = np.empty_like(k_own)
    for s in range(c.n_seq):
        k0, n = int(w.kv_off[s]), int(w.n_ctx[s])
        for bi, a in enumerate(w.seq_anchors(s)):
            a = int(a)
            if a + c.block > n:
                raise ValueError("anchor + block runs past the context")
            t0 = int(w.q_off[s]) + bi * c.block
            k_own[t0:t0 + c.block] = w.k[k0 + a:k0 + a + c.block]
            v_own[t0:t0 + c.block] = w.v[k0 + a:k0 + a + c.block]
    w.k_own, w.v_own = k_own, v_own
    return w
