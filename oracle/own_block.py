"""Own-block mask variant: plain float64 attention and gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reading (the other reading of the mask; the pages print none): draft queries
cross-attend over the context with a block-sparse mask ([P1] lede; [P3]
Abstract), and a draft block also attends to its own draft tokens, whose keys
and values are a query-sized segment held with the queries rather than
context positions.  Draft block b of a sequence (anchor a_b, B rows) sees the
context keys [0, min(a_b, N)) and all B keys of its own block: k_own, v_own
[M, Hkv, D] hold one key and value per draft token, row t of the sequence's
queries belonging to block t // B.  Every row sees at least its own B keys, so
LSE is always finite.  In Split-KV terms the own-block keys form one more,
query-sized partial next to the context chunks' partials ([P1] "Split-KV's
Core Mechanism": shard-local results merged exactly).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def context_ends(anchors, n_ctx: int) -> np.ndarray:
    """min(a_b, N): the exclusive end of the context prefix block b sees."""
    return np.minimum(np.asarray(anchors, dtype=np.int64), int(n_ctx))


def _keys(k, v, k_own, v_own, n: int, rows: slice, g: int):
    """The keys and values block b sees: context [0, n) then its own B."""
    return np.concatenate([k[:n, g], k_own[rows, g]]), np.concatenate([v[:n, g], v_own[rows, g]])


def attention_own(q, k, v, k_own, v_own, anchors, block: int, sm_scale: float,
                  heads: Optional[Iterable[int]] = None):
    """O [M, Hq, D] and LSE [M, Hq] of one sequence under the own-block mask."""
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    e = context_ends(anchors, N)
    O = np.zeros((M, Hq, D))
    LSE = np.full((M, Hq), -np.inf)
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        for b, n in enumerate(e):
            rows = slice(b * block, (b + 1) * block)
            kk, vv = _keys(k, v, k_own, v_own, int(n), rows, g)
            s = sm_scale * (q[rows, h] @ kk.T)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1)
            O[rows, h] = (p @ vv) / l[:, None]
            LSE[rows, h] = m + np.log(l)
    return O, LSE


def own_partial(q, k_own, v_own, block: int, sm_scale: float, hkv: int):
    """The own-block partial alone: unnormalised O [Hq, M, D], m and LSE [Hq, M]."""
    M, Hq, D = q.shape
    G = Hq // hkv
    o = np.zeros((Hq, M, D))
    m_out = np.full((Hq, M), -np.inf)
    lse = np.full((Hq, M), -np.inf)
    for h in range(Hq):
        g = h // G
        for b in range(M // block):
            rows = slice(b * block, (b + 1) * block)
            s = sm_scale * (q[rows, h] @ k_own[rows, g].T)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            o[h, rows] = p @ v_own[rows, g]
            m_out[h, rows] = m
            lse[h, rows] = m + np.log(p.sum(axis=1))
    return o, m_out, lse


def attention_own_bwd(q, k, v, k_own, v_own, anchors, block: int, sm_scale: float, do,
                      kv_heads: Optional[Iterable[int]] = None):
    """Gradients of L = sum(O * dO) under the own-block mask, reusing the row LSE:
    P = exp(s - LSE), Delta = sum_d dO * O, dS = P * (dO.v - Delta),
    dQ = scale * dS K, dK = scale * dS^T q, dV = P^T dO over the keys each block
    sees (context prefix and own block), summed over the query heads sharing a
    KV head.  Returns dq, dk, dv, dk_own, dv_own, O, LSE."""
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    heads = None if kv_heads is None else [h for g in kv_heads for h in range(g * G, (g + 1) * G)]
    O, LSE = attention_own(q, k, v, k_own, v_own, anchors, block, sm_scale, heads=heads)
    e = context_ends(anchors, N)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dk_own, dv_own = np.zeros_like(k_own), np.zeros_like(v_own)
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        for b, n in enumerate(e):
            n = int(n)
            rows = slice(b * block, (b + 1) * block)
            kk, vv = _keys(k, v, k_own, v_own, n, rows, g)
            s = sm_scale * (q[rows, h] @ kk.T)
            p = np.exp(s - LSE[rows, h][:, None])
            delta = (do[rows, h] * O[rows, h]).sum(axis=1)
            dvv = p.T @ do[rows, h]
            ds = p * (do[rows, h] @ vv.T - delta[:, None])
            dkk = sm_scale * (ds.T @ q[rows, h])
            dq[rows, h] = sm_scale * (ds @ kk)
            dk[:n, g] += dkk[:n]
            dv[:n, g] += dvv[:n]
            dk_own[rows, g] += dkk[n:]
            dv_own[rows, g] += dvv[n:]
    return dq, dk, dv, dk_own, dv_own, O, LSE


def _seq(w, s: int):
    qs = slice(int(w.q_off[s]), int(w.q_off[s + 1]))
    ks = slice(int(w.kv_off[s]), int(w.kv_off[s + 1]))
    f = w.as_f64
    return f("q", rows=qs), f("k", rows=ks), f("v", rows=ks), f("k_own", rows=qs), f("v_own", rows=qs), qs, ks


def attention_own_workload(w, heads: Optional[Iterable[int]] = None):
    """O, LSE over every sequence of a workload that carries k_own / v_own."""
    cfg = w.cfg
    tq = int(w.q_off[-1])
    O = np.zeros((tq, cfg.hq, cfg.d))
    LSE = np.full((tq, cfg.hq), -np.inf)
    for s in range(cfg.n_seq):
        q, k, v, ko, vo, qs, _ = _seq(w, s)
        O[qs], LSE[qs] = attention_own(q, k, v, ko, vo, w.seq_anchors(s), cfg.block, w.sm_scale, heads=heads)
    return O, LSE


def bwd_own_workload(w, kv_heads: Optional[Iterable[int]] = None, seqs: Optional[Iterable[int]] = None):
    """dq, dk, dv, dk_own, dv_own over the workload (restricted to kv_heads / seqs)."""
    cfg = w.cfg
    tq, tk = int(w.q_off[-1]), int(w.kv_off[-1])
    dq = np.zeros((tq, cfg.hq, cfg.d))
    dk, dv = np.zeros((tk, cfg.hkv, cfg.d)), np.zeros((tk, cfg.hkv, cfg.d))
    dko, dvo = np.zeros((tq, cfg.hkv, cfg.d)), np.zeros((tq, cfg.hkv, cfg.d))
    for s in (range(cfg.n_seq) if seqs is None else seqs):
        q, k, v, ko, vo, qs, ks = _seq(w, s)
        do = w.as_f64("do", rows=qs)
        r = attention_own_bwd(q, k, v, ko, vo, w.seq_anchors(s), cfg.block, w.sm_scale, do, kv_heads=kv_heads)
        dq[qs], dk[ks], dv[ks], dko[qs], dvo[qs] = r[:5]
    return dq, dk, dv, dko, dvo
