"""Plain float64 masked softmax attention, its Split-KV partials and merge, and
its gradients — the definitions written out, one (head, draft block) at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:
  * Draft queries attend over a much longer context with a block-sparse mask
    ([P1] lede; [P3] Abstract).  Reading of the mask (the pages print none):
    draft block b is anchored at context position a_b and its B rows see the
    context prefix [0, e_b) with e_b = min(a_b + B, N), i.e. the context before
    the anchor plus the block's own B positions, clipped at the end of the
    context.
  * Split-KV keeps each KV shard local and aggregates the shard-local results
    exactly, so the result equals the unsharded one ([P1] "Split-KV's Core
    Mechanism").  Reading: a shard (KV chunk) yields an unnormalised output
    O_c = sum_j exp(s_j - m_c) v_j with its row max m_c and log-sum-exp LSE_c
    (natural log); shards are merged by log-sum-exp rescaling.
  * The exactness matters for gradient correctness in training ([P1] "Split-KV's
    Core Mechanism"); the backward reuses the merged LSE.

Conventions: a row with no visible key has O = 0 and LSE = -inf (never NaN);
in a partial such a row has m_c = LSE_c = -inf and its O_c is unspecified
(returned as 0 here).  KV head of query head h is h // (Hq / Hkv).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def block_ends(anchors, block: int, n_ctx: int) -> np.ndarray:
    """e_b = min(a_b + B, N): the exclusive end of the context prefix block b sees."""
    return np.minimum(np.asarray(anchors, dtype=np.int64) + int(block), int(n_ctx))


def visible_mask(anchors, block: int, n_ctx: int) -> np.ndarray:
    """Dense boolean mask [Mq, N]: query row r sees key j iff j < e_{r // B}."""
    e = block_ends(anchors, block, n_ctx)
    e_row = np.repeat(e, block)
    return np.arange(n_ctx)[None, :] < e_row[:, None]


def _softmax_rows(s: np.ndarray):
    """Row max, exp(s - max) and row sum of a [rows, keys] logit block (keys > 0)."""
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p, p.sum(axis=1)


def attention(q, k, v, anchors, block: int, sm_scale: float, heads: Optional[Iterable[int]] = None):
    """Masked softmax attention of one sequence.

    q [M, Hq, D], k/v [N, Hkv, D] (float64).  Returns O [M, Hq, D] and
    LSE [M, Hq]; rows of heads not in ``heads`` are left 0 / -inf.
    """
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    e = block_ends(anchors, block, N)
    O = np.zeros((M, Hq, D))
    LSE = np.full((M, Hq), -np.inf)
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        for b, n in enumerate(e):
            if n <= 0:
                continue
            rows = slice(b * block, (b + 1) * block)
            s = sm_scale * (q[rows, h] @ k[:n, g].T)
            m, p, l = _softmax_rows(s)
            O[rows, h] = (p @ v[:n, g]) / l[:, None]
            LSE[rows, h] = m + np.log(l)
    return O, LSE


def chunk_partials(q, k, v, anchors, block: int, sm_scale: float, chunk: int,
                   heads: Optional[Iterable[int]] = None):
    """Per-KV-chunk partials of one sequence.

    Chunk c holds keys [c*L, min((c+1)*L, N)).  For each row the visible keys of
    the chunk are those below e_b.  Returns o_part [C, Hq, M, D] (unnormalised),
    m_part [C, Hq, M] (row max of the scaled logits) and lse_part [C, Hq, M].
    """
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    C = -(-N // chunk)
    e = block_ends(anchors, block, N)
    o_part = np.zeros((C, Hq, M, D))
    m_part = np.full((C, Hq, M), -np.inf)
    lse_part = np.full((C, Hq, M), -np.inf)
    for c in range(C):
        lo = c * chunk
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            for b, n in enumerate(e):
                hi = min((c + 1) * chunk, N, int(n))
                if hi <= lo:
                    continue
                rows = slice(b * block, (b + 1) * block)
                s = sm_scale * (q[rows, h] @ k[lo:hi, g].T)
                m, p, l = _softmax_rows(s)
                o_part[c, h, rows] = p @ v[lo:hi, g]
                m_part[c, h, rows] = m
                lse_part[c, h, rows] = m + np.log(l)
    return o_part, m_part, lse_part


def lse_merge(o_part, m_part, lse_part):
    """Exact merge of C partials by log-sum-exp rescaling.

    LSE = M + ln sum_c exp(LSE_c - M) with M = max_c LSE_c, and
    O = sum over partials with LSE_c > -inf of exp(m_c - LSE) * O_c.
    A row whose partials are all -inf gets O = 0, LSE = -inf.
    Inputs [C, Hq, M(, D)]; returns O [M, Hq, D], LSE [M, Hq].
    """
    C, Hq, M, D = o_part.shape
    Mx = lse_part.max(axis=0)                                  # [Hq, M]
    live = np.isfinite(Mx)
    Ms = np.where(live, Mx, 0.0)
    with np.errstate(invalid="ignore"):
        ssum = np.exp(lse_part - Ms[None]).sum(axis=0)         # exp(-inf) = 0
    lse = np.where(live, Ms + np.log(np.where(live, ssum, 1.0)), -np.inf)
    O = np.zeros((Hq, M, D))
    for c in range(C):
        vis = np.isfinite(lse_part[c]) & live
        with np.errstate(invalid="ignore"):
            w = np.where(vis, np.exp(np.where(vis, m_part[c] - lse, 0.0)), 0.0)
        O += w[..., None] * np.where(vis[..., None], o_part[c], 0.0)
    return O.transpose(1, 0, 2).copy(), lse.T.copy()


def attention_bwd(q, k, v, anchors, block: int, sm_scale: float, do, heads: Optional[Iterable[int]] = None,
                  kv_heads: Optional[Iterable[int]] = None):
    """Gradients of L = sum(O * dO) for one sequence, reusing the row LSE.

    With s = scale * q.k, P = exp(s - LSE) on visible entries (0 elsewhere),
    Delta = sum_d dO * O, dS = P * (dO.v - Delta):
        dV_j = sum_rows P dO,   dQ = scale * dS K,   dK_j = scale * sum_rows dS q,
    summed over the query heads sharing a KV head.  Keys no query sees get
    dK = dV = 0.  ``kv_heads`` restricts work to those KV groups (others 0).
    Returns dq, dk, dv, O, LSE (O, LSE from this module's own forward).
    """
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    if kv_heads is not None:
        heads = [h for g in kv_heads for h in range(g * G, (g + 1) * G)]
    O, LSE = attention(q, k, v, anchors, block, sm_scale, heads=heads)
    e = block_ends(anchors, block, N)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        for b, n in enumerate(e):
            if n <= 0:
                continue
            rows = slice(b * block, (b + 1) * block)
            s = sm_scale * (q[rows, h] @ k[:n, g].T)
            p = np.exp(s - LSE[rows, h][:, None])
            delta = (do[rows, h] * O[rows, h]).sum(axis=1)
            dv[:n, g] += p.T @ do[rows, h]
            dp = do[rows, h] @ v[:n, g].T
            ds = p * (dp - delta[:, None])
            dq[rows, h] = sm_scale * (ds @ k[:n, g])
            dk[:n, g] += sm_scale * (ds.T @ q[rows, h])
    return dq, dk, dv, O, LSE


# ---------------------------------------------------------------------------
# Whole-workload wrappers (sequences are independent; heads may be sub-sampled)
# ---------------------------------------------------------------------------

def _seq_inputs(w, s: int, names=("q", "k", "v")):
    qs = slice(int(w.q_off[s]), int(w.q_off[s + 1]))
    ks = slice(int(w.kv_off[s]), int(w.kv_off[s + 1]))
    out = []
    for nm in names:
        out.append(w.as_f64(nm, rows=qs if nm in ("q", "do") else ks))
    return out


def attention_workload(w, heads: Optional[Iterable[int]] = None):
    """O [sum Mq, Hq, D] and LSE [sum Mq, Hq] for every sequence of a workload."""
    cfg = w.cfg
    tq = int(w.q_off[-1])
    O = np.zeros((tq, cfg.hq, cfg.d))
    LSE = np.full((tq, cfg.hq), -np.inf)
    for s in range(cfg.n_seq):
        q, k, v = _seq_inputs(w, s)
        o, l = attention(q, k, v, w.seq_anchors(s), cfg.block, w.sm_scale, heads=heads)
        O[int(w.q_off[s]):int(w.q_off[s + 1])] = o
        LSE[int(w.q_off[s]):int(w.q_off[s + 1])] = l
    return O, LSE


def partials_workload(w, s: int, heads: Optional[Iterable[int]] = None):
    """chunk_partials for sequence s of a workload (layout [C, Hq, Mq_s(, D)])."""
    q, k, v = _seq_inputs(w, s)
    return chunk_partials(q, k, v, w.seq_anchors(s), w.cfg.block, w.sm_scale, w.cfg.chunk, heads=heads)


def bwd_workload(w, kv_heads: Optional[Iterable[int]] = None, seqs: Optional[Iterable[int]] = None):
    """dq, dk, dv, O, LSE over the workload (restricted to kv_heads / seqs if given)."""
    cfg = w.cfg
    tq, tk = int(w.q_off[-1]), int(w.kv_off[-1])
    dq = np.zeros((tq, cfg.hq, cfg.d))
    dk = np.zeros((tk, cfg.hkv, cfg.d))
    dv = np.zeros((tk, cfg.hkv, cfg.d))
    O = np.zeros((tq, cfg.hq, cfg.d))
    LSE = np.full((tq, cfg.hq), -np.inf)
    for s in (range(cfg.n_seq) if seqs is None else seqs):
        q, k, v, do = _seq_inputs(w, s, ("q", "k", "v", "do"))
        a, b = int(w.q_off[s]), int(w.q_off[s + 1])
        c, d = int(w.kv_off[s]), int(w.kv_off[s + 1])
        r = attention_bwd(q, k, v, w.seq_anchors(s), cfg.block, w.sm_scale, do, kv_heads=kv_heads)
        dq[a:b], dk[c:d], dv[c:d], O[a:b], LSE[a:b] = r
    return dq, dk, dv, O, LSE
