"""Pins of the own-block mask oracle (CPU): the exact identity with the
prefix-mask oracle when the own keys are copies of the context keys at
[a_b, a_b + B), finite differences for every gradient, and the anchor-0 case
against torch's scaled-dot-product attention."""
import numpy as np
import pytest
import torch

import oracle
from synthetic import add_own_block, make_custom



def _w(from_context: bool, seed=2, dtype="f32"):
    w = make_custom([300, 200], [[0, 40, 41, 250], [5, 100, 150, 184]], block=16, hq=4, hkv=2, d=8,
                    dtype=dtype, chunk=64, seed=seed, with_do=True)
    return add_own_block(w, from_context=from_context)


def test_own_block_equals_prefix_mask_when_own_keys_are_the_context_keys():
    w = _w(True)
    O, L = oracle.attention_own_workload(w)
    O1, L1 = oracle.attention_workload(w)
    assert np.isfinite(L).all()
    np.testing.assert_allclose(O, O1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L1, rtol=0, atol=1e-12)
    dq, dk, dv, dko, dvo = oracle.bwd_own_workload(w)
    dq1, dk1, dv1 = oracle.bwd_workload(w)[:3]
    np.testing.assert_allclose(dq, dq1, rtol=0, atol=1e-12)
    # the prefix mask's dK, dV of context keys [a_b, a_b + B) = own-block gradients
    # of block b plus the context gradients of later blocks' prefixes
    dk_sum, dv_sum = dk.copy(), dv.copy()
    B = w.cfg.block
    for s in range(w.cfg.n_seq):
        k0, t0 = int(w.kv_off[s]), int(w.q_off[s])
        for bi, a in enumerate(w.seq_anchors(s)):
            rows = slice(t0 + bi * B, t0 + (bi + 1) * B)
            dk_sum[k0 + a:k0 + a + B] += dko[rows]
            dv_sum[k0 + a:k0 + a + B] += dvo[rows]
    np.testing.assert_allclose(dk_sum, dk1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_sum, dv1, rtol=0, atol=1e-12)


def test_own_block_gradients_match_finite_differences():
    w = _w(False, seed=5)
    s = 1
    qs = slice(int(w.q_off[s]), int(w.q_off[s + 1]))
    ks = slice(int(w.kv_off[s]), int(w.kv_off[s + 1]))
    x = {n: w.as_f64(n, rows=qs if n in ("q", "do", "k_own", "v_own") else ks).copy()
         for n in ("q", "k", "v", "k_own", "v_own", "do")}
    anc, B, sc = w.seq_anchors(s), w.cfg.block, w.sm_scale

    def loss():
        O, _ = oracle.attention_own(x["q"], x["k"], x["v"], x["k_own"], x["v_own"], anc, B, sc)
        return float((O * x["do"]).sum())

    dq, dk, dv, dko, dvo = oracle.attention_own_bwd(x["q"], x["k"], x["v"], x["k_own"], x["v_own"], anc, B, sc,
                                                    x["do"])[:5]
    grads = {"q": dq, "k": dk, "v": dv, "k_own": dko, "v_own": dvo}
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, g in grads.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in g.shape)
            if name in ("k", "v"):      # a context key some block sees
                idx = (int(rng.integers(0, int(np.max(anc)))),) + idx[1:]
            old = x[name][idx]
            x[name][idx] = old + eps
            lp = loss()
            x[name][idx] = old - eps
            lm = loss()
            x[name][idx] = old
            assert abs((lp - lm) / (2 * eps) - g[idx]) < 1e-6 * max(1.0, abs(g[idx])), (name, idx)


def test_anchor_zero_sees_only_its_own_block_like_sdpa():
    w = _w(False, seed=9)
    O, L = oracle.attention_own_workload(w)
    B, G = w.cfg.block, w.cfg.hq // w.cfg.hkv
    q = w.as_f64("q")[0:B]                 # sequence 0, block 0 has anchor 0
    ko, vo = w.as_f64("k_own")[0:B], w.as_f64("v_own")[0:B]
    for h in range(w.cfg.hq):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None], torch.from_numpy(ko[:, h // G])[None],
            torch.from_numpy(vo[:, h // G])[None], scale=w.sm_scale)[0].numpy()
        np.testing.assert_allclose(O[0:B, h], ref, rtol=0, atol=1e-12)
    # the own partial alone, merged with nothing, is the same output
    o, m, lse = oracle.own_partial(q, ko, vo, B, w.sm_scale, w.cfg.hkv)
    np.testing.assert_allclose((o * np.exp(m - lse)[..., None]).transpose(1, 0, 2), O[0:B], rtol=0, atol=1e-12)
    # its max and log-sum-exp (and the merged LSE of an anchor-0 block) are
    # those of the own-block scores, from torch's max and logsumexp
    for h in range(w.cfg.hq):
        s = w.sm_scale * (torch.from_numpy(q[:, h]) @ torch.from_numpy(ko[:, h // G]).T)
        np.testing.assert_allclose(m[h], s.max(dim=-1).values.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0:B, h], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)
