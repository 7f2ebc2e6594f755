"""Pins for the float64 attention oracle: each test checks it against something
other than itself (brute force, a library routine, closed forms, finite
differences).  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic import make, make_custom


def _rand_problem(rng, N, A, B, Hq, Hkv, D, anchor_lo=0):
    anchors = np.sort(rng.integers(anchor_lo, N, size=A))
    q = rng.standard_normal((A * B, Hq, D))
    k = rng.standard_normal((N, Hkv, D))
    v = rng.standard_normal((N, Hkv, D))
    do = rng.standard_normal((A * B, Hq, D))
    return anchors, q, k, v, do


def _brute_attention(q, k, v, anchors, B, scale):
    """Pure-Python loops with math.exp: row r of block r//B sees keys j < min(a+B, N)."""
    M, Hq, D = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    O = [[[0.0] * D for _ in range(Hq)] for _ in range(M)]
    L = [[-math.inf] * Hq for _ in range(M)]
    for r in range(M):
        end = min(int(anchors[r // B]) + B, N)
        for h in range(Hq):
            g = h // G
            logits = []
            for j in range(end):
                logits.append(scale * sum(q[r, h, t] * k[j, g, t] for t in range(D)))
            if not logits:
                continue
            mx = max(logits)
            ws = [math.exp(x - mx) for x in logits]
            den = sum(ws)
            for t in range(D):
                O[r][h][t] = sum(ws[j] * v[j, g, t] for j in range(end)) / den
            L[r][h] = mx + math.log(den)
    return np.array(O), np.array(L)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, N, A = 2, 4, 2, 5, 37, 3
    anchors, q, k, v, _ = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    anchors[-1] = N - 1  # one block clipped at the end of the context
    O, L = oracle.attention(q, k, v, anchors, B, 0.37)
    Ob, Lb = _brute_attention(q, k, v, anchors, B, 0.37)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_dense_case_equals_torch_sdpa_with_grads():
    """All blocks see the whole context (anchors at N-1): plain dense attention."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, N, A = 4, 6, 2, 8, 50, 3
    anchors = np.full(A, N - 1)
    _, q, k, v, do = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    scale = 1.0 / math.sqrt(D)
    O, L = oracle.attention(q, k, v, anchors, B, scale)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, anchors, B, scale, do)
    G = Hq // Hkv
    tq = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)            # [Hq, M, D]
    tk = torch.tensor(k.transpose(1, 0, 2), requires_grad=True)            # [Hkv, N, D]
    tv = torch.tensor(v.transpose(1, 0, 2), requires_grad=True)
    ke = tk.repeat_interleave(G, dim=0)
    ve = tv.repeat_interleave(G, dim=0)
    to = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, scale=scale)
    to.backward(torch.tensor(do.transpose(1, 0, 2)))
    np.testing.assert_allclose(O, to.detach().numpy().transpose(1, 0, 2), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy().transpose(1, 0, 2), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy().transpose(1, 0, 2), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy().transpose(1, 0, 2), atol=1e-11)
    tl = torch.logsumexp(scale * tq @ ke.transpose(1, 2), dim=-1).detach().numpy().T
    np.testing.assert_allclose(L, tl, atol=1e-12)


def test_single_visible_key():
    """B = 1 and anchor 0: the row sees key 0 only, so O = v0, LSE = s0,
    dQ = 0, dK = 0 and dV_0 = sum over the group's heads of dO."""
    rng = np.random.default_rng(7)
    _, q, k, v, do = _rand_problem(rng, 9, 1, 1, 2, 1, 4)
    anchors = np.array([0])
    O, L = oracle.attention(q, k, v, anchors, 1, 0.5)
    np.testing.assert_allclose(O[0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(O[0, 1], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(L[0], 0.5 * q[0] @ k[0, 0], atol=1e-15)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, anchors, 1, 0.5, do)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0, 0], do[0, 0] + do[0, 1], atol=1e-15)
    assert np.abs(dv[1:]).max() == 0.0


@pytest.mark.parametrize("chunk", [1, 7, 64, 100, 101, 1000])
def test_split_then_merge_equals_unsplit(chunk):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, N, A = 4, 4, 2, 8, 100, 5
    anchors, q, k, v, _ = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    O, L = oracle.attention(q, k, v, anchors, B, 0.3)
    op, mp, lp = oracle.chunk_partials(q, k, v, anchors, B, 0.3, chunk)
    Om, Lm = oracle.lse_merge(op, mp, lp)
    np.testing.assert_allclose(Om, O, atol=1e-12)
    np.testing.assert_allclose(Lm, L, atol=1e-12)


def test_partials_are_chunk_restricted_attention():
    """Each partial equals plain attention over the chunk's keys alone:
    O_c / exp(LSE_c - m_c) is the normalised chunk output."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, N, A, L = 2, 2, 1, 4, 40, 3, 16
    anchors, q, k, v, _ = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    op, mp, lp = oracle.chunk_partials(q, k, v, anchors, B, 0.5, L)
    for c in range(op.shape[0]):
        lo, hi = c * L, min((c + 1) * L, N)
        for r in range(A * B):
            end = min(int(anchors[r // B]) + B, N)
            for h in range(Hq):
                if end <= lo:
                    assert mp[c, h, r] == -np.inf and lp[c, h, r] == -np.inf
                    continue
                s = 0.5 * (k[lo:min(hi, end), 0] @ q[r, h])
                assert mp[c, h, r] == pytest.approx(s.max(), abs=1e-14)
                w = np.exp(s - s.max())
                np.testing.assert_allclose(op[c, h, r], w @ v[lo:min(hi, end), 0], atol=1e-12)
                assert lp[c, h, r] == pytest.approx(s.max() + np.log(w.sum()), abs=1e-13)


def test_fully_masked_partials_change_nothing():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, D, N, A = 4, 2, 2, 8, 64, 2
    anchors, q, k, v, _ = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    op, mp, lp = oracle.chunk_partials(q, k, v, anchors, B, 0.3, 16)
    Om, Lm = oracle.lse_merge(op, mp, lp)
    # append partials that are empty for every row (and garbage in O_c)
    extra = 3
    op2 = np.concatenate([op, np.full((extra,) + op.shape[1:], np.nan)])
    mp2 = np.concatenate([mp, np.full((extra,) + mp.shape[1:], -np.inf)])
    lp2 = np.concatenate([lp, np.full((extra,) + lp.shape[1:], -np.inf)])
    Om2, Lm2 = oracle.lse_merge(op2, mp2, lp2)
    assert np.array_equal(Om, Om2) and np.array_equal(Lm, Lm2)
    # all partials empty: O = 0, LSE = -inf, no NaN
    Oe, Le = oracle.lse_merge(op2[-extra:], mp2[-extra:], lp2[-extra:])
    assert np.all(Oe == 0) and np.all(Le == -np.inf)


def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(14)
    B, Hq, Hkv, D, N, A = 4, 2, 1, 6, 30, 3
    anchors, q, k, v, do = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    k[:] = k[0:1]
    O, L = oracle.attention(q, k, v, anchors, B, 0.7)
    e = np.minimum(anchors + B, N)
    for r in range(A * B):
        n = int(e[r // B])
        for h in range(Hq):
            np.testing.assert_allclose(O[r, h], v[:n, 0].mean(axis=0), atol=1e-13)
            assert L[r, h] == pytest.approx(0.7 * q[r, h] @ k[0, 0] + math.log(n), abs=1e-13)
    dq, _, _, _, _ = oracle.attention_bwd(q, k, v, anchors, B, 0.7, do)
    assert np.abs(dq).max() < 1e-12


def test_constant_values_give_that_value():
    rng = np.random.default_rng(15)
    B, Hq, Hkv, D, N, A = 4, 4, 2, 6, 33, 4
    anchors, q, k, v, _ = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    v[:] = v[0:1]
    O, _ = oracle.attention(q, k, v, anchors, B, 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(O[:, h], np.broadcast_to(v[0, h // 2], O[:, h].shape), atol=1e-13)


def test_gradients_match_finite_differences():
    rng = np.random.default_rng(16)
    B, Hq, Hkv, D, N, A = 3, 4, 2, 5, 20, 3
    anchors, q, k, v, do = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    scale = 0.45
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, anchors, B, scale, do)

    def loss(qq, kk, vv):
        O, _ = oracle.attention(qq, kk, vv, anchors, B, scale)
        return float((O * do).sum())

    eps = 1e-5
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = plus
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = minus
            lm = loss(args["q"], args["k"], args["v"])
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-7, (name, idx)


def test_gradient_closed_forms():
    """sum_j dK_j = 0 per KV head and sum_j dV_j = sum of dO over the group."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, D, N, A = 4, 6, 3, 8, 90, 6
    anchors, q, k, v, do = _rand_problem(rng, N, A, B, Hq, Hkv, D)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, anchors, B, 0.2, do)
    G = Hq // Hkv
    for g in range(Hkv):
        assert np.abs(dk[:, g].sum(axis=0)).max() < 1e-12
        np.testing.assert_allclose(dv[:, g].sum(axis=0), do[:, g * G:(g + 1) * G].sum(axis=(0, 1)), atol=1e-12)
    # keys beyond the furthest block end receive nothing
    e_max = int(min(anchors.max() + B, N))
    assert np.all(dk[e_max:] == 0) and np.all(dv[e_max:] == 0)


def test_workload_wrappers_and_generator_are_consistent():
    w = make("c3", seed=3, n_ctx_range=(300, 700), n_anchor=5, hq=4, hkv=2, d=16, chunk=128)
    assert np.all(np.diff(w.q_off) == 5 * 16)
    assert np.all(np.diff(w.kv_off) == w.n_ctx)
    for s in range(w.cfg.n_seq):
        a = w.seq_anchors(s)
        assert np.all(np.diff(a) >= 0) and a.min() >= 256 and a.max() < w.n_ctx[s]
    O, L = oracle.attention_workload(w)
    s = 2
    q = w.as_f64("q", rows=slice(int(w.q_off[s]), int(w.q_off[s + 1])))
    k = w.as_f64("k", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
    v = w.as_f64("v", rows=slice(int(w.kv_off[s]), int(w.kv_off[s + 1])))
    O2, L2 = oracle.attention(q, k, v, w.seq_anchors(s), 16, w.sm_scale)
    assert np.array_equal(O[int(w.q_off[s]):int(w.q_off[s + 1])], O2)
    # the same seed gives identical bits; another seed does not
    w2 = make("c3", seed=3, n_ctx_range=(300, 700), n_anchor=5, hq=4, hkv=2, d=16, chunk=128)
    assert np.array_equal(w.k, w2.k) and np.array_equal(w.anchors, w2.anchors)
    w3 = make("c3", seed=4, n_ctx_range=(300, 700), n_anchor=5, hq=4, hkv=2, d=16, chunk=128)
    assert not np.array_equal(w.k, w3.k)


def test_bf16_rounding_is_nearest_even():
    from synthetic import bf16_bits_from_f32, f64_from_bf16_bits
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    y = f64_from_bf16_bits(bf16_bits_from_f32(x))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... i.e. 1.015625)
    assert list(y) == [1.0, 1.0, 1.015625, -2.5, 1.0]
    z = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    zb = f64_from_bf16_bits(bf16_bits_from_f32(z))
    assert np.max(np.abs(zb - z) / np.abs(z)) <= 2 ** -8   # unit roundoff of an 8-bit significand


def test_custom_workload():
    w = make_custom([100, 70], [[90, 3], [69, 10]], block=4, hq=2, hkv=1, d=8, dtype="f32", chunk=64)
    assert list(w.anchors) == [3, 90, 10, 69]
    O, L = oracle.attention_workload(w)
    assert np.isfinite(L).all()
