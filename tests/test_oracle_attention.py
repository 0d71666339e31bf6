"""Pins of the attention oracle against things other than itself.

Each pin is chosen so that a plausible slip in ``oracle.attention`` (wrong
sign of the score, a dropped scale, an off-by-one causal bound, K and V
swapped, a transposed operand) fails at least one of them; the mutation test
at the end demonstrates that on planted mistakes.

Sources: "vLLM / PagedAttention" (awesome.papernotes.org), key design 1:
eq. 1 (exact attention) and eq. 2 (the same attention evaluated block by
block over KV blocks of B tokens).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oa


def _rng(seed=0):
    return np.random.default_rng(seed)


# --- library routine: float64 SDPA -------------------------------------------------

def _sdpa(q, K, V, scale, causal):
    # torch's CPU math path in float64; q [n][d], K/V [L][d]
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    kt = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("L,d", [(1, 8), (7, 8), (33, 16), (200, 128)])
def test_decode_matches_float64_sdpa(L, d):
    r = _rng(L * 1000 + d)
    H = 3
    q = r.standard_normal((H, d))
    K = r.standard_normal((L, H, d))
    V = r.standard_normal((L, H, d))
    got = oa.decode(q, K, V)
    for h in range(H):
        ref = _sdpa(q[h][None], K[:, h], V[:, h], 1 / math.sqrt(d), causal=False)[0]
        np.testing.assert_allclose(got[h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,d", [(1, 8), (9, 8), (64, 32)])
def test_prefill_matches_float64_causal_sdpa(L, d):
    r = _rng(7 + L)
    H = 2
    Q = r.standard_normal((L, H, d))
    K = r.standard_normal((L, H, d))
    V = r.standard_normal((L, H, d))
    got = oa.prefill(Q, K, V)
    for h in range(H):
        ref = _sdpa(Q[:, h], K[:, h], V[:, h], 1 / math.sqrt(d), causal=True)
        np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=1e-12)


# --- closed forms ------------------------------------------------------------------

def test_zero_query_gives_mean_of_values():
    r = _rng(1)
    K = r.standard_normal((13, 1, 8))
    V = r.standard_normal((13, 1, 8))
    o = oa.decode(np.zeros((1, 8)), K, V)
    np.testing.assert_allclose(o[0], V[:, 0].mean(axis=0), atol=1e-14)


def test_constant_values_give_that_constant():
    r = _rng(2)
    c = r.standard_normal(16)
    K = r.standard_normal((21, 1, 16)) * 3
    V = np.broadcast_to(c, (21, 1, 16)).copy()
    o = oa.decode(r.standard_normal((1, 16)), K, V)
    np.testing.assert_allclose(o[0], c, atol=1e-13)


def test_single_token_history_returns_its_value_exactly():
    r = _rng(3)
    K = r.standard_normal((1, 2, 8))
    V = r.standard_normal((1, 2, 8))
    o = oa.decode(r.standard_normal((2, 8)), K, V)
    assert np.array_equal(o, V[0])


def test_two_keys_follow_the_logistic_function():
    # a = exp(s0)/(exp(s0)+exp(s1)) = 1/(1+exp(s1-s0)); catches a wrong sign or scale
    r = _rng(4)
    d = 8
    q = r.standard_normal(d)
    K = r.standard_normal((2, d))
    V = r.standard_normal((2, d))
    scale = 0.37
    s0, s1 = scale * float(q @ K[0]), scale * float(q @ K[1])
    a0 = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = a0 * V[0] + (1 - a0) * V[1]
    np.testing.assert_allclose(oa.attend(q, K, V, scale), expect, atol=1e-14)


def test_dominant_key_selects_its_value():
    r = _rng(5)
    d, L, star = 16, 40, 17
    q = r.standard_normal(d)
    K = r.standard_normal((L, d)) * 0.1
    K[star] = q / np.linalg.norm(q) * 200.0   # score gap >> 30
    V = r.standard_normal((L, d))
    scale = 1 / math.sqrt(d)
    s = scale * (K @ q)
    gap = s[star] - np.max(np.delete(s, star))
    assert gap > 30
    bound = (L - 1) * math.exp(-gap) * np.max(np.abs(V - V[star]))
    assert np.max(np.abs(oa.attend(q, K, V, scale) - V[star])) <= bound + 1e-15


def test_weights_are_a_distribution_and_shift_invariant():
    r = _rng(6)
    d, L = 32, 50
    q = r.standard_normal(d)
    K = r.standard_normal((L, d))
    a = oa.attention_weights(q, K, 0.2)
    assert np.all(a >= 0)
    assert abs(a.sum() - 1.0) < 1e-14
    # adding u with q.u = const to every key adds a constant to every score
    u = q * (5.0 / float(q @ q))
    np.testing.assert_allclose(oa.attention_weights(q, K + u, 0.2), a, atol=1e-14)


def test_weights_follow_exp_of_score_differences():
    # a_i / a_j = exp(s_i - s_j): numerator and denominator of eq. 1
    r = _rng(9)
    d, L = 8, 6
    q = r.standard_normal(d)
    K = r.standard_normal((L, d))
    a = oa.attention_weights(q, K, 0.5)
    s = 0.5 * (K @ q)
    for i in range(L):
        for j in range(L):
            assert abs(a[i] / a[j] - math.exp(s[i] - s[j])) < 1e-12 * math.exp(abs(s[i] - s[j]))


# --- eq. 2: block-by-block evaluation over KV blocks ---------------------------------

def _blockwise(q, K, V, scale, B):
    # one pass over blocks of B tokens keeping (running max, running sum, running
    # numerator): the per-block softmax slices of eq. 2 merged exactly
    m, l, acc = -math.inf, 0.0, np.zeros(V.shape[1])
    for j0 in range(0, K.shape[0], B):
        s = scale * (K[j0:j0 + B] @ q)
        m_new = max(m, float(s.max()))
        f = 0.0 if m == -math.inf else math.exp(m - m_new)
        p = np.exp(s - m_new)
        l = l * f + p.sum()
        acc = acc * f + p @ V[j0:j0 + B]
        m = m_new
    return acc / l


@pytest.mark.parametrize("B", [1, 4, 16, 32])
def test_blockwise_eq2_equals_eq1(B):
    r = _rng(10 + B)
    d, L = 16, 75
    q = r.standard_normal(d)
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, d))
    np.testing.assert_allclose(oa.attend(q, K, V, 0.25), _blockwise(q, K, V, 0.25, B), atol=1e-13)


# --- brute force on tiny inputs ------------------------------------------------------

def test_brute_force_loops_on_the_tiny_shape():
    # the worked-example shape: B=4, 1 head, d=8, contexts 8..10
    r = _rng(11)
    d = 8
    for L in (8, 9, 10):
        q = r.standard_normal(d).tolist()
        K = r.standard_normal((L, d)).tolist()
        V = r.standard_normal((L, d)).tolist()
        sc = 1 / math.sqrt(d)
        e = [math.exp(sc * sum(q[c] * K[t][c] for c in range(d))) for t in range(L)]
        z = math.fsum(e)
        ref = [math.fsum(e[t] * V[t][c] for t in range(L)) / z for c in range(d)]
        got = oa.decode(np.array([q]), np.array(K)[:, None, :], np.array(V)[:, None, :])[0]
        np.testing.assert_allclose(got, ref, atol=1e-13)


def test_prefill_rows_are_decodes_of_prefixes_and_row0_is_v0():
    r = _rng(12)
    L, H, d = 12, 2, 8
    Q = r.standard_normal((L, H, d))
    K = r.standard_normal((L, H, d))
    V = r.standard_normal((L, H, d))
    P = oa.prefill(Q, K, V)
    assert np.array_equal(P[0], V[0])
    for i in range(L):
        np.testing.assert_allclose(P[i], oa.decode(Q[i], K[: i + 1], V[: i + 1]), atol=1e-14)
    # the last n rows alone (q_len < ctx_len)
    np.testing.assert_allclose(oa.prefill(Q[-5:], K, V), P[-5:], atol=1e-14)


# --- the pins catch planted mistakes -------------------------------------------------

def _mutants():
    def wrong_sign(q, K, V, scale):
        s = -(np.asarray(K) @ np.asarray(q)) * scale
        e = np.exp(s - s.max())
        return (e / e.sum()) @ V

    def no_scale(q, K, V, scale):
        s = np.asarray(K) @ np.asarray(q)
        e = np.exp(s - s.max())
        return (e / e.sum()) @ V

    def swapped_kv(q, K, V, scale):
        s = (np.asarray(V) @ np.asarray(q)) * scale
        e = np.exp(s - s.max())
        return (e / e.sum()) @ K

    def drops_last_token(q, K, V, scale):
        K, V = np.asarray(K)[:-1] if len(K) > 1 else K, np.asarray(V)[:-1] if len(V) > 1 else V
        s = (K @ np.asarray(q)) * scale
        e = np.exp(s - s.max())
        return (e / e.sum()) @ V

    return [wrong_sign, no_scale, swapped_kv, drops_last_token]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_fail_the_sdpa_pin(mutant, monkeypatch):
    monkeypatch.setattr(oa, "attend", mutant)
    r = _rng(13)
    L, d = 9, 8
    q = r.standard_normal((1, d))
    K = r.standard_normal((L, 1, d))
    V = r.standard_normal((L, 1, d))
    got = oa.decode(q, K, V)[0]
    ref = _sdpa(q, K[:, 0], V[:, 0], 1 / math.sqrt(d), causal=False)[0]
    assert np.max(np.abs(got - ref)) > 1e-6


def _prefill_mutants():
    # whole-function copies of a causal prefill with one planted slip each
    def masked(Q, K, V, scale, keep):
        n, L = Q.shape[0], K.shape[0]
        pos = L - n + np.arange(n)
        s = (Q @ K.T) * scale
        s = np.where(keep(np.arange(L)[None, :], pos[:, None]), s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        return (e / e.sum(axis=1, keepdims=True)) @ V

    def excludes_self(Q, K, V, scale):
        # every row but the first (which would be empty) drops its own key
        out = masked(Q, K, V, scale, lambda t, p: t < p)
        out[0] = V[0]
        return out

    def one_too_many(Q, K, V, scale):
        return masked(Q, K, V, scale, lambda t, p: t <= p + 1)

    def no_mask(Q, K, V, scale):
        return masked(Q, K, V, scale, lambda t, p: t >= 0)

    return [excludes_self, one_too_many, no_mask]


@pytest.mark.parametrize("mutant", _prefill_mutants(), ids=lambda f: f.__name__)
def test_planted_causal_mistakes_fail_the_sdpa_pin(mutant):
    # the causal SDPA pin above separates the oracle's prefill from
    # off-by-one and missing causal bounds
    r = _rng(14)
    L, d = 10, 8
    Q, K, V = (r.standard_normal((L, d)) for _ in range(3))
    ref = _sdpa(Q, K, V, 1 / math.sqrt(d), causal=True)
    np.testing.assert_allclose(oa.prefill(Q[:, None], K[:, None], V[:, None])[:, 0], ref, rtol=0, atol=1e-12)
    assert np.max(np.abs(mutant(Q, K, V, 1 / math.sqrt(d)) - ref)) > 1e-6
