"""Pins of the gated-delta-rule oracle against values fixed by the rule and by
linear algebra, not by the oracle itself: a hand-worked two-token example, the
delta rule's write and keep properties, pure decay, exact retrieval from an
orthonormal memory, the closed product form over several tokens, the grouped
head mapping, invariance under rescaled q and k, and independence of the
sequences of a batch.  The last test plants one plausible mistake at a time in
the oracle and checks that some pin fails."""

import json
import os

import numpy as np
import pytest

from oracle import gdn_oracle as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gdn_worked.json")


def _unit(rng, n):
    x = rng.standard_normal(n)
    return x / np.linalg.norm(x)


def _one_head(S, q, k, v, alpha, beta, scale=1.0, eps=0.0):
    """Run the oracle's batched entry point on a single head and token."""
    dv, dk = S.shape
    shape = G.GdnShape(1, 1, dk, dv, scale, eps)
    out, S1 = G.gdn_recurrence(shape, np.reshape(q, (1, 1, 1, dk)), np.reshape(k, (1, 1, 1, dk)),
                               np.reshape(v, (1, 1, 1, dv)), np.full((1, 1, 1), alpha),
                               np.full((1, 1, 1), beta), S.reshape(1, 1, dv, dk))
    return out[0, 0, 0], S1[0, 0]


def test_worked_two_tokens():
    g = json.load(open(GOLDEN))
    S = np.array(g["state0"], dtype=np.float64)
    for st in g["steps"]:
        o, S = _one_head(S, st["q"], st["k"], st["v"], st["alpha"], st["beta"], st["scale"], g["eps"])
        np.testing.assert_allclose(S, st["state"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(o, st["out"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("dk,dv", [(8, 8), (16, 8), (8, 24)])
def test_full_write_stores_v_at_k_and_keeps_the_rest(dk, dv):
    """alpha = beta = 1: the new state maps k to v exactly and acts as the old
    state on every direction orthogonal to k."""
    rng = np.random.default_rng(dk * 100 + dv)
    S = rng.standard_normal((dv, dk))
    k = _unit(rng, dk)
    v = rng.standard_normal(dv)
    _, S1 = _one_head(S, rng.standard_normal(dk), k, v, 1.0, 1.0)
    np.testing.assert_allclose(S1 @ k, v, atol=1e-12)
    w = rng.standard_normal(dk)
    w -= (w @ k) * k
    np.testing.assert_allclose(S1 @ w, S @ w, atol=1e-12)


def test_partial_write_closed_form():
    """S' k = alpha (1 - beta) S k + beta v and S' w = alpha S w for w
    orthogonal to a unit k."""
    rng = np.random.default_rng(7)
    dk, dv = 12, 10
    for alpha, beta in [(0.9, 0.3), (0.25, 0.75), (1.0, 0.5), (0.5, 1.0)]:
        S = rng.standard_normal((dv, dk))
        k = _unit(rng, dk)
        v = rng.standard_normal(dv)
        _, S1 = _one_head(S, rng.standard_normal(dk), k, v, alpha, beta)
        np.testing.assert_allclose(S1 @ k, alpha * (1 - beta) * (S @ k) + beta * v, atol=1e-12)
        w = rng.standard_normal(dk)
        w -= (w @ k) * k
        np.testing.assert_allclose(S1 @ w, alpha * (S @ w), atol=1e-12)


def test_zero_write_is_pure_decay_and_output_reads_the_state():
    rng = np.random.default_rng(8)
    S = rng.standard_normal((6, 4))
    q = rng.standard_normal(4)
    o, S1 = _one_head(S, q, rng.standard_normal(4), rng.standard_normal(6), 0.375, 0.0, scale=0.5)
    np.testing.assert_allclose(S1, 0.375 * S, atol=1e-14)
    np.testing.assert_allclose(o, S1 @ (0.5 * q / np.linalg.norm(q)), atol=1e-13)


def test_orthonormal_memory_is_recalled_exactly():
    """From a zero state, writing value i at basis key pi(i) with alpha = beta
    = 1 builds S = sum_i v_i e_pi(i)^T; querying e_j returns the value stored at
    key j (brute force over all j)."""
    rng = np.random.default_rng(9)
    dk, dv = 6, 5
    perm = rng.permutation(dk)
    vals = rng.standard_normal((dk, dv))
    shape = G.GdnShape(1, 1, dk, dv, 1.0, 0.0)
    q = np.zeros((1, dk, 1, dk))
    k = np.zeros((1, dk, 1, dk))
    for i in range(dk):
        k[0, i, 0, perm[i]] = 3.0          # any positive length: k is normalised
        q[0, i, 0, 0] = 1.0
    _, S = G.gdn_recurrence(shape, q, k, vals.reshape(1, dk, 1, dv), np.ones((1, dk, 1)), np.ones((1, dk, 1)),
                            np.zeros((1, 1, dv, dk)))
    for j in range(dk):
        e = np.zeros(dk)
        e[j] = 1.0
        o, _ = _one_head(S[0, 0], e, np.ones(dk), np.zeros(dv), 1.0, 0.0)
        np.testing.assert_allclose(o, vals[list(perm).index(j)], atol=1e-14)


def test_several_tokens_match_the_product_form():
    """S_T = S_0 P_1 ... P_T + sum_t beta_t v_t k_t^T P_{t+1} ... P_T with
    P_t = alpha_t (I - beta_t k_t k_t^T): the recurrence unrolled, built here
    from the products, not from the oracle's step."""
    rng = np.random.default_rng(10)
    dk, dv, T = 7, 5, 6
    eps = 1e-6
    S0 = rng.standard_normal((dv, dk))
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    alpha = rng.uniform(0.3, 1.0, (1, T, 1))
    beta = rng.uniform(0.0, 1.0, (1, T, 1))
    shape = G.GdnShape(1, 1, dk, dv, 0.7, eps)
    out, S = G.gdn_recurrence(shape, q, k, v, alpha, beta, S0.reshape(1, 1, dv, dk))
    kn = k[0, :, 0] / np.sqrt((k[0, :, 0] ** 2).sum(1, keepdims=True) + eps)
    qn = 0.7 * q[0, :, 0] / np.sqrt((q[0, :, 0] ** 2).sum(1, keepdims=True) + eps)
    P = [alpha[0, t, 0] * (np.eye(dk) - beta[0, t, 0] * np.outer(kn[t], kn[t])) for t in range(T)]

    def tail(a, b):                     # P_a ... P_{b-1}
        m = np.eye(dk)
        for t in range(a, b):
            m = m @ P[t]
        return m
    for t_end in range(1, T + 1):
        St = S0 @ tail(0, t_end)
        for t in range(t_end):
            St = St + beta[0, t, 0] * np.outer(v[0, t, 0], kn[t]) @ tail(t + 1, t_end)
        np.testing.assert_allclose(out[0, t_end - 1, 0], St @ qn[t_end - 1], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], St, atol=1e-12)


def test_grouped_heads_read_their_key_head():
    """Four value heads over two key heads: value head h equals a single-head
    run on key head h // 2, and differs from one on the other key head."""
    rng = np.random.default_rng(11)
    dk, dv = 4, 3
    shape = G.GdnShape(2, 4, dk, dv, 1.0, 0.0)
    q = rng.standard_normal((1, 1, 2, dk))
    k = rng.standard_normal((1, 1, 2, dk))
    v = rng.standard_normal((1, 1, 4, dv))
    a = rng.uniform(0.5, 1, (1, 1, 4))
    bt = rng.uniform(0.2, 0.8, (1, 1, 4))
    S0 = rng.standard_normal((1, 4, dv, dk))
    out, S = G.gdn_recurrence(shape, q, k, v, a, bt, S0)
    for h in range(4):
        own, other = h // 2, 1 - h // 2
        o1, s1 = _one_head(S0[0, h], q[0, 0, own], k[0, 0, own], v[0, 0, h], a[0, 0, h], bt[0, 0, h])
        o2, _ = _one_head(S0[0, h], q[0, 0, other], k[0, 0, other], v[0, 0, h], a[0, 0, h], bt[0, 0, h])
        np.testing.assert_allclose(out[0, 0, h], o1, atol=1e-13)
        np.testing.assert_allclose(S[0, h], s1, atol=1e-13)
        assert np.max(np.abs(out[0, 0, h] - o2)) > 1e-3


def test_rescaled_q_and_k_give_the_same_result():
    rng = np.random.default_rng(12)
    S = rng.standard_normal((5, 6))
    q, k, v = rng.standard_normal(6), rng.standard_normal(6), rng.standard_normal(5)
    o1, S1 = _one_head(S, q, k, v, 0.8, 0.6, scale=0.25)
    o2, S2 = _one_head(S, 7.5 * q, 0.01 * k, v, 0.8, 0.6, scale=0.25)
    np.testing.assert_allclose(S1, S2, atol=1e-12)
    np.testing.assert_allclose(o1, o2, atol=1e-12)


def test_sequences_of_a_batch_are_independent():
    rng = np.random.default_rng(13)
    shape = G.GdnShape(1, 2, 4, 4, 0.5)
    B, T = 3, 2
    q, k = rng.standard_normal((B, T, 1, 4)), rng.standard_normal((B, T, 1, 4))
    v = rng.standard_normal((B, T, 2, 4))
    a, bt = rng.uniform(0, 1, (B, T, 2)), rng.uniform(0, 1, (B, T, 2))
    S0 = rng.standard_normal((B, 2, 4, 4))
    out, S = G.gdn_recurrence(shape, q, k, v, a, bt, S0)
    for b in range(B):
        ob, sb = G.gdn_recurrence(shape, q[b:b + 1], k[b:b + 1], v[b:b + 1], a[b:b + 1], bt[b:b + 1], S0[b:b + 1])
        np.testing.assert_array_equal(out[b], ob[0])
        np.testing.assert_array_equal(S[b], sb[0])


def test_zero_key_leaves_only_decay():
    """A zero k (normalised with eps > 0 to the zero vector) writes nothing."""
    rng = np.random.default_rng(14)
    S = rng.standard_normal((3, 4))
    _, S1 = _one_head(S, rng.standard_normal(4), np.zeros(4), rng.standard_normal(3), 0.5, 0.9, eps=1e-6)
    np.testing.assert_allclose(S1, 0.5 * S, atol=1e-15)


PINS = [
    test_worked_two_tokens,
    lambda: test_full_write_stores_v_at_k_and_keeps_the_rest(8, 8),
    lambda: test_full_write_stores_v_at_k_and_keeps_the_rest(16, 8),
    test_partial_write_closed_form,
    test_zero_write_is_pure_decay_and_output_reads_the_state,
    test_orthonormal_memory_is_recalled_exactly,
    test_several_tokens_match_the_product_form,
    test_grouped_heads_read_their_key_head,
    test_rescaled_q_and_k_give_the_same_result,
]


def _mut(kind):
    def step(S, q_hat, k_hat, v, alpha, beta):
        S = np.asarray(S, dtype=np.float64)
        k = np.asarray(k_hat, dtype=np.float64).reshape(-1, 1)
        vv = np.asarray(v, dtype=np.float64).reshape(-1, 1)
        eye = np.eye(S.shape[1])
        if kind == "alpha_on_the_write_too":
            S_new = alpha * (S @ (eye - beta * (k @ k.T)) + beta * (vv @ k.T))
        elif kind == "no_alpha":
            S_new = S @ (eye - beta * (k @ k.T)) + beta * (vv @ k.T)
        elif kind == "projection_without_beta":
            S_new = alpha * (S @ (eye - k @ k.T)) + beta * (vv @ k.T)
        elif kind == "projection_sign":
            S_new = alpha * (S @ (eye + beta * (k @ k.T))) + beta * (vv @ k.T)
        elif kind == "projection_on_the_left":        # (I - b k k^T) S needs d_k == d_v; else transpose
            P = eye - beta * (k @ k.T)
            S_new = alpha * (P @ S) if S.shape[0] == S.shape[1] else alpha * (S @ P.T @ P)
            S_new = S_new + beta * (vv @ k.T)
        elif kind == "write_without_beta":
            S_new = alpha * (S @ (eye - beta * (k @ k.T))) + vv @ k.T
        elif kind == "output_reads_old_state":
            S_new = alpha * (S @ (eye - beta * (k @ k.T))) + beta * (vv @ k.T)
            return S_new, S @ np.asarray(q_hat)
        else:
            raise AssertionError(kind)
        return S_new, S_new @ np.asarray(q_hat)
    return step


MUTATIONS = {
    **{k: ("delta_rule_step", _mut(k)) for k in ["alpha_on_the_write_too", "no_alpha", "projection_without_beta",
                                                  "projection_sign", "projection_on_the_left", "write_without_beta",
                                                  "output_reads_old_state"]},
    "key_head_modulo": ("key_head", lambda shape, h: h % shape.n_k_heads),
    "normalise_by_squared_norm": ("l2_normalize",
                                  lambda x, eps: np.asarray(x, float) / (np.sum(np.asarray(x, float) ** 2, axis=-1,
                                                                                keepdims=True) + eps)),
    "normalise_by_max_abs": ("l2_normalize",
                                          lambda x, eps: np.asarray(x, float) / np.max(np.abs(np.asarray(x, float)),
                                                                                       axis=-1, keepdims=True)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(G, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin catches the mutation {name}"
