"""Pins of the oracle's attention value-projection scores (CPU only).

The scores are the inner-mode loss change of the explainer's "The real work" for a perturbed
value projection: c = -<Delta o, g> with Delta o the change of the attention output when the
values move by sigma a. The oracle uses that the attention weights do not depend on the values.
The pins do not: they re-run a causal attention with numpy on explicit values v and v + sigma a
(noise taken from the oracle's generator, itself pinned in test_oracle_generator.py) and take
numpy's inner product; with identity attention every token sees only itself and the score is
-sigma <a_t, g_t>; the score is linear in sigma; weights above the diagonal are never read.
"""
import numpy as np
import pytest

import oracle


def _causal_weights(g, B, H, S, scale=1.0):
    z = g.standard_normal((B, H, S, S)) * scale
    mask = np.tril(np.ones((S, S), dtype=bool))
    z = np.where(mask, z, -np.inf)
    z = np.exp(z - z.max(-1, keepdims=True))
    return z / z.sum(-1, keepdims=True)


def _attend(P, v, H):
    """o[b, t, h*dh + j] = sum_s P[b, h, t, s] v[b, s, h*dh + j]."""
    B, S, d = v.shape
    vh = v.reshape(B, S, H, d // H)
    return np.einsum("bhts,bshj->bthj", P, vh).reshape(B, S, d)


@pytest.mark.parametrize("B,H,S,dh,K,chan0,draw0,tok0", [
    (2, 2, 16, 8, 3, 0, 0, 0),
    (1, 3, 24, 4, 2, 64, 5, 100),
])
def test_scores_equal_an_explicit_attention_rerun(B, H, S, dh, K, chan0, draw0, tok0):
    g = np.random.default_rng(60)
    T, d, sigma, seed, tag = B * S, H * dh, 0.05, 0x5EED, 4
    P = _causal_weights(g, B, H, S)
    v = g.standard_normal((B, S, d))
    go = g.standard_normal((T, d))
    a = oracle.normals(seed, tag, draw0, tok0, chan0, K, T, d)        # [K, T, d]
    o = _attend(P, v, H)
    ref = np.empty((K, T))
    for i in range(K):
        do = _attend(P, v + sigma * a[i].reshape(B, S, d), H) - o
        ref[i] = -np.einsum("tj,tj->t", do.reshape(T, d), go)
    got = oracle.attn_value_scores(P, go, K, sigma, seed, tag, draw0, tok0, chan0)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_identity_attention_is_the_own_token_inner_product():
    g = np.random.default_rng(61)
    B, H, S, dh, K, sigma = 2, 2, 8, 4, 3, 0.3
    T, d = B * S, H * dh
    P = np.broadcast_to(np.eye(S), (B, H, S, S)).copy()
    go = g.standard_normal((T, d))
    a = oracle.normals(7, 1, 0, 0, 0, K, T, d)
    ref = oracle.loss_delta_inner(sigma * a, go)
    np.testing.assert_allclose(oracle.attn_value_scores(P, go, K, sigma, 7, 1), ref,
                               rtol=1e-12, atol=1e-14)


def test_linear_in_sigma_and_blind_above_the_diagonal():
    g = np.random.default_rng(62)
    B, H, S, dh, K = 1, 2, 12, 4, 2
    P = _causal_weights(g, B, H, S)
    go = g.standard_normal((B * S, H * dh))
    c1 = oracle.attn_value_scores(P, go, K, 0.01, 9, 2)
    np.testing.assert_allclose(oracle.attn_value_scores(P, go, K, 0.02, 9, 2), 2 * c1, rtol=1e-12)
    assert np.all(oracle.attn_value_scores(P, go, K, 0.0, 9, 2) == 0.0)
    Pj = P + np.triu(g.standard_normal((S, S)), 1)[None, None]
    assert np.array_equal(oracle.attn_value_scores(Pj, go, K, 0.01, 9, 2), c1)


def test_sampled_scores_equal_the_full_array():
    g = np.random.default_rng(63)
    B, H, S, dh, K = 2, 2, 16, 8, 3
    P = _causal_weights(g, B, H, S)
    go = g.standard_normal((B * S, H * dh))
    full = oracle.attn_value_scores(P, go, K, 0.03, 11, 5, 2, 7, 16)
    k, t = np.array([0, 2, 1, 2]), np.array([0, 31, 17, 16])
    np.testing.assert_array_equal(oracle.attn_value_scores_at(P, go, k, t, 0.03, 11, 5, 2, 7, 16),
                                  full[k, t])
