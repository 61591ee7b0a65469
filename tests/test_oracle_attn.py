"""Pins of the oracle's attention scores (CPU only).

The scores are the inner-mode loss change of the explainer's "The real work" for a perturbed
attention projection: c = -<Delta o, g> with Delta o the change of the attention output when
the values (or the keys) move by sigma a.

Values: the oracle uses that the attention weights do not depend on the values. The pins do
not: they re-run a causal attention with numpy on explicit values v and v + sigma a (noise
taken from the oracle's generator, itself pinned in test_oracle_generator.py) and take numpy's
inner product; with identity attention every token sees only itself and the score is
-sigma <a_t, g_t>; the score is linear in sigma; weights above the diagonal are never read.

Keys: the oracle re-runs the softmax from the given weights with the logits moved by
sigma tau <q_t, a_s>. The pins build explicit queries and keys, take the causal softmax of
tau q k^T and of tau q (k + sigma a)^T with numpy, and compare the output change's inner
product; the first-order term is the textbook softmax Jacobian P_s (delta_sr - P_r); a row's
weights count only relative to their sum, so rescaling rows changes nothing; sigma = 0 and a
query that attends only to itself give exactly zero; weights above the diagonal are ignored.

Queries: the same softmax re-run with the logits moved by sigma tau <a_t, k_s> (the noise at the
query token), pinned the same way against softmax(tau (q + sigma a) k^T).
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


def _softmax_causal(z):
    S = z.shape[-1]
    z = np.where(np.tril(np.ones((S, S), dtype=bool)), z, -np.inf)
    z = np.exp(z - z.max(-1, keepdims=True))
    return z / z.sum(-1, keepdims=True)


def _heads(x, B, S, H):
    """[B*S, H*dh] -> [B, H, S, dh]."""
    return x.reshape(B, S, H, -1).transpose(0, 2, 1, 3)


@pytest.mark.parametrize("B,H,S,dh,K,chan0,draw0,tok0", [
    (2, 2, 12, 8, 3, 0, 0, 0),
    (1, 3, 20, 4, 2, 64, 5, 100),
])
def test_key_scores_equal_an_explicit_attention_rerun(B, H, S, dh, K, chan0, draw0, tok0):
    g = np.random.default_rng(64)
    T, d, sigma, tau, seed, tag = B * S, H * dh, 0.3, 1.0 / np.sqrt(dh), 0x5EED, 4
    q, k, v, go = (g.standard_normal((T, d)) for _ in range(4))
    P = _softmax_causal(tau * _heads(q, B, S, H) @ _heads(k, B, S, H).transpose(0, 1, 3, 2))
    o = np.einsum("bhts,bhsj->bhtj", P, _heads(v, B, S, H))
    a = oracle.normals(seed, tag, draw0, tok0, chan0, K, T, d)
    ref = np.empty((K, T))
    for i in range(K):
        kp = _heads(k + sigma * a[i], B, S, H)
        Pp = _softmax_causal(tau * _heads(q, B, S, H) @ kp.transpose(0, 1, 3, 2))
        do = np.einsum("bhts,bhsj->bhtj", Pp, _heads(v, B, S, H)) - o       # [B, H, S, dh]
        ref[i] = -np.einsum("bhtj,bhtj->bt", do, _heads(go, B, S, H)).reshape(T)
    got = oracle.attn_key_scores(P, q, v, go, K, sigma, tau, seed, tag, draw0, tok0, chan0)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_key_scores_first_order_is_the_softmax_jacobian():
    g = np.random.default_rng(65)
    B, H, S, dh, K, tau = 1, 2, 16, 8, 2, 0.4
    T, d = B * S, H * dh
    q, v, go = (g.standard_normal((T, d)) for _ in range(3))
    P = _causal_weights(g, B, H, S)
    a = oracle.normals(3, 7, 0, 0, 0, K, T, d)
    qh, vh, gh = _heads(q, B, S, H), _heads(v, B, S, H), _heads(go, B, S, H)
    u = gh @ vh.transpose(0, 1, 3, 2)                        # u[b,h,t,s] = <g_t, v_s>
    lin = np.empty((K, T))
    for i in range(K):
        D = tau * qh @ _heads(a[i], B, S, H).transpose(0, 1, 3, 2)     # d logit_ts / d sigma
        # d o_t / d sigma = sum_s P_ts (D_ts - sum_r P_tr D_tr) v_s
        dP = P * (D - (P * D).sum(-1, keepdims=True))
        lin[i] = -(dP * u).sum(-1).sum(1).reshape(T)
    for sigma in (1e-5, 1e-6):
        got = oracle.attn_key_scores(P, q, v, go, K, sigma, tau, 3, 7) / sigma
        np.testing.assert_allclose(got, lin, rtol=3 * sigma * 1e2, atol=1e-9)


def test_key_scores_invariant_to_row_scale_and_blind_above_the_diagonal():
    g = np.random.default_rng(66)
    B, H, S, dh, K, sigma, tau = 2, 2, 12, 4, 2, 0.2, 0.5
    T, d = B * S, H * dh
    q, v, go = (g.standard_normal((T, d)) for _ in range(3))
    P = _causal_weights(g, B, H, S)
    c = oracle.attn_key_scores(P, q, v, go, K, sigma, tau, 9, 2)
    scaled = P * np.exp(g.standard_normal((B, H, S, 1)))
    np.testing.assert_allclose(oracle.attn_key_scores(scaled, q, v, go, K, sigma, tau, 9, 2), c,
                               rtol=1e-10, atol=1e-13)
    junk = P + np.triu(np.abs(g.standard_normal((S, S))), 1)[None, None]
    assert np.array_equal(oracle.attn_key_scores(junk, q, v, go, K, sigma, tau, 9, 2), c)


def test_key_scores_vanish_at_sigma_zero_and_for_self_attention():
    g = np.random.default_rng(67)
    B, H, S, dh, K = 1, 2, 10, 4, 3
    T, d = B * S, H * dh
    q, v, go = (g.standard_normal((T, d)) for _ in range(3))
    P = _causal_weights(g, B, H, S)
    assert np.all(oracle.attn_key_scores(P, q, v, go, K, 0.0, 0.5, 1, 1) == 0.0)
    eye = np.broadcast_to(np.eye(S), (B, H, S, S)).copy()
    assert np.all(oracle.attn_key_scores(eye, q, v, go, K, 0.7, 0.5, 1, 1) == 0.0)
    assert np.any(oracle.attn_key_scores(P, q, v, go, K, 0.7, 0.5, 1, 1) != 0.0)


def test_sampled_key_scores_equal_the_full_array():
    g = np.random.default_rng(68)
    B, H, S, dh, K = 2, 2, 16, 8, 3
    q, v, go = (g.standard_normal((B * S, H * dh)) for _ in range(3))
    P = _causal_weights(g, B, H, S)
    full = oracle.attn_key_scores(P, q, v, go, K, 0.03, 0.35, 11, 5, 2, 7, 16)
    k, t = np.array([0, 2, 1, 2]), np.array([0, 31, 17, 16])
    np.testing.assert_array_equal(
        oracle.attn_key_scores_at(P, q, v, go, k, t, 0.03, 0.35, 11, 5, 2, 7, 16), full[k, t])


@pytest.mark.parametrize("B,H,S,dh,K,chan0,draw0,tok0", [
    (2, 2, 12, 8, 3, 0, 0, 0),
    (1, 3, 20, 4, 2, 64, 5, 100),
])
def test_query_scores_equal_an_explicit_attention_rerun(B, H, S, dh, K, chan0, draw0, tok0):
    g = np.random.default_rng(69)
    T, d, sigma, tau, seed, tag = B * S, H * dh, 0.3, 1.0 / np.sqrt(dh), 0x5EEE, 5
    q, k, v, go = (g.standard_normal((T, d)) for _ in range(4))
    kT = _heads(k, B, S, H).transpose(0, 1, 3, 2)
    P = _softmax_causal(tau * _heads(q, B, S, H) @ kT)
    o = np.einsum("bhts,bhsj->bhtj", P, _heads(v, B, S, H))
    a = oracle.normals(seed, tag, draw0, tok0, chan0, K, T, d)
    ref = np.empty((K, T))
    for i in range(K):
        Pp = _softmax_causal(tau * _heads(q + sigma * a[i], B, S, H) @ kT)
        do = np.einsum("bhts,bhsj->bhtj", Pp, _heads(v, B, S, H)) - o
        ref[i] = -np.einsum("bhtj,bhtj->bt", do, _heads(go, B, S, H)).reshape(T)
    got = oracle.attn_query_scores(P, k, v, go, K, sigma, tau, seed, tag, draw0, tok0, chan0)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_query_scores_first_order_is_the_softmax_jacobian():
    g = np.random.default_rng(70)
    B, H, S, dh, K, tau = 1, 2, 16, 8, 2, 0.4
    T, d = B * S, H * dh
    k, v, go = (g.standard_normal((T, d)) for _ in range(3))
    P = _causal_weights(g, B, H, S)
    a = oracle.normals(3, 8, 0, 0, 0, K, T, d)
    kh, vh, gh = _heads(k, B, S, H), _heads(v, B, S, H), _heads(go, B, S, H)
    u = gh @ vh.transpose(0, 1, 3, 2)
    lin = np.empty((K, T))
    for i in range(K):
        D = tau * _heads(a[i], B, S, H) @ kh.transpose(0, 1, 3, 2)     # d logit_ts / d sigma
        dP = P * (D - (P * D).sum(-1, keepdims=True))
        lin[i] = -(dP * u).sum(-1).sum(1).reshape(T)
    for sigma in (1e-5, 1e-6):
        got = oracle.attn_query_scores(P, k, v, go, K, sigma, tau, 3, 8) / sigma
        np.testing.assert_allclose(got, lin, rtol=3 * sigma * 1e2, atol=1e-9)


def test_query_scores_row_scale_diagonal_and_zeros():
    g = np.random.default_rng(71)
    B, H, S, dh, K, sigma, tau = 2, 2, 12, 4, 2, 0.2, 0.5
    T, d = B * S, H * dh
    k, v, go = (g.standard_normal((T, d)) for _ in range(3))
    P = _causal_weights(g, B, H, S)
    c = oracle.attn_query_scores(P, k, v, go, K, sigma, tau, 9, 3)
    scaled = P * np.exp(g.standard_normal((B, H, S, 1)))
    np.testing.assert_allclose(oracle.attn_query_scores(scaled, k, v, go, K, sigma, tau, 9, 3), c,
                               rtol=1e-10, atol=1e-13)
    junk = P + np.triu(np.abs(g.standard_normal((S, S))), 1)[None, None]
    assert np.array_equal(oracle.attn_query_scores(junk, k, v, go, K, sigma, tau, 9, 3), c)
    assert np.all(oracle.attn_query_scores(P, k, v, go, K, 0.0, tau, 9, 3) == 0.0)
    eye = np.broadcast_to(np.eye(S), (B, H, S, S)).copy()
    assert np.all(oracle.attn_query_scores(eye, k, v, go, K, sigma, tau, 9, 3) == 0.0)
    assert np.any(c != 0.0)
    full = oracle.attn_query_scores(P, k, v, go, K, sigma, tau, 9, 3, 2, 7, 16)
    kk, t = np.array([0, 1, 1]), np.array([0, 23, 12])
    np.testing.assert_array_equal(
        oracle.attn_query_scores_at(P, k, v, go, kk, t, sigma, tau, 9, 3, 2, 7, 16), full[kk, t])


# Row weights: the draw-independent part of the softmax re-run that the key and query scorers
# share. Pinned against an explicit numpy re-run under arbitrary logit shifts, and by their
# invariants.

@pytest.mark.parametrize("B,H,S,dh", [(2, 2, 12, 8), (1, 3, 20, 4)])
def test_row_weights_reproduce_an_explicit_softmax_rerun(B, H, S, dh):
    """For any logit shifts delta, sum_s W_ts (e^delta - 1) / (Z (Z + N0)) is the change of
    <o_t, g_t> when head h's weights become P e^delta renormalised, against the rows of P
    normalised by Z (rows are rescaled on purpose so that Z != 1)."""
    g = np.random.default_rng(70)
    T, d = B * S, H * dh
    P = _causal_weights(g, B, H, S) * g.uniform(0.5, 2.0, (B, H, S, 1))
    v, go = g.standard_normal((T, d)), g.standard_normal((T, d))
    W, Z = oracle.attn_row_weights(P, v, go)
    vh, gh = _heads(v, B, S, H), _heads(go, B, S, H)
    tri = np.tril(np.ones((S, S), dtype=bool))
    for trial in range(3):
        delta = np.where(tri, g.standard_normal((B, H, S, S)) * 0.7, 0.0)
        Pp = P * np.exp(delta) * tri
        Pp = Pp / Pp.sum(-1, keepdims=True)
        Pc = P * tri / (P * tri).sum(-1, keepdims=True)
        ref = np.einsum("bhtj,bhtj->bht", np.einsum("bhts,bhsj->bhtj", Pp - Pc, vh), gh)
        em1 = np.expm1(delta) * tri
        N0 = (P * tri * em1).sum(-1)
        got = (W * em1).sum(-1) / (Z * (Z + N0))
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-13)


def test_row_weights_invariants():
    """Rows of W sum to zero; Z is the causal row sum; W vanishes above the diagonal, for
    self-attention only (a row with one key has nothing to move toward), and ignores the
    weights above the diagonal."""
    g = np.random.default_rng(71)
    B, H, S, dh = 2, 2, 16, 4
    T, d = B * S, H * dh
    P = _causal_weights(g, B, H, S)
    v, go = g.standard_normal((T, d)), g.standard_normal((T, d))
    W, Z = oracle.attn_row_weights(P, v, go)
    scale = np.abs(W).max()
    assert scale > 0.1
    np.testing.assert_allclose(W.sum(-1), 0.0, atol=1e-12 * S * scale)
    np.testing.assert_allclose(Z, np.tril(P).sum(-1), rtol=1e-15)
    assert np.all(W[..., ~np.tril(np.ones((S, S), dtype=bool))] == 0.0)
    junk = P + np.triu(g.standard_normal((B, H, S, S)), 1)
    W2, Z2 = oracle.attn_row_weights(junk, v, go)
    assert np.array_equal(W2, W) and np.array_equal(Z2, Z)
    eye = np.broadcast_to(np.eye(S), (B, H, S, S)).copy()
    We, Ze = oracle.attn_row_weights(eye, v, go)
    assert np.all(We == 0.0) and np.all(Ze == 1.0)


def test_row_weights_recover_the_key_and_query_scores():
    """The oracle's key and query scores (explicit re-runs) equal the row-weight form under the
    logit shifts of the same draws: sigma tau <q_t, a_s> for keys, sigma tau <a_t, k_s> for
    queries, noise from the oracle's generator."""
    g = np.random.default_rng(72)
    B, H, S, dh, K = 1, 2, 12, 4, 2
    T, d, sigma, tau, seed, tag = B * S, H * dh, 0.2, 0.5, 0x5EED, 9
    q, k, v, go = (g.standard_normal((T, d)) for _ in range(4))
    P = _softmax_causal(tau * _heads(q, B, S, H) @ _heads(k, B, S, H).transpose(0, 1, 3, 2))
    W, Z = oracle.attn_row_weights(P, v, go)
    tri = np.tril(np.ones((S, S), dtype=bool))
    a = oracle.normals(seed, tag, 0, 0, 0, K, T, d)
    ck = oracle.attn_key_scores(P, q, v, go, K, sigma, tau, seed, tag)
    cq = oracle.attn_query_scores(P, k, v, go, K, sigma, tau, seed, tag)
    for i in range(K):
        ah = _heads(a[i], B, S, H)
        for got, delta in ((ck[i], _heads(q, B, S, H) @ ah.transpose(0, 1, 3, 2)),
                           (cq[i], ah @ _heads(k, B, S, H).transpose(0, 1, 3, 2))):
            em1 = np.expm1(sigma * tau * delta) * tri
            val = (W * em1).sum(-1) / (Z * (Z + (P * tri * em1).sum(-1)))   # [B, H, S]
            np.testing.assert_allclose(got, -val.sum(1).reshape(T), rtol=1e-9, atol=1e-13)


@pytest.mark.parametrize("which", ["keys", "queries"])
@pytest.mark.parametrize("sigma", [30.0, 300.0])
def test_key_and_query_scores_at_large_shifts(which, sigma):
    """Logit shifts of hundreds (sigma = 300 reaches past fp64's e^x range, about 709): the
    oracle's re-run, which subtracts each row's maximum, equals the explicit numpy re-run, and
    every score is finite."""
    B, H, S, dh, K = 1, 2, 16, 8, 3
    g = np.random.default_rng(70)
    T, d, tau, seed, tag = B * S, H * dh, 1.0 / np.sqrt(dh), 0x5EEF, 6
    q, k, v, go = (g.standard_normal((T, d)) for _ in range(4))
    kT = _heads(k, B, S, H).transpose(0, 1, 3, 2)
    P = _softmax_causal(tau * _heads(q, B, S, H) @ kT)
    o = np.einsum("bhts,bhsj->bhtj", P, _heads(v, B, S, H))
    a = oracle.normals(seed, tag, 0, 0, 0, K, T, d)
    ref = np.empty((K, T))
    worst = 0.0
    for i in range(K):
        if which == "keys":
            z = tau * _heads(q, B, S, H) @ _heads(k + sigma * a[i], B, S, H).transpose(0, 1, 3, 2)
        else:
            z = tau * _heads(q + sigma * a[i], B, S, H) @ kT
        worst = max(worst, float(np.abs(np.tril(z[0, 0] - (tau * _heads(q, B, S, H) @ kT)[0, 0])).max()))
        do = np.einsum("bhts,bhsj->bhtj", _softmax_causal(z), _heads(v, B, S, H)) - o
        ref[i] = -np.einsum("bhtj,bhtj->bt", do, _heads(go, B, S, H)).reshape(T)
    if sigma == 300.0:
        assert worst > 709.0
    f = oracle.attn_key_scores if which == "keys" else oracle.attn_query_scores
    got = f(P, q if which == "keys" else k, v, go, K, sigma, tau, seed, tag, 0, 0, 0)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9)
