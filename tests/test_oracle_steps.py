"""Pins of the oracle's estimator steps against what the pages and the mathematics fix (CPU).

Source: the Dust explainer, cnblogs.com/32bin/p/23212811, section "Credit assignment: one
forward, two rewards" (perturbation, loss change, reward, output-error estimate, weight
gradient) and section "The real work: suppressing interference" (attention scoring, LM-head
chunk). Each pin is independent of the oracle's own code: closed forms, special cases stated on
the pages, library routines (numpy, torch), brute force, or statistical limits.
"""
import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------------------------ perturbation
def test_inject_sigma_zero_is_identity():
    y = np.random.default_rng(0).standard_normal((7, 12))
    assert np.array_equal(oracle.noise_inject(y, 0.0, 3, 1, 2)[2], y)


def test_inject_adds_sigma_times_standard_normal():
    g = np.random.default_rng(1)
    y = g.standard_normal((64, 256))
    yp = oracle.noise_inject(y, 0.25, 16, seed=3, tag=9)
    a = (yp - y[None]) / 0.25
    n = a.size
    assert abs(a.mean()) < 5 / np.sqrt(n) and abs(a.var() - 1) < 5 * np.sqrt(2 / n)


def test_inject_leading_dimension_and_offsets():
    g = np.random.default_rng(2)
    ywide = g.standard_normal((10, 40))
    full = oracle.noise_inject(ywide, 0.1, 5, seed=4, tag=2)
    # columns 8..27 of y with chan0 = 8, tokens 3..9 with tok0 = 3, draws 1..3 with draw0 = 1
    part = oracle.noise_inject(ywide[3:, 8:28], 0.1, 3, seed=4, tag=2, draw0=1, tok0=3, chan0=8)
    assert np.array_equal(part, full[1:4, 3:, 8:28])


# ------------------------------------------------------------------------------ loss change
def test_loss_delta_loss_is_clean_minus_perturbed():
    g = np.random.default_rng(3)
    lc = g.standard_normal(33) + 8
    lp = lc[None] + 1e-2 * g.standard_normal((5, 33))
    assert np.array_equal(oracle.loss_delta_loss(lc, lp), np.subtract(lc[None], lp))
    # no perturbation -> no change
    assert np.all(oracle.loss_delta_loss(lc, np.tile(lc, (4, 1))) == 0.0)


def test_loss_delta_inner_matches_einsum():
    g = np.random.default_rng(4)
    do = g.standard_normal((6, 11, 37))
    go = g.standard_normal((11, 37))
    np.testing.assert_allclose(oracle.loss_delta_inner(do, go), -np.einsum("ksj,sj->ks", do, go),
                               rtol=1e-13, atol=1e-13)


def test_loss_delta_inner_along_the_error_is_minus_eps_norm():
    go = np.random.default_rng(5).standard_normal((9, 20))
    eps = 0.003
    c = oracle.loss_delta_inner(eps * go[None], go)
    np.testing.assert_allclose(c[0], -eps * (go ** 2).sum(axis=1), rtol=1e-13)


# ------------------------------------------------------------------------------ reward scan
def _brute_scan(c, seg, gamma):
    K, T = c.shape
    r = np.zeros_like(c)
    for t in range(T):
        end = (t // seg + 1) * seg
        for s in range(t, end):
            r[:, t] += gamma ** (s - t) * c[:, s]
    return r


def test_scan_gamma_zero_keeps_own_token():
    # explainer: gamma = 0 reduces the reward to the token's own score
    c = np.random.default_rng(6).standard_normal((4, 50))
    assert np.array_equal(oracle.reward_scan(c, 10, 0.0), c)


def test_scan_impulse_response():
    seg, gamma = 16, 0.7
    c = np.zeros((1, 48))
    c[0, 21] = 1.0                     # inside the second sequence [16, 32)
    r = oracle.reward_scan(c, seg, gamma)[0]
    expect = np.zeros(48)
    expect[16:22] = gamma ** (21 - np.arange(16, 22))
    np.testing.assert_allclose(r, expect, rtol=1e-15, atol=0)


def test_scan_constant_input_geometric_series():
    seg, gamma, v = 100, 0.93, 2.5
    r = oracle.reward_scan(np.full((2, 300), v), seg, gamma)
    n = seg - (np.arange(300) % seg)   # tokens from t to its sequence end, inclusive
    np.testing.assert_allclose(r[1], v * (1 - gamma ** n) / (1 - gamma), rtol=1e-13)


def test_scan_gamma_one_is_suffix_sum_per_sequence():
    c = np.random.default_rng(7).standard_normal((3, 40))
    r = oracle.reward_scan(c, 8, 1.0)
    cs = c.reshape(3, 5, 8)
    expect = np.flip(np.cumsum(np.flip(cs, -1), -1), -1).reshape(3, 40)
    np.testing.assert_allclose(r, expect, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("gamma", [0.0, 0.5, 0.9, 0.99, 1.0])
def test_scan_brute_force(gamma):
    c = np.random.default_rng(8).standard_normal((3, 36))
    np.testing.assert_allclose(oracle.reward_scan(c, 12, gamma), _brute_scan(c, 12, gamma),
                               rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ error estimate
def test_error_estimate_brute_force_tiny():
    g = np.random.default_rng(9)
    K, T, d, sigma = 3, 4, 6, 0.05
    r = g.standard_normal((K, T))
    gh = oracle.error_estimate(r, d, sigma, seed=5, tag=1, draw0=2, tok0=7, chan0=4, K_total=10)
    expect = np.zeros((T, d))
    for t in range(T):
        for j in range(d):
            acc = sum(r[i, t] * oracle.normal(5, 1, 2 + i, 7 + t, 4 + j) for i in range(K))
            expect[t, j] = -acc / (10 * sigma)
    np.testing.assert_allclose(gh, expect, rtol=1e-13, atol=1e-15)


def test_error_estimate_chunked_population_equals_one_pass():
    g = np.random.default_rng(10)
    K, T, d, sigma = 12, 9, 10, 0.02
    r = g.standard_normal((K, T))
    one = oracle.error_estimate(r, d, sigma, seed=1, tag=3)
    a = oracle.error_estimate(r[:5], d, sigma, seed=1, tag=3, K_total=K)
    b = oracle.error_estimate(r[5:], d, sigma, seed=1, tag=3, draw0=5, K_total=K, g_in=a)
    np.testing.assert_allclose(b, one, rtol=1e-12, atol=1e-15)
    at = oracle.error_estimate_at(r, [0, 8, 3], [9, 0, 4], sigma, seed=1, tag=3)
    np.testing.assert_allclose(at, one[[0, 8, 3], [9, 0, 4]], rtol=1e-13)


@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_error_estimate_recovers_linear_loss_gradient(gamma):
    """Linear per-token loss l_t = <w_t, y_t>: the loss reduction of a draw is exactly
    c_t = -sigma <w_t, a_t>, the true output error is w_t, and the estimate's mean is w_t for
    any gamma (noise of other tokens is independent of a_t). Pins the sign of c, the reading
    that the estimate is +dl/dy, and the 1/(K sigma) scale."""
    g = np.random.default_rng(11)
    K, T, d, sigma, seg = 20000, 6, 8, 0.01, 6
    w = g.standard_normal((T, d))
    y = g.standard_normal((T, d))
    yp = oracle.noise_inject(y, sigma, K, seed=21, tag=4)
    lc = (w * y).sum(-1)
    lp = (w[None] * yp).sum(-1)
    c = oracle.loss_delta_loss(lc, lp)
    r = oracle.reward_scan(c, seg, gamma)
    gh = oracle.error_estimate(r, d, sigma, seed=21, tag=4)
    # per-element sd of the mean: sqrt((|w_t|^2 + w_tj^2 + gamma-terms) / K)
    extra = np.array([sum(gamma ** (2 * (s - t)) * (w[s] ** 2).sum() for s in range(t + 1, T))
                      for t in range(T)])
    sd = np.sqrt(((w ** 2).sum(1, keepdims=True) + w ** 2 + extra[:, None]) / K)
    z = (gh - w) / sd
    assert np.abs(z).max() < 5.0, np.abs(z).max()


# ------------------------------------------------------------------------------ weight gradient
def test_weight_grad_is_the_backprop_outer_product():
    """Explainer: with the chain-rule output error in place of the estimate, the contraction is
    exactly backprop's weight gradient. Pinned against torch autograd (fp64) on the tiny
    linear + softmax model."""
    g = np.random.default_rng(12)
    d_in, d_out, V, T = 16, 12, 30, 25
    W = g.standard_normal((d_out, d_in)) / 4
    H = g.standard_normal((V, d_out)) / 4
    x = g.standard_normal((T, d_in))
    tgt = g.integers(0, V, T)
    gy, _ = oracle.tiny_analytic_grad(W, H, x, tgt)
    G = oracle.weight_grad(gy, x)

    Wt = torch.tensor(W, requires_grad=True)
    z = torch.tensor(x) @ Wt.T @ torch.tensor(H).T
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(tgt), reduction="sum")
    loss.backward()
    np.testing.assert_allclose(G, Wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.tiny_forward_losses(W, H, x, tgt),
                               torch.nn.functional.cross_entropy(z, torch.tensor(tgt),
                                                                 reduction="none").detach().numpy(),
                               rtol=1e-12)


# ------------------------------------------------------------------------------ LM-head chunk
@pytest.mark.parametrize("V,v0,C", [(50, 0, 50), (64, 12, 20), (97, 88, 9), (40, 0, 4)])
def test_head_ce_matches_torch_cross_entropy(V, v0, C):
    g = np.random.default_rng(13)
    T, K, sigma = 7, 5, 0.3
    z = g.standard_normal((T, V)) * np.sqrt(2)
    tgt = g.integers(0, V, T).astype(np.int32)
    tgt[0] = v0           # a target inside the chunk
    tgt[1] = (v0 + C) % V  # one just past it
    lp, lc = oracle.head_ce_chunk(z, tgt, v0, C, K, sigma, seed=6, tag=2, draw0=3, tok0=11)
    a = oracle.normals(6, 2, 3, 11, v0, K, T, C)          # [K, T, C]
    zp = np.repeat(z[None], K, axis=0)
    zp[:, :, v0:v0 + C] += sigma * a
    ref = torch.nn.functional.cross_entropy(torch.tensor(zp.reshape(K * T, V)),
                                            torch.tensor(np.tile(tgt, K)).long(),
                                            reduction="none").numpy().reshape(K, T)
    np.testing.assert_allclose(lp, ref, rtol=0, atol=1e-12)
    ref_c = torch.nn.functional.cross_entropy(torch.tensor(z), torch.tensor(tgt).long(),
                                              reduction="none").numpy()
    np.testing.assert_allclose(lc, ref_c, rtol=0, atol=1e-12)


def test_head_ce_sigma_zero_and_large_logits():
    g = np.random.default_rng(14)
    z = g.standard_normal((4, 30)) + 1000.0      # log-sum-exp must be shift-invariant
    tgt = np.array([0, 5, 29, 17], dtype=np.int32)
    lp, lc = oracle.head_ce_chunk(z, tgt, 8, 12, 3, 0.0, seed=1, tag=1)
    assert np.all(lp == lc[None])
    ref = oracle.head_ce_chunk(z - 1000.0, tgt, 8, 12, 3, 0.0, seed=1, tag=1)[1]
    np.testing.assert_allclose(lc, ref, atol=1e-10)


def test_head_chunk_estimate_recovers_softmax_minus_onehot():
    """With the head's own logits as the perturbed layer, the output error of token t is
    softmax(z_t) - e_target. The chunk estimate (loss change -> gamma = 0 -> g_hat on channels
    v0..v0+C) must converge to it on the chunk."""
    g = np.random.default_rng(15)
    T, V, v0, C, K, sigma = 4, 24, 8, 8, 40000, 0.01
    z = g.standard_normal((T, V)) * np.sqrt(2)
    tgt = np.array([9, 3, 15, 20], dtype=np.int32)
    lp, lc = oracle.head_ce_chunk(z, tgt, v0, C, K, sigma, seed=8, tag=5)
    c = oracle.loss_delta_loss(lc, lp)
    gh = oracle.error_estimate(c, C, sigma, seed=8, tag=5, chan0=v0)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    p[np.arange(T), tgt] -= 1.0
    exact = p[:, v0:v0 + C]
    sd = np.sqrt(((exact ** 2).sum(1, keepdims=True) + exact ** 2) / K)
    assert np.abs((gh - exact) / sd).max() < 5.0
