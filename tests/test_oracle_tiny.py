"""Whole-estimator pin on the tiny linear + fixed-head model (CPU oracle).

Dust explainer (cnblogs.com/32bin/p/23212811): "Credit assignment" argues that each
reward-weighted noise sample is the gradient plus an error with no preferred direction, so the
signal grows with the population K while the error grows with its square root; "Gradients
grow" reports that the cosine to backprop follows cos(K) = c_max / sqrt(1 + c/K).

For ONE perturbed layer with a smooth loss the estimate is unbiased for the gradient of the
sigma-smoothed loss (bias O(sigma^2)), so c_max -> 1 here. To first order in sigma a single
draw has Cov(g_hat_t) = |g_t|^2 I + g_t g_t^T + sum_{s>t in t's sequence} gamma^{2(s-t)} |g_s|^2 I
and tokens are uncorrelated, which predicts
    c = sum_t |x_t|^2 [(d_out + 1)|g_t|^2 + d_out sum_{s>t} gamma^{2(s-t)} |g_s|^2] / |G_W|_F^2.
(This constant is derived here from the estimator's definition; the pages print none.)
"""
import numpy as np
import pytest
from scipy.optimize import curve_fit

import oracle
import synth

CFG = synth.WORKLOADS[1]


def _estimate(W, H, x, tgt, K, gamma, seed, block=512):
    """The oracle's chain on the tiny model: inject -> forward CE -> loss change -> reward scan
    -> output-error estimate -> weight gradient."""
    T, d_out, sigma = CFG["T"], CFG["d_out"], CFG["sigma"]
    y = x @ W.T
    lc = oracle.tiny_forward_losses(W, H, x, tgt)
    gh = np.zeros((T, d_out))
    for k0 in range(0, K, block):
        kb = min(block, K - k0)
        yp = oracle.noise_inject(y, sigma, kb, seed=seed, tag=1, draw0=k0)
        lp = oracle.tiny_forward_losses(W, H, x, tgt, y=yp)
        c = oracle.loss_delta_loss(lc, lp)
        r = oracle.reward_scan(c, CFG["seg_len"], gamma)
        gh = oracle.error_estimate(r, d_out, sigma, seed=seed, tag=1, draw0=k0, K_total=K, g_in=gh)
    return oracle.weight_grad(gh, x)


def _predicted_c(W, H, x, tgt, gamma):
    g, G = oracle.tiny_analytic_grad(W, H, x, tgt)
    d = g.shape[1]
    g2 = (g ** 2).sum(1)
    T = len(g2)
    tail = np.array([sum(gamma ** (2 * (s - t)) * g2[s] for s in range(t + 1, T)) for t in range(T)])
    return ((x ** 2).sum(1) * ((d + 1) * g2 + d * tail)).sum() / (G ** 2).sum()


def _cos(a, b):
    return float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()))


@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_cosine_to_analytic_gradient_approaches_one(gamma):
    W, H, x, tgt = (a.astype(np.float64) if a.dtype != np.int32 else a for a in synth.tiny_model())
    _, G = oracle.tiny_analytic_grad(W, H, x, tgt)
    c_pred = _predicted_c(W, H, x, tgt, gamma)
    Ks = np.array([16, 64, 256, 1024, 4096])
    cos = np.array([_cos(_estimate(W, H, x, tgt, int(K), gamma, synth.noise_seed(1)), G) for K in Ks])
    # monotone towards 1, and close to 1 at the largest population
    assert np.all(np.diff(cos) > 0), cos
    assert cos[-1] > 1.0 / np.sqrt(1.0 + 2.0 * c_pred / Ks[-1]), (cos, c_pred)
    # every point is near the first-order law with c_max = 1 (sampling spread ~ 1/sqrt(K T))
    law = 1.0 / np.sqrt(1.0 + c_pred / Ks)
    assert np.all(np.abs(cos - law) < 0.08), (cos, law)
    # a two-parameter fit of the pages' law recovers c_max ~ 1 and c ~ the prediction
    (cmax, c), _ = curve_fit(lambda k, a, b: a / np.sqrt(1.0 + b / k), Ks, cos, p0=(1.0, c_pred))
    assert cmax > 0.97, (cmax, c)
    assert 0.7 * c_pred < c < 1.3 * c_pred, (c, c_pred)


def test_wrong_sign_reading_gives_cosine_minus_one():
    """The other reading of the loss change (perturbed minus clean) flips the estimate: the
    cosine goes to -1, so the +1 limit above pins the sign."""
    W, H, x, tgt = (a.astype(np.float64) if a.dtype != np.int32 else a for a in synth.tiny_model())
    _, G = oracle.tiny_analytic_grad(W, H, x, tgt)
    assert _cos(-_estimate(W, H, x, tgt, 1024, 0.0, 5), G) < -0.9
