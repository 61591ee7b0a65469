"""Pins of the oracle's optimizer steps (CPU only).

The explainer's section "Results" names the optimizers Dust's estimate was used with (SGD with
momentum at a constant learning rate; Adam) without printing formulas, so the oracle states the
textbook ones.
They are pinned here to torch.optim's implementations run in fp64 on the CPU (a library routine
doing the same step), and to closed forms: with zero momentum SGD is w - lr g; Adam's first step
from zero moments moves every weight by lr g / (|g| + eps), i.e. by about lr against the sign
of its gradient; decoupled weight decay alone scales w by 1 - lr wd.
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_steps(opt_cls, w0, grads, **kw):
    p = torch.nn.Parameter(torch.tensor(w0, dtype=torch.float64))
    opt = opt_cls([p], **kw)
    out = []
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        out.append(p.detach().numpy().copy())
    return out


def _grads(n, steps, seed):
    g = np.random.default_rng(seed)
    return [g.standard_normal(n) * (0.1 + g.random()) for _ in range(steps)]


@pytest.mark.parametrize("lr,mu", [(0.05, 0.9), (0.3, 0.0), (0.01, 0.99)])
def test_sgd_momentum_matches_torch(lr, mu):
    w0 = np.random.default_rng(1).standard_normal(257)
    grads = _grads(257, 6, 2)
    ref = _torch_steps(torch.optim.SGD, w0, grads, lr=lr, momentum=mu)
    w, buf = w0.copy(), np.zeros_like(w0)
    for g, r in zip(grads, ref):
        w, buf = oracle.sgd_momentum(w, g, buf, lr, mu)
        np.testing.assert_allclose(w, r, rtol=1e-13, atol=1e-13)


def test_sgd_without_momentum_is_plain_gradient_step():
    w0, g = np.array([1.0, -2.0, 0.5]), np.array([0.5, 0.25, -4.0])
    w, buf = oracle.sgd_momentum(w0, g, np.zeros(3), 0.1, 0.0)
    assert np.array_equal(w, w0 - 0.1 * g) and np.array_equal(buf, g)


@pytest.mark.parametrize("lr,b1,b2,eps,wd", [
    (1e-3, 0.9, 0.999, 1e-8, 0.0),
    (3e-2, 0.8, 0.95, 1e-6, 0.0),
    (1e-2, 0.9, 0.999, 1e-8, 0.1),
])
def test_adam_matches_torch(lr, b1, b2, eps, wd):
    w0 = np.random.default_rng(3).standard_normal(300)
    grads = _grads(300, 7, 4)
    cls = torch.optim.AdamW if wd else torch.optim.Adam
    ref = _torch_steps(cls, w0, grads, lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for t, (g, r) in enumerate(zip(grads, ref), start=1):
        w, m, v = oracle.adam(w, g, m, v, lr, b1, b2, eps, wd, t)
        np.testing.assert_allclose(w, r, rtol=1e-12, atol=1e-14)


def test_adam_first_step_and_weight_decay_closed_forms():
    w0 = np.array([1.0, -1.0, 2.0, 0.0])
    g = np.array([3.0, -0.5, 1e-3, -2.0])
    lr, eps = 0.01, 1e-8
    w, m, v = oracle.adam(w0, g, np.zeros(4), np.zeros(4), lr, 0.9, 0.999, eps, 0.0, 1)
    np.testing.assert_allclose(w, w0 - lr * g / (np.abs(g) + eps), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-13)
    # a zero gradient on zero moments leaves only the decay
    w, _, _ = oracle.adam(w0, np.zeros(4), np.zeros(4), np.zeros(4), lr, 0.9, 0.999, eps, 0.5, 3)
    np.testing.assert_allclose(w, w0 * (1 - lr * 0.5), rtol=1e-15)


def test_cosine_terms_are_the_exact_sums_and_closed_forms():
    """The screening cosine's three sums: equal the exactly rounded sums (math.fsum of the exact
    fp64 products of fp32 inputs); basis vectors, a vector with itself, its negative and an
    orthogonal pair give the closed forms."""
    import math
    g = np.random.default_rng(90)
    a = g.standard_normal(1001).astype(np.float32).astype(np.float64)
    b = g.standard_normal(1001).astype(np.float32).astype(np.float64)
    t = oracle.cosine_terms(a, b)
    exact = [math.fsum(a * b), math.fsum(a * a), math.fsum(b * b)]
    np.testing.assert_allclose(t, exact, rtol=1e-13, atol=0)
    e = np.eye(5)
    assert list(oracle.cosine_terms(e[1], e[1])) == [1.0, 1.0, 1.0]
    assert list(oracle.cosine_terms(e[1], e[3])) == [0.0, 1.0, 1.0]
    x = np.array([3.0, -4.0])
    assert list(oracle.cosine_terms(x, -x)) == [-25.0, 25.0, 25.0]
    assert list(oracle.cosine_terms(x, np.array([4.0, 3.0]))) == [0.0, 25.0, 25.0]
