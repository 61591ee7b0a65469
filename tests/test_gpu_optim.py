"""GPU parity of the optimizer steps (dust_sgd_momentum, dust_adam) with the oracle (MI355X only).

Each step starts both sides from the same fp32 state (the device's state after the previous
step) and the same hyperparameters (the fp32 values the device receives), so the comparison
bounds one step's rounding: the device computes in fp32 with the bias corrections formed in
fp64, the oracle in fp64. A sum of two terms is rounded once or twice on the device, so its
error is bounded by ulps of its terms' magnitudes (they may cancel); the weight then moves by
lr / (1 - b1^t) times the first moment over the denominator, which carries that error along.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, announce, dust, f32, host_f32

pytestmark = pytest.mark.gpu

SIZES = [
    (1, 0),           # one weight: the scalar path
    (4099, 0),        # ragged: the scalar path
    (1 << 20, 0),     # 16-byte pieces
    (4096, 1),        # arrays one element off a 16-byte boundary: the scalar path
]


def _ulp(a):
    return np.spacing(np.abs(a.astype(np.float32))).astype(np.float64)


def _f32(x):
    return float(np.float32(x))


def _dev(a, off):
    t = torch.zeros(a.size + off, dtype=torch.float32, device=DEV)
    t[off:] = torch.from_numpy(a.astype(np.float32)).to(DEV)
    return t[off:]


@pytest.mark.parametrize("n,off", SIZES)
@pytest.mark.parametrize("lr,mu", [(0.05, 0.9), (1e-3, 0.0)])
def test_sgd_momentum_steps(n, off, lr, mu):
    announce("sgd momentum %s" % ((n, off, lr, mu),))
    lr, mu = _f32(lr), _f32(mu)
    g = np.random.default_rng(50)
    w, buf = _dev(g.standard_normal(n), off), _dev(np.zeros(n), off)
    for step in range(4):
        gr = _dev(g.standard_normal(n) * 0.5, off)
        w0, b0, g0 = host_f32(w).astype(np.float64), host_f32(buf).astype(np.float64), host_f32(gr)
        dust.dust_sgd_momentum(w, gr, buf, n, lr, mu)
        rw, rb = oracle.sgd_momentum(w0, g0, b0, lr, mu)
        gw, gb = host_f32(w).astype(np.float64), host_f32(buf).astype(np.float64)
        db = _ulp(np.abs(mu * b0) + np.abs(g0))      # one rounding of mu b + g
        assert np.all(np.abs(gb - rb) <= db), step
        assert np.all(np.abs(gw - rw) <= _ulp(np.abs(w0) + lr * np.abs(rb)) + lr * db), step


@pytest.mark.parametrize("n,off", SIZES)
@pytest.mark.parametrize("lr,b1,b2,eps,wd", [(1e-3, 0.9, 0.999, 1e-8, 0.0),
                                             (1e-2, 0.8, 0.95, 1e-6, 0.1)])
def test_adam_steps(n, off, lr, b1, b2, eps, wd):
    announce("adam %s" % ((n, off, lr, b1, b2, eps, wd),))
    lr, b1, b2, eps, wd = (_f32(x) for x in (lr, b1, b2, eps, wd))
    g = np.random.default_rng(51)
    w = _dev(g.standard_normal(n), off)
    m, v = _dev(np.zeros(n), off), _dev(np.zeros(n), off)
    for t in range(1, 6):
        gr = _dev(g.standard_normal(n) * (0.01 + t), off)
        w0, m0, v0 = (host_f32(x).astype(np.float64) for x in (w, m, v))
        g0 = host_f32(gr)
        dust.dust_adam(w, gr, m, v, n, lr, b1, b2, eps, wd, t)
        rw, rm, rv = oracle.adam(w0, g0, m0, v0, lr, b1, b2, eps, wd, t)
        gw, gm, gv = (host_f32(x).astype(np.float64) for x in (w, m, v))
        dm = 2 * _ulp(np.abs(b1 * m0) + np.abs((1 - b1) * g0)) + 1e-30
        assert np.all(np.abs(gm - rm) <= dm), t
        assert np.all(np.abs(gv - rv) <= 3 * _ulp(rv) + 1e-30), t
        denom = np.sqrt(rv / (1 - b2 ** t)) + eps
        move = np.abs(w0 * (1 - lr * wd) - rw)          # the Adam move of this step
        dw = 2 * _ulp(np.abs(w0) + move) + 1e-6 * move + lr / (1 - b1 ** t) * dm / denom
        assert np.all(np.abs(gw - rw) <= dw), t


def test_optimizer_zero_size_touches_nothing():
    w = torch.full((4,), 3.0, device=DEV)
    dust.dust_sgd_momentum(w, w, w, 0, 0.1, 0.9)
    dust.dust_adam(w, w, w, w, 0, 0.1, 0.9, 0.999, 1e-8, 0.0, 1)
    assert torch.all(w == 3.0)


@pytest.mark.parametrize("n", [1, 1000, 1025, (1 << 22) + 3])
def test_cosine_terms(n):
    """dust_cosine_terms against the oracle's fp64 sums: the fp32 products are exact in fp64,
    only the summation order differs (relative 1e-12 allows n 2^-53 and more)."""
    announce("cosine terms n=%d" % n)
    g = np.random.default_rng(91)
    a = g.standard_normal(n).astype(np.float32)
    b = (0.3 * a + g.standard_normal(n)).astype(np.float32)
    t = torch.full((3,), float("nan"), dtype=torch.float64, device=DEV)
    dust.dust_cosine_terms(f32(a), f32(b), n, t)
    np.testing.assert_allclose(t.cpu().numpy(), oracle.cosine_terms(a, b), rtol=1e-12, atol=0)


def test_cosine_terms_zero_size_and_identical_arrays():
    t = torch.full((3,), 7.0, dtype=torch.float64, device=DEV)
    dust.dust_cosine_terms(None, None, 0, t)
    assert torch.all(t == 7.0)
    from activation_perturbation_es_amd.screen import cosine
    x = f32(np.random.default_rng(92).standard_normal(5000).astype(np.float32))
    assert abs(cosine(x, x) - 1.0) < 1e-14 and abs(cosine(x, -x) + 1.0) < 1e-14
