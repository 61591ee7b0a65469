"""The key and query scorers' e^x - 1 (attn_scores.hip): x + x^2 q(x) with a fitted quadratic q for
|x| <= kPolyRange, evaluated in fp32 by Horner's rule in the unscaled product D (x = s1 D). Host
check of the accuracy its comment states, from the constants in the source: within 8.5e-7 of
e^x - 1 over the range at any scale s1, and near x = 0 (where the leading term is exact) at
fp32 rounding level. Explainer cnblogs.com/32bin/p/23212811, "The real work: suppressing
interference" (the key and query projections scored through the attention output)."""
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "activation_perturbation_es_amd", "csrc", "attn_scores.hip")


def _constants():
    text = open(SRC).read()
    q = [float(re.search(r"kExpm1Q%d = ([0-9.eE+-]+)" % k, text).group(1)) for k in range(3)]
    rng = float(re.search(r"constexpr float kPolyRange = ([0-9.]+)f;", text).group(1))
    return q, rng


def _fma32(a, b, c):
    """fp32 fused multiply-add: the product of two fp32 values is exact in fp64."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _expm1_fp32(D, s1, q):
    s = np.float32(s1)
    a2, a3, a4 = (np.float32(float(s) ** (k + 2) * q[k]) for k in range(3))
    f = lambda v: np.full_like(D, v, dtype=np.float32)
    p = _fma32(D, f(a4), f(a3))
    p = _fma32(D, p, f(a2))
    p = _fma32(D, p, f(s))
    return (D * p).astype(np.float32), s


def test_expm1_form_within_its_stated_bound():
    q, rng = _constants()
    assert rng == 0.15
    g = np.random.default_rng(5)
    for s1 in (1e-3, 4.9e-3, 0.0123, 0.31, 1.0, 2.5, -0.7):
        lim = rng / abs(s1)
        D = np.concatenate([np.linspace(-lim, lim, 200001), g.uniform(-lim, lim, 100000)])
        D = D[D != 0].astype(np.float32)
        e, s = _expm1_fp32(D, s1, q)
        ref = np.expm1(np.float64(s) * D.astype(np.float64))
        rel = np.abs(e.astype(np.float64) / ref - 1.0)
        assert rel.max() <= 8.5e-7, (s1, rel.max())
        small = np.abs(np.float64(s) * D) <= 0.01
        assert rel[small].max() <= 2.5e-7, (s1, rel[small].max())


def test_expm1_form_leading_term_exact():
    """x + x^2 q(x): the coefficient of x is s1 itself, so at tiny x the result is e^x - 1 to
    within the fp32 roundings of the last multiply-add and multiply; a fitted leading
    coefficient off by its 1e-7 would show here."""
    q, _ = _constants()
    for s1 in (0.0123, 1.7):
        D = np.float32([1e-6, -3e-5, 2e-4, -7e-4]) / np.float32(s1)
        e, s = _expm1_fp32(D, s1, q)
        ref = np.expm1(np.float64(s) * D.astype(np.float64))
        assert np.all(np.abs(e.astype(np.float64) / ref - 1.0) <= 1.2e-7), (s1, e, ref)
