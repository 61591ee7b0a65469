"""Pins of the perturbed downstream product (CPU only).

Explainer, "The real work: suppressing interference", first measure: a perturbed layer is scored
by re-running the network from that layer onward; the first operation of the re-run is the next
linear layer applied to the activated perturbed output,
    out[k][t][n] = sum_j act(y[t][j] + sigma a^{(draw0+k)}_{tok0+t, chan0+j}) w[n][j].
The oracle states it as the perturbation, the activation and a matrix product. Pins:
  - the activations equal torch's relu, relu squared and gelu(approximate="tanh") in fp64;
  - the product equals torch.nn.functional.linear (fp64) of explicitly formed act(y + sigma a),
    the noise taken from the bulk normals (pinned by the generator tests), under draw, token and
    channel offsets (channels beyond 2^32);
  - sigma = 0 without an activation is y w^T; without an activation the output is affine in
    sigma with slope a w^T;
  - the sampled rows equal rows of the bulk product's operand.
"""
import numpy as np
import pytest
import torch

import oracle

ACTS = [(oracle.ACT_NONE, lambda x: x), (oracle.ACT_RELU, torch.relu),
        (oracle.ACT_RELU2, lambda x: torch.relu(x) ** 2),
        (oracle.ACT_GELU_TANH, lambda x: torch.nn.functional.gelu(x, approximate="tanh"))]


@pytest.mark.parametrize("act,ref", ACTS, ids=["none", "relu", "relu2", "gelu_tanh"])
def test_activation_equals_torch(act, ref):
    x = np.concatenate([np.linspace(-8, 8, 1601), [0.0, -0.0, 1e-30, -1e-30, 30.0, -30.0]])
    got = oracle.activation(x, act)
    # far in the negative tail both sides round 0.5 x (1 + tanh u) near zero: absolute 1e-15
    np.testing.assert_allclose(got, ref(torch.tensor(x)).numpy(), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("act,ref", ACTS, ids=["none", "relu", "relu2", "gelu_tanh"])
@pytest.mark.parametrize("draw0,tok0,chan0", [(0, 0, 0), (7, 300, 2**32 + 64)])
def test_perturbed_linear_equals_torch_linear_of_explicit_inputs(act, ref, draw0, tok0, chan0):
    g = np.random.default_rng(81)
    K, T, d, n_out, sigma = 3, 9, 64, 40, 0.3
    y = g.standard_normal((T, d))
    w = g.standard_normal((n_out, d)) / 8
    got = oracle.perturbed_linear(y, w, K, sigma, 5, 9, act, draw0=draw0, tok0=tok0, chan0=chan0)
    a = oracle.normals(5, 9, draw0, tok0, chan0, K, T, d)
    x = ref(torch.tensor(y[None] + sigma * a))
    want = torch.nn.functional.linear(x, torch.tensor(w)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_sigma_zero_is_the_clean_product_and_the_output_is_affine_in_sigma():
    g = np.random.default_rng(82)
    K, T, d, n_out = 2, 7, 64, 24
    y = g.standard_normal((T, d))
    w = g.standard_normal((n_out, d))
    out0 = oracle.perturbed_linear(y, w, K, 0.0, 3, 4, oracle.ACT_NONE)
    np.testing.assert_allclose(out0, np.broadcast_to(y @ w.T, (K, T, n_out)), rtol=1e-13, atol=1e-12)
    out1 = oracle.perturbed_linear(y, w, K, 0.25, 3, 4, oracle.ACT_NONE, draw0=2)
    out2 = oracle.perturbed_linear(y, w, K, 0.5, 3, 4, oracle.ACT_NONE, draw0=2)
    np.testing.assert_allclose(out2 - out0, 2.0 * (out1 - out0), rtol=1e-10, atol=1e-12)
    a = oracle.normals(3, 4, 2, 0, 0, K, T, d)
    np.testing.assert_allclose(out1 - out0, 0.25 * a @ w.T, rtol=1e-10, atol=1e-12)


def test_sampled_rows_equal_the_bulk_operand():
    g = np.random.default_rng(83)
    K, T, d, sigma = 3, 6, 64, 0.7
    y = g.standard_normal((T, d))
    k = np.array([0, 2, 1, 2])
    t = np.array([5, 0, 3, 3])
    for act, ref in ACTS:
        rows = oracle.perturbed_rows_at(y, k, t, sigma, 11, 2, act, draw0=4, tok0=10, chan0=8)
        full = ref(torch.tensor(y[None] + sigma * oracle.normals(11, 2, 4, 10, 8, K, T, d))).numpy()
        np.testing.assert_allclose(rows, full[k, t], rtol=1e-13, atol=1e-300)
