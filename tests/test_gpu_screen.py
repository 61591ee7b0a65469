"""Hyperparameter screening by cosine on the small random-weight GPT (MI355X only).

The explainer ("The real work") tunes Dust cheaply by ranking candidate settings on one batch by
the cosine between the estimate and the backpropagation gradient, and leaves the final choice to
training. Here the screen runs the library's chain (inject, the harness's suffix forward, loss
change and reward, output error, weight gradient) for each (sigma, gamma) on a grid, for the two
layer types of test_gpu_gpt.py, against autograd's gradient of the same batch, at K = 4096.

What it must find follows from the credit-assignment limit of test_gpu_gpt.py: the attention
value projection mixes tokens directly, so its gradient is the gamma = 1 limit and gamma = 1 wins;
block 0's MLP output reaches other tokens only through block 1's attention, so most of its
gradient is the own token's and gamma = 0, the lowest-variance reward, wins at this population.
In the small-sigma regime the cosine does not depend on sigma; sigma = 1 leaves the linear
regime: it loses at the layer's best gamma and elsewhere moves the cosine by less than 0.01. The
screen's cosines must also equal a host fp64 cosine of the same arrays.
"""
import numpy as np
import pytest
import torch

import test_gpu_gpt as gpt
from activation_perturbation_es_amd.screen import screen
from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu

K = 4096
GRID = [(s, g) for s in (0.01, 1.0) for g in (0.0, 0.9, 1.0)]


def _estimate_dev(net, sigma, gamma):
    saved = gpt.SIGMA
    gpt.SIGMA = sigma
    try:
        return torch.tensor(gpt._estimate(net, K, gamma), dtype=torch.float32, device=DEV)
    finally:
        gpt.SIGMA = saved


@pytest.mark.parametrize("layer,best_gamma", [("attn_v", 1.0), ("mlp_up", 0.0)])
def test_screen_picks_the_layer_types_gamma(layer, best_gamma):
    announce("screen %s" % layer)
    net = gpt.Net(layer)
    G_true, _, _ = gpt._limits(net)
    ref = torch.tensor(G_true, dtype=torch.float32, device=DEV)
    ests = {c: _estimate_dev(net, *c) for c in GRID}
    ranked = screen(GRID, lambda c: ests[c], ref)
    print(layer, ["%.3f s%g g%.1f" % (cs, c[0], c[1]) for cs, c in ranked])
    for cs, c in ranked:   # the device cosine against the host's
        e = ests[c].double().cpu().numpy().ravel()
        r = ref.double().cpu().numpy().ravel()
        assert abs(cs - e @ r / np.sqrt((e @ e) * (r @ r))) < 1e-9
    assert [cs for cs, _ in ranked] == sorted((cs for cs, _ in ranked), reverse=True)
    (_, (s_best, g_best)) = ranked[0]
    assert g_best == best_gamma and s_best == 0.01, ranked[0]
    cos = dict((c, cs) for cs, c in ranked)
    for g in (0.0, 0.9, 1.0):   # leaving the linear regime costs cosine
        assert cos[(1.0, g)] < cos[(0.01, g)] + 0.01
    assert len(screen(GRID, lambda c: ests[c], ref, keep=2)) == 2
