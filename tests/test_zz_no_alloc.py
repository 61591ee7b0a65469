"""dust_weight_grad_noalloc (the weight-gradient entry point for callers that cannot allocate)
against dust_weight_grad with a caller-allocated workspace, through the C ABI (MI355X only).

Same kernels, so the two must agree bit for bit; both are also checked against the oracle's fp64
product of the same bf16 inputs (relative Frobenius error <= 1e-5, the bar of the weight
gradient on identical bf16 inputs). Two calls in a row, the second smaller, so the second runs
on scratch that still holds the first call's partial sums.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, announce, bf16, bits_to_f64, dust, frob_rel, host_f32

pytestmark = pytest.mark.gpu


def _inputs(seed, T, d_out, d_in):
    g = np.random.default_rng(seed)
    a = (g.standard_normal((d_out, T)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = (g.standard_normal((T, d_in)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return a, x


def _with_workspace(at, xt, T, d_out, d_in):
    G = torch.full((d_out, d_in), float("nan"), device=DEV)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    dust.dust_weight_grad(at, xt, G, T, d_out, d_in, ws, ws_bytes)
    return G


@pytest.mark.parametrize("shapes", [
    # large-tile kernel with 16 splits (64 MiB of partials), then the same kernel with fewer
    [(16384, 2048, 512), (4096, 1024, 512)],
    # large-tile kernel, then the small-tile kernel with a ragged output
    [(16384, 4096, 1024), (2048, 200, 136)],
])
def test_noalloc_equals_workspace_entry_point(shapes):
    for n, (T, d_out, d_in) in enumerate(shapes):
        announce("weight_grad_noalloc call %d %s" % (n, (T, d_out, d_in)))
        assert dust.dust_weight_grad_workspace(T, d_out, d_in) <= 64 << 20
        abits, xbits = _inputs(100 + n, T, d_out, d_in)
        at, xt = bf16(abits), bf16(xbits)
        G_ref = _with_workspace(at, xt, T, d_out, d_in)
        G = torch.full((d_out, d_in), float("nan"), device=DEV)
        dust.dust_weight_grad_noalloc(at, xt, G, T, d_out, d_in)
        got, ref = host_f32(G), host_f32(G_ref)
        assert np.array_equal(got, ref)
        rows = np.arange(0, d_out, max(1, d_out // 64))
        exact = oracle.weight_grad(bits_to_f64(abits[rows]).T, bits_to_f64(xbits))
        assert frob_rel(got[rows], exact) <= 1e-5


def test_noalloc_rejects_shapes_beyond_the_scratch():
    T, d_out, d_in = 16384, 768, 11008
    assert dust.dust_weight_grad_workspace(T, d_out, d_in) > 64 << 20
    G = torch.empty((d_out, d_in), device=DEV)
    a = torch.empty((d_out, T), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((T, d_in), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dust.DustError) as e:
        dust.dust_weight_grad_noalloc(a, x, G, T, d_out, d_in)
    assert e.value.status == dust.DUST_ERR_UNSUPPORTED
