"""GPU parity of dust_perturbed_linear, the next linear layer applied to the activated perturbed
outputs with the noise regenerated inside the matrix-core operand path (MI355X only).

Explainer, "The real work: suppressing interference", first measure (the re-run from a
perturbed layer onward). Expected values come from the oracle's plain statement: perturbation,
activation and an fp64 matrix product. Tolerances:
  - against the fp64 product of the unrounded operand: relative Frobenius error <= 2e-2, the
    bound for bf16 matrix-core products (the operand act(y + sigma a) is rounded to bf16, which
    alone gives about 1e-3);
  - against the fp64 product of the operand rounded to bf16 by the oracle (nearest even):
    relative Frobenius error <= 2e-4 with an fp32 output (fp32 accumulation; the kernel rounds
    its fp32 operand, so an element whose fp32 and fp64 values straddle a rounding boundary can
    differ by one bf16 ulp), <= 3e-3 with a bf16 output (one more rounding, 2^-9 relative).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, announce, bf16, bits_to_f64, dust, frob_rel, host_f32

pytestmark = pytest.mark.gpu


def _run(ybits, wbits, T, d, n_out, Kc, act, out_bf16, sigma, seed, tag, draw0, tok0, chan0):
    out = torch.full((Kc, T, n_out), float("nan"), device=DEV,
                     dtype=torch.bfloat16 if out_bf16 else torch.float32)
    dust.dust_perturbed_linear(bf16(ybits), bf16(wbits), out,
                               dust.DUST_BF16 if out_bf16 else dust.DUST_F32, act, T, d, n_out,
                               chan0, Kc, sigma, seed, tag, draw0, tok0)
    return host_f32(out).astype(np.float64)


CASES = [
    # T, d, n_out, Kc, act, out_bf16, draw0, tok0, chan0
    (128, 64, 512, 1, oracle.ACT_RELU, False, 0, 0, 0),              # one whole tile
    (200, 128, 544, 2, oracle.ACT_GELU_TANH, False, 3, 17, 8),        # ragged tokens, partial n-tile
    (300, 256, 96, 3, oracle.ACT_RELU2, True, 1, 5, 2**32 + 4),       # bf16 out, channels past 2^32
    (64, 64, 32, 2, oracle.ACT_NONE, True, 0, 2**32 - 64, 0),         # one n-tile, last tokens
    (257, 192, 1024, 1, oracle.ACT_GELU_TANH, False, 2**31, 0, 64),   # odd tile count
]


@pytest.mark.parametrize("T,d,n_out,Kc,act,out_bf16,draw0,tok0,chan0", CASES)
def test_perturbed_linear(T, d, n_out, Kc, act, out_bf16, draw0, tok0, chan0):
    announce("perturbed_linear %s" % ((T, d, n_out, Kc, act, out_bf16, draw0, tok0, chan0),))
    g = np.random.default_rng(91)
    sigma, seed, tag = 0.05, 0xFEED, 6
    ybits = synth.normal_bf16(g, (T, d))
    wbits = synth.normal_bf16(g, (n_out, d), 1.0 / np.sqrt(d))
    got = _run(ybits, wbits, T, d, n_out, Kc, act, out_bf16, sigma, seed, tag, draw0, tok0, chan0)
    y, w = bits_to_f64(ybits), bits_to_f64(wbits)
    ref = oracle.perturbed_linear(y, w, Kc, sigma, seed, tag, act, draw0, tok0, chan0)
    assert frob_rel(got, ref) <= 2e-2
    k, t = np.meshgrid(np.arange(Kc), np.arange(T), indexing="ij")
    rows = oracle.perturbed_rows_at(y, k.ravel(), t.ravel(), sigma, seed, tag, act, draw0, tok0,
                                    chan0)
    ref_b = (oracle.round_bf16(rows) @ w.T).reshape(Kc, T, n_out)
    err = frob_rel(got, ref_b)
    print("perturbed_linear rel err: %.2e (unrounded operand %.2e)" % (err, frob_rel(got, ref)))
    assert err <= (3e-3 if out_bf16 else 2e-4)


def test_perturbed_linear_full_size_sampled_rows():
    """The 240M shape's MLP: y [16384, 4096] (the up-projection's output), the down-projection
    w [1024, 4096], GELU, 2 draws; sampled (draw, token) rows against the oracle, and the call
    repeats bit for bit."""
    announce("perturbed_linear full size")
    T, d, n_out, Kc, sigma, seed, tag, draw0 = 16384, 4096, 1024, 2, 0.01, synth.noise_seed(5), 1, 30
    g = synth.rng(5, 9)
    ybits = synth.normal_bf16(g, (T, d))
    wbits = synth.normal_bf16(g, (n_out, d), 1.0 / np.sqrt(d))
    yt, wt = bf16(ybits), bf16(wbits)
    out = torch.empty((Kc, T, n_out), dtype=torch.float32, device=DEV)
    dust.dust_perturbed_linear(yt, wt, out, dust.DUST_F32, dust.DUST_ACT_GELU_TANH, T, d, n_out, 0,
                               Kc, sigma, seed, tag, draw0, 0)
    again = torch.empty_like(out)
    dust.dust_perturbed_linear(yt, wt, again, dust.DUST_F32, dust.DUST_ACT_GELU_TANH, T, d, n_out,
                               0, Kc, sigma, seed, tag, draw0, 0)
    assert torch.equal(out, again)
    k = np.array([0, 1, 0, 1, 0, 1, 0, 1, 1, 0, 1, 0])
    t = np.array([0, 1, 127, 128, 129, 4095, 8191, 8192, 12345, 16255, 16256, 16383])
    rows = oracle.perturbed_rows_at(bits_to_f64(ybits), k, t, sigma, seed, tag,
                                    oracle.ACT_GELU_TANH, draw0=draw0)
    w = bits_to_f64(wbits)
    got = host_f32(out)[k, t].astype(np.float64)
    assert frob_rel(got, rows @ w.T) <= 2e-2
    err = frob_rel(got, oracle.round_bf16(rows) @ w.T)
    print("perturbed_linear full size, sampled rows: rel err %.2e" % err)
    assert err <= 2e-4
