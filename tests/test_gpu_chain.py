"""End-to-end estimator chain on the tiny workload (linear 64 -> 64 feeding a fixed head 64 -> 256,
T = 128 tokens as one sequence, K = 16 draws, sigma = 0.01, gamma in {0, 0.9}) on the GPU,
against the oracle's chain in fp64.

The downstream forward (perturbed output -> head logits -> per-token cross-entropy) is the
model's job, not the estimator's: here it is a harness computed with torch in fp64 on the GPU,
and the oracle side computes the same forward in fp64 on the host. The library receives fp32
losses, so the loss change carries the fp32 rounding of l (about 2^-24 * 5.5 ~ 3e-7 against
|c| ~ 1e-2): the output-error estimate is compared at relative Frobenius 1e-3, and the weight
gradient, whose bf16 matrix-core product rounds g_hat^T and x to bf16, at the 2e-2 bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, announce, bf16, dust, f32, frob_rel, host_f32, rne_bf16_bits_of_f32

pytestmark = pytest.mark.gpu


def _harness_losses(yp: torch.Tensor, H: torch.Tensor, tgt: torch.Tensor) -> torch.Tensor:
    z = yp.double() @ H.double().T
    K, T, V = z.shape
    return torch.nn.functional.cross_entropy(z.reshape(K * T, V), tgt.repeat(K).long(),
                                             reduction="none").reshape(K, T).float()


def _cos(a, b):
    return float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()))


@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_tiny_chain(gamma):
    announce("tiny chain gamma=%g" % gamma)
    cfg = synth.WORKLOADS[1]
    T, d_in, d_out, K, sigma, S = cfg["T"], cfg["d_in"], cfg["d_out"], cfg["K"], cfg["sigma"], cfg["seg_len"]
    seed, tag = synth.noise_seed(1), synth.NOISE_TAG
    W, H, x, tgt = synth.tiny_model()
    y = (x.astype(np.float64) @ W.astype(np.float64).T).astype(np.float32)   # cached clean output

    # ---- GPU: library calls, with the harness forward in between
    yd, Hd, td = f32(y), f32(H), torch.from_numpy(tgt).to(DEV)
    yp = torch.empty((K, T, d_out), dtype=torch.float32, device=DEV)
    dust.dust_noise_inject(yd, yp, dust.DUST_F32, T, d_out, d_out, 0, K, sigma, seed, tag, 0, 0)
    lp = _harness_losses(yp, Hd, td)
    lc = _harness_losses(yd[None], Hd, td)[0]
    c = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_LOSS, lc, lp, None, None, dust.DUST_F32, c, K, T, 0)
    r = torch.empty_like(c)
    dust.dust_reward_scan(c, r, K, T, S, gamma)
    gh = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    ght = torch.empty((d_out, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(r, gh, ght, K, K, T, d_out, 0, sigma, seed, tag, 0, 0, 0)
    xb = bf16(rne_bf16_bits_of_f32(x))
    G = torch.empty((d_out, d_in), dtype=torch.float32, device=DEV)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    dust.dust_weight_grad(ght, xb, G, T, d_out, d_in, ws, ws_bytes)

    # ---- oracle chain in fp64 (its own forward of the same model)
    y64 = y.astype(np.float64)
    o_yp = oracle.noise_inject(y64, sigma, K, seed, tag)
    o_lp = oracle.tiny_forward_losses(W, H, x, tgt, y=o_yp)
    o_lc = oracle.tiny_forward_losses(W, H, x, tgt, y=y64)
    o_c = oracle.loss_delta_loss(o_lc, o_lp)
    o_r = oracle.reward_scan(o_c, S, gamma)
    o_g = oracle.error_estimate(o_r, d_out, sigma, seed, tag)
    o_G = oracle.weight_grad(o_g, x)

    assert frob_rel(host_f32(gh), o_g) <= 1e-3
    assert frob_rel(host_f32(G), o_G) <= 2e-2
    _, G_true = oracle.tiny_analytic_grad(W, H, x, tgt)
    assert abs(_cos(host_f32(G), G_true) - _cos(o_G, G_true)) <= 1e-2
