"""Reentrancy on concurrent streams and run-to-run determinism (MI355X only).

include/dust.h promises reentrant entry points that only enqueue work on the caller's stream
and keep no global state. Two whole estimates (inject, loss change and reward, output error,
weight gradient; different seeds, shapes and gammas) are issued at the same time on two side
streams and must equal, bit for bit, the same estimates issued one after the other on the
default stream. The attention scorers must also repeat bit for bit (fixed-order sums, no
atomics).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import DEV, announce, bf16, dust, f32, row_weights

pytestmark = pytest.mark.gpu


class Estimate:
    def __init__(self, T, d_in, d_out, K, S, sigma, gamma, seed, tag, rng):
        self.a = (T, d_in, d_out, K, S, sigma, gamma, seed, tag)
        g = synth.rng(7, rng)
        self.y = bf16(synth.normal_bf16(g, (T, d_out)))
        self.x = bf16(synth.normal_bf16(g, (T, d_in)))
        lc, lp = synth.losses(g, K, T)
        self.lc, self.lp = f32(lc), f32(lp)
        self.yp = torch.empty((K, T, d_out), dtype=torch.bfloat16, device=DEV)
        self.r = torch.empty((K, T), dtype=torch.float32, device=DEV)
        self.gh = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
        self.ght = torch.empty((d_out, T), dtype=torch.bfloat16, device=DEV)
        self.G = torch.empty((d_out, d_in), dtype=torch.float32, device=DEV)
        self.ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=DEV)

    def run(self, stream):
        T, d_in, d_out, K, S, sigma, gamma, seed, tag = self.a
        dust.dust_noise_inject(self.y, self.yp, dust.DUST_BF16, T, d_out, d_out, 0, K, sigma, seed,
                               tag, 0, 0, stream)
        dust.dust_loss_reward(self.lc, self.lp, self.r, K, T, S, gamma, stream)
        dust.dust_error_estimate(self.r, self.gh, self.ght, K, K, T, d_out, 0, sigma, seed, tag, 0,
                                 0, 0, stream)
        dust.dust_weight_grad(self.ght, self.x, self.G, T, d_out, d_in, self.ws, self.ws_bytes,
                              stream)

    def outputs(self):
        return [t.clone() for t in (self.yp, self.r, self.gh, self.ght, self.G)]


def test_two_estimates_on_concurrent_streams_equal_sequential():
    announce("concurrent streams")
    ea = Estimate(4096, 512, 2048, 8, 1024, 0.01, 0.0, 0x1111, 1, 1)
    eb = Estimate(2048, 256, 1024, 16, 512, 0.02, 0.9, 0x2222, 2, 2)
    ea.run(None)
    eb.run(None)
    torch.cuda.synchronize()
    ref_a, ref_b = ea.outputs(), eb.outputs()
    for e in (ea, eb):   # the reruns must recompute everything
        for t in (e.yp, e.r, e.gh, e.ght, e.G):
            t.zero_()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(2):   # the second round overlaps with the first's tail on each stream
        ea.run(s1)
        eb.run(s2)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)
    for got, ref in zip(ea.outputs() + eb.outputs(), ref_a + ref_b):
        assert torch.equal(bits(got), bits(ref))


def test_attention_scorers_repeat_bit_for_bit():
    announce("attention determinism")
    B, H, S, dh, Kc = 2, 2, 128, 64, 12
    T, d = B * S, H * dh
    g = torch.Generator(device=DEV).manual_seed(5)
    z = torch.randn((B, H, S, S), generator=g, device=DEV)
    z.masked_fill_(~torch.ones((S, S), dtype=torch.bool, device=DEV).tril(), float("-inf"))
    P = torch.softmax(z, -1).to(torch.bfloat16)
    q, k, v, go = (torch.randn((T, d), generator=g, device=DEV).to(torch.bfloat16) for _ in range(4))
    W, Z = row_weights(P, v, go, B, H, S, dh)
    W2, Z2 = row_weights(P, v, go, B, H, S, dh)
    assert torch.equal(W.view(torch.int32), W2.view(torch.int32))
    assert torch.equal(Z.view(torch.int32), Z2.view(torch.int32))
    calls = [
        lambda c: dust.dust_attn_value_scores(P, go, c, Kc, B, H, S, dh, 0, 0.05, 3, 1, 0, 0),
        lambda c: dust.dust_attn_key_scores(P, q, W, Z, c, Kc, B, H, S, dh, 0, 0.05, 0.125, 3, 1, 0, 0),
        lambda c: dust.dust_attn_query_scores(P, k, W, Z, c, Kc, B, H, S, dh, 0, 0.05, 0.125, 3, 1, 0, 0),
    ]
    for call in calls:
        c1 = torch.empty((Kc, T), device=DEV)
        c2 = torch.full((Kc, T), float("nan"), device=DEV)
        call(c1)
        call(c2)
        assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))
