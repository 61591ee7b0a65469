"""GPU parity of the attention scorers and of their row weights with the oracle (MI355X only).

The scores c = -<Delta o, g_o> of a perturbed attention value projection, computed on the
device without forming Delta o, are compared with the oracle's fp64 sum element by element at
sizes the oracle finishes in seconds: several 32-key and 32-query tiles, several heads, all
supported head widths' layouts (dh = 16 .. 128), ragged draw groups (the device runs four
draws per block), channel, draw and token offsets, and weights above the diagonal that must be
ignored. Tolerance: relative Frobenius 1e-5, the bar of the inner-mode scores (the noise enters
the bf16 matrix cores as a high part plus a bf16 remainder, about 2^-17 relative). With
identity attention the call must agree with the inner-mode loss change of sigma a computed by
two other entry points (dust_noise_inject into zeros, then dust_loss_delta).

The key scores (a softmax re-run with the logits moved by sigma tau <q_t, a_s>) are compared the
same way, at the same bar, over the same layouts, with logit shifts both inside and beyond the
range where the kernel takes e^x - 1 from a polynomial (|x| <= 0.2), and on tiles that mix the
two; sigma = 0 must give exactly zero and attention to the own token only (nearly) zero. The
query scores (shifts sigma tau <a_t, k_s>) are checked the same way, including the widest heads
(which run 8 waves per block instead of 12) and the longest sequences. Both take the values and
the output error through the row weights W and Z of dust_attn_row_weights, which are themselves
compared with the oracle's element by element.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DEV, announce, bf16, bits_to_f64, dust, f32, frob_rel, host_f32,
                         rne_bf16_bits_of_f32, row_weights)

pytestmark = pytest.mark.gpu


def _causal_weights(g, B, H, S, garbage_above=False):
    z = g.standard_normal((B, H, S, S)) * 2.0
    mask = np.tril(np.ones((S, S), dtype=bool))
    p = np.exp(np.where(mask, z, -np.inf) - np.where(mask, z, -np.inf).max(-1, keepdims=True))
    p = p / p.sum(-1, keepdims=True)
    if garbage_above:
        p = p + np.triu(np.abs(g.standard_normal((S, S))), 1)[None, None]
    return p


@pytest.mark.parametrize("B,H,S,dh,Kc,chan0,draw0,tok0,garbage", [
    (2, 2, 32, 16, 5, 0, 3, 7, False),       # one tile, ragged draw group
    (1, 3, 64, 32, 6, 64, 0, 0, True),       # channel offset, weights above the diagonal
    (2, 2, 128, 64, 3, 0, 11, 1000, False),  # 4 x 4 tiles, the workload's head width
    (1, 1, 96, 128, 9, 8, 2, 5, True),       # widest heads, three groups of draws
    (1, 4, 64, 48, 4, 4, 0, 0, False),       # three k-slices
    (1, 1, 2048, 16, 2, 0, 0, 0, False),     # long sequence: more than 64 KB of LDS per block
    (1, 1, 4096, 16, 1, 0, 0, 0, True),      # the longest sequence supported
    (1, 2, 256, 128, 17, 0, 5, 0, False),    # widest heads, three draw blocks, a ragged one
])
def test_attn_value_scores(B, H, S, dh, Kc, chan0, draw0, tok0, garbage):
    announce("attn value scores %s" % ((B, H, S, dh, Kc, chan0, draw0, tok0, garbage),))
    g = np.random.default_rng(70)
    T, d, sigma, seed, tag = B * S, H * dh, 0.02, 0xA77E, 6
    Pbits = rne_bf16_bits_of_f32(_causal_weights(g, B, H, S, garbage).astype(np.float32))
    gbits = rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32))
    c = torch.full((Kc, T), float("nan"), dtype=torch.float32, device=DEV)
    dust.dust_attn_value_scores(bf16(Pbits), bf16(gbits), c, Kc, B, H, S, dh, chan0, sigma, seed, tag,
                                draw0, tok0)
    ref = oracle.attn_value_scores(bits_to_f64(Pbits), bits_to_f64(gbits), Kc, sigma, seed, tag,
                                   draw0, tok0, chan0)
    assert frob_rel(host_f32(c), ref) <= 1e-5


def test_identity_attention_equals_inner_mode_of_injected_noise():
    announce("attn value scores vs inject + inner mode")
    B, H, S, dh, Kc, sigma, seed, tag = 2, 4, 64, 32, 6, 0.05, 77, 9
    T, d = B * S, H * dh
    g = np.random.default_rng(71)
    P = np.broadcast_to(np.eye(S, dtype=np.float32), (B, H, S, S)).copy()
    gbits = rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32))
    c = torch.empty((Kc, T), dtype=torch.float32, device=DEV)
    dust.dust_attn_value_scores(bf16(rne_bf16_bits_of_f32(P)), bf16(gbits), c, Kc, B, H, S, dh, 0,
                                sigma, seed, tag, 0, 0)
    zeros = torch.zeros((T, d), dtype=torch.float32, device=DEV)
    do = torch.empty((Kc, T, d), dtype=torch.float32, device=DEV)      # sigma a
    dust.dust_noise_inject(zeros, do, dust.DUST_F32, T, d, d, 0, Kc, sigma, seed, tag, 0, 0)
    c2 = torch.empty((Kc, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_INNER, None, None, do, f32(bits_to_f64(gbits)), dust.DUST_F32,
                         c2, Kc, T, d)
    assert frob_rel(host_f32(c), host_f32(c2).astype(np.float64)) <= 1e-5


def test_attn_value_scores_zero_draws_touch_nothing():
    c = torch.full((2, 64), 5.0, device=DEV)
    dust.dust_attn_value_scores(None, None, c, 0, 2, 2, 32, 16, 0, 0.01, 1, 1, 0, 0)
    assert torch.all(c == 5.0)


@pytest.mark.parametrize("B,H,S,dh,Kc,chan0,draw0,tok0,garbage,sigma,tau", [
    (2, 2, 32, 16, 5, 0, 3, 7, False, 0.05, 0.25),       # one tile, ragged draw group
    (1, 3, 64, 32, 6, 64, 0, 0, True, 0.05, 0.18),       # channel offset, weights above the diagonal
    (2, 2, 128, 64, 3, 0, 11, 1000, False, 0.01, 0.125), # 4 x 4 tiles, the workload's head width
    (1, 1, 96, 128, 9, 8, 2, 5, True, 0.02, 0.09),       # widest heads, three groups of draws
    (1, 4, 64, 48, 4, 4, 0, 0, False, 0.05, 0.144),      # three k-slices
    (1, 2, 1024, 16, 2, 0, 0, 0, False, 0.05, 0.25),     # longest sequence
    (1, 2, 64, 32, 4, 0, 0, 0, False, 1.5, 0.18),        # large shifts: e^x - 1 from exp
    (1, 2, 128, 32, 4, 0, 0, 0, False, 0.15, 0.18),      # tiles that mix both forms
    (1, 1, 1024, 128, 2, 0, 0, 0, True, 0.02, 0.09),     # longest sequence at the widest heads
    (1, 1, 512, 80, 3, 0, 0, 0, False, 0.02, 0.11),      # the widest heads on 12 waves
    (2, 1, 32, 64, 17, 4, 9, 3, False, 0.05, 0.125),     # one tile per sequence, ragged blocks
    (1, 1, 1024, 96, 13, 0, 0, 0, True, 0.02, 0.1),      # 8 waves of one draw: 8 + 5 draws
    (1, 2, 2048, 16, 5, 0, 1, 0, False, 0.05, 0.25),     # 4 waves per block, 4 + 1 draws
    (1, 1, 4096, 16, 3, 4, 0, 0, True, 0.05, 0.25),      # 2 waves per block, 2 + 1 draws
    (1, 1, 4096, 128, 2, 0, 0, 0, False, 0.02, 0.09),    # the widest heads at the longest sequence
    (1, 1, 1024, 64, 33, 0, 5, 0, False, 0.01, 0.125),   # 33 draws: 12 + 12 + 9
])
def test_attn_key_scores(B, H, S, dh, Kc, chan0, draw0, tok0, garbage, sigma, tau):
    announce("attn key scores %s" % ((B, H, S, dh, Kc, chan0, draw0, tok0, garbage, sigma, tau),))
    g = np.random.default_rng(72)
    T, d, seed, tag = B * S, H * dh, 0xA77F, 7
    Pbits = rne_bf16_bits_of_f32(_causal_weights(g, B, H, S, garbage).astype(np.float32))
    qb, vb, gb = (rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)) for _ in range(3))
    c = torch.full((Kc, T), float("nan"), dtype=torch.float32, device=DEV)
    Pd = bf16(Pbits)
    W, Z = row_weights(Pd, bf16(vb), bf16(gb), B, H, S, dh)
    dust.dust_attn_key_scores(Pd, bf16(qb), W, Z, c, Kc, B, H, S, dh, chan0, sigma, tau, seed, tag,
                              draw0, tok0)
    ref = oracle.attn_key_scores(bits_to_f64(Pbits), bits_to_f64(qb), bits_to_f64(vb),
                                 bits_to_f64(gb), Kc, sigma, tau, seed, tag, draw0, tok0, chan0)
    err = frob_rel(host_f32(c), ref)
    print("key scores rel. Frobenius error %.2e" % err)
    assert err <= 1e-5


def test_attn_key_scores_vanish_at_sigma_zero_and_for_self_attention():
    announce("attn key scores sigma = 0, self attention")
    B, H, S, dh, Kc = 1, 2, 64, 32, 4
    T, d = B * S, H * dh
    g = np.random.default_rng(73)
    qb, vb, gb = (bf16(rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)))
                  for _ in range(3))
    P = bf16(rne_bf16_bits_of_f32(_causal_weights(g, B, H, S).astype(np.float32)))
    c = torch.full((Kc, T), float("nan"), dtype=torch.float32, device=DEV)
    W, Z = row_weights(P, vb, gb, B, H, S, dh)
    dust.dust_attn_key_scores(P, qb, W, Z, c, Kc, B, H, S, dh, 0, 0.0, 0.2, 5, 1, 0, 0)
    assert torch.all(c == 0)
    eye = bf16(rne_bf16_bits_of_f32(np.broadcast_to(np.eye(S, dtype=np.float32), (B, H, S, S)).copy()))
    W, Z = row_weights(eye, vb, gb, B, H, S, dh)
    dust.dust_attn_key_scores(eye, qb, W, Z, c, Kc, B, H, S, dh, 0, 0.05, 0.2, 5, 1, 0, 0)
    assert float(c.abs().max()) <= 1e-6


def test_attn_key_scores_zero_draws_touch_nothing():
    c = torch.full((2, 64), 5.0, device=DEV)
    dust.dust_attn_key_scores(None, None, None, None, c, 0, 2, 2, 32, 16, 0, 0.01, 0.25, 1, 1, 0, 0)
    dust.dust_attn_query_scores(None, None, None, None, c, 0, 2, 2, 32, 16, 0, 0.01, 0.25, 1, 1, 0, 0)
    assert torch.all(c == 5.0)


def test_attn_scores_channels_beyond_32_bits():
    """chan0 above 2^32 (the noise's channel index goes to 2^34): the kernels take chan0 / 4."""
    announce("attn scores chan0 >= 2^32")
    B, H, S, dh, Kc, sigma, tau, chan0 = 1, 2, 32, 16, 3, 0.05, 0.25, (1 << 32) + 64
    T, d = B * S, H * dh
    g = np.random.default_rng(74)
    Pbits = rne_bf16_bits_of_f32(_causal_weights(g, B, H, S).astype(np.float32))
    qb, vb, gb = (rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)) for _ in range(3))
    c = torch.empty((Kc, T), dtype=torch.float32, device=DEV)
    dust.dust_attn_value_scores(bf16(Pbits), bf16(gb), c, Kc, B, H, S, dh, chan0, sigma, 3, 1, 0, 0)
    ref = oracle.attn_value_scores(bits_to_f64(Pbits), bits_to_f64(gb), Kc, sigma, 3, 1, 0, 0, chan0)
    assert frob_rel(host_f32(c), ref) <= 1e-5
    W, Z = row_weights(bf16(Pbits), bf16(vb), bf16(gb), B, H, S, dh)
    dust.dust_attn_key_scores(bf16(Pbits), bf16(qb), W, Z, c, Kc, B, H, S, dh, chan0, sigma, tau, 3,
                              1, 0, 0)
    ref = oracle.attn_key_scores(bits_to_f64(Pbits), bits_to_f64(qb), bits_to_f64(vb),
                                 bits_to_f64(gb), Kc, sigma, tau, 3, 1, 0, 0, chan0)
    assert frob_rel(host_f32(c), ref) <= 1e-5
    dust.dust_attn_query_scores(bf16(Pbits), bf16(qb), W, Z, c, Kc, B, H, S, dh, chan0, sigma, tau,
                                3, 1, 0, 0)
    ref = oracle.attn_query_scores(bits_to_f64(Pbits), bits_to_f64(qb), bits_to_f64(vb),
                                   bits_to_f64(gb), Kc, sigma, tau, 3, 1, 0, 0, chan0)
    assert frob_rel(host_f32(c), ref) <= 1e-5


@pytest.mark.parametrize("B,H,S,dh,Kc,chan0,draw0,tok0,garbage,sigma,tau", [
    (2, 2, 32, 16, 5, 0, 3, 7, False, 0.05, 0.25),       # one tile, ragged draw group
    (1, 3, 64, 32, 6, 64, 0, 0, True, 0.05, 0.18),       # channel offset, weights above the diagonal
    (2, 2, 128, 64, 3, 0, 11, 1000, False, 0.01, 0.125), # 4 x 4 tiles, the workload's head width
    (1, 1, 96, 128, 9, 8, 2, 5, True, 0.02, 0.09),       # widest heads (8 waves a block), 2 blocks
    (1, 4, 64, 48, 4, 4, 0, 0, False, 0.05, 0.144),      # three k-slices
    (1, 1, 96, 112, 5, 0, 0, 0, False, 0.05, 0.094),     # seven k-slices (8 waves a block)
    (1, 1, 4096, 16, 2, 0, 0, 0, False, 0.05, 0.25),     # the longest sequence
    (1, 2, 64, 32, 4, 0, 0, 0, False, 1.5, 0.18),        # large shifts: e^x - 1 from exp
    (1, 2, 128, 32, 4, 0, 0, 0, False, 0.15, 0.18),      # tiles that mix both forms
    (2, 1, 32, 64, 17, 4, 9, 3, False, 0.05, 0.125),     # one tile per sequence, ragged blocks
    (1, 1, 2048, 64, 13, 0, 0, 0, True, 0.02, 0.125),    # long sequence, 13 draws in one block
    (1, 1, 128, 80, 9, 0, 0, 0, False, 0.05, 0.11),      # the narrowest heads of one draw a wave
    (1, 1, 1024, 64, 33, 0, 5, 0, False, 0.01, 0.125),   # 33 draws: 12 + 12 + 9
    # 16 sequences x 201 draws: on 256 compute units 8 waves of two draws end in one round of
    # blocks against two for 12 waves of one, so this launch takes the two-draw layout; the
    # odd count leaves one wave with its second draw past the last
    (16, 1, 64, 64, 201, 0, 3, 0, False, 0.05, 0.125),
])
def test_attn_query_scores(B, H, S, dh, Kc, chan0, draw0, tok0, garbage, sigma, tau):
    announce("attn query scores %s" % ((B, H, S, dh, Kc, chan0, draw0, tok0, garbage, sigma, tau),))
    g = np.random.default_rng(75)
    T, d, seed, tag = B * S, H * dh, 0xA780, 8
    Pbits = rne_bf16_bits_of_f32(_causal_weights(g, B, H, S, garbage).astype(np.float32))
    kb, vb, gb = (rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)) for _ in range(3))
    c = torch.full((Kc, T), float("nan"), dtype=torch.float32, device=DEV)
    Pd = bf16(Pbits)
    W, Z = row_weights(Pd, bf16(vb), bf16(gb), B, H, S, dh)
    dust.dust_attn_query_scores(Pd, bf16(kb), W, Z, c, Kc, B, H, S, dh, chan0, sigma, tau, seed,
                                tag, draw0, tok0)
    ref = oracle.attn_query_scores(bits_to_f64(Pbits), bits_to_f64(kb), bits_to_f64(vb),
                                   bits_to_f64(gb), Kc, sigma, tau, seed, tag, draw0, tok0, chan0)
    err = frob_rel(host_f32(c), ref)
    print("query scores rel. Frobenius error %.2e" % err)
    assert err <= 1e-5


def _max_shift(x64, B, H, S, dh, Kc, sigma, tau, seed, tag, noise_on_keys):
    """Largest |sigma tau <q_t, a_s>| (or <a_t, k_s>) over the causal pairs, from the oracle's
    normals: how far the draws reach beyond e^delta's fp32 range."""
    a = oracle.normals(seed, tag, 0, 0, 0, Kc, B * S, H * dh)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            xs = x64[b * S:(b + 1) * S, h * dh:(h + 1) * dh]
            for k in range(Kc):
                an = a[k, b * S:(b + 1) * S, h * dh:(h + 1) * dh]
                D = xs @ an.T if noise_on_keys else an @ xs.T      # [query, key]
                worst = max(worst, float(np.abs(np.tril(D)).max()))
    return abs(sigma * tau) * worst


@pytest.mark.parametrize("which,B,H,S,dh,Kc,garbage,sigma,tau,reach", [
    ("keys", 1, 2, 64, 32, 4, False, 40.0, 0.18, 100),     # nearly every query beyond e^x's range
    ("queries", 1, 2, 64, 32, 4, False, 40.0, 0.18, 100),
    ("keys", 1, 2, 64, 32, 4, False, 10.0, 0.18, 20),      # within range, rows' mass far below Z
    ("queries", 1, 2, 64, 32, 4, False, 10.0, 0.18, 20),
    ("keys", 2, 1, 96, 16, 5, True, 26.0, 0.25, 100),      # some queries of some draws
    ("queries", 2, 1, 96, 16, 5, True, 26.0, 0.25, 100),
    ("keys", 1, 1, 288, 128, 3, False, 30.0, 0.09, 100),   # two groups of queries, the widest heads
    ("queries", 1, 1, 288, 128, 3, False, 30.0, 0.09, 100),
    ("keys", 1, 1, 2048, 16, 3, False, 24.0, 0.25, 100),   # a long sequence on 4 waves a block
])
def test_attn_softmax_scores_beyond_exp_range(which, B, H, S, dh, Kc, garbage, sigma, tau, reach):
    """Large logit shifts: past fp32's e^x range, or moving a row's mass far below Z (where the
    fast form cancels). The fast pass marks those queries and the exact pass with the row maximum
    subtracted recomputes them; every score finite, and equal to the oracle's (which subtracts
    the row maximum throughout)."""
    announce("attn %s scores beyond e^x %s" % (which, (B, H, S, dh, Kc, garbage, sigma, tau)))
    g = np.random.default_rng(78)
    T, d, seed, tag = B * S, H * dh, 0xA781, 9
    Pbits = rne_bf16_bits_of_f32(_causal_weights(g, B, H, S, garbage).astype(np.float32))
    xb, vb, gb = (rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)) for _ in range(3))
    assert _max_shift(bits_to_f64(xb), B, H, S, dh, Kc, sigma, tau, seed, tag, which == "keys") > reach
    c = torch.full((Kc, T), float("nan"), dtype=torch.float32, device=DEV)
    Pd = bf16(Pbits)
    W, Z = row_weights(Pd, bf16(vb), bf16(gb), B, H, S, dh)
    fn = dust.dust_attn_key_scores if which == "keys" else dust.dust_attn_query_scores
    fn(Pd, bf16(xb), W, Z, c, Kc, B, H, S, dh, 0, sigma, tau, seed, tag, 0, 0)
    of = oracle.attn_key_scores if which == "keys" else oracle.attn_query_scores
    ref = of(bits_to_f64(Pbits), bits_to_f64(xb), bits_to_f64(vb), bits_to_f64(gb), Kc, sigma, tau,
             seed, tag, 0, 0, 0)
    got = host_f32(c)
    assert np.all(np.isfinite(got))
    err = frob_rel(got, ref)
    print("%s scores beyond e^x: rel. Frobenius error %.2e" % (which, err))
    assert err <= 1e-5


def test_attn_query_scores_vanish_at_sigma_zero_and_for_self_attention():
    announce("attn query scores sigma = 0, self attention")
    B, H, S, dh, Kc = 1, 2, 64, 32, 4
    T, d = B * S, H * dh
    g = np.random.default_rng(76)
    kb, vb, gb = (bf16(rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)))
                  for _ in range(3))
    P = bf16(rne_bf16_bits_of_f32(_causal_weights(g, B, H, S).astype(np.float32)))
    c = torch.full((Kc, T), float("nan"), dtype=torch.float32, device=DEV)
    W, Z = row_weights(P, vb, gb, B, H, S, dh)
    dust.dust_attn_query_scores(P, kb, W, Z, c, Kc, B, H, S, dh, 0, 0.0, 0.2, 5, 1, 0, 0)
    assert torch.all(c == 0)
    eye = bf16(rne_bf16_bits_of_f32(np.broadcast_to(np.eye(S, dtype=np.float32), (B, H, S, S)).copy()))
    W, Z = row_weights(eye, vb, gb, B, H, S, dh)
    dust.dust_attn_query_scores(eye, kb, W, Z, c, Kc, B, H, S, dh, 0, 0.05, 0.2, 5, 1, 0, 0)
    assert float(c.abs().max()) <= 1e-6


@pytest.mark.parametrize("B,H,S,dh,garbage", [
    (2, 2, 32, 16, False),     # one tile
    (1, 3, 64, 32, True),      # weights above the diagonal must be ignored
    (2, 2, 128, 64, False),    # 4 x 4 tiles, the workload's head width
    (1, 1, 96, 128, True),     # widest heads
    (1, 4, 64, 48, False),     # three k-slices
    (1, 1, 4096, 16, False),   # the longest sequence
    (3, 1, 64, 112, False),    # a partly filled last block of query tiles
    (1, 2, 1024, 96, True),    # six k-slices, long sequence
])
def test_attn_row_weights(B, H, S, dh, garbage):
    """W and Z of dust_attn_row_weights against the oracle's: relative Frobenius 1e-5 for W (fp32
    sums of bf16 products over dh and of S weights), 2e-5 per row sum for Z, and W exactly zero
    above the diagonal."""
    announce("attn row weights %s" % ((B, H, S, dh, garbage),))
    g = np.random.default_rng(77)
    T, d = B * S, H * dh
    Pbits = rne_bf16_bits_of_f32(_causal_weights(g, B, H, S, garbage).astype(np.float32))
    vb, gb = (rne_bf16_bits_of_f32(g.standard_normal((T, d)).astype(np.float32)) for _ in range(2))
    W, Z = row_weights(bf16(Pbits), bf16(vb), bf16(gb), B, H, S, dh)
    Wr, Zr = oracle.attn_row_weights(bits_to_f64(Pbits), bits_to_f64(vb), bits_to_f64(gb))
    Wg, Zg = host_f32(W), host_f32(Z)
    err = frob_rel(Wg, Wr)
    print("row weights rel. Frobenius error %.2e" % err)
    assert err <= 1e-5
    assert np.all(np.abs(Zg - Zr) <= 2e-5 * np.abs(Zr))
    assert np.all(Wg[..., ~np.tril(np.ones((S, S), dtype=bool))] == 0.0)


def test_attn_row_weights_zero_size_touches_nothing():
    W = torch.full((2, 2, 32, 32), 5.0, device=DEV)
    dust.dust_attn_row_weights(None, None, None, W, W, 0, 2, 32, 16)
    assert torch.all(W == 5.0)
