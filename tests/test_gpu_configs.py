"""GPU parity at the full workload sizes, in the launch configurations the benchmark times, on
sampled outputs the oracle computes one by one (MI355X only).

Workloads (see synth.WORKLOADS): 2 = MLP up-projection 512 -> 2048, T = 16384, K = 64;
3 = LM-head chunk [0, 1024) of V = 4096, T = 16384, K = 1024; 4 = attention k/v 512 -> 512
scored by inner products, gamma = 0.99, K = 16384 in blocks of 512; 5 = MLP up-projection
1024 -> 4096, T = 16384, K = 1024. Tolerances are those of test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (DEV, announce, bf16, bf16_ulp, bits_to_f64, dust, f32, frob_rel,
                         host_bf16_bits, host_f32, i32, rne_bf16_bits_of_f32, row_weights)

pytestmark = pytest.mark.gpu
NS = 20000   # sampled elements per check


def _gather_bits(t: torch.Tensor, *idx) -> np.ndarray:
    """bf16 bit patterns of the sampled elements, gathered on the device."""
    ii = tuple(torch.from_numpy(np.asarray(i, dtype=np.int64)).to(DEV) for i in idx)
    return host_bf16_bits(t[ii].contiguous())


def _check_inject_block(cfg, d_key):
    c = synth.WORKLOADS[cfg]
    T, d, sigma, Kb = c["T"], c[d_key], c["sigma"], c["inject_block"]
    draw0 = c["K"] - Kb                         # last block of the population
    seed, tag = synth.noise_seed(cfg), synth.NOISE_TAG
    ybits = synth.normal_bf16(synth.rng(cfg, 1), (T, d))
    out = torch.empty((Kb, T, d), dtype=torch.bfloat16, device=DEV)
    dust.dust_noise_inject(bf16(ybits), out, dust.DUST_BF16, T, d, d, 0, Kb, sigma, seed, tag, draw0, 0)
    g = np.random.default_rng(100 + cfg)
    k, t, j = g.integers(0, Kb, NS), g.integers(0, T, NS), g.integers(0, d, NS)
    k[:2], t[:2], j[:2] = [0, Kb - 1], [0, T - 1], [0, d - 1]
    got = _gather_bits(out, k, t, j)
    del out
    n = oracle.normals_at(seed, tag, k, t, j, draw0=draw0)
    ref = oracle.round_bf16(bits_to_f64(ybits[t, j]) + sigma * n)
    gv = bits_to_f64(got)
    assert np.all(np.abs(gv - ref) <= bf16_ulp(ref))
    assert np.mean(gv != ref) < 0.01


def _check_error_estimate(cfg, K, T, d, chan0=0):
    sigma, seed, tag = synth.WORKLOADS[cfg]["sigma"], synth.noise_seed(cfg), synth.NOISE_TAG
    r = synth.normal_f32(synth.rng(cfg, 3), (K, T), 0.01)
    gh = torch.empty((T, d), dtype=torch.float32, device=DEV)
    gt = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(f32(r), gh, gt, K, K, T, d, chan0, sigma, seed, tag, 0, 0, 0)
    got = host_f32(gh)
    gtb = host_bf16_bits(gt)
    g = np.random.default_rng(200 + cfg)
    ns = 2000 if K <= 1024 else 600
    tok, ch = g.integers(0, T, ns), g.integers(0, d, ns)
    tok[:2], ch[:2] = [0, T - 1], [0, d - 1]
    ref = oracle.error_estimate_at(r, tok, ch, sigma, seed, tag, chan0=chan0)
    assert frob_rel(got[tok, ch], ref) <= 1e-5
    assert np.array_equal(gtb[ch, tok], rne_bf16_bits_of_f32(got[tok, ch]))


def _check_weight_grad(cfg, T, d_out, d_in, nrows):
    g = synth.rng(cfg, 4)
    a = synth.normal_bf16(g, (d_out, T))
    b = synth.normal_bf16(g, (T, d_in))
    G = torch.empty((d_out, d_in), dtype=torch.float32, device=DEV)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    dust.dust_weight_grad(bf16(a), bf16(b), G, T, d_out, d_in, ws, ws_bytes)
    got = host_f32(G)
    rows = np.random.default_rng(300 + cfg).choice(d_out, size=min(nrows, d_out), replace=False)
    rows[0] = d_out - 1
    ref = oracle.weight_grad(bits_to_f64(a[rows]).T, bits_to_f64(b))
    assert frob_rel(got[rows], ref) <= 1e-5


# ------------------------------------------------------------------------------ workload 2
def test_w2_inject_block():
    announce("w2 inject block")
    _check_inject_block(2, "d_out")


def test_w2_loss_delta_and_scan():
    announce("w2 loss delta + scan")
    c = synth.WORKLOADS[2]
    K, T, S = c["K"], c["T"], c["seg_len"]
    lc, lp = synth.losses(synth.rng(2, 2), K, T)
    cd = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_LOSS, f32(lc), f32(lp), None, None, dust.DUST_F32, cd, K, T, 0)
    ref = oracle.loss_delta_loss(lc, lp)
    assert np.array_equal(host_f32(cd), ref.astype(np.float32))
    rd = torch.empty_like(cd)
    dust.dust_reward_scan(cd, rd, K, T, S, c["gamma"])
    assert np.array_equal(host_f32(rd), host_f32(cd))    # gamma = 0
    rf = torch.empty_like(cd)                             # the fused call the benchmark times
    dust.dust_loss_reward(f32(lc), f32(lp), rf, K, T, S, c["gamma"])
    assert np.array_equal(host_f32(rf), host_f32(rd))


def test_w2_error_estimate():
    announce("w2 error estimate")
    c = synth.WORKLOADS[2]
    _check_error_estimate(2, c["K"], c["T"], c["d_out"])


def test_w2_weight_grad():
    announce("w2 weight grad")
    c = synth.WORKLOADS[2]
    _check_weight_grad(2, c["T"], c["d_out"], c["d_in"], 256)


# ------------------------------------------------------------------------------ workload 3
def test_w3_head_chunk():
    announce("w3 head chunk")
    c = synth.WORKLOADS[3]
    T, V, v0, C, K, sigma = c["T"], c["V"], c["v0"], c["C"], c["K"], c["sigma"]
    seed, tag = synth.noise_seed(3), synth.NOISE_TAG
    g = synth.rng(3, 1)
    z = synth.normal_f32(g, (T, V), np.sqrt(2.0))
    tgt = synth.targets(g, T, V)
    lp = torch.empty((K, T), dtype=torch.float32, device=DEV)
    lc = torch.empty((T,), dtype=torch.float32, device=DEV)
    dust.dust_head_ce_chunk(f32(z), i32(tgt), lp, lc, T, V, v0, C, K, sigma, seed, tag, 0, 0)
    got_p, got_c = host_f32(lp), host_f32(lc)
    _, ref_c = oracle.head_ce_chunk(z, tgt, v0, C, 0, sigma, seed, tag)
    assert np.abs(got_c - ref_c).max() <= 1e-4
    s = np.random.default_rng(403)
    k, t = s.integers(0, K, 400), s.integers(0, T, 400)
    k[:2], t[:2] = [0, K - 1], [0, T - 1]
    ref_p = oracle.head_ce_at(z, tgt, v0, C, k, t, sigma, seed, tag)
    assert np.abs(got_p[k, t] - ref_p).max() <= 1e-4


def test_w3_error_estimate():
    announce("w3 error estimate")
    c = synth.WORKLOADS[3]
    _check_error_estimate(3, c["K"], c["T"], c["C"], chan0=c["v0"])


def test_w3_weight_grad():
    announce("w3 weight grad")
    c = synth.WORKLOADS[3]
    _check_weight_grad(3, c["T"], c["C"], c["hidden"], 256)


# ------------------------------------------------------------------------------ workload 4
def test_w4_delta_o_block_generation():
    """The synthetic attention-output change of one 512-draw block, N(0, 1e-4) in bf16, drawn on
    the device from its own Philox tag."""
    announce("w4 delta_o block")
    c = synth.WORKLOADS[4]
    T, d, Kb, std = c["T"], c["d"], c["draw_block"], c["delta_o_std"]
    seed = synth.noise_seed(4)
    zero = torch.zeros((T, d), dtype=torch.bfloat16, device=DEV)
    do = torch.empty((Kb, T, d), dtype=torch.bfloat16, device=DEV)
    draw0 = c["K"] - Kb
    dust.dust_noise_inject(zero, do, dust.DUST_BF16, T, d, d, 0, Kb, std, seed, synth.DELTA_O_TAG, draw0, 0)
    g = np.random.default_rng(404)
    k, t, j = g.integers(0, Kb, NS), g.integers(0, T, NS), g.integers(0, d, NS)
    got = _gather_bits(do, k, t, j)
    del do
    ref = oracle.round_bf16(std * oracle.normals_at(seed, synth.DELTA_O_TAG, k, t, j, draw0=draw0))
    gv = bits_to_f64(got)
    assert np.all(np.abs(gv - ref) <= bf16_ulp(ref))


def test_w4_inner_scores():
    announce("w4 inner scores")
    c = synth.WORKLOADS[4]
    T, d, std = c["T"], c["d"], c["delta_o_std"]
    Kb = 8
    g = synth.rng(4, 1)
    go = synth.normal_bf16(g, (T, d))
    do = synth.normal_bf16(g, (Kb, T, d), std)
    cd = torch.empty((Kb, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_INNER, None, None, bf16(do), bf16(go), dust.DUST_BF16, cd, Kb, T, d)
    ref = oracle.loss_delta_inner(bits_to_f64(do), bits_to_f64(go))
    assert frob_rel(host_f32(cd), ref) <= 1e-5


def test_w4_inner_scores_bench_launch():
    """The attention workload's inner-product scores in the bench's own launch: 512 draws at the
    full T x d (the kernel splits the draws 8 ways at this size). The 4.3-billion-element output
    change is built on the device by plain torch from a host block D [7, T, d]:
    delta_o[i][s] = D[i % 7][(s - i) mod T] (a per-draw roll, so every (draw, token) pair is
    distinct); sampled scores are checked against the oracle on the host copy of D."""
    announce("w4 inner scores, 512-draw launch")
    c = synth.WORKLOADS[4]
    T, d, std, Kb = c["T"], c["d"], c["delta_o_std"], 512
    g = synth.rng(4, 3)
    go = synth.normal_bf16(g, (T, d))
    D = synth.normal_bf16(g, (7, T, d), std)
    Dd = bf16(D)
    do = torch.empty((Kb, T, d), dtype=torch.bfloat16, device=DEV)
    for i in range(Kb):
        do[i] = torch.roll(Dd[i % 7], shifts=i, dims=0)
    del Dd
    cd = torch.full((Kb, T), float("nan"), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_INNER, None, None, do, bf16(go), dust.DUST_BF16, cd, Kb,
                         T, d)
    got = host_f32(cd)
    del do
    assert np.all(np.isfinite(got))
    rs = np.random.default_rng(406)
    k = np.concatenate([[0, Kb - 1, 7, 255], rs.integers(0, Kb, 60)])
    t = np.concatenate([[0, T - 1, 16383, 8192], rs.integers(0, T, 60)])
    ref = np.array([oracle.loss_delta_inner(bits_to_f64(D[i % 7][(s - i) % T])[None, None, :],
                                            bits_to_f64(go[s])[None, :])[0, 0]
                    for i, s in zip(k, t)])
    assert frob_rel(got[k, t], ref) <= 1e-5


def test_w4_scan():
    announce("w4 scan")
    c = synth.WORKLOADS[4]
    K, T, S, gamma = c["K"], c["T"], c["seg_len"], c["gamma"]
    cc = synth.normal_f32(synth.rng(4, 2), (K, T))
    r = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_reward_scan(f32(cc), r, K, T, S, gamma)
    rows = np.random.default_rng(405).choice(K, 48, replace=False)
    rows[0] = K - 1
    got = host_f32(r[torch.from_numpy(rows).to(DEV)])
    ref = oracle.reward_scan(cc[rows], S, gamma)
    assert frob_rel(got, ref) <= 1e-5


def test_w4_error_estimate():
    announce("w4 error estimate")
    c = synth.WORKLOADS[4]
    _check_error_estimate(4, c["K"], c["T"], c["d"])


def test_w4_weight_grad():
    announce("w4 weight grad")
    c = synth.WORKLOADS[4]
    _check_weight_grad(4, c["T"], c["d"], c["d"], 512)


def test_w4_attention_value_scores():
    """The attention workload scored through a re-run of the attention with perturbed values
    (8 heads of 64, bench.py --attention-values), at full size: all 16384 draws in one call as
    the benchmark times it, sampled outputs against the oracle."""
    announce("w4 attention value scores")
    c = synth.WORKLOADS[4]
    T, d, S, K, sigma = c["T"], c["d"], c["seg_len"], c["K"], c["sigma"]
    B, H = T // S, 8
    seed, tag = synth.noise_seed(4), synth.NOISE_TAG
    g = np.random.default_rng(404)
    z = g.standard_normal((B, H, S, S)).astype(np.float32)
    z[:, :, np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] = -np.inf
    z = np.exp(z - z.max(-1, keepdims=True))
    Pbits = rne_bf16_bits_of_f32((z / z.sum(-1, keepdims=True)).astype(np.float32))
    del z
    gbits = synth.normal_bf16(synth.rng(4, 1), (T, d))
    cd = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_attn_value_scores(bf16(Pbits), bf16(gbits), cd, K, B, H, S, d // H, 0, sigma, seed,
                                tag, 0, 0)
    got = host_f32(cd)
    s = np.random.default_rng(405)
    k, t = s.integers(0, K, 120), s.integers(0, T, 120)
    k[:3], t[:3] = [0, K - 1, K - 1], [0, T - 1, S - 1]
    ref = oracle.attn_value_scores_at(bits_to_f64(Pbits), bits_to_f64(gbits), k, t, sigma, seed, tag)
    assert frob_rel(got[k, t], ref) <= 1e-5


def test_w4_attention_key_scores():
    """The attention workload scored through a softmax re-run with perturbed keys (8 heads of
    64, softmax scale 1/8, bench.py --attention-keys), at full size: all 16384 draws in one call
    as the benchmark times it, sampled outputs against the oracle."""
    announce("w4 attention key scores")
    c = synth.WORKLOADS[4]
    T, d, S, K, sigma = c["T"], c["d"], c["seg_len"], c["K"], c["sigma"]
    B, H = T // S, 8
    tau = 1.0 / np.sqrt(d // H)
    seed, tag = synth.noise_seed(4), synth.NOISE_TAG
    g = np.random.default_rng(406)
    z = g.standard_normal((B, H, S, S)).astype(np.float32)
    z[:, :, np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] = -np.inf
    z = np.exp(z - z.max(-1, keepdims=True))
    Pbits = rne_bf16_bits_of_f32((z / z.sum(-1, keepdims=True)).astype(np.float32))
    del z
    qb, vb, gb = (synth.normal_bf16(synth.rng(4, j), (T, d)) for j in (3, 4, 1))
    cd = torch.empty((K, T), dtype=torch.float32, device=DEV)
    Pd = bf16(Pbits)
    W, Z = row_weights(Pd, bf16(vb), bf16(gb), B, H, S, d // H)
    dust.dust_attn_key_scores(Pd, bf16(qb), W, Z, cd, K, B, H, S, d // H, 0, sigma, tau, seed, tag,
                              0, 0)
    del W, Z
    got = host_f32(cd)
    s = np.random.default_rng(407)
    k, t = s.integers(0, K, 96), s.integers(0, T, 96)
    k[:3], t[:3] = [0, K - 1, K - 1], [0, T - 1, S - 1]
    ref = oracle.attn_key_scores_at(bits_to_f64(Pbits), bits_to_f64(qb), bits_to_f64(vb),
                                    bits_to_f64(gb), k, t, sigma, tau, seed, tag)
    assert frob_rel(got[k, t], ref) <= 1e-5


def test_w4_attention_query_scores():
    """The attention workload scored through a softmax re-run with perturbed queries (8 heads of
    64, softmax scale 1/8, bench.py --attention-queries), at full size: all 16384 draws in one
    call as the benchmark times it, sampled outputs against the oracle."""
    announce("w4 attention query scores")
    c = synth.WORKLOADS[4]
    T, d, S, K, sigma = c["T"], c["d"], c["seg_len"], c["K"], c["sigma"]
    B, H = T // S, 8
    tau = 1.0 / np.sqrt(d // H)
    seed, tag = synth.noise_seed(4), synth.NOISE_TAG
    g = np.random.default_rng(408)
    z = g.standard_normal((B, H, S, S)).astype(np.float32)
    z[:, :, np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] = -np.inf
    z = np.exp(z - z.max(-1, keepdims=True))
    Pbits = rne_bf16_bits_of_f32((z / z.sum(-1, keepdims=True)).astype(np.float32))
    del z
    kb, vb, gb = (synth.normal_bf16(synth.rng(4, j), (T, d)) for j in (4, 5, 1))
    cd = torch.empty((K, T), dtype=torch.float32, device=DEV)
    Pd = bf16(Pbits)
    W, Z = row_weights(Pd, bf16(vb), bf16(gb), B, H, S, d // H)
    dust.dust_attn_query_scores(Pd, bf16(kb), W, Z, cd, K, B, H, S, d // H, 0, sigma, tau, seed,
                                tag, 0, 0)
    del W, Z
    got = host_f32(cd)
    s = np.random.default_rng(409)
    k, t = s.integers(0, K, 96), s.integers(0, T, 96)
    k[:3], t[:3] = [0, K - 1, K - 1], [0, T - 1, S - 1]
    ref = oracle.attn_query_scores_at(bits_to_f64(Pbits), bits_to_f64(kb), bits_to_f64(vb),
                                      bits_to_f64(gb), k, t, sigma, tau, seed, tag)
    assert frob_rel(got[k, t], ref) <= 1e-5


# ------------------------------------------------------------------------------ workload 5
def test_w5_inject_block():
    announce("w5 inject block")
    _check_inject_block(5, "d_out")


def test_w5_loss_reward():
    announce("w5 loss -> reward")
    c = synth.WORKLOADS[5]
    K, T, S = c["K"], c["T"], c["seg_len"]
    lc, lp = synth.losses(synth.rng(5, 2), K, T)
    rf = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_reward(f32(lc), f32(lp), rf, K, T, S, c["gamma"])
    assert np.array_equal(host_f32(rf), oracle.loss_delta_loss(lc, lp).astype(np.float32))


def test_w5_error_estimate():
    announce("w5 error estimate")
    c = synth.WORKLOADS[5]
    _check_error_estimate(5, c["K"], c["T"], c["d_out"])


def test_w5_weight_grad():
    announce("w5 weight grad")
    c = synth.WORKLOADS[5]
    _check_weight_grad(5, c["T"], c["d_out"], c["d_in"], 128)


# ------------------------------------------------------------------------------ maximum sizes
@pytest.mark.parametrize("Kc,T,d", [
    (80, 16384, 4096),    # rows inside one block each: 5.4e9 output elements, 10.7 GB
    (1100, 16384, 256),   # several rows per block: 4.6e9 output elements, 9.2 GB
])
def test_inject_beyond_32_bit_element_offsets(Kc, T, d):
    """One call whose output has more than 2^32 elements, so element offsets, and not only byte
    offsets, leave 32 bits; sampled outputs include the very last element."""
    assert Kc * T * d > 1 << 32
    announce("inject beyond 32-bit offsets %s" % ((Kc, T, d),))
    seed, tag, sigma, draw0 = 0x1234_5678_9ABC, 9, 0.01, 7
    ybits = synth.normal_bf16(np.random.default_rng(31), (T, d))
    out = torch.empty((Kc, T, d), dtype=torch.bfloat16, device=DEV)
    dust.dust_noise_inject(bf16(ybits), out, dust.DUST_BF16, T, d, d, 0, Kc, sigma, seed, tag, draw0, 0)
    g = np.random.default_rng(32)
    k, t, j = g.integers(0, Kc, NS), g.integers(0, T, NS), g.integers(0, d, NS)
    k[:3], t[:3], j[:3] = [0, Kc - 1, Kc - 1], [0, T - 1, T - 1], [0, d - 1, 0]
    got = _gather_bits(out, k, t, j)
    del out
    n = oracle.normals_at(seed, tag, k, t, j, draw0=draw0)
    ref = oracle.round_bf16(bits_to_f64(ybits[t, j]) + sigma * n)
    gv = bits_to_f64(got)
    assert np.all(np.abs(gv - ref) <= bf16_ulp(ref))
    assert np.mean(gv != ref) < 0.01
