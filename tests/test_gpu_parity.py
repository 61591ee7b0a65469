"""GPU parity: every C-ABI entry point against the CPU oracle, element by element, at sizes that
span several tiles and ragged tails (MI355X only).

Tolerances (stated per test):
  * Philox words and indexing: bit-exact.
  * Normals: |n_gpu - n_oracle| <= 2.5e-6 (fp32 Box-Muller with the hardware log2 / sqrt / sin /
    cos, measured <= 1 ulp, <= 1 ulp, <= 1.3e-7 abs on this part, and one multiply by
    sqrt(2 ln 2): relative error <= 4 ulp plus 1.3e-7 rho absolute, <= 2.1e-6 at the largest
    radius 5.77).
  * Perturbed outputs: fp32 within 2^-23 |y'| + 3e-6 sigma; bf16 within one bf16 ulp of the
    oracle's nearest-even rounding of the fp64 value.
  * Loss mode of the loss change: bit-exact (one correctly rounded fp32 subtraction).
  * Inner mode, reward scan, error estimate: relative Frobenius error <= 1e-5.
  * Weight gradient on identical bf16 inputs: relative Frobenius error <= 1e-5 (fp32 MFMA
    accumulation over the token axis).
  * Chunk cross-entropy: |l_gpu - l_oracle| <= 1e-4 per token.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DEV, announce, bf16, bf16_ulp, bits_to_f64, dust, f32, frob_rel,
                         host_bf16_bits, host_f32, i32, rne_bf16_bits_of_f32)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------ generator
@pytest.mark.parametrize("Kc,T,G,group0,seed,tag,draw0,tok0", [
    (3, 37, 70, 0, 1, 0, 0, 0),
    (2, 5, 300, 123456, 0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, 4294967290, 4294967000),
    (1, 1, 1, 0, 0, 0, 0, 0),
    (4, 3, 257, 7, 0x0D057002, 1, 60, 16380),
])
def test_noise_words_bit_exact(Kc, T, G, group0, seed, tag, draw0, tok0):
    announce("noise_words %s" % ((Kc, T, G, group0, seed, tag, draw0, tok0),))
    w = torch.zeros((Kc, T, G, 4), dtype=torch.int32, device=DEV)
    dust.dust_noise_words(w, Kc, T, G, group0, seed, tag, draw0, tok0)
    got = host_f32(w.view(torch.float32)).view(np.uint32)
    ref = np.array([[[oracle.noise_words(seed, tag, draw0 + k, tok0 + t, group0 + g)
                      for g in range(G)] for t in range(T)] for k in range(Kc)], dtype=np.uint32)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("T,d,ld,chan0,Kc,draw0,tok0", [
    (29, 72, 72, 8, 3, 5, 100),      # vector path
    (31, 70, 75, 0, 2, 0, 0),        # ragged channel group, leading dimension > d
    (300, 1028, 1028, 4, 2, 9, 7),   # rows spanning several blocks
])
def test_normals_through_f32_inject(T, d, ld, chan0, Kc, draw0, tok0):
    announce("inject f32 normals %s" % ((T, d, ld, chan0, Kc, draw0, tok0),))
    seed, tag = 0xABCDEF0123, 3
    y = torch.zeros((T, ld), dtype=torch.float32, device=DEV)
    out = torch.full((Kc, T, d), float("nan"), dtype=torch.float32, device=DEV)
    dust.dust_noise_inject(y, out, dust.DUST_F32, T, d, ld, chan0, Kc, 1.0, seed, tag, draw0, tok0)
    ref = oracle.normals(seed, tag, draw0, tok0, chan0, Kc, T, d)
    got = host_f32(out)
    assert np.abs(got - ref).max() <= 2.5e-6


@pytest.mark.parametrize("T,d,ld,chan0,Kc", [
    (33, 72, 72, 8, 4), (17, 70, 80, 0, 3), (5, 1, 1, 0, 2),
    # <= 4 draws with many threads: each thread walks 4 adjacent tokens (ragged last slot),
    # with several tokens per block (d = 256) and several blocks per token (d = 4096)
    (4099, 256, 256, 0, 3), (301, 4096, 4096, 16, 2),
])
def test_inject_f32_and_bf16(T, d, ld, chan0, Kc):
    announce("inject f32/bf16 %s" % ((T, d, ld, chan0, Kc),))
    g = np.random.default_rng(20)
    seed, tag, sigma, draw0, tok0 = 77, 1, 0.01, 3, 11
    # fp32
    y32 = g.standard_normal((T, ld)).astype(np.float32)
    out = torch.empty((Kc, T, d), dtype=torch.float32, device=DEV)
    dust.dust_noise_inject(f32(y32), out, dust.DUST_F32, T, d, ld, chan0, Kc, sigma, seed, tag, draw0, tok0)
    ref = oracle.noise_inject(y32, sigma, Kc, seed, tag, draw0, tok0, chan0, d=d)
    got = host_f32(out)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 3e-6 * sigma)
    # bf16
    ybits = (g.standard_normal((T, ld)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    outb = torch.empty((Kc, T, d), dtype=torch.bfloat16, device=DEV)
    dust.dust_noise_inject(bf16(ybits), outb, dust.DUST_BF16, T, d, ld, chan0, Kc, sigma, seed, tag,
                           draw0, tok0)
    exact = oracle.noise_inject(bits_to_f64(ybits), sigma, Kc, seed, tag, draw0, tok0, chan0, d=d)
    refb = oracle.round_bf16(exact)
    gotb = bits_to_f64(host_bf16_bits(outb))
    assert np.all(np.abs(gotb - refb) <= bf16_ulp(refb))
    assert np.mean(gotb != refb) < 0.01


def test_inject_zero_sizes_touch_nothing():
    out = torch.full((4,), 7.0, device=DEV)
    dust.dust_noise_inject(out, out, dust.DUST_F32, 0, 4, 4, 0, 3, 0.1, 1, 1, 0, 0)
    dust.dust_noise_inject(out, out, dust.DUST_F32, 1, 4, 4, 0, 0, 0.1, 1, 1, 0, 0)
    assert torch.all(out == 7.0)


# ------------------------------------------------------------------------------ loss change
@pytest.mark.parametrize("Kc,T,inplace", [(5, 1003, False), (4, 1024, False), (3, 4096, True)])
def test_loss_delta_loss_bit_exact(Kc, T, inplace):
    announce("loss_delta LOSS %s" % ((Kc, T, inplace),))
    g = np.random.default_rng(21)
    lc = (8 + g.standard_normal(T)).astype(np.float32)
    lp = (lc[None] - 0.01 * g.standard_normal((Kc, T))).astype(np.float32)
    lpt = f32(lp)
    c = lpt if inplace else torch.empty((Kc, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_LOSS, f32(lc), lpt, None, None, dust.DUST_F32, c, Kc, T, 0)
    ref = oracle.loss_delta_loss(lc, lp).astype(np.float32)   # exact difference, rounded once
    assert np.array_equal(host_f32(c), ref)


@pytest.mark.parametrize("dt,Kc,T,d", [
    ("bf16", 9, 37, 512), ("bf16", 6, 21, 1000), ("bf16", 5, 13, 100), ("bf16", 3, 9, 5000),
    ("f32", 9, 37, 512), ("f32", 7, 11, 6), ("f32", 2, 5, 3000),
    # 4-token tiles: ragged last tile, fp32 rows, short rows, one token, draws split over waves
    ("f32", 5, 23, 256), ("bf16", 33, 7, 64), ("bf16", 1, 1, 8), ("bf16", 64, 37, 512),
    ("bf16", 100, 6, 504),
])
def test_loss_delta_inner(dt, Kc, T, d):
    announce("loss_delta INNER %s" % ((dt, Kc, T, d),))
    g = np.random.default_rng(22)
    do = (0.01 * g.standard_normal((Kc, T, d))).astype(np.float32)
    go = g.standard_normal((T, d)).astype(np.float32)
    if dt == "bf16":
        do_b = rne_bf16_bits_of_f32(do)
        go_b = rne_bf16_bits_of_f32(go)
        dev_do, dev_go, code = bf16(do_b), bf16(go_b), dust.DUST_BF16
        do64, go64 = bits_to_f64(do_b), bits_to_f64(go_b)
    else:
        dev_do, dev_go, code = f32(do), f32(go), dust.DUST_F32
        do64, go64 = do.astype(np.float64), go.astype(np.float64)
    c = torch.empty((Kc, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_INNER, None, None, dev_do, dev_go, code, c, Kc, T, d)
    ref = oracle.loss_delta_inner(do64, go64)
    assert frob_rel(host_f32(c), ref) <= 1e-5


# ------------------------------------------------------------------------------ reward scan
SCAN_CASES = [(3, 4096, 1024), (5, 300, 100), (2, 201, 67), (1, 5000, 5000), (4, 64, 1), (2, 96, 32)]


@pytest.mark.parametrize("K,T,S", SCAN_CASES)
@pytest.mark.parametrize("gamma", [0.0, 0.5, 0.9, 0.99, 1.0])
def test_reward_scan(K, T, S, gamma):
    announce("reward_scan %s" % ((K, T, S, gamma),))
    c = np.random.default_rng(23).standard_normal((K, T)).astype(np.float32)
    r = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_reward_scan(f32(c), r, K, T, S, gamma)
    got = host_f32(r)
    ref = oracle.reward_scan(c, S, gamma)
    if gamma == 0.0:
        assert np.array_equal(got, c)      # gamma = 0 keeps each token's own score, exactly
    assert frob_rel(got, ref) <= 1e-5
    bound = oracle.reward_scan(np.abs(c), S, gamma)   # sum_s gamma^(s-t) |c_s|
    assert np.all(np.abs(got - ref) <= 1e-5 * bound + 1e-30)


# more (draw, sequence) units than the chip keeps waves resident: every wave walks several units
# (whole sequences in registers, or streamed chunk by chunk past 4 chunks), in place or not
MANY_UNITS = [(6000, 64, 32), (9000, 1300, 1300), (20000, 67, 67), (700, 16384, 1024)]


@pytest.mark.parametrize("K,T,S", MANY_UNITS)
@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_reward_scan_many_units_per_wave(K, T, S, gamma):
    announce("reward_scan many units %s" % ((K, T, S, gamma),))
    g = np.random.default_rng(27)
    c = g.standard_normal((K, T)).astype(np.float32)
    r = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_reward_scan(f32(c), r, K, T, S, gamma)
    got = host_f32(r)
    ref = oracle.reward_scan(c, S, gamma)
    if gamma == 0.0:
        assert np.array_equal(got, c)
    assert frob_rel(got, ref) <= 1e-5
    bound = oracle.reward_scan(np.abs(c), S, gamma)
    assert np.all(np.abs(got - ref) <= 1e-5 * bound + 1e-30)
    lc = g.standard_normal(T).astype(np.float32)
    buf = f32(c)
    dust.dust_loss_reward(f32(lc), buf, buf, K, T, S, gamma)   # fused, in place
    ref_f = oracle.reward_scan(oracle.loss_delta_loss(lc, c), S, gamma)
    assert frob_rel(host_f32(buf), ref_f) <= 1e-5


def test_reward_scan_in_place():
    announce("reward_scan in place")
    K, T, S, gamma = 3, 2048, 1024, 0.99
    c = np.random.default_rng(24).standard_normal((K, T)).astype(np.float32)
    buf = f32(c)
    dust.dust_reward_scan(buf, buf, K, T, S, gamma)
    assert frob_rel(host_f32(buf), oracle.reward_scan(c, S, gamma)) <= 1e-5


# ------------------------------------------------------------------------------ fused loss -> reward
@pytest.mark.parametrize("K,T,S", SCAN_CASES)
@pytest.mark.parametrize("gamma", [0.0, 0.9, 1.0])
def test_loss_reward(K, T, S, gamma):
    announce("loss_reward %s" % ((K, T, S, gamma),))
    g = np.random.default_rng(25)
    lc = g.standard_normal(T).astype(np.float32)
    lp = (lc + 0.01 * g.standard_normal((K, T))).astype(np.float32)
    r = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_reward(f32(lc), f32(lp), r, K, T, S, gamma)
    got = host_f32(r)
    c = oracle.loss_delta_loss(lc, lp)
    ref = oracle.reward_scan(c, S, gamma)
    assert frob_rel(got, ref) <= 1e-5
    bound = oracle.reward_scan(np.abs(c), S, gamma)
    assert np.all(np.abs(got - ref) <= 1e-5 * bound + 1e-30)
    # the two-kernel path gives the same bits
    c2 = torch.empty((K, T), dtype=torch.float32, device=DEV)
    r2 = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_LOSS, f32(lc), f32(lp), None, None, dust.DUST_F32, c2, K, T, 0)
    dust.dust_reward_scan(c2, r2, K, T, S, gamma)
    assert np.array_equal(got, host_f32(r2))


def test_loss_reward_in_place_and_unaligned():
    announce("loss_reward in place / unaligned")
    K, T, S, gamma = 3, 2048, 1024, 0.99
    g = np.random.default_rng(26)
    lc = g.standard_normal(T).astype(np.float32)
    lp = g.standard_normal((K, T)).astype(np.float32)
    ref = oracle.reward_scan(oracle.loss_delta_loss(lc, lp), S, gamma)
    buf = f32(lp)
    dust.dust_loss_reward(f32(lc), buf, buf, K, T, S, gamma)
    assert frob_rel(host_f32(buf), ref) <= 1e-5
    # loss_clean one element off a 16-byte boundary: the scalar path
    lcs = torch.zeros(T + 1, dtype=torch.float32, device=DEV)
    lcs[1:] = f32(lc)
    r = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_reward(lcs[1:], f32(lp), r, K, T, S, gamma)
    assert frob_rel(host_f32(r), ref) <= 1e-5


# ------------------------------------------------------------------------------ error estimate
@pytest.mark.parametrize("K,K_total,T,d,chan0,draw0,tok0", [
    (37, 100, 50, 300, 16, 7, 3),     # ragged token tile and channel tile, vector path
    (5, 5, 19, 6, 0, 0, 0),           # d not a multiple of 4: scalar path
    (64, 64, 256, 2048, 0, 0, 0),     # full 256-channel tiles
])
def test_error_estimate(K, K_total, T, d, chan0, draw0, tok0):
    announce("error_estimate %s" % ((K, K_total, T, d, chan0, draw0, tok0),))
    seed, tag, sigma = 0x5EED, 2, 0.01
    r = np.random.default_rng(25).standard_normal((K, T)).astype(np.float32) * 1e-3
    gh = torch.full((T, d), float("nan"), dtype=torch.float32, device=DEV)
    gt = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(f32(r), gh, gt, K, K_total, T, d, chan0, sigma, seed, tag, draw0, tok0, 0)
    ref = oracle.error_estimate(r, d, sigma, seed, tag, draw0, tok0, chan0, K_total)
    got = host_f32(gh)
    assert frob_rel(got, ref) <= 1e-5
    # the transpose is the nearest-even bf16 of the kernel's own fp32 result
    assert np.array_equal(host_bf16_bits(gt), rne_bf16_bits_of_f32(got.T))


def test_error_estimate_accumulates_draw_chunks():
    announce("error_estimate accumulate")
    K, T, d, sigma, seed, tag = 40, 33, 260, 0.02, 9, 4
    r = np.random.default_rng(26).standard_normal((K, T)).astype(np.float32)
    gh = torch.empty((T, d), dtype=torch.float32, device=DEV)
    gt = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
    rd = f32(r)
    dust.dust_error_estimate(rd[:15], gh, None, 15, K, T, d, 0, sigma, seed, tag, 0, 0, 0)
    dust.dust_error_estimate(rd[15:], gh, gt, 25, K, T, d, 0, sigma, seed, tag, 15, 0, 1)
    ref = oracle.error_estimate(r, d, sigma, seed, tag, K_total=K)
    got = host_f32(gh)
    assert frob_rel(got, ref) <= 1e-5
    assert np.array_equal(host_bf16_bits(gt), rne_bf16_bits_of_f32(got.T))


@pytest.mark.parametrize("T,d", [(131072, 64), (65536, 64)])   # 16- and 8-token tiles
def test_error_estimate_wide_token_tiles(T, d):
    announce("error_estimate tiles %s" % ((T, d),))
    K, sigma, seed, tag = 6, 0.01, 31, 1
    g = np.random.default_rng(27)
    r = g.standard_normal((K, T)).astype(np.float32)
    gh = torch.empty((T, d), dtype=torch.float32, device=DEV)
    gt = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(f32(r), gh, gt, K, K, T, d, 0, sigma, seed, tag, 0, 0, 0)
    got = host_f32(gh)
    tok = np.concatenate([g.integers(0, T, 3000), [0, T - 1]])
    ch = np.concatenate([g.integers(0, d, 3000), [0, d - 1]])
    ref = oracle.error_estimate_at(r, tok, ch, sigma, seed, tag)
    assert frob_rel(got[tok, ch], ref) <= 1e-5
    gtb = host_bf16_bits(gt)
    assert np.array_equal(gtb[ch, tok], rne_bf16_bits_of_f32(got[tok, ch]))


def test_error_estimate_zero_draws_writes_zero():
    T, d = 10, 12
    gh = torch.full((T, d), 3.0, device=DEV)
    gt = torch.full((d, T), 3.0, dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(None, gh, gt, 0, 1, T, d, 0, 0.1, 1, 1, 0, 0, 0)
    assert torch.all(gh == 0) and torch.all(gt == 0)


# ------------------------------------------------------------------------------ weight gradient
@pytest.mark.parametrize("T,d_out,d_in", [
    (1024, 256, 256),    # split over tokens
    (4096, 200, 136),    # ragged output tiles
    (512, 128, 128),     # one tile, one split
    (1000, 64, 64),      # T not a multiple of the 64-token step
    (1001, 33, 17),      # plain path (T, d_in not multiples of 8)
    (64, 1, 8),
    (1024, 1024, 512),   # large-tile path, whole tiles, 4 splits
    (1056, 1040, 520),   # large-tile path, ragged row and column tiles, last split shorter
    (32, 2048, 512),     # large-tile path, one 32-token step, one split
    (4096, 520, 1016),   # large-tile path, N not a multiple of 16
])
def test_weight_grad(T, d_out, d_in):
    announce("weight_grad %s" % ((T, d_out, d_in),))
    g = np.random.default_rng(28)
    a = rne_bf16_bits_of_f32(g.standard_normal((d_out, T)).astype(np.float32))
    b = rne_bf16_bits_of_f32(g.standard_normal((T, d_in)).astype(np.float32))
    G = torch.full((d_out, d_in), float("nan"), dtype=torch.float32, device=DEV)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    dust.dust_weight_grad(bf16(a), bf16(b), G, T, d_out, d_in, ws, ws_bytes)
    got = host_f32(G)
    ref = oracle.weight_grad(bits_to_f64(a).T, bits_to_f64(b))
    assert frob_rel(got, ref) <= 1e-5
    # deterministic: the split partial sums are added in a fixed order
    G2 = torch.empty_like(G)
    dust.dust_weight_grad(bf16(a), bf16(b), G2, T, d_out, d_in, ws, ws_bytes)
    assert torch.equal(G, G2)


def test_weight_grad_short_workspace_is_rejected():
    T, d_out, d_in = 1024, 256, 256
    need = dust.dust_weight_grad_workspace(T, d_out, d_in)
    assert need > 0
    z = torch.zeros(8, dtype=torch.uint8, device=DEV)
    with pytest.raises(dust.DustError) as e:
        dust.dust_weight_grad(z, z, z, T, d_out, d_in, z, need - 1)
    assert e.value.status == dust.DUST_ERR_WORKSPACE


def test_weight_grad_zero_tokens_writes_zero():
    G = torch.full((5, 8), 1.0, device=DEV)
    dust.dust_weight_grad(None, None, G, 0, 5, 8, None, 0)
    assert torch.all(G == 0)


# ------------------------------------------------------------------------------ scores folded into the estimate
@pytest.mark.parametrize("K,T,d,chan0,draw0,tok0", [
    (5, 96, 256, 0, 0, 0),
    (7, 37, 70, 8, 3, 11),        # ragged token tile and channel group
    (33, 4096, 512, 4, 100, 0),   # several channel tiles, 8-token tiles
])
def test_error_estimate_losses_equals_loss_delta_then_estimate(K, T, d, chan0, draw0, tok0):
    announce("error_estimate_losses %s" % ((K, T, d, chan0, draw0, tok0),))
    g = np.random.default_rng(33)
    seed, tag, sigma = 0x5EED, 2, 0.05
    lc = (8.0 + g.standard_normal(T)).astype(np.float32)
    lp = (lc + 0.05 * g.standard_normal((K, T))).astype(np.float32)
    c = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_delta(dust.DUST_DELTA_LOSS, f32(lc), f32(lp), None, None, dust.DUST_F32, c, K, T, 0)
    g1 = torch.empty((T, d), device=DEV)
    t1 = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(c, g1, t1, K, 2 * K, T, d, chan0, sigma, seed, tag, draw0, tok0, 0)
    g2 = torch.full((T, d), float("nan"), device=DEV)
    t2 = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate_losses(f32(lc), f32(lp), g2, t2, K, 2 * K, T, d, chan0, sigma, seed,
                                    tag, draw0, tok0, 0)
    assert torch.equal(g1, g2) and torch.equal(t1.view(torch.int16), t2.view(torch.int16))
    # a second block of draws accumulated, as with chunked populations
    dust.dust_error_estimate_losses(f32(lc), f32(lp), g2, None, K, 2 * K, T, d, chan0, sigma, seed,
                                    tag, draw0 + K, tok0, 1)
    # the second block's draws draw0 + K .. reuse the same losses
    ref = (oracle.error_estimate(oracle.loss_delta_loss(lc, lp), d, sigma, seed, tag, draw0=draw0,
                                 tok0=tok0, chan0=chan0, K_total=2 * K)
           + oracle.error_estimate(oracle.loss_delta_loss(lc, lp), d, sigma, seed, tag,
                                   draw0=draw0 + K, tok0=tok0, chan0=chan0, K_total=2 * K))
    assert frob_rel(host_f32(g2), ref) <= 1e-5


# ------------------------------------------------------------------------------ LM-head chunk
@pytest.mark.parametrize("T,V,v0,C,Kc", [
    (37, 1000, 200, 300, 5),
    (16, 4096, 0, 1024, 3),
    (9, 64, 60, 4, 4),
    (5, 5000, 0, 4096, 2),
    (11, 300, 100, 130, 3),    # ragged last channel group
    (13, 700, 64, 256, 37),    # draws in batches of 16: two whole batches and a ragged one
    (6, 512, 0, 512, 16),      # exactly one whole batch
])
def test_head_ce_chunk(T, V, v0, C, Kc):
    announce("head_ce_chunk %s" % ((T, V, v0, C, Kc),))
    g = np.random.default_rng(29)
    seed, tag, sigma, draw0, tok0 = 4242, 7, 0.3, 2, 5
    z = (g.standard_normal((T, V)) * np.sqrt(2)).astype(np.float32)
    tgt = g.integers(0, V, T).astype(np.int32)
    tgt[0] = v0
    tgt[1] = v0 + C - 1
    tgt[2] = (v0 + C) % V
    lp = torch.full((Kc, T), float("nan"), device=DEV)
    lc = torch.full((T,), float("nan"), device=DEV)
    dust.dust_head_ce_chunk(f32(z), i32(tgt), lp, lc, T, V, v0, C, Kc, sigma, seed, tag, draw0, tok0)
    ref_p, ref_c = oracle.head_ce_chunk(z, tgt, v0, C, Kc, sigma, seed, tag, draw0, tok0)
    assert np.abs(host_f32(lp) - ref_p).max() <= 1e-4
    assert np.abs(host_f32(lc) - ref_c).max() <= 1e-4


@pytest.mark.parametrize("V,v0,C", [(700, 256, 256), (300, 0, 100)])
def test_head_ce_chunk_masked_logits(V, v0, C):
    """Masked vocabulary entries (logit -inf) outside the chunk, at the lowest ids so that a lane
    meets them before any finite logit, and inside the chunk: they contribute nothing to the
    log-sum-exp, as in the oracle."""
    announce("head_ce_chunk masked %s" % ((V, v0, C),))
    g = np.random.default_rng(31)
    T, Kc, seed, tag, sigma = 9, 20, 77, 3, 0.3
    z = (g.standard_normal((T, V)) * np.sqrt(2)).astype(np.float32)
    z[:, :200 if v0 >= 200 else 0] = -np.inf          # every lane's first logits, out of chunk
    z[1:, v0 + C:v0 + C + 70] = -np.inf                # a run after the chunk
    z[2, v0 + 5:v0 + 9] = -np.inf                      # inside the chunk
    z[3, :] = -np.inf
    z[3, v0 + 3] = 1.5                                 # one finite logit, inside the chunk
    tgt = g.integers(v0, v0 + C, T).astype(np.int32)
    tgt[2] = v0 + 10
    tgt[3] = v0 + 3
    tgt[4] = v0 + C + 80 if v0 + C + 80 < V else 0    # a finite target outside the chunk
    lp = torch.full((Kc, T), float("nan"), device=DEV)
    lc = torch.full((T,), float("nan"), device=DEV)
    dust.dust_head_ce_chunk(f32(z), i32(tgt), lp, lc, T, V, v0, C, Kc, sigma, seed, tag, 0, 0)
    ref_p, ref_c = oracle.head_ce_chunk(z, tgt, v0, C, Kc, sigma, seed, tag, 0, 0)
    assert np.all(np.isfinite(ref_p)) and np.all(np.isfinite(ref_c))
    assert np.abs(host_f32(lp) - ref_p).max() <= 1e-4
    assert np.abs(host_f32(lc) - ref_c).max() <= 1e-4


def test_head_ce_bad_target_gives_nan():
    T, V = 4, 64
    z = np.zeros((T, V), dtype=np.float32)
    tgt = np.array([0, -1, 64, 3], dtype=np.int32)
    lp = torch.zeros((2, T), device=DEV)
    dust.dust_head_ce_chunk(f32(z), i32(tgt), lp, None, T, V, 0, 16, 2, 0.1, 1, 1, 0, 0)
    got = host_f32(lp)
    assert np.all(np.isfinite(got[:, [0, 3]])) and np.all(np.isnan(got[:, [1, 2]]))


# ------------------------------------------------------------------------------ determinism
def test_noise_kernels_are_deterministic():
    announce("determinism")
    T, d, K = 512, 1024, 8
    y = torch.randn((T, d), device=DEV).to(torch.bfloat16)
    a = torch.empty((K, T, d), dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    dust.dust_noise_inject(y, a, dust.DUST_BF16, T, d, d, 0, K, 0.01, 5, 1, 0, 0)
    dust.dust_noise_inject(y, b, dust.DUST_BF16, T, d, d, 0, K, 0.01, 5, 1, 0, 0)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    r = torch.randn((K, T), device=DEV)
    g1 = torch.empty((T, d), device=DEV)
    g2 = torch.empty((T, d), device=DEV)
    dust.dust_error_estimate(r, g1, None, K, K, T, d, 0, 0.01, 5, 1, 0, 0, 0)
    dust.dust_error_estimate(r, g2, None, K, K, T, d, 0, 0.01, 5, 1, 0, 0, 0)
    assert torch.equal(g1, g2)
