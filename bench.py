#!/usr/bin/env python3
"""Throughput of the Dust estimator chain on one MI355X.

One step = one whole estimate, with every input resident in HBM before the timed region. The
default workload is the largest one that fits one GPU: the MLP up-projection 1024 -> 4096 of the
~240M-parameter GPT shape (T = 16 x 1024 tokens, K = 1024 draws, gamma = 0, sigma = 0.01):
    dust_noise_inject   (32 calls of 32 draws, [32, 16384, 4096] bf16 perturbed outputs each)
    dust_loss_reward    (loss change and reward scan in one pass, [1024, 16384]; --unfused runs
                         dust_loss_delta and dust_reward_scan instead)
    dust_error_estimate (g_hat [16384, 4096] fp32 + its bf16 transpose)
    dust_weight_grad    (G_W [4096, 1024], bf16 matrix cores)
The perturbed forward of the rest of the model, between the perturbation and the loss change,
is not part of the estimator; its per-token losses are synthetic inputs here.
--workload 2 / 3 / 4 time the MLP up-projection 512 -> 2048 (K = 64), the LM-head chunk and the
attention k/v inner-product chains the same way. With --workload 4, --attention-values,
--attention-keys or --attention-queries scores the draws by re-running the attention with
perturbed values, keys or queries (dust_attn_value_scores / _key_scores / _query_scores; keys and
queries after dust_attn_row_weights, once per step) instead of streaming a synthetic
attention-output change.

Metric: draws x tokens per second (K * T / step time). Prints one JSON line with the per-kernel
HIP-event durations measured inside the timed region, the roofline of the dominant kernel, and
the CPU oracle's throughput on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 30] [--workload 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "Dust estimator draws·tokens/sec on 1 GPU + % of HBM/MFMA roofline"
UNIT = "draws·tokens/s"
# What the path computes in: bf16 activations, perturbed outputs and matrix-core operands (the
# weight-gradient contraction runs on the bf16 matrix cores), fp32 noise, scores, rewards,
# output error and every accumulation; the generator itself is 32-bit integer arithmetic.
DTYPE = "bf16 storage and MFMA operands, fp32 accumulate"

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# Vector ALU issue rate: 256 CUs x 64 lanes x 2.4 GHz = 39.32e12 lane-operations per second.
# This is the roof of the noise generator's instruction mix (64-bit integer multiplies, bit
# operations, transcendentals), which issues one wave64 instruction per SIMD every 4 cycles.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# fp32 multiply-adds from two or more waves per SIMD issue twice as fast: the published fp32
# vector peak, 157.3 TFLOP/s = 78.6e12 fma lane-operations per second. It is the roof of
# fp32-dominated vector work (the key scores' e^x - 1 and weighted sums).
FP32_VALU_PEAK_TOPS = 2 * VALU_PEAK_TOPS

# Algorithmic vector operations per generated standard normal (one issue slot each).
# Philox4x32-10: a round is 2 32x32->64 multiplies (v_mad_u64_u32) + 2 three-input XORs
# (v_bitop3_b32). Of the counter (channel group, token, draw, tag), the channel group and tag
# are fixed per lane and token and draw are uniform across the wave, so the first round and half
# of the second run once per lane or on the scalar unit, not per draw: 2 + 8 x 4 = 34 operations
# per 4 words -> 8.5 per normal. Box-Muller per pair, in polar form: funnel shift + subtract for
# the radius uniform, one funnel shift for the angle (in turns, the whole turn is free), log2,
# sqrt of the negated log, cos, sin = 7 -> 3.5 per normal. The consumer multiplies the radius by
# its own coefficient (which carries sqrt(2 ln 2)) once per pair and applies it to cos and sin.
OPS_PER_NORMAL = 8.5 + 3.5
OPS_INJECT_EXTRA = 2.0    # half the coefficient x radius multiply, fma with y, half a bf16 pack
OPS_EE_EXTRA = 1.5        # half the reward x radius multiply, fma into the accumulator
OPS_HEAD_EXTRA = 3.5      # half the coefficient x radius multiply, multiply, exp2, fma
# Key scores, per (draw, head, query, key <= query): e^x - 1 of the logit shift (x + x^2 q(x),
# q a quadratic: 3 fma + 1 multiply) and the two weighted sums N1, N0 (2 fma).
OPS_KEY_SCORE = 6.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the shader clock takes tens of milliseconds under load to settle; 30 untimed steps put the
    # timed ones in steady state (about +1 % against 3 on the headline workload)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=5, choices=(2, 3, 4, 5))
    ap.add_argument("--draw-block", type=int, default=0,
                    help="draws per perturbation call of workloads 2 and 5 (a divisor of K; "
                         "default: the workload's own block)")
    ap.add_argument("--cpu-scale", type=float, default=1.0,
                    help="scale of the CPU oracle's sample (1.0 = about 10-30 s on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of an estimate, measure the denominators the design notes read "
                         "fractions against: a 1 GiB device copy (GB/s), the library's noise "
                         "generator alone (normals/s) and back-to-back bf16 MFMAs on random "
                         "operands (TFLOP/s); prints one JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--optimizer", choices=("none", "sgd", "adam"), default="none",
                    help="also apply the estimate to synthetic fp32 weights each step: SGD with "
                         "momentum or Adam (not part of the estimate; off by default)")
    ap.add_argument("--attention-values", action="store_true",
                    help="workload 4: score by re-running the attention with perturbed values "
                         "(dust_attn_value_scores on synthetic attention weights, 8 heads of 64) "
                         "instead of streaming a synthetic attention-output change")
    ap.add_argument("--attention-keys", action="store_true",
                    help="workload 4: score by re-running the softmax with perturbed keys "
                         "(dust_attn_key_scores on synthetic queries, keys and values, 8 heads of "
                         "64) instead of streaming a synthetic attention-output change")
    ap.add_argument("--attention-queries", action="store_true",
                    help="workload 4: score by re-running the softmax with perturbed queries "
                         "(dust_attn_query_scores on synthetic queries, keys and values, 8 heads "
                         "of 64) instead of streaming a synthetic attention-output change")
    ap.add_argument("--downstream", choices=("none", "fused", "unfused"), default="none",
                    help="workloads 2 and 5: also run the first operation of the perturbed "
                         "forward, the down-projection of the activated perturbed outputs "
                         "(GELU, then [d_in x d_out]): 'fused' with dust_perturbed_linear "
                         "(noise regenerated in the matrix-core operand path, y' never written), "
                         "'unfused' as dust_noise_inject + torch GELU + torch matmul")
    ap.add_argument("--fold", action="store_true",
                    help="loss-scored workloads with gamma = 0 (2, 3, 5): form the scores inside "
                         "the error estimate (dust_error_estimate_losses) instead of running "
                         "dust_loss_reward first")
    ap.add_argument("--unfused", action="store_true",
                    help="loss mode: run the loss change and the reward scan as two kernels "
                         "instead of dust_loss_reward")
    return ap.parse_args()


def _alu(normals, extra):
    return ("alu", normals * (OPS_PER_NORMAL + extra), 1e12, VALU_PEAK_TOPS, "Tops/s", normals)


def _hbm(nbytes):
    return ("hbm", float(nbytes), 1e9, HBM_PEAK_GBS, "GB/s")


def _mfma(flops):
    return ("mfma", float(flops), 1e12, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s")


class Chain:
    """Device buffers, one step of the estimator, the work model per kernel, and the oracle
    sample of one workload."""

    def __init__(self, cfg_id, dust, torch, dev):
        self.cfg_id, self.dust, self.torch, self.dev = cfg_id, dust, torch, dev
        self.c = synth.WORKLOADS[cfg_id]
        self.seed, self.tag = synth.noise_seed(cfg_id), synth.NOISE_TAG
        self.fused = True   # loss mode: scores and rewards in one pass (dust_loss_reward)
        self.fold = False   # gamma = 0: scores formed inside the error estimate
        self.draw_block = 0  # draws per perturbation call (0: the workload's own)

    # ---- optional optimizer step on the estimate (dust_sgd_momentum / dust_adam)
    optimizer = "none"

    def opt_setup(self):
        if self.optimizer == "none":
            return
        n = self.G.numel()
        self.W = self.f32(synth.normal_f32(synth.rng(self.cfg_id, 7), (n,), 0.02))
        self.s1 = self.torch.zeros(n, dtype=self.torch.float32, device=self.dev)
        self.s2 = self.torch.zeros(n, dtype=self.torch.float32, device=self.dev)
        self.opt_t = 0

    def opt_step(self, run, sh):
        d, n = self.dust, self.G.numel()
        if self.optimizer == "sgd":
            run("dust_sgd_momentum", d.dust_sgd_momentum, self.W, self.G, self.s1, n, 0.01, 0.9, sh)
        elif self.optimizer == "adam":
            self.opt_t += 1
            run("dust_adam", d.dust_adam, self.W, self.G, self.s1, self.s2, n, 1e-3, 0.9, 0.999,
                1e-8, 0.0, self.opt_t, sh)

    def opt_model(self):
        n = self.G.numel()
        return {"dust_sgd_momentum": _hbm(20.0 * n), "dust_adam": _hbm(28.0 * n)}

    def serial_roofs(self):
        """Kernels whose matrix-core and vector work do not overlap on this part: the sum of
        their parts at the published peaks, ms per launch."""
        return {}

    def bf(self, bits):
        return self.torch.from_numpy(bits.view(np.int16)).to(self.dev).view(self.torch.bfloat16)

    def f32(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.dev)

    def empty(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.dev)


class LinearChain(Chain):
    """Workloads 2 and 5: perturb a linear layer's output, score by the loss change."""

    def setup(self):
        c, t = self.c, self.torch
        self.T, self.d_in, self.d_out, self.K = c["T"], c["d_in"], c["d_out"], c["K"]
        self.KB, self.S, self.gamma, self.sigma = c["inject_block"], c["seg_len"], c["gamma"], c["sigma"]
        if self.draw_block:
            if self.K % self.draw_block:
                raise SystemExit("--draw-block must divide K = %d" % self.K)
            self.KB = self.draw_block
        g = synth.rng(self.cfg_id, 1)
        self.ybits = synth.normal_bf16(g, (self.T, self.d_out))
        self.xbits = synth.normal_bf16(g, (self.T, self.d_in))
        self.lc_h, self.lp_h = synth.losses(synth.rng(self.cfg_id, 2), self.K, self.T)
        self.y, self.x = self.bf(self.ybits), self.bf(self.xbits)
        self.lc, self.lp = self.f32(self.lc_h), self.f32(self.lp_h)
        self.ybuf = self.empty((self.KB, self.T, self.d_out), t.bfloat16)
        self.cbuf = self.empty((self.K, self.T), t.float32)
        self.rbuf = self.empty((self.K, self.T), t.float32)
        self.gh = self.empty((self.T, self.d_out), t.float32)
        self.ght = self.empty((self.d_out, self.T), t.bfloat16)
        self.G = self.empty((self.d_out, self.d_in), t.float32)
        self.ws_bytes = self.dust.dust_weight_grad_workspace(self.T, self.d_out, self.d_in)
        self.ws = self.empty(max(self.ws_bytes, 16), t.uint8)
        if self.downstream != "none":
            # the next layer: the MLP down-projection [d_in, d_out], W ~ N(0, 1/d_out), bf16
            self.wnbits = synth.normal_bf16(synth.rng(self.cfg_id, 8), (self.d_in, self.d_out),
                                            1.0 / np.sqrt(self.d_out))
            self.wn = self.bf(self.wnbits)
            self.dbuf = self.empty((self.KB, self.T, self.d_in), t.bfloat16)

    downstream = "none"   # "none", "fused" or "unfused"

    def step(self, run, sh):
        d, T, K, KB, t = self.dust, self.T, self.K, self.KB, self.torch
        for blk in range(K // KB):
            if self.downstream == "fused":
                run("dust_perturbed_linear", d.dust_perturbed_linear, self.y, self.wn, self.dbuf,
                    d.DUST_BF16, d.DUST_ACT_GELU_TANH, T, self.d_out, self.d_in, 0, KB, self.sigma,
                    self.seed, self.tag, blk * KB, 0, sh)
                continue
            run("dust_noise_inject", d.dust_noise_inject, self.y, self.ybuf, d.DUST_BF16, T, self.d_out,
                self.d_out, 0, KB, self.sigma, self.seed, self.tag, blk * KB, 0, sh)
            if self.downstream == "unfused":
                run("torch_gelu_matmul", lambda: t.matmul(
                    t.nn.functional.gelu(self.ybuf, approximate="tanh"), self.wn.t(),
                    out=self.dbuf))
        if self.fold:
            run("dust_error_estimate_losses", d.dust_error_estimate_losses, self.lc, self.lp,
                self.gh, self.ght, K, K, T, self.d_out, 0, self.sigma, self.seed, self.tag, 0, 0,
                0, sh)
        else:
            if self.fused:
                run("dust_loss_reward", d.dust_loss_reward, self.lc, self.lp, self.rbuf, K, T,
                    self.S, self.gamma, sh)
            else:
                run("dust_loss_delta", d.dust_loss_delta, d.DUST_DELTA_LOSS, self.lc, self.lp,
                    None, None, d.DUST_F32, self.cbuf, K, T, 0, sh)
                run("dust_reward_scan", d.dust_reward_scan, self.cbuf, self.rbuf, K, T, self.S,
                    self.gamma, sh)
            run("dust_error_estimate", d.dust_error_estimate, self.rbuf, self.gh, self.ght, K, K,
                T, self.d_out, 0, self.sigma, self.seed, self.tag, 0, 0, 0, sh)
        run("dust_weight_grad", d.dust_weight_grad, self.ght, self.x, self.G, T, self.d_out, self.d_in,
            self.ws, self.ws_bytes, sh)

    def draws_tokens(self):
        return self.K * self.T

    def model(self):
        T, K, do = self.T, self.K, self.d_out
        return {
            "dust_noise_inject": _alu(self.KB * T * do, OPS_INJECT_EXTRA),
            "dust_loss_delta": _hbm((8.0 + 4.0 / K) * K * T),
            "dust_reward_scan": _hbm(8.0 * K * T),
            "dust_loss_reward": _hbm((8.0 + 4.0 / K) * K * T),
            "dust_error_estimate": _alu(K * T * do, OPS_EE_EXTRA),
            "dust_error_estimate_losses": _alu(K * T * do, OPS_EE_EXTRA),
            "dust_weight_grad": _mfma(2.0 * T * do * self.d_in),
            # the down-projection of the block's activated perturbed outputs
            "dust_perturbed_linear": _mfma(2.0 * self.KB * T * do * self.d_in),
            "torch_gelu_matmul": _mfma(2.0 * self.KB * T * do * self.d_in),
        }

    def config(self):
        cfg = {"workload": self.c["name"], "d_in": self.d_in, "d_out": self.d_out, "tokens": self.T,
               "seq_len": self.S, "draws": self.K, "gamma": self.gamma, "sigma": self.sigma,
               "inject_block": self.KB, "storage": "bf16 activations, fp32 rewards/g_hat/G_W"}
        if self.downstream != "none":
            cfg["workload"] += "_downstream_" + self.downstream
            cfg["downstream"] = ("GELU (tanh form) then the down-projection [%d x %d], bf16 out, "
                                 "%s" % (self.d_in, self.d_out,
                                         "dust_perturbed_linear" if self.downstream == "fused"
                                         else "dust_noise_inject + torch gelu + torch matmul"))
        return cfg

    def cpu_baseline(self, scale):
        """The oracle's chain (as it stands) on whole sequences with all K draws: several
        sequences at workload 2, one at workload 5 (a subset of the draws when scale < 1)."""
        import oracle
        S = self.S
        if self.cfg_id == 2:
            K_s, T_s = self.K, min(self.T, max(S, int(16 * S * scale) // S * S))
        else:
            K_s, T_s = min(self.K, max(4, int(1024 * scale) // 4 * 4)), S
        if self.downstream != "none":
            K_s = max(1, int(64 * scale))  # the product costs d_out d_in multiply-adds per token
        KB = min(self.KB, K_s)
        y = synth.bf16_bits_to_f32(self.ybits[:T_s]).astype(np.float64)
        x = synth.bf16_bits_to_f32(self.xbits[:T_s]).astype(np.float64)
        oracle.threads()
        t0 = time.perf_counter()
        for b in range(K_s // KB):
            if self.downstream != "none":
                oracle.perturbed_linear(y, synth.bf16_bits_to_f32(self.wnbits).astype(np.float64),
                                        KB, self.sigma, self.seed, self.tag, oracle.ACT_GELU_TANH,
                                        draw0=b * KB)
                continue
            oracle.noise_inject(y, self.sigma, KB, self.seed, self.tag, draw0=b * KB)
        r = oracle.reward_scan(oracle.loss_delta_loss(self.lc_h[:T_s], self.lp_h[:K_s, :T_s]), S, self.gamma)
        g = oracle.error_estimate(r, self.d_out, self.sigma, self.seed, self.tag, K_total=self.K)
        oracle.weight_grad(g, x)
        dt = time.perf_counter() - t0
        return {"value": K_s * T_s / dt, "unit": UNIT, "cores": oracle.threads(), "kind": "oracle",
                "sample": "%d of %d draws x first %d of %d tokens (%d whole sequences), whole chain "
                          "incl. %sthe full G_W contraction over those tokens; %.1f s"
                          % (K_s, self.K, T_s, self.T, T_s // S,
                             "the down-projection of the perturbed outputs and "
                             if self.downstream != "none" else "", dt)}


class HeadChain(Chain):
    """Workload 3: LM head perturbed on cached logits, one vocabulary chunk."""

    def setup(self):
        c, t = self.c, self.torch
        self.T, self.V, self.v0, self.C, self.K = c["T"], c["V"], c["v0"], c["C"], c["K"]
        self.H, self.S, self.gamma, self.sigma = c["hidden"], c["seg_len"], c["gamma"], c["sigma"]
        g = synth.rng(self.cfg_id, 1)
        self.z_h = synth.normal_f32(g, (self.T, self.V), np.sqrt(2.0))
        self.tgt_h = synth.targets(g, self.T, self.V)
        self.hbits = synth.normal_bf16(g, (self.T, self.H))
        self.z, self.h = self.f32(self.z_h), self.bf(self.hbits)
        self.tgt = self.torch.from_numpy(self.tgt_h).to(self.dev)
        self.lp = self.empty((self.K, self.T), t.float32)
        self.lc = self.empty((self.T,), t.float32)
        self.cbuf = self.empty((self.K, self.T), t.float32)
        self.gh = self.empty((self.T, self.C), t.float32)
        self.ght = self.empty((self.C, self.T), t.bfloat16)
        self.G = self.empty((self.C, self.H), t.float32)
        self.ws_bytes = self.dust.dust_weight_grad_workspace(self.T, self.C, self.H)
        self.ws = self.empty(max(self.ws_bytes, 16), t.uint8)

    def step(self, run, sh):
        d, T, K = self.dust, self.T, self.K
        run("dust_head_ce_chunk", d.dust_head_ce_chunk, self.z, self.tgt, self.lp, self.lc, T, self.V,
            self.v0, self.C, K, self.sigma, self.seed, self.tag, 0, 0, sh)
        if self.fold:
            run("dust_error_estimate_losses", d.dust_error_estimate_losses, self.lc, self.lp,
                self.gh, self.ght, K, K, T, self.C, self.v0, self.sigma, self.seed, self.tag, 0, 0,
                0, sh)
        else:
            if self.fused:
                run("dust_loss_reward", d.dust_loss_reward, self.lc, self.lp, self.cbuf, K, T,
                    self.S, self.gamma, sh)
            else:
                run("dust_loss_delta", d.dust_loss_delta, d.DUST_DELTA_LOSS, self.lc, self.lp,
                    None, None, d.DUST_F32, self.cbuf, K, T, 0, sh)
                run("dust_reward_scan", d.dust_reward_scan, self.cbuf, self.cbuf, K, T, self.S,
                    self.gamma, sh)
            run("dust_error_estimate", d.dust_error_estimate, self.cbuf, self.gh, self.ght, K, K,
                T, self.C, self.v0, self.sigma, self.seed, self.tag, 0, 0, 0, sh)
        run("dust_weight_grad", d.dust_weight_grad, self.ght, self.h, self.G, T, self.C, self.H,
            self.ws, self.ws_bytes, sh)

    def draws_tokens(self):
        return self.K * self.T

    def model(self):
        T, K, C = self.T, self.K, self.C
        return {
            "dust_head_ce_chunk": _alu(K * T * C, OPS_HEAD_EXTRA),
            "dust_loss_delta": _hbm((8.0 + 4.0 / K) * K * T),
            "dust_reward_scan": _hbm(8.0 * K * T),
            "dust_loss_reward": _hbm((8.0 + 4.0 / K) * K * T),
            "dust_error_estimate": _alu(K * T * C, OPS_EE_EXTRA),
            "dust_error_estimate_losses": _alu(K * T * C, OPS_EE_EXTRA),
            "dust_weight_grad": _mfma(2.0 * T * C * self.H),
        }

    def config(self):
        return {"workload": self.c["name"], "vocab": self.V, "chunk": [self.v0, self.v0 + self.C],
                "hidden": self.H, "tokens": self.T, "draws": self.K, "gamma": self.gamma,
                "sigma": self.sigma, "storage": "fp32 logits, bf16 hidden"}

    def cpu_baseline(self, scale):
        import oracle
        K_s, T_s = self.K, max(2, int(2048 * scale))
        oracle.threads()
        t0 = time.perf_counter()
        lp, lc = oracle.head_ce_chunk(self.z_h[:T_s], self.tgt_h[:T_s], self.v0, self.C, K_s,
                                      self.sigma, self.seed, self.tag)
        r = oracle.reward_scan(oracle.loss_delta_loss(lc, lp), T_s, self.gamma)
        g = oracle.error_estimate(r, self.C, self.sigma, self.seed, self.tag, chan0=self.v0)
        oracle.weight_grad(g, synth.bf16_bits_to_f32(self.hbits[:T_s]).astype(np.float64))
        dt = time.perf_counter() - t0
        return {"value": K_s * T_s / dt, "unit": UNIT, "cores": oracle.threads(), "kind": "oracle",
                "sample": "all %d draws x first %d of %d tokens, whole chain; %.1f s"
                          % (K_s, T_s, self.T, dt)}


class InnerChain(Chain):
    """Workload 4: attention k/v projection scored by inner products, gamma = 0.99."""

    def setup(self):
        c, t = self.c, self.torch
        self.T, self.d, self.K, self.KB = c["T"], c["d"], c["K"], c["draw_block"]
        self.S, self.gamma, self.sigma, self.std = c["seg_len"], c["gamma"], c["sigma"], c["delta_o_std"]
        g = synth.rng(self.cfg_id, 1)
        self.gobits = synth.normal_bf16(g, (self.T, self.d))
        self.xbits = synth.normal_bf16(g, (self.T, self.d))
        self.go, self.x = self.bf(self.gobits), self.bf(self.xbits)
        B, S, H = self.T // self.S, self.S, self.HEADS
        if self.attn_mode == "values":
            # attention weights of the clean forward: a causal softmax of N(0, 1) scores per
            # head and sequence, drawn on the device from a seeded generator before timing
            gen = t.Generator(device=self.dev).manual_seed(7000 + self.cfg_id)
            z = t.randn((B, H, S, S), generator=gen, device=self.dev)
            z.masked_fill_(~t.ones((S, S), dtype=t.bool, device=self.dev).tril(), float("-inf"))
            self.P = t.softmax(z, -1).to(t.bfloat16)
            del z
        elif self.attn_mode in ("keys", "queries"):
            # queries, keys and values N(0, 1) in bf16; the clean forward's weights are the
            # causal softmax of tau q k^T per head (fp32 on the device, before timing)
            self.tau = 1.0 / np.sqrt(self.d // H)
            self.qbits, self.kbits, self.vbits = (synth.normal_bf16(synth.rng(self.cfg_id, j),
                                                                    (self.T, self.d))
                                                  for j in (3, 4, 5))
            self.q, self.k, self.v = self.bf(self.qbits), self.bf(self.kbits), self.bf(self.vbits)
            heads = lambda a: a.float().reshape(B, S, H, -1).permute(0, 2, 1, 3)
            z = self.tau * heads(self.q) @ heads(self.k).transpose(-1, -2).contiguous()
            z.masked_fill_(~t.ones((S, S), dtype=t.bool, device=self.dev).tril(), float("-inf"))
            self.P = t.softmax(z, -1).to(t.bfloat16)
            del z
            # the draw-independent row weights of the re-run, recomputed in every timed step
            self.W = self.empty((B, H, S, S), t.float32)
            self.Z = self.empty((B, H, S), t.float32)
        else:
            # One 512-draw block of the synthetic attention-output change, drawn on the device
            # before timing; every block of the timed step streams this buffer (the kernel's work
            # does not depend on the values).
            zero = self.torch.zeros((self.T, self.d), dtype=t.bfloat16, device=self.dev)
            self.do = self.empty((self.KB, self.T, self.d), t.bfloat16)
            self.dust.dust_noise_inject(zero, self.do, self.dust.DUST_BF16, self.T, self.d, self.d,
                                        0, self.KB, self.std, self.seed, synth.DELTA_O_TAG, 0, 0)
            del zero
        self.cbuf = self.empty((self.K, self.T), t.float32)
        self.gh = self.empty((self.T, self.d), t.float32)
        self.ght = self.empty((self.d, self.T), t.bfloat16)
        self.G = self.empty((self.d, self.d), t.float32)
        self.ws_bytes = self.dust.dust_weight_grad_workspace(self.T, self.d, self.d)
        self.ws = self.empty(max(self.ws_bytes, 16), t.uint8)

    attn_mode = None   # None, "values", "keys" or "queries"
    HEADS = 8

    def step(self, run, sh):
        d, T, K, KB = self.dust, self.T, self.K, self.KB
        if self.attn_mode == "values":
            run("dust_attn_value_scores", d.dust_attn_value_scores, self.P, self.go, self.cbuf, K,
                T // self.S, self.HEADS, self.S, self.d // self.HEADS, 0, self.sigma, self.seed,
                self.tag, 0, 0, sh)
        elif self.attn_mode in ("keys", "queries"):
            B, H, S, dh = T // self.S, self.HEADS, self.S, self.d // self.HEADS
            run("dust_attn_row_weights", d.dust_attn_row_weights, self.P, self.v, self.go, self.W,
                self.Z, B, H, S, dh, sh)
            if self.attn_mode == "keys":
                run("dust_attn_key_scores", d.dust_attn_key_scores, self.P, self.q, self.W, self.Z,
                    self.cbuf, K, B, H, S, dh, 0, self.sigma, self.tau, self.seed, self.tag, 0, 0,
                    sh)
            else:
                run("dust_attn_query_scores", d.dust_attn_query_scores, self.P, self.k, self.W,
                    self.Z, self.cbuf, K, B, H, S, dh, 0, self.sigma, self.tau, self.seed,
                    self.tag, 0, 0, sh)
        else:
            for blk in range(K // KB):
                run("dust_loss_delta", d.dust_loss_delta, d.DUST_DELTA_INNER, None, None, self.do,
                    self.go, d.DUST_BF16, self.cbuf[blk * KB:(blk + 1) * KB], KB, T, self.d, sh)
        run("dust_reward_scan", d.dust_reward_scan, self.cbuf, self.cbuf, K, T, self.S, self.gamma, sh)
        run("dust_error_estimate", d.dust_error_estimate, self.cbuf, self.gh, self.ght, K, K, T, self.d,
            0, self.sigma, self.seed, self.tag, 0, 0, 0, sh)
        run("dust_weight_grad", d.dust_weight_grad, self.ght, self.x, self.G, T, self.d, self.d,
            self.ws, self.ws_bytes, sh)

    def draws_tokens(self):
        return self.K * self.T

    def model(self):
        T, K, d = self.T, self.K, self.d
        S, H = self.S, self.HEADS
        return {
            "dust_loss_delta": _hbm(self.KB * T * (2.0 * d + 4.0) + 2.0 * T * d),
            # the key-query inner products over the causal triangle: 2 (S (S + 1) / 2) dh flops
            # per draw, head and sequence
            "dust_attn_value_scores": _mfma(2.0 * K * (T // S) * H * (S * (S + 1) / 2) * (d // H)),
            # per causal (draw, head, query, key) element: e^x - 1 and two weighted sums, fp32
            "dust_attn_key_scores": ("alu", OPS_KEY_SCORE * K * (T // S) * H * (S * (S + 1) / 2),
                                     1e12, FP32_VALU_PEAK_TOPS, "Tops/s"),
            "dust_attn_query_scores": ("alu", OPS_KEY_SCORE * K * (T // S) * H * (S * (S + 1) / 2),
                                       1e12, FP32_VALU_PEAK_TOPS, "Tops/s"),
            # once per estimate: P read once (bf16), W written (fp32, zero above the diagonal)
            # and Z
            "dust_attn_row_weights": _hbm((T // S) * H * (6.0 * S * S + 4.0 * S)),
            "dust_reward_scan": _hbm(8.0 * K * T),
            "dust_error_estimate": _alu(K * T * d, OPS_EE_EXTRA),
            "dust_weight_grad": _mfma(2.0 * T * d * d),
        }

    def serial_roofs(self):
        # The attention scorers, each part at its published peak: the products of the causal
        # elements as executed (the noise's high part and remainder: 4 dh flops per element) on
        # the matrix cores, the per-element fp32 work on the vector units (6 ops for the key and
        # query scores, 1 fma for the value scores), and the noise, K T d normals regenerated
        # once each at the generator's 12 operations
        T, K, S, H = self.T, self.K, self.S, self.HEADS
        elems = K * (T // S) * H * (S * (S + 1) / 2)
        common = (4.0 * (self.d // H) * elems / (BF16_MFMA_PEAK_TFLOPS * 1e12) +
                  OPS_PER_NORMAL * K * T * self.d / (VALU_PEAK_TOPS * 1e12))
        ms_kq = 1e3 * (common + OPS_KEY_SCORE * elems / (FP32_VALU_PEAK_TOPS * 1e12))
        ms_v = 1e3 * (common + elems / (FP32_VALU_PEAK_TOPS * 1e12))
        return {"dust_attn_key_scores": ms_kq, "dust_attn_query_scores": ms_kq,
                "dust_attn_value_scores": ms_v}

    def config(self):
        cfg = {"workload": self.c["name"], "d": self.d, "tokens": self.T, "seq_len": self.S,
               "draws": self.K, "draw_block": self.KB, "gamma": self.gamma, "sigma": self.sigma,
               "storage": "bf16 delta_o / g_o / x, fp32 scores, rewards, g_hat, G_W"}
        if self.attn_mode == "values":
            cfg.update({"workload": self.c["name"] + "_attention_values", "heads": self.HEADS,
                        "head_dim": self.d // self.HEADS, "draw_block": self.K,
                        "delta_o": "attention re-run with perturbed values (synthetic weights)",
                        "storage": "bf16 attention weights / g_o / x, fp32 scores, rewards, "
                                   "g_hat, G_W"})
        elif self.attn_mode == "keys":
            cfg.update({"workload": self.c["name"] + "_attention_keys", "heads": self.HEADS,
                        "head_dim": self.d // self.HEADS, "draw_block": self.K,
                        "softmax_scale": self.tau,
                        "delta_o": "softmax re-run with perturbed keys (synthetic q, k, v)",
                        "storage": "bf16 attention weights / q / v / g_o / x, fp32 row weights, "
                                   "scores, rewards, g_hat, G_W"})
        elif self.attn_mode == "queries":
            cfg.update({"workload": self.c["name"] + "_attention_queries", "heads": self.HEADS,
                        "head_dim": self.d // self.HEADS, "draw_block": self.K,
                        "softmax_scale": self.tau,
                        "delta_o": "softmax re-run with perturbed queries (synthetic q, k, v)",
                        "storage": "bf16 attention weights / k / v / g_o / x, fp32 row weights, "
                                   "scores, rewards, g_hat, G_W"})
        return cfg

    def cpu_baseline(self, scale):
        import oracle
        if self.attn_mode is not None:
            return self._cpu_baseline_attention(scale)
        S, d = self.S, self.d
        K_s, T_s = max(8, int(8192 * scale) // 8 * 8), S
        oracle.threads()
        go = synth.bf16_bits_to_f32(self.gobits[:T_s]).astype(np.float64)
        c = np.empty((K_s, T_s))
        t_gen = t_inner = 0.0
        for k0 in range(0, K_s, 1024):   # blocks of draws bound the host memory
            kb = min(1024, K_s - k0)
            t1 = time.perf_counter()
            do = self.std * oracle.normals(self.seed, synth.DELTA_O_TAG, k0, 0, 0, kb, T_s, d)
            t2 = time.perf_counter()
            c[k0:k0 + kb] = oracle.loss_delta_inner(do, go)
            t3 = time.perf_counter()
            t_gen += t2 - t1
            t_inner += t3 - t2
            del do
        t0 = time.perf_counter()
        r = oracle.reward_scan(c, S, self.gamma)
        g = oracle.error_estimate(r, d, self.sigma, self.seed, self.tag, K_total=self.K)
        oracle.weight_grad(g, synth.bf16_bits_to_f32(self.xbits[:T_s]).astype(np.float64))
        dt = t_inner + time.perf_counter() - t0
        return {"value": K_s * T_s / dt, "unit": UNIT, "cores": oracle.threads(), "kind": "oracle",
                "sample": "%d of %d draws x first %d tokens (one sequence): inner-product scores, "
                          "scan, error estimate, G_W; the attention-output change is drawn "
                          "untimed (%.1f s), as on the device; %.1f s"
                          % (K_s, self.K, T_s, t_gen, dt)}


    def _cpu_baseline_attention(self, scale):
        import oracle
        S, d, H = self.S, self.d, self.HEADS
        # about 10 s on 16 cores: the value and key oracles regenerate the noise of every key
        # for every query (0.5 s per draw), the query oracle once per query (2.5 ms per draw)
        K_s = max(1, int((128 if self.attn_mode == "queries" else 16) * scale))
        P = self.P[:1].float().cpu().numpy().astype(np.float64)          # the first sequence
        go = synth.bf16_bits_to_f32(self.gobits[:S]).astype(np.float64)
        t0 = time.perf_counter()
        if self.attn_mode == "keys":
            q, v = (synth.bf16_bits_to_f32(a[:S]).astype(np.float64) for a in (self.qbits, self.vbits))
            c = oracle.attn_key_scores(P, q, v, go, K_s, self.sigma, self.tau, self.seed, self.tag)
        elif self.attn_mode == "queries":
            k, v = (synth.bf16_bits_to_f32(a[:S]).astype(np.float64) for a in (self.kbits, self.vbits))
            c = oracle.attn_query_scores(P, k, v, go, K_s, self.sigma, self.tau, self.seed,
                                         self.tag)
        else:
            c = oracle.attn_value_scores(P, go, K_s, self.sigma, self.seed, self.tag)
        r = oracle.reward_scan(c, S, self.gamma)
        g = oracle.error_estimate(r, d, self.sigma, self.seed, self.tag, K_total=self.K)
        oracle.weight_grad(g, synth.bf16_bits_to_f32(self.xbits[:S]).astype(np.float64))
        dt = time.perf_counter() - t0
        return {"value": K_s * S / dt, "unit": UNIT, "cores": oracle.threads(), "kind": "oracle",
                "sample": "%d of %d draws x first %d tokens (one sequence, %d heads): attention "
                          "%s scores, scan, error estimate, G_W; %.1f s"
                          % (K_s, self.K, S, H, self.attn_mode[:-1].replace("querie", "query"),
                             dt)}


CHAINS = {2: LinearChain, 3: HeadChain, 4: InnerChain, 5: LinearChain}


def ceilings(torch, dev) -> dict:
    """The measured ceilings: a device copy, the noise generator alone and the matrix cores alone
    (activation_perturbation_es_amd/csrc/probes.hip), each run until the clock has settled and
    then timed with HIP events; medians of 10 launches."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "activation_perturbation_es_amd", "libdust_probes.so"))
    lib.dust_probe_generator.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_void_p]
    lib.dust_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                    ctypes.c_uint32, ctypes.c_void_p]
    sh = torch.cuda.current_stream().cuda_stream

    def timed(fn, warm=20, n=10):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)          # 1 GiB
    b = torch.empty_like(a)
    t_copy = timed(lambda: b.copy_(a))
    del a, b
    gb, gd = 8192, 2048                                                 # 32 waves per CU
    gout = torch.empty(gb * 256, dtype=torch.float32, device=dev)
    t_gen = timed(lambda: lib.dust_probe_generator(gout.data_ptr(), gb, gd, sh))
    mb, mi = 256, 8192                                                  # one wave per SIMD
    src = torch.randn(mb * 256 * 16, device=dev).to(torch.bfloat16)
    mout = torch.empty(mb * 256, dtype=torch.float32, device=dev)
    t_mfma = timed(lambda: lib.dust_probe_mfma(src.data_ptr(), mout.data_ptr(), mb, mi, sh))
    normals = gb * 256 * 4 * gd
    flops = mb * 4 * mi * 16 * 32768
    copy_gbs = 2.0 * (1 << 30) / t_copy / 1e9
    clock = clock_under_load(torch, dev, lib, timed)
    return {
        "clock_under_load": clock,
        "device_copy": {"GB_per_s": round(copy_gbs, 1), "frac_of_hbm_peak":
                        round(copy_gbs / HBM_PEAK_GBS, 4), "bytes_moved": 2 * (1 << 30)},
        "noise_generator": {"normals_per_s": float("%.4g" % (normals / t_gen)),
                            "ops_per_s_at_13_per_normal": float("%.4g" % (13 * normals / t_gen)),
                            "frac_of_valu_peak": round(13 * normals / t_gen / 1e12 / VALU_PEAK_TOPS, 4),
                            "normals": normals},
        "mfma_bf16_random_operands": {"TFLOP_per_s": round(flops / t_mfma / 1e12, 1),
                                      "frac_of_peak": round(flops / t_mfma / 1e12 /
                                                            BF16_MFMA_PEAK_TFLOPS, 4),
                                      "flops": flops},
    }


def clock_under_load(torch, dev, lib, timed) -> dict:
    """Shader clock and rates while four waves per CU issue MFMAs and four others read LDS, run
    the noise generator or idle, and while LDS reads or the generator run alone: per-wave
    s_memtime cycles over s_memrealtime ticks, averaged over the 256 blocks (one per CU) of the
    last of the timed launches."""
    import ctypes
    lib.dust_probe_clock.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    lib.dust_probe_wallclock_khz.restype = ctypes.c_int
    khz = lib.dust_probe_wallclock_khz()
    if khz <= 0:
        raise RuntimeError("hipDeviceAttributeWallClockRate unavailable")
    sh = torch.cuda.current_stream().cuda_stream
    blocks, iters = 256, 4000
    out = torch.zeros(blocks * 8 * 2, dtype=torch.int64, device=dev)
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    # (name, MFMA waves, LDS bytes per LDS wave per iteration, LDS waves)
    modes = [("mfma_alone", 4, 0, 0), ("mfma_with_lds_b128_reads", 4, 16384, 4),
             ("mfma_with_lds_tr_reads", 4, 16384, 4), ("lds_b128_reads_alone", 0, 8192, 8),
             ("lds_tr_reads_alone", 0, 8192, 8), ("mfma_with_generator", 4, 0, 0),
             ("generator_alone", 0, 0, 0)]
    res = {}
    for mode, (name, mw, lbytes, lw) in enumerate(modes):
        rc = []
        timed(lambda: rc.append(lib.dust_probe_clock(mode, out.data_ptr(), sink.data_ptr(),
                                                     blocks, iters, sh)), warm=5, n=5)
        if any(rc):
            raise RuntimeError("dust_probe_clock failed: %r" % rc)
        o = out.view(blocks, 8, 2).double()
        gen = name in ("mfma_with_generator", "generator_alone")
        waves = slice(0, 4) if mw else (slice(4, 8) if gen else slice(0, 8))
        cyc = o[:, waves, 0].mean().item()
        sec = o[:, waves, 1].mean().item() / (khz * 1e3)
        r = {"clock_GHz": round(cyc / sec / 1e9, 3)}
        if mw:
            fl = blocks * mw * iters * 16 * 32768
            r["mfma_TFLOP_per_s"] = round(fl / sec / 1e12, 1)
            r["mfma_frac_of_peak"] = round(fl / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        if gen:   # 4 generator waves, 64 lanes, 8 normals per lane per iteration
            gsec = o[:, 4:8, 1].mean().item() / (khz * 1e3)
            r["generator_normals_per_s"] = float("%.4g" % (blocks * 4 * 64 * 8 * iters / gsec))
            r["generator_clock_GHz"] = round(o[:, 4:8, 0].mean().item() / gsec / 1e9, 3)
        if lw:
            lo = slice(4, 8) if mw else slice(0, 8)
            lcyc = o[:, lo, 0].mean().item()
            r["lds_bytes_per_clock_per_CU"] = round(lw * lbytes * iters / lcyc, 1)
        res[name] = r
    res["wallclock_kHz"] = khz
    return res


def cfg_name(chain) -> str:
    """The workload name the bench line carries (and profiles/traffic.json is keyed by)."""
    return chain.config()["workload"]


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the estimator runs on a single MI355X here "
              "(the path shards by sequences across GPUs, but only the one-GPU case is built). "
              "Use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import activation_perturbation_es_amd as dust

    dev = "cuda:0"
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(torch, dev), "n_gpus": 1}), flush=True)
        return 0
    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    chain = CHAINS[args.workload](args.workload, dust, torch, dev)
    chain.fused = not args.unfused
    if args.draw_block:
        if args.workload not in (2, 5):
            print("--draw-block applies to the MLP workloads 2 and 5 only", file=sys.stderr)
            return 2
        chain.draw_block = args.draw_block
    if args.fold:
        if args.workload not in (2, 3, 5) or chain.c["gamma"] != 0.0:
            print("--fold applies to the loss-scored workloads with gamma = 0 (2, 3, 5)",
                  file=sys.stderr)
            return 2
        chain.fold = True
    if args.downstream != "none":
        if args.workload not in (2, 5):
            print("--downstream applies to the MLP workloads 2 and 5 only", file=sys.stderr)
            return 2
        chain.downstream = args.downstream
    chain.optimizer = args.optimizer
    modes = [m for m, on in (("values", args.attention_values), ("keys", args.attention_keys),
                             ("queries", args.attention_queries)) if on]
    if modes:
        if args.workload != 4 or len(modes) > 1:
            print("--attention-values, --attention-keys or --attention-queries (one of them) "
                  "applies to workload 4 only", file=sys.stderr)
            return 2
        chain.attn_mode = modes[0]
    chain.setup()
    chain.opt_setup()

    def full_step(run):
        chain.step(run, sh)
        if chain.optimizer != "none":
            chain.opt_step(run, sh)

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    events = []   # (kernel, start event, end event) inside the timed region

    def plain(name, fn, *a):
        fn(*a)

    def recorded(name, fn, *a):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*a)
        e1.record(stream)
        events.append((name, e0, e1))

    for _ in range(args.warmup):
        full_step(plain)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        full_step(recorded)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = chain.draws_tokens() / (elapsed / args.steps)

    # ---- per-kernel durations (HIP events on the launch stream)
    per = {}
    for name, e0, e1 in events:
        per.setdefault(name, []).append(e0.elapsed_time(e1))
    model = chain.model()
    model.update(chain.opt_model())
    serial = chain.serial_roofs()
    kernels = {}
    for name, ms in per.items():
        bound, work, scale, peak, unit = model[name][:5]
        avg_ms = float(np.mean(ms))
        ach = work / (avg_ms * 1e-3) / scale
        kernels[name] = {"launches_per_step": len(ms) // args.steps, "avg_ms": round(avg_ms, 5),
                         "ms_per_step": round(sum(ms) / args.steps, 5), "bound": bound,
                         "achieved": round(ach, 3), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4)}
        if len(model[name]) > 5:   # generating kernels: normals per second, free of the op model
            kernels[name]["normals_per_s"] = float("%.4g" % (model[name][5] / (avg_ms * 1e-3)))
        if name in serial:
            kernels[name]["serial_roof_ms"] = round(serial[name], 3)
            kernels[name]["serial_frac"] = round(serial[name] / avg_ms, 4)
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dominant]
    roofline = {"kernel": dominant, "bound": dk["bound"], "achieved": dk["achieved"],
                "peak": dk["peak"], "unit": dk["unit"], "frac": dk["frac"], "traffic": None}
    # HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE,
    # scaled by the copy-kernel calibration (profiles/); null unless they were taken for this
    # workload, this kernel and the current kernel sources.
    traffic_file = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(traffic_file):
        with open(traffic_file) as f:
            tr = json.load(f).get(cfg_name(chain), {})
        if tr.get("kernel") == dominant and tr.get("build") == _kernel_build_id(dominant):
            roofline["traffic"] = tr.get("bytes_per_launch")

    cfg = chain.config()
    cfg["parallelism"] = "single GPU"
    cfg["precision"] = ("bf16 activations, perturbed outputs and matrix-core operands; fp32 "
                        "noise, scores, rewards, output error and accumulation")
    if args.workload != 4:
        cfg["loss_to_reward"] = ("inside the error estimate" if chain.fold else
                                 "one kernel" if chain.fused else "two kernels")
    if chain.optimizer != "none":
        cfg["optimizer"] = chain.optimizer
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic", "config": cfg, "roofline": roofline, "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = chain.cpu_baseline(args.cpu_scale)
    print(json.dumps(line), flush=True)
    return 0


# HIP translation unit of each entry point's kernels; every unit also includes the two shared
# device headers, and build.py fixes the compile flags.
KERNEL_SOURCES = {
    "dust_noise_inject": "noise.hip", "dust_loss_delta": "delta_scan.hip",
    "dust_reward_scan": "delta_scan.hip", "dust_loss_reward": "delta_scan.hip",
    "dust_error_estimate": "error_estimate.hip", "dust_error_estimate_losses": "error_estimate.hip",
    "dust_weight_grad": "weight_grad.hip", "dust_head_ce_chunk": "head_ce.hip",
    "dust_sgd_momentum": "optim.hip", "dust_adam": "optim.hip",
    "dust_attn_value_scores": "attn_scores.hip", "dust_attn_key_scores": "attn_scores.hip",
    "dust_attn_query_scores": "attn_scores.hip", "dust_attn_row_weights": "attn_scores.hip",
    "dust_perturbed_linear": "perturbed_linear.hip",
}


def _kernel_build_id(kernel: str) -> str:
    """Hash of the sources one entry point's kernels are compiled from, so recorded counter
    traffic is tied to the kernels it measured and goes stale when any of them changes."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "activation_perturbation_es_amd")
    for rel in (os.path.join("csrc", KERNEL_SOURCES[kernel]), os.path.join("csrc", "dust_internal.hpp"),
                os.path.join("csrc", "dust_noise.hpp"), "build.py"):
        with open(os.path.join(pkg, rel), "rb") as f:
            h.update(rel.encode() + f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
