#!/usr/bin/env python3
"""Throughput of the Dust estimator chain on one MI355X.

One step = one whole estimate for the MLP up-projection 512 -> 2048 of the 8-layer width-512
GPT (T = 16 x 1024 tokens, K = 64 draws, gamma = 0, sigma = 0.01), with every input resident in
HBM before the timed region:
    dust_noise_inject   x 8 (8-draw blocks into a rotating perturbed-output buffer)
    dust_loss_delta     (loss mode, [64, 16384])
    dust_reward_scan    (gamma = 0, sequences of 1024)
    dust_error_estimate (g_hat [16384, 2048] fp32 + its bf16 transpose)
    dust_weight_grad    (G_W [2048, 512], bf16 matrix cores)
The perturbed forward of the rest of the model that sits between the perturbation and the loss
change is not part of the estimator; its per-token losses are synthetic inputs here.

Metric: draws x tokens per second (K * T / step time). Prints one JSON line; with the per-kernel
HIP-event durations measured inside the timed region it adds the roofline of the dominant
kernel, and the CPU oracle's throughput on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--cpu-tokens 8192 | --no-cpu-baseline]
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
CFG_ID = 2

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# Vector ALU issue rate: 256 CUs x 64 lanes x 2.4 GHz = 39.32e12 lane-operations per second.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12

# Algorithmic vector operations per generated standard normal (one issue slot each; derivation
# in the design doc). Philox4x32-10: a round is 2 32x32->64 multiplies (v_mad_u64_u32) + 2 three-input
# XORs (v_bitop3_b32). Of the counter (channel group, token, draw, tag), the channel group and
# tag are fixed per lane and draw is uniform across the wave, so the first round and the
# multiplies of the second run once per lane or on the scalar unit, not per draw: 2 + 8 x 4 = 34
# operations per 4 words -> 8.5 per normal. Box-Muller per pair: 2 x 2 for the uniforms
# (funnel shift, subtract), log2, scale, sqrt, cos, sin, 2 multiplies = 11 -> 5.5 per normal.
OPS_PER_NORMAL = 8.5 + 5.5
OPS_INJECT_EXTRA = 1.5    # fma with y, and half of a packed fp32 -> bf16 conversion
OPS_EE_EXTRA = 1.0        # fma of reward x normal into the accumulator


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens (whole sequences) of the CPU oracle's sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def cpu_baseline(c, ybits, xbits, lc, lp, tokens: int) -> dict:
    """The oracle's chain (as it stands) on the first `tokens` tokens with all K draws."""
    import oracle
    T_s = min(tokens, c["T"])
    T_s -= T_s % c["seg_len"]
    K, KB, d_out, sigma = c["K"], c["inject_block"], c["d_out"], c["sigma"]
    seed, tag = synth.noise_seed(CFG_ID), synth.NOISE_TAG
    y = synth.bf16_bits_to_f32(ybits[:T_s]).astype(np.float64)
    x = synth.bf16_bits_to_f32(xbits[:T_s]).astype(np.float64)
    oracle.threads()   # load before timing
    t0 = time.perf_counter()
    for b in range(K // KB):
        oracle.noise_inject(y, sigma, KB, seed, tag, draw0=b * KB)
    r = oracle.reward_scan(oracle.loss_delta_loss(lc[:T_s], lp[:, :T_s]), c["seg_len"], c["gamma"])
    g = oracle.error_estimate(r, d_out, sigma, seed, tag)
    oracle.weight_grad(g, x)
    dt = time.perf_counter() - t0
    return {"value": K * T_s / dt, "unit": UNIT, "cores": oracle.threads(), "kind": "oracle",
            "sample": "all %d draws x first %d of %d tokens (%d whole sequences), whole chain "
                      "incl. the full G_W contraction over those tokens; %.1f s"
                      % (K, T_s, c["T"], T_s // c["seg_len"], dt)}


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the estimator runs on a single MI355X here "
              "(multi-GPU sharding is described in DESIGN.md, not built). Use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import activation_perturbation_es_amd as dust

    c = synth.CONFIGS[CFG_ID]
    T, d_in, d_out, K, KB = c["T"], c["d_in"], c["d_out"], c["K"], c["inject_block"]
    S, gamma, sigma = c["seg_len"], c["gamma"], c["sigma"]
    seed, tag = synth.noise_seed(CFG_ID), synth.NOISE_TAG
    dev = "cuda:0"

    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---- inputs, resident in HBM before timing
    g = synth.rng(CFG_ID, 1)
    ybits = synth.normal_bf16(g, (T, d_out))
    xbits = synth.normal_bf16(g, (T, d_in))
    lc_h, lp_h = synth.losses(synth.rng(CFG_ID, 2), K, T)

    def bf(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    y, x = bf(ybits), bf(xbits)
    lc, lp = torch.from_numpy(lc_h).to(dev), torch.from_numpy(lp_h).to(dev)
    ybuf = torch.empty((KB, T, d_out), dtype=torch.bfloat16, device=dev)
    cbuf = torch.empty((K, T), dtype=torch.float32, device=dev)
    rbuf = torch.empty((K, T), dtype=torch.float32, device=dev)
    gh = torch.empty((T, d_out), dtype=torch.float32, device=dev)
    ght = torch.empty((d_out, T), dtype=torch.bfloat16, device=dev)
    G = torch.empty((d_out, d_in), dtype=torch.float32, device=dev)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    events = []   # (kernel, start event, end event) inside the timed region

    def timed(name, fn, *a, record):
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(*a)
            e1.record(stream)
            events.append((name, e0, e1))
        else:
            fn(*a)

    def step(record=False):
        for blk in range(K // KB):
            timed("dust_noise_inject", dust.dust_noise_inject, y, ybuf, dust.DUST_BF16, T, d_out,
                  d_out, 0, KB, sigma, seed, tag, blk * KB, 0, sh, record=record)
        timed("dust_loss_delta", dust.dust_loss_delta, dust.DUST_DELTA_LOSS, lc, lp, None, None,
              dust.DUST_F32, cbuf, K, T, 0, sh, record=record)
        timed("dust_reward_scan", dust.dust_reward_scan, cbuf, rbuf, K, T, S, gamma, sh, record=record)
        timed("dust_error_estimate", dust.dust_error_estimate, rbuf, gh, ght, K, K, T, d_out, 0,
              sigma, seed, tag, 0, 0, 0, sh, record=record)
        timed("dust_weight_grad", dust.dust_weight_grad, ght, x, G, T, d_out, d_in, ws, ws_bytes, sh,
              record=record)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = K * T / (elapsed / args.steps)

    # ---- per-kernel durations (HIP events on the launch stream)
    per = {}
    for name, e0, e1 in events:
        per.setdefault(name, []).append(e0.elapsed_time(e1))
    steps = args.steps
    normals_inject = KB * T * d_out
    normals_ee = K * T * d_out
    model = {
        # name: (bound, algorithmic work per launch, unit scale, peak, unit)
        "dust_noise_inject": ("alu", normals_inject * (OPS_PER_NORMAL + OPS_INJECT_EXTRA), 1e12,
                              VALU_PEAK_TOPS, "Tops/s"),
        "dust_error_estimate": ("alu", normals_ee * (OPS_PER_NORMAL + OPS_EE_EXTRA), 1e12,
                                VALU_PEAK_TOPS, "Tops/s"),
        "dust_loss_delta": ("hbm", (8.0 + 4.0 / K) * K * T, 1e9, HBM_PEAK_GBS, "GB/s"),
        "dust_reward_scan": ("hbm", 8.0 * K * T, 1e9, HBM_PEAK_GBS, "GB/s"),
        "dust_weight_grad": ("mfma", 2.0 * T * d_out * d_in, 1e12, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"),
    }
    kernels = {}
    for name, ms in per.items():
        bound, work, scale, peak, unit = model[name]
        avg_ms = float(np.mean(ms))
        ach = work / (avg_ms * 1e-3) / scale
        kernels[name] = {"launches_per_step": len(ms) // steps, "avg_ms": round(avg_ms, 5),
                         "ms_per_step": round(sum(ms) / steps, 5), "bound": bound,
                         "achieved": round(ach, 3), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4)}
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dominant]
    roofline = {"kernel": dominant, "bound": dk["bound"], "achieved": dk["achieved"],
                "peak": dk["peak"], "unit": dk["unit"], "frac": dk["frac"],
                "traffic": None}
    # HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE,
    # scaled by the copy-kernel calibration (see profiles/); null when not measured for the
    # current kernel build.
    traffic_file = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(traffic_file):
        with open(traffic_file) as f:
            tr = json.load(f)
        if tr.get("kernel") == dominant and tr.get("build") == _kernel_build_id():
            roofline["traffic"] = tr.get("bytes_per_launch")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": c["name"], "d_in": d_in, "d_out": d_out, "tokens": T,
                   "seq_len": S, "draws": K, "gamma": gamma, "sigma": sigma,
                   "inject_block": KB, "storage": "bf16 activations, fp32 rewards/g_hat/G_W",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, ybits, xbits, lc_h, lp_h, args.cpu_tokens)
    print(json.dumps(line), flush=True)
    return 0


def _kernel_build_id() -> str:
    """Hash of the HIP sources, so recorded counter traffic is tied to the kernels it measured."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_perturbation_es_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
