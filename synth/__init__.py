"""Seeded synthetic inputs for the Dust estimator's tests, smoke check and benchmark.

This module holds none of the estimator's arithmetic: only the workload shapes, seeds, random
draws (numpy PCG64) and the conversion of fp32 draws to bf16 bit patterns. Both the HIP path and
the CPU oracle receive their inputs from here; neither is imported by this module.

The workloads stand in for the pages' setting (a GPT with 8 layers, width 512, a 4096-token BPE
vocabulary and 16k-token batches; a ~240M-parameter variant of width 1024) with synthetic data of
those shapes and value distributions. Notation N(mu, v) uses the VARIANCE v.
"""
from __future__ import annotations

import numpy as np

# Workload definitions (sizes are element counts).
WORKLOADS = {
    # Tiny CPU-checkable model: linear 64 -> 64 (fp32) feeding a fixed LM head 64 -> 256.
    1: dict(name="tiny_linear_64x64_head256", d_in=64, d_out=64, V=256, T=128, seg_len=128,
            K=16, sigma=0.01, gammas=(0.0, 0.9)),
    # MLP up-projection 512 -> 2048 of the 8-layer width-512 GPT, 16 x 1024 tokens, 64 draws.
    # The whole population is perturbed in one call (a 4.3 GB perturbed-output buffer).
    2: dict(name="mlp_up_512x2048_T16384_K64", d_in=512, d_out=2048, V=4096, T=16384,
            seg_len=1024, K=64, gamma=0.0, sigma=0.01, inject_block=64),
    # LM head on cached logits: vocabulary 4096, chunk [0, 1024), hidden 512, 1024 draws.
    3: dict(name="lm_head_chunk1024_V4096_T16384_K1024", hidden=512, V=4096, v0=0, C=1024,
            T=16384, seg_len=1024, K=1024, gamma=0.0, sigma=0.01),
    # Attention key/value projection 512 -> 512 scored by the inner product with the attention
    # output error, gamma = 0.99 over 16 x 1024 tokens, 16384 draws in blocks of 512.
    4: dict(name="attn_kv_inner_512_T16384_K16384", d=512, T=16384, seg_len=1024, K=16384,
            draw_block=512, gamma=0.99, sigma=0.01, delta_o_std=0.01),
    # ~240M-parameter GPT (width 1024): MLP up-projection 1024 -> 4096, 1024 draws, perturbed
    # in blocks of 32 draws (a 4.3 GB perturbed-output buffer).
    5: dict(name="mlp_up_1024x4096_T16384_K1024", d_in=1024, d_out=4096, V=4096, T=16384,
            seg_len=1024, K=1024, gamma=0.0, sigma=0.01, inject_block=32),
}

NOISE_TAG = 1          # Philox tag of the estimator's noise
DELTA_O_TAG = 0x100    # Philox tag of the synthetic attention-output change (workload 4)


def noise_seed(cfg: int) -> int:
    """Philox seed of workload `cfg`."""
    return 0x0D057000 + cfg


def rng(cfg: int, stream: int = 0) -> np.random.Generator:
    """Host generator of workload `cfg`; `stream` separates independent arrays."""
    return np.random.Generator(np.random.PCG64([1000 + cfg, stream]))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact fp32 values of bf16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, std^2) draws."""
    return f32_to_bf16_bits(normal_f32(g, shape, std))


def targets(g: np.random.Generator, T: int, V: int) -> np.ndarray:
    return g.integers(0, V, size=T, dtype=np.int32)


def losses(g: np.random.Generator, K: int, T: int):
    """Synthetic per-token losses standing in for the downstream forward, which is outside the
    estimator: clean losses around the cross-entropy level of a 4096-token vocabulary and
    perturbed losses that differ by N(0, 1e-4) per draw. Returns (loss_clean [T],
    loss_pert [K, T]) as fp32."""
    lc = (np.float32(8.3) + normal_f32(g, (T,), 0.5)).astype(np.float32)
    dc = normal_f32(g, (K, T), 0.01)
    lp = (lc[None, :] - dc).astype(np.float32)
    return lc, lp


def tiny_model(cfg: int = 1):
    """Workload 1: W ~ N(0, 1/64) [d_out, d_in], H ~ N(0, 1/64) [V, d_out], x ~ N(0, 1)
    [T, d_in], targets uniform in [0, V). All fp32."""
    c = WORKLOADS[cfg]
    g = rng(cfg)
    W = normal_f32(g, (c["d_out"], c["d_in"]), 1.0 / 8.0)
    H = normal_f32(g, (c["V"], c["d_out"]), 1.0 / 8.0)
    x = normal_f32(g, (c["T"], c["d_in"]))
    tgt = targets(g, c["T"], c["V"])
    return W, H, x, tgt
