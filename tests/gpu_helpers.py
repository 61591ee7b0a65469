"""Helpers of the GPU parity tests: device transfers and comparison measures (no arithmetic of
the estimator lives here)."""
import sys

import numpy as np
import torch

import activation_perturbation_es_amd as dust  # noqa: F401  (re-exported for the tests)

DEV = "cuda:0"


def announce(msg: str) -> None:
    """Name the GPU case about to run, flushed, so a failing box still says which one it was."""
    print("[gpu case] " + msg, flush=True)
    sys.stdout.flush()


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def bf16(bits) -> torch.Tensor:
    """Device bf16 tensor holding the given uint16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_bf16_bits_of_f32(a) -> np.ndarray:
    """bf16 bit patterns of fp32 values, nearest-even (to check a kernel's own rounding of its
    own fp32 result)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (normal range)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def frob_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def row_weights(P, v, g_o, B, H, S, dh):
    """W [B, H, S, S] and Z [B, H, S] of dust_attn_row_weights, on the device (the key and query
    scorers take them in place of the values and the output error)."""
    W = torch.full((B, H, S, S), float("nan"), dtype=torch.float32, device=DEV)
    Z = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    dust.dust_attn_row_weights(P, v, g_o, W, Z, B, H, S, dh)
    return W, Z
