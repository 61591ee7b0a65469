"""The library driven from plain C (MI355X only).

tests/c_abi/estimate.c makes one estimate through include/dust.h alone: hipMalloc'd device
memory, the entry points called from C (inject, loss change and reward in one pass, output
error, weight gradient), no Python or torch in the process. The same inputs go through the
Python binding here; the two must agree bit for bit (the same kernels on the same inputs), and
the C program's first perturbed draw must equal the oracle's y + sigma a rounded to bf16 within
one bf16 ulp. Build: __graft_entry__.build() compiles the program with gcc.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, announce, bf16, bf16_ulp, bits_to_f64, dust, f32, host_f32

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "estimate")


def test_estimate_from_c_equals_the_binding(tmp_path):
    announce("C client estimate")
    assert os.path.exists(EXE), "tests/c_abi/estimate is missing: run __graft_entry__.build()"
    T, d_in, d_out, K, S, sigma, gamma = 256, 64, 96, 16, 64, 0.01, 0.9
    seed, tag = synth.noise_seed(1), synth.NOISE_TAG
    g = synth.rng(1, 9)
    ybits = synth.normal_bf16(g, (T, d_out))
    xbits = synth.normal_bf16(g, (T, d_in))
    lc, lp = synth.losses(g, K, T)
    ybits.tofile(tmp_path / "y.bin")
    xbits.tofile(tmp_path / "x.bin")
    lc.astype(np.float32).tofile(tmp_path / "lc.bin")
    lp.astype(np.float32).tofile(tmp_path / "lp.bin")
    out = subprocess.run([EXE, str(tmp_path), str(T), str(d_in), str(d_out), str(K), str(S),
                          repr(sigma), repr(gamma), str(seed), str(tag)],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    G_c = np.fromfile(tmp_path / "G.bin", dtype=np.float32).reshape(d_out, d_in)
    yp0_c = np.fromfile(tmp_path / "yp0.bin", dtype=np.uint16).reshape(T, d_out)

    yp = torch.empty((K, T, d_out), dtype=torch.bfloat16, device=DEV)
    dust.dust_noise_inject(bf16(ybits), yp, dust.DUST_BF16, T, d_out, d_out, 0, K, sigma, seed, tag, 0, 0)
    r = torch.empty((K, T), dtype=torch.float32, device=DEV)
    dust.dust_loss_reward(f32(lc), f32(lp), r, K, T, S, gamma)
    gh = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    ght = torch.empty((d_out, T), dtype=torch.bfloat16, device=DEV)
    dust.dust_error_estimate(r, gh, ght, K, K, T, d_out, 0, sigma, seed, tag, 0, 0, 0)
    G = torch.empty((d_out, d_in), dtype=torch.float32, device=DEV)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    dust.dust_weight_grad(ght, bf16(xbits), G, T, d_out, d_in, ws, ws_bytes)
    assert np.array_equal(G_c.view(np.uint32), host_f32(G).view(np.uint32))

    ref = oracle.round_bf16(bits_to_f64(ybits) + sigma * oracle.normals(seed, tag, 0, 0, 0, 1, T, d_out)[0])
    assert np.all(np.abs(bits_to_f64(yp0_c) - ref) <= bf16_ulp(ref))
