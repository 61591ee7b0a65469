"""The estimator chain captured into a HIP graph (torch.cuda.CUDAGraph) replays exactly like the
eager calls (MI355X only).

The library allocates nothing and clears nothing with memset, so a caller may capture a whole
estimate (inject -> loss and reward -> output error -> weight gradient, with a preallocated
weight-gradient workspace) and replay it. Each replay here follows eager work of the program's
own and a synchronisation, and every output is poisoned before the replay and compared with the
eager result bit for bit afterwards.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import DEV, announce, bf16, dust, f32

pytestmark = pytest.mark.gpu


def _chain(buf, stream):
    T, d_out, d_in, K, S, gamma, sigma, seed, tag = buf["shape"]
    dust.dust_noise_inject(buf["y"], buf["yp"], dust.DUST_BF16, T, d_out, d_out, 0, K, sigma, seed,
                           tag, 0, 0, stream)
    dust.dust_loss_reward(buf["lc"], buf["lp"], buf["r"], K, T, S, gamma, stream)
    dust.dust_error_estimate(buf["r"], buf["gh"], buf["ght"], K, K, T, d_out, 0, sigma, seed, tag,
                             0, 0, 0, stream)
    dust.dust_weight_grad(buf["ght"], buf["x"], buf["G"], T, d_out, d_in, buf["ws"],
                          buf["ws_bytes"], stream)


def _buffers(T, d_out, d_in, K, S, gamma, sigma):
    g = np.random.default_rng(41)
    lc, lp = synth.losses(g, K, T)
    ws_bytes = dust.dust_weight_grad_workspace(T, d_out, d_in)
    return {
        "shape": (T, d_out, d_in, K, S, gamma, sigma, 0xC0FFEE, 5),
        "y": bf16(synth.normal_bf16(g, (T, d_out))), "x": bf16(synth.normal_bf16(g, (T, d_in))),
        "lc": f32(lc), "lp": f32(lp),
        "yp": torch.empty((K, T, d_out), dtype=torch.bfloat16, device=DEV),
        "r": torch.empty((K, T), dtype=torch.float32, device=DEV),
        "gh": torch.empty((T, d_out), dtype=torch.float32, device=DEV),
        "ght": torch.empty((d_out, T), dtype=torch.bfloat16, device=DEV),
        "G": torch.empty((d_out, d_in), dtype=torch.float32, device=DEV),
        "ws": torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV), "ws_bytes": ws_bytes,
    }


OUTS = ("yp", "r", "gh", "ght", "G")


@pytest.mark.parametrize("T,d_out,d_in,K,S,gamma", [
    (2048, 256, 128, 16, 512, 0.9),     # small-tile contraction with split partials
    (4096, 1024, 512, 8, 1024, 0.0),    # large-tile contraction with split partials
])
def test_captured_chain_replays_like_eager(T, d_out, d_in, K, S, gamma):
    announce("graph replay %s" % ((T, d_out, d_in, K, S, gamma),))
    buf = _buffers(T, d_out, d_in, K, S, gamma, 0.01)
    assert buf["ws_bytes"] > 0      # the split-K path, whose partials live in the workspace
    _chain(buf, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = {k: buf[k].clone() for k in OUTS}

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        _chain(buf, side.cuda_stream)     # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            _chain(buf, side.cuda_stream)
    torch.cuda.synchronize()

    other = _buffers(T, d_out, d_in, K, S, gamma, 0.02)
    for rep in range(3):
        for k in OUTS:
            buf[k].view(torch.uint8).fill_(0xFF)          # NaN in every float format
        _chain(other, torch.cuda.current_stream().cuda_stream)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(buf[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)


def _attention(buf, stream):
    B, H, S, dh, Kc, sigma, tau, seed, tag = buf["shape"]
    dust.dust_attn_row_weights(buf["P"], buf["v"], buf["g"], buf["W"], buf["Z"], B, H, S, dh, stream)
    dust.dust_attn_key_scores(buf["P"], buf["q"], buf["W"], buf["Z"], buf["ck"], Kc, B, H, S, dh, 0,
                              sigma, tau, seed, tag, 0, 0, stream)
    dust.dust_attn_query_scores(buf["P"], buf["k"], buf["W"], buf["Z"], buf["cq"], Kc, B, H, S, dh,
                                0, sigma, tau, seed, tag + 1, 0, 0, stream)
    dust.dust_attn_value_scores(buf["P"], buf["g"], buf["cv"], Kc, B, H, S, dh, 0, sigma, seed,
                                tag + 2, 0, 0, stream)
    dust.dust_perturbed_linear(buf["y"], buf["wn"], buf["po"], dust.DUST_F32, dust.DUST_ACT_GELU_TANH,
                               B * S, H * dh, 64, 0, Kc, sigma, seed, tag + 3, 0, 0, stream)


def _attention_buffers(B, H, S, dh, Kc, sigma, tau, rng_seed):
    g = np.random.default_rng(rng_seed)
    T, d = B * S, H * dh
    z = g.standard_normal((B, H, S, S))
    z = np.where(np.tril(np.ones((S, S), dtype=bool)), z, -np.inf)
    P = np.exp(z - z.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    nb = lambda shape: bf16(synth.normal_bf16(g, shape))
    return {
        "shape": (B, H, S, dh, Kc, sigma, tau, 0xBEEF, 21),
        "P": torch.from_numpy(P.astype(np.float32)).to(DEV).to(torch.bfloat16).contiguous(),
        "q": nb((T, d)), "k": nb((T, d)), "v": nb((T, d)), "g": nb((T, d)), "y": nb((T, d)),
        "wn": nb((64, d)),
        "W": torch.empty((B, H, S, S), dtype=torch.float32, device=DEV),
        "Z": torch.empty((B, H, S), dtype=torch.float32, device=DEV),
        "ck": torch.empty((Kc, T), dtype=torch.float32, device=DEV),
        "cq": torch.empty((Kc, T), dtype=torch.float32, device=DEV),
        "cv": torch.empty((Kc, T), dtype=torch.float32, device=DEV),
        "po": torch.empty((Kc, T, 64), dtype=torch.float32, device=DEV),
    }


AOUTS = ("W", "Z", "ck", "cq", "cv", "po")


@pytest.mark.parametrize("sigma", [0.05, 20.0])   # the second sends rows through the repair pass
# the second shape (16 sequences x 201 draws) runs the query scores on 8 waves of two draws on a
# 256-CU device, the first on 12 waves of one
@pytest.mark.parametrize("B,H,S,dh,Kc", [(1, 2, 128, 32, 6), (16, 2, 64, 32, 201)])
def test_captured_attention_scores_replay_like_eager(sigma, B, H, S, dh, Kc):
    """Row weights, the three attention scorers (the key and query scores with their repair pass)
    and the perturbed down-projection, captured and replayed: bit-identical to the eager calls."""
    announce("graph replay attention sigma=%g shape %s" % (sigma, (B, H, S, dh, Kc)))
    tau = 0.18
    buf = _attention_buffers(B, H, S, dh, Kc, sigma, tau, 43)
    _attention(buf, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = {k: buf[k].clone() for k in AOUTS}
    for k in ("ck", "cq", "cv"):
        assert torch.isfinite(ref[k]).all(), k

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        _attention(buf, side.cuda_stream)
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            _attention(buf, side.cuda_stream)
    torch.cuda.synchronize()

    other = _attention_buffers(B, H, S, dh, Kc, sigma / 2, tau, 44)
    for rep in range(3):
        for k in AOUTS:
            buf[k].view(torch.uint8).fill_(0xFF)
        _attention(other, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in AOUTS:
            assert torch.equal(buf[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
