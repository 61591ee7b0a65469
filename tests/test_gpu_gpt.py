"""The whole estimator inside a small random-weight GPT, against autograd (MI355X only).

A 2-block causal GPT (vocabulary 128, width 64, 4 heads, MLP 256, 8 sequences of 64 tokens,
seeded weights; the forward is a torch harness: the model's forward is not the library's job)
gives two perturbed layers of different types: block 0's MLP up-projection (its output reaches
later tokens only through block 1's attention) and block 1's attention value projection (its
output is mixed across tokens directly). For each, the library runs the chain -- inject, the
harness's suffix forward per draw, loss change and reward, output error, weight gradient -- and
the estimate is compared with autograd.

What the estimate converges to follows from the explainer's "Credit assignment" definitions: to
first order in sigma, c_s = -sigma sum_u (dl_s/dy_u) a_u with independent unit noise per token,
so E[g_hat_t] = sum_{s >= t} gamma^(s-t) dl_s/dy_t and the weight gradient tends to
G_gamma = sum_t x_t E[g_hat_t]^T. gamma = 1 gives autograd's gradient of the summed loss (a
token's output only reaches its own and later losses); gamma < 1 discounts the credit a token
gets for later tokens' losses, so G_gamma differs from it. The test assembles G_gamma from
autograd's per-loss gradients, checks G_1 against autograd's own weight gradient, and requires
  - the estimate's cosine with its own limit G_gamma to grow with K;
  - the law cos(K) = c_max / sqrt(1 + c / K) (explainer, "Gradients grow") fitted to the cosine
    with autograd's gradient to give c_max = cos(G_gamma, G_true) within 0.02;
  - the gamma = 1 estimate to approach autograd's gradient itself.
"""
import numpy as np
import pytest
import torch
from scipy.optimize import curve_fit

from gpu_helpers import DEV, announce, dust

pytestmark = pytest.mark.gpu

V, DM, NH, S, B = 128, 64, 4, 64, 8
T, DF = B * S, 4 * DM
SIGMA, SEED, TAG = 0.01, 0xD057, 3
KS = (256, 1024, 4096, 16384)


def _model():
    g = np.random.default_rng(7)

    def w(*shape, std=None):
        std = std if std is not None else 1.0 / np.sqrt(shape[-1])
        return torch.tensor(g.standard_normal(shape) * std, dtype=torch.float32, device=DEV)

    P = {"emb": w(V, DM, std=1.0), "pos": w(S, DM, std=0.5), "head": w(V, DM)}
    for l in range(2):
        P["qkv%d" % l], P["ao%d" % l] = w(3 * DM, DM), w(DM, DM)
        P["fc%d" % l], P["pr%d" % l] = w(DF, DM), w(DM, DF)
    tok = torch.tensor(g.integers(0, V, (B, S)), device=DEV)
    tgt = torch.tensor(g.integers(0, V, (B, S)), device=DEV)
    return P, tok, tgt


def _ln(x):
    return torch.nn.functional.layer_norm(x, (x.shape[-1],))


def _attend(q, k, v):
    n = q.shape[0]
    sh = lambda a: a.reshape(n, S, NH, DM // NH).permute(0, 2, 1, 3)
    sc = (sh(q) @ sh(k).transpose(-1, -2)) / np.sqrt(DM // NH)
    mask = torch.ones(S, S, dtype=torch.bool, device=DEV).tril()
    o = torch.softmax(sc.masked_fill(~mask, float("-inf")), -1) @ sh(v)
    return o.permute(0, 2, 1, 3).reshape(n, S, DM)


class Net:
    """The harness forward, split at one layer's output y = x W^T."""

    def __init__(self, layer):
        self.P, self.tok, self.tgt = _model()
        self.layer = layer
        self.wkey, self.rows = ("fc0", slice(0, DF)) if layer == "mlp_up" else ("qkv1", slice(2 * DM, 3 * DM))

    def weight(self):
        return self.P[self.wkey][self.rows]

    def losses(self, h):
        z = _ln(h) @ self.P["head"].T
        n = h.shape[0] // B
        return torch.nn.functional.cross_entropy(z.reshape(-1, V), self.tgt.repeat(n, 1).reshape(-1),
                                                 reduction="none").reshape(n, T)

    def block(self, h, l):
        a = _ln(h)
        q, k, v = (a @ self.P["qkv%d" % l].T).split(DM, -1)
        h = h + _attend(q, k, v) @ self.P["ao%d" % l].T
        return h + torch.nn.functional.gelu(_ln(h) @ self.P["fc%d" % l].T) @ self.P["pr%d" % l].T

    def prefix(self, W):
        """(context, x, y) with y = x W^T the perturbed layer's output."""
        P = self.P
        h = P["emb"][self.tok] + P["pos"][None]
        if self.layer == "mlp_up":
            a = _ln(h)
            q, k, v = (a @ P["qkv0"].T).split(DM, -1)
            h = h + _attend(q, k, v) @ P["ao0"].T
            x = _ln(h)
            return h, x, x @ W.T
        h = self.block(h, 0)
        a = _ln(h)
        q, k, _ = (a @ P["qkv1"].T).split(DM, -1)
        return (h, q, k), a, a @ W.T

    def suffix_losses(self, ctx, y):
        """Per-token losses [n, T] for n copies of the batch with the layer output y [n*B, S, d]."""
        P = self.P
        n = y.shape[0] // B
        if self.layer == "mlp_up":
            h = ctx.repeat(n, 1, 1) + torch.nn.functional.gelu(y) @ P["pr0"].T
            return self.losses(self.block(h, 1))
        h, q, k = ctx
        h = h.repeat(n, 1, 1) + _attend(q.repeat(n, 1, 1), k.repeat(n, 1, 1), y) @ P["ao1"].T
        h = h + torch.nn.functional.gelu(_ln(h) @ P["fc1"].T) @ P["pr1"].T
        return self.losses(h)


def _cos(a, b):
    return float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()))


def _limits(net):
    """autograd's weight gradient of the summed loss, and sum_t x_t (dl_s/dy_t)_{s,t} per sequence."""
    W = net.weight().clone().requires_grad_(True)
    ctx, x, y = net.prefix(W)
    net.suffix_losses(ctx, y).sum().backward()
    G_true = W.grad.double().cpu().numpy()
    with torch.no_grad():
        ctx, x, y = net.prefix(net.weight())
    d = y.shape[-1]
    J = torch.zeros((S, B, S, d), dtype=torch.float64, device=DEV)   # dl_{b,s} / dy_{b,t}
    for s in range(S):
        yv = y.detach().clone().requires_grad_(True)
        l = net.suffix_losses(ctx, yv).reshape(B, S)[:, s].sum()
        (gy,) = torch.autograd.grad(l, yv)
        J[s] = gy.double()
    return G_true, J, x.detach().double()


def _G_gamma(J, x, gamma):
    s, t = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    wts = torch.tensor(np.where(s >= t, gamma ** np.maximum(s - t, 0), 0.0), dtype=torch.float64,
                       device=DEV)
    g = torch.einsum("st,sbtf->btf", wts, J)
    return torch.einsum("btf,btm->fm", g, x).cpu().numpy()


def _estimate(net, K, gamma, chunk=512):
    with torch.no_grad():
        ctx, x, y = net.prefix(net.weight())
        d = y.shape[-1]
        yf = y.reshape(T, d).contiguous()
        lc = net.suffix_losses(ctx, y)[0].contiguous()
        lp = torch.empty((K, T), dtype=torch.float32, device=DEV)
        for k0 in range(0, K, chunk):
            kc = min(chunk, K - k0)
            yp = torch.empty((kc, T, d), dtype=torch.float32, device=DEV)
            dust.dust_noise_inject(yf, yp, dust.DUST_F32, T, d, d, 0, kc, SIGMA, SEED, TAG, k0, 0)
            lp[k0:k0 + kc] = net.suffix_losses(ctx, yp.reshape(kc * B, S, d))
        r = torch.empty_like(lp)
        dust.dust_loss_reward(lc, lp, r, K, T, S, gamma)
        gh = torch.empty((T, d), dtype=torch.float32, device=DEV)
        ght = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
        dust.dust_error_estimate(r, gh, ght, K, K, T, d, 0, SIGMA, SEED, TAG, 0, 0, 0)
        xb = x.reshape(T, DM).to(torch.bfloat16).contiguous()
        G = torch.empty((d, DM), dtype=torch.float32, device=DEV)
        ws_bytes = dust.dust_weight_grad_workspace(T, d, DM)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
        dust.dust_weight_grad(ght, xb, G, T, d, DM, ws, ws_bytes)
        torch.cuda.synchronize()
        return G.double().cpu().numpy()


@pytest.mark.parametrize("layer", ["mlp_up", "attn_v"])
def test_estimate_converges_to_its_credit_assignment_limit(layer):
    announce("gpt %s" % layer)
    net = Net(layer)
    G_true, J, x = _limits(net)
    assert _cos(_G_gamma(J, x, 1.0), G_true) > 0.99999      # gamma = 1 is the full gradient
    law = lambda K, cm, c: cm / np.sqrt(1 + c / K)
    for gamma in (0.0, 0.9):
        G_lim = _G_gamma(J, x, gamma)
        ests = [_estimate(net, K, gamma) for K in KS]
        to_lim = [_cos(G, G_lim) for G in ests]
        to_true = np.array([_cos(G, G_true) for G in ests])
        print("%s gamma %.1f: cos to limit %s, to autograd %s, limit vs autograd %.4f"
              % (layer, gamma, np.round(to_lim, 4), np.round(to_true, 4), _cos(G_lim, G_true)))
        assert all(b > a for a, b in zip(to_lim, to_lim[1:]))
        (c_max, _), _ = curve_fit(law, np.array(KS, dtype=float), to_true, p0=(1.0, 100.0),
                                  bounds=([0.0, 0.0], [2.0, 1e9]))
        assert abs(c_max - _cos(G_lim, G_true)) <= 0.02, (c_max, _cos(G_lim, G_true))
    to_true = [_cos(_estimate(net, K, 1.0), G_true) for K in KS]
    print("%s gamma 1.0: cos to autograd %s" % (layer, np.round(to_true, 4)))
    assert all(b > a for a, b in zip(to_true, to_true[1:])) and to_true[-1] >= 0.7


# ------------------------------------------------------------------------------ layer-type groups
# The explainer ("The real work: suppressing interference") perturbs several layers of one type
# in the same forward, each with its own noise, and gives every layer type its own forward and
# its own sigma. Here both blocks' MLP up-projections form one group: one forward per draw
# perturbs both, under distinct tags, and each layer's estimate is formed from the same per-token
# loss changes. To first order in sigma the other layer's noise adds a zero-mean term to every
# loss change, so it adds variance but no bias: at a fixed population the group's cosines sit
# below the single-layer ones (a larger c in the law cos(K) = c_max / sqrt(1 + c/K) of "Gradients
# grow"), while the fitted c_max stays that of the single layer -- the estimate recovers with K.
# A second layer type in the same forward at its own, larger sigma (block 1's attention value
# projection) swamps the group's loss changes: that is why layer types get separate forwards.
GROUP_TAGS = {"fc0": 11, "fc1": 12, "v1": 13}
GROUP_KS = (256, 1024, 4096, 16384)


class GroupNet:
    """The harness forward with optional noise on block 0's and block 1's MLP up-projection
    outputs and on block 1's attention values."""

    def __init__(self):
        self.P, self.tok, self.tgt = _model()

    def forward(self, n=1, W=None, noise=None):
        """Per-token losses [n, T] of n copies of the batch, and the clean inputs of the two
        up-projections; noise maps a layer ('fc0', 'fc1', 'v1') to [n*B, S, width] additions."""
        P, W, noise = self.P, W or {}, noise or {}
        h = (P["emb"][self.tok] + P["pos"][None]).repeat(n, 1, 1)
        a = _ln(h)
        q, k, v = (a @ P["qkv0"].T).split(DM, -1)
        h = h + _attend(q, k, v) @ P["ao0"].T
        x0 = _ln(h)
        y0 = x0 @ W.get("fc0", P["fc0"]).T
        if "fc0" in noise:
            y0 = y0 + noise["fc0"]
        h = h + torch.nn.functional.gelu(y0) @ P["pr0"].T
        a = _ln(h)
        q, k, v = (a @ P["qkv1"].T).split(DM, -1)
        if "v1" in noise:
            v = v + noise["v1"]
        h = h + _attend(q, k, v) @ P["ao1"].T
        x1 = _ln(h)
        y1 = x1 @ W.get("fc1", P["fc1"]).T
        if "fc1" in noise:
            y1 = y1 + noise["fc1"]
        h = h + torch.nn.functional.gelu(y1) @ P["pr1"].T
        z = _ln(h) @ P["head"].T
        l = torch.nn.functional.cross_entropy(z.reshape(-1, V), self.tgt.repeat(n, 1).reshape(-1),
                                              reduction="none").reshape(n, T)
        return l, x0, x1


def _group_truth(net):
    W = {k: net.P[k].clone().requires_grad_(True) for k in ("fc0", "fc1")}
    l, _, _ = net.forward(W=W)
    l.sum().backward()
    return {k: W[k].grad.double().cpu().numpy() for k in W}


def _group_estimate(net, K, sigmas, estimated, chunk=512):
    """One forward per draw with every layer in `sigmas` perturbed (its own tag and sigma); the
    library's chain turns the shared loss changes into each estimated layer's weight gradient."""
    width = {"fc0": DF, "fc1": DF, "v1": DM}
    with torch.no_grad():
        lc, x0, x1 = net.forward()
        lc = lc[0].contiguous()
        xs = {"fc0": x0, "fc1": x1}
        lp = torch.empty((K, T), dtype=torch.float32, device=DEV)
        for k0 in range(0, K, chunk):
            kc = min(chunk, K - k0)
            noise = {}
            for layer, sg in sigmas.items():
                d = width[layer]
                zero = torch.zeros((T, d), dtype=torch.float32, device=DEV)
                a = torch.empty((kc, T, d), dtype=torch.float32, device=DEV)
                dust.dust_noise_inject(zero, a, dust.DUST_F32, T, d, d, 0, kc, sg, SEED,
                                       GROUP_TAGS[layer], k0, 0)          # sigma a, draws k0..
                noise[layer] = a.reshape(kc * B, S, d)
            lp[k0:k0 + kc] = net.forward(kc, noise=noise)[0]
        r = torch.empty_like(lp)
        dust.dust_loss_reward(lc, lp, r, K, T, S, 0.0)
        out = {}
        for layer in estimated:
            d, sg = width[layer], sigmas[layer]
            gh = torch.empty((T, d), dtype=torch.float32, device=DEV)
            ght = torch.empty((d, T), dtype=torch.bfloat16, device=DEV)
            dust.dust_error_estimate(r, gh, ght, K, K, T, d, 0, sg, SEED, GROUP_TAGS[layer], 0, 0, 0)
            xb = xs[layer].reshape(T, DM).to(torch.bfloat16).contiguous()
            G = torch.empty((d, DM), dtype=torch.float32, device=DEV)
            ws_bytes = dust.dust_weight_grad_workspace(T, d, DM)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
            dust.dust_weight_grad(ght, xb, G, T, d, DM, ws, ws_bytes)
            out[layer] = G
        torch.cuda.synchronize()
        return {k: v.double().cpu().numpy() for k, v in out.items()}


def test_layer_type_group_interference():
    announce("gpt layer-type group")
    net = GroupNet()
    G_true = _group_truth(net)
    law = lambda K, cm, c: cm / np.sqrt(1 + c / K)
    runs = {
        "alone": {layer: [_group_estimate(net, K, {layer: SIGMA}, [layer])[layer]
                          for K in GROUP_KS] for layer in ("fc0", "fc1")},
        "group": [_group_estimate(net, K, {"fc0": SIGMA, "fc1": SIGMA}, ["fc0", "fc1"])
                  for K in GROUP_KS],
        "mixed": [_group_estimate(net, K, {"fc0": SIGMA, "fc1": SIGMA, "v1": 0.3},
                                  ["fc0", "fc1"]) for K in GROUP_KS[:3]],
    }
    for layer in ("fc0", "fc1"):
        alone = np.array([_cos(G, G_true[layer]) for G in runs["alone"][layer]])
        group = np.array([_cos(run[layer], G_true[layer]) for run in runs["group"]])
        mixed = np.array([_cos(run[layer], G_true[layer]) for run in runs["mixed"]])
        fa, _ = curve_fit(law, np.array(GROUP_KS, float), alone, p0=(1.0, 100.0),
                          bounds=([0.0, 0.0], [2.0, 1e9]))
        fg, _ = curve_fit(law, np.array(GROUP_KS, float), group, p0=(1.0, 100.0),
                          bounds=([0.0, 0.0], [2.0, 1e9]))
        print("%s: alone cos %s (c_max %.3f, c %.0f); group cos %s (c_max %.3f, c %.0f); "
              "with attention values at sigma 0.3 in the same forward: cos %s"
              % (layer, np.round(alone, 4), fa[0], fa[1], np.round(group, 4), fg[0], fg[1],
                 np.round(mixed, 4)))
        # interference: lower cosines at every population up to 4096 draws, a larger c
        assert np.all(group[:3] < alone[:3])
        assert fg[1] > 1.3 * fa[1]
        # no bias: the group's estimate recovers with K towards the single layer's limit
        assert all(b > a for a, b in zip(group, group[1:]))
        assert abs(fg[0] - fa[0]) <= 0.02
        # another layer type at a larger sigma in the same forward swamps the group
        assert mixed[-1] < 0.5 * group[2]
