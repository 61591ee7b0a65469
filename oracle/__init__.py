"""Dust gradient estimator -- CPU ORACLE. TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 statement of what the Dust estimator computes, used to check the HIP library.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. It shares no code with ``activation_perturbation_es_amd`` and never imports
it. The element loops live in ``dust_oracle.c`` (plain C, fp64); this module marshals numpy
arrays to it and states the two steps that are library primitives (a matrix product) or small
closed forms (the tiny linear + softmax model) in numpy.

Method source: the "Dust" explainer at cnblogs.com/32bin/p/23212811, sections
"Credit assignment: one forward, two rewards" (noise, loss change, reward, error estimate,
weight gradient) and "The real work: suppressing interference" (attention scoring, LM-head
chunk). Generator: Philox4x32-10 (Salmon et al., SC'11) and Box-Muller; the counter layout is
stated in ``dust_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dust_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdust_oracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64


def build(force: bool = False) -> str:
    """Compile dust_oracle.c into libdust_oracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _configure(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures on a loaded oracle library."""
    lib.dust_or_philox4x32_10.argtypes = [ctypes.POINTER(_u32), ctypes.POINTER(_u32),
                                          ctypes.POINTER(_u32)]
    lib.dust_or_attn_value_scores.argtypes = [_d, _d, _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                              _u64, _u32, _u32, _u32, _i64, _d]
    lib.dust_or_attn_value_scores_at.argtypes = [_d, _d, _i64, _i64, _i64, _i64, ctypes.c_double,
                                                 _u64, _u32, _u32, _u32, _i64,
                                                 ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i64,
                                                 _d]
    lib.dust_or_attn_key_scores.argtypes = [_d, _d, _d, _d, _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_double, ctypes.c_double, _u64, _u32, _u32,
                                            _u32, _i64, _d]
    lib.dust_or_attn_key_scores_at.argtypes = [_d, _d, _d, _d, _i64, _i64, _i64, ctypes.c_double,
                                               ctypes.c_double, _u64, _u32, _u32, _u32, _i64,
                                               ctypes.POINTER(_i64), ctypes.POINTER(_i64), _i64,
                                               _d]
    lib.dust_or_attn_query_scores.argtypes = lib.dust_or_attn_key_scores.argtypes
    lib.dust_or_attn_row_weights.argtypes = [_d, _d, _d, _i64, _i64, _i64, _i64, _d, _d]
    lib.dust_or_attn_query_scores_at.argtypes = lib.dust_or_attn_key_scores_at.argtypes
    lib.dust_or_sgd_momentum.argtypes = [_d, _d, _d, _i64, ctypes.c_double, ctypes.c_double]
    lib.dust_or_adam.argtypes = [_d, _d, _d, _d, _i64, ctypes.c_double, ctypes.c_double,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_double, _i64]
    lib.dust_or_noise_words.argtypes = [_u64, _u32, _u32, _u32, _u32, ctypes.POINTER(_u32)]
    lib.dust_or_uniform.argtypes = [_u32]
    lib.dust_or_uniform.restype = ctypes.c_double
    lib.dust_or_angle.argtypes = [_u32]
    lib.dust_or_angle.restype = ctypes.c_double
    lib.dust_or_box_muller.argtypes = [_u32, _u32, ctypes.c_int]
    lib.dust_or_box_muller.restype = ctypes.c_double
    lib.dust_or_normal.argtypes = [_u64, _u32, _u32, _u32, _u64]
    lib.dust_or_normal.restype = ctypes.c_double
    lib.dust_or_normals.argtypes = [_u64, _u32, _u32, _u32, _i64, _i64, _i64, _i64, _d]
    lib.dust_or_noise_inject.argtypes = [_d, _i64, _i64, _i64, _i64, _i64, ctypes.c_double, _u64,
                                         _u32, _u32, _u32, _d]
    lib.dust_or_loss_delta_loss.argtypes = [_d, _d, _i64, _i64, _d]
    lib.dust_or_loss_delta_inner.argtypes = [_d, _d, _i64, _i64, _i64, _d]
    lib.dust_or_reward_scan.argtypes = [_d, _i64, _i64, _i64, ctypes.c_double, _d]
    lib.dust_or_error_estimate.argtypes = [_d, _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                           _u64, _u32, _u32, _u32, ctypes.c_int, _d]
    lib.dust_or_error_estimate_at.argtypes = [_d, _i64, _i64, _i64, _i64, ctypes.c_double, _u64,
                                              _u32, _u32, _u32, ctypes.POINTER(_i64),
                                              ctypes.POINTER(_i64), _i64, _d]
    lib.dust_or_head_ce_chunk.argtypes = [_d, ctypes.POINTER(ctypes.c_int32), _i64, _i64, _i64,
                                          _i64, _i64, ctypes.c_double, _u64, _u32, _u32, _u32,
                                          _d, _d]
    _pi64 = ctypes.POINTER(_i64)
    lib.dust_or_normals_at.argtypes = [_u64, _u32, _u32, _u32, _i64, _pi64, _pi64, _pi64, _i64, _d]
    lib.dust_or_head_ce_at.argtypes = [_d, ctypes.POINTER(ctypes.c_int32), _i64, _i64, _i64, _i64,
                                       ctypes.c_double, _u64, _u32, _u32, _u32, _pi64, _pi64, _i64,
                                       _d]
    lib.dust_or_activation.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.dust_or_activation.restype = ctypes.c_double
    lib.dust_or_perturbed_linear.argtypes = [_d, _d, _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                             _u64, _u32, _u32, _u32, ctypes.c_int, _d]
    lib.dust_or_perturbed_rows_at.argtypes = [_d, _i64, _i64, ctypes.c_double, _u64, _u32, _u32,
                                              _u32, ctypes.c_int, _pi64, _pi64, _i64, _d]
    lib.dust_or_threads.restype = ctypes.c_int
    lib.dust_or_round_bf16.argtypes = [ctypes.c_double]
    lib.dust_or_round_bf16.restype = ctypes.c_double
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_d)


def threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().dust_or_threads())


# ------------------------------------------------------------------------------ generator
def philox4x32_10(counter, key) -> np.ndarray:
    """Philox4x32-10 (SC'11) of one 4-word counter under a 2-word key."""
    lib = _load()
    c = (_u32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (_u32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (_u32 * 4)()
    lib.dust_or_philox4x32_10(c, k, out)
    return np.array(list(out), dtype=np.uint32)


def noise_words(seed: int, tag: int, draw: int, token: int, q: int) -> np.ndarray:
    """Words carrying channels 4q..4q+3 of (draw, token): counter (q, token, draw, tag)."""
    lib = _load()
    out = (_u32 * 4)()
    lib.dust_or_noise_words(seed, tag, draw, token, q, out)
    return np.array(list(out), dtype=np.uint32)


def uniform(w: int) -> float:
    """Radius uniform u(w) in (0, 1)."""
    return _load().dust_or_uniform(int(w) & 0xFFFFFFFF)


def angle(w: int) -> float:
    """Angle uniform v(w) in [0, 1), in turns."""
    return _load().dust_or_angle(int(w) & 0xFFFFFFFF)


def box_muller(wa: int, wb: int, sine: bool) -> float:
    """One normal of the word pair (wa, wb): rho(wa) sin or cos (2 pi v(wb))."""
    return _load().dust_or_box_muller(int(wa) & 0xFFFFFFFF, int(wb) & 0xFFFFFFFF, int(bool(sine)))


def normal(seed: int, tag: int, draw: int, token: int, ch: int) -> float:
    """a^{(draw)}_{token, ch} ~ N(0, 1)."""
    return _load().dust_or_normal(seed, tag, draw, token, ch)


def normals(seed: int, tag: int, draw0: int, tok0: int, chan0: int, K: int, T: int, d: int) -> np.ndarray:
    """Normals for draws draw0.., tokens tok0.., channels chan0..: array [K, T, d]."""
    out = np.empty((K, T, d), dtype=np.float64)
    _load().dust_or_normals(seed, tag, draw0, tok0, chan0, K, T, d, _p(out))
    return out


def _idx(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


def _pidx(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(_i64))


def normals_at(seed: int, tag: int, k, t, j, draw0: int = 0, tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """Normals at chosen local (draw, token, channel) triples."""
    k, t, j = _idx(k), _idx(t), _idx(j)
    out = np.empty(len(k), dtype=np.float64)
    _load().dust_or_normals_at(seed, tag, draw0, tok0, chan0, _pidx(k), _pidx(t), _pidx(j), len(k),
                               _p(out))
    return out


# ------------------------------------------------------------------------------ estimator steps
def noise_inject(y, sigma: float, K: int, seed: int, tag: int, draw0: int = 0, tok0: int = 0,
                 chan0: int = 0, d: int | None = None) -> np.ndarray:
    """y'^{(i)}_t = y_t + sigma a^{(i)}_t for i = draw0 .. draw0+K-1: returns [K, T, d] fp64."""
    y = _f64(y)
    T, ld = y.shape
    d = ld if d is None else d
    out = np.empty((K, T, d), dtype=np.float64)
    _load().dust_or_noise_inject(_p(y), T, d, ld, chan0, K, sigma, seed, tag, draw0, tok0, _p(out))
    return out


def loss_delta_loss(loss_clean, loss_pert) -> np.ndarray:
    """c^{(i)}_t = l_clean,t - l^{(i)}_pert,t: returns [K, T]."""
    lc, lp = _f64(loss_clean), _f64(loss_pert)
    K, T = lp.shape
    c = np.empty((K, T), dtype=np.float64)
    _load().dust_or_loss_delta_loss(_p(lc), _p(lp), K, T, _p(c))
    return c


def loss_delta_inner(delta_o, g_o) -> np.ndarray:
    """c^{(i)}_s = -<delta_o^{(i)}_s, g^o_s>: delta_o [K, T, d], g_o [T, d] -> [K, T]."""
    do, go = _f64(delta_o), _f64(g_o)
    K, T, d = do.shape
    c = np.empty((K, T), dtype=np.float64)
    _load().dust_or_loss_delta_inner(_p(do), _p(go), K, T, d, _p(c))
    return c


def attn_value_scores(P, g_o, K: int, sigma: float, seed: int, tag: int, draw0: int = 0,
                      tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """Scores c [K, T] of K draws perturbing an attention value projection (dust_oracle.c
    states the formula): P [B, H, S, S] attention weights (query rows), g_o [T, H*dh]."""
    Pd, gd = _f64(P), _f64(g_o)
    B, H, S, _ = Pd.shape
    T = B * S
    dh = gd.shape[1] // H
    c = np.empty((K, T), dtype=np.float64)
    _load().dust_or_attn_value_scores(_p(Pd), _p(gd), K, B, H, S, dh, sigma, seed, tag, draw0,
                                      tok0, chan0, _p(c))
    return c


def attn_value_scores_at(P, g_o, k, t, sigma: float, seed: int, tag: int, draw0: int = 0,
                         tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """attn_value_scores at chosen local (draw, token) pairs."""
    Pd, gd = _f64(P), _f64(g_o)
    B, H, S, _ = Pd.shape
    dh = gd.shape[1] // H
    k, t = _idx(k), _idx(t)
    out = np.empty(len(k), dtype=np.float64)
    _load().dust_or_attn_value_scores_at(_p(Pd), _p(gd), B, H, S, dh, sigma, seed, tag, draw0,
                                         tok0, chan0, _pidx(k), _pidx(t), len(k), _p(out))
    return out


def attn_key_scores(P, q, v, g_o, K: int, sigma: float, tau: float, seed: int, tag: int,
                    draw0: int = 0, tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """Scores c [K, T] of K draws perturbing an attention key projection (dust_oracle.c states
    the formula): P [B, H, S, S] attention weights (query rows), q, v, g_o [T, H*dh], tau the
    softmax scale."""
    Pd, qd, vd, gd = _f64(P), _f64(q), _f64(v), _f64(g_o)
    B, H, S, _ = Pd.shape
    T = B * S
    dh = gd.shape[1] // H
    c = np.empty((K, T), dtype=np.float64)
    _load().dust_or_attn_key_scores(_p(Pd), _p(qd), _p(vd), _p(gd), K, B, H, S, dh, sigma, tau,
                                    seed, tag, draw0, tok0, chan0, _p(c))
    return c


def attn_key_scores_at(P, q, v, g_o, k, t, sigma: float, tau: float, seed: int, tag: int,
                       draw0: int = 0, tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """attn_key_scores at chosen local (draw, token) pairs."""
    Pd, qd, vd, gd = _f64(P), _f64(q), _f64(v), _f64(g_o)
    B, H, S, _ = Pd.shape
    dh = gd.shape[1] // H
    k, t = _idx(k), _idx(t)
    out = np.empty(len(k), dtype=np.float64)
    _load().dust_or_attn_key_scores_at(_p(Pd), _p(qd), _p(vd), _p(gd), H, S, dh, sigma, tau, seed,
                                       tag, draw0, tok0, chan0, _pidx(k), _pidx(t), len(k),
                                       _p(out))
    return out


def attn_row_weights(P, v, g_o):
    """Draw-independent row weights of the softmax re-run (dust_oracle.c states the formula):
    W [B, H, S, S] with W_ts = P_ts (Z_t u_ts - base_t) on and below the diagonal, 0 above it,
    and the causal row sums Z [B, H, S]; P [B, H, S, S], v, g_o [T, H*dh]."""
    Pd, vd, gd = _f64(P), _f64(v), _f64(g_o)
    B, H, S, _ = Pd.shape
    dh = gd.shape[1] // H
    W = np.empty((B, H, S, S), dtype=np.float64)
    Z = np.empty((B, H, S), dtype=np.float64)
    _load().dust_or_attn_row_weights(_p(Pd), _p(vd), _p(gd), B, H, S, dh, _p(W), _p(Z))
    return W, Z


def attn_query_scores(P, k, v, g_o, K: int, sigma: float, tau: float, seed: int, tag: int,
                      draw0: int = 0, tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """Scores c [K, T] of K draws perturbing an attention query projection (dust_oracle.c states
    the formula): P [B, H, S, S] attention weights (query rows), k, v, g_o [T, H*dh], tau the
    softmax scale."""
    Pd, kd, vd, gd = _f64(P), _f64(k), _f64(v), _f64(g_o)
    B, H, S, _ = Pd.shape
    T = B * S
    dh = gd.shape[1] // H
    c = np.empty((K, T), dtype=np.float64)
    _load().dust_or_attn_query_scores(_p(Pd), _p(kd), _p(vd), _p(gd), K, B, H, S, dh, sigma, tau,
                                      seed, tag, draw0, tok0, chan0, _p(c))
    return c


def attn_query_scores_at(P, k, v, g_o, kk, t, sigma: float, tau: float, seed: int, tag: int,
                         draw0: int = 0, tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """attn_query_scores at chosen local (draw, token) pairs."""
    Pd, kd, vd, gd = _f64(P), _f64(k), _f64(v), _f64(g_o)
    B, H, S, _ = Pd.shape
    dh = gd.shape[1] // H
    kk, t = _idx(kk), _idx(t)
    out = np.empty(len(kk), dtype=np.float64)
    _load().dust_or_attn_query_scores_at(_p(Pd), _p(kd), _p(vd), _p(gd), H, S, dh, sigma, tau,
                                         seed, tag, draw0, tok0, chan0, _pidx(kk), _pidx(t),
                                         len(kk), _p(out))
    return out


def cosine_terms(a, b) -> np.ndarray:
    """(sum a b, sum a^2, sum b^2) of two arrays in fp64: the sums of their cosine."""
    a, b = _f64(a).ravel(), _f64(b).ravel()
    return np.array([np.dot(a, b), np.dot(a, a), np.dot(b, b)])


def reward_scan(c, seg_len: int, gamma: float) -> np.ndarray:
    """r_t = sum_{s>=t in t's sequence} gamma^(s-t) c_s along the last axis of c [K, T]."""
    c = _f64(c)
    K, T = c.shape
    assert T % seg_len == 0
    r = np.empty_like(c)
    _load().dust_or_reward_scan(_p(c), K, T, seg_len, gamma, _p(r))
    return r


def error_estimate(r, d: int, sigma: float, seed: int, tag: int, draw0: int = 0, tok0: int = 0,
                   chan0: int = 0, K_total: int | None = None, g_in=None) -> np.ndarray:
    """g_t = -(1/(K_total sigma)) sum_i r^{(i)}_t a^{(i)}_t (+ g_in): r [K, T] -> [T, d]."""
    r = _f64(r)
    K, T = r.shape
    K_total = K if K_total is None else K_total
    g = np.zeros((T, d), dtype=np.float64) if g_in is None else _f64(g_in).copy()
    _load().dust_or_error_estimate(_p(r), K, K_total, T, d, chan0, sigma, seed, tag, draw0, tok0,
                                   0 if g_in is None else 1, _p(g))
    return g


def error_estimate_at(r, tok, ch, sigma: float, seed: int, tag: int, draw0: int = 0, tok0: int = 0,
                      chan0: int = 0, K_total: int | None = None) -> np.ndarray:
    """g at chosen (token, channel) pairs only (no accumulate term)."""
    r = _f64(r)
    K, T = r.shape
    K_total = K if K_total is None else K_total
    tok = np.ascontiguousarray(tok, dtype=np.int64)
    ch = np.ascontiguousarray(ch, dtype=np.int64)
    out = np.empty(len(tok), dtype=np.float64)
    _load().dust_or_error_estimate_at(_p(r), K, K_total, T, chan0, sigma, seed, tag, draw0, tok0,
                                      tok.ctypes.data_as(ctypes.POINTER(_i64)),
                                      ch.ctypes.data_as(ctypes.POINTER(_i64)), len(tok), _p(out))
    return out


def weight_grad(g_hat, x) -> np.ndarray:
    """G_W = sum_t g_t x_t^T (explainer, "Credit assignment", weight-gradient outer product),
    taken as one fp64 library matrix product: g_hat [T, d_out], x [T, d_in] -> [d_out, d_in]."""
    return _f64(g_hat).T @ _f64(x)


def head_ce_chunk(logits, targets, v0: int, C: int, K: int, sigma: float, seed: int, tag: int,
                  draw0: int = 0, tok0: int = 0):
    """Per-token cross-entropy with vocabulary chunk [v0, v0+C) perturbed, all other logits
    clean: returns (loss_pert [K, T], loss_clean [T])."""
    z = _f64(logits)
    T, V = z.shape
    y = np.ascontiguousarray(targets, dtype=np.int32)
    lp = np.empty((K, T), dtype=np.float64)
    lc = np.empty(T, dtype=np.float64)
    _load().dust_or_head_ce_chunk(_p(z), y.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), T, V, v0,
                                  C, K, sigma, seed, tag, draw0, tok0, _p(lp), _p(lc))
    return lp, lc


def head_ce_at(logits, targets, v0: int, C: int, k, t, sigma: float, seed: int, tag: int,
               draw0: int = 0, tok0: int = 0) -> np.ndarray:
    """loss_pert of draw draw0 + k[m] at token t[m], for chosen pairs only."""
    z = _f64(logits)
    T, V = z.shape
    y = np.ascontiguousarray(targets, dtype=np.int32)
    k, t = _idx(k), _idx(t)
    out = np.empty(len(k), dtype=np.float64)
    _load().dust_or_head_ce_at(_p(z), y.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), T, V, v0, C,
                               sigma, seed, tag, draw0, tok0, _pidx(k), _pidx(t), len(k), _p(out))
    return out


ACT_NONE, ACT_RELU, ACT_RELU2, ACT_GELU_TANH = 0, 1, 2, 3


def activation(x, act: int) -> np.ndarray:
    """Elementwise activation (dust_oracle.c states the four forms) of an array, fp64."""
    f = np.vectorize(lambda v: _load().dust_or_activation(v, act), otypes=[np.float64])
    return f(_f64(x))


def perturbed_linear(y, w, K: int, sigma: float, seed: int, tag: int, act: int, draw0: int = 0,
                     tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """out[k][t][n] = sum_j act(y[t][j] + sigma a^{(draw0+k)}_{tok0+t, chan0+j}) w[n][j]: the next
    linear layer applied to the activated perturbed output (explainer, "The real work", first
    measure). y [T, d], w [n_out, d] -> [K, T, n_out], fp64."""
    y, w = _f64(y), _f64(w)
    T, d = y.shape
    n_out = w.shape[0]
    out = np.empty((K, T, n_out), dtype=np.float64)
    _load().dust_or_perturbed_linear(_p(y), _p(w), T, d, n_out, chan0, K, sigma, seed, tag, draw0,
                                     tok0, act, _p(out))
    return out


def perturbed_rows_at(y, k, t, sigma: float, seed: int, tag: int, act: int, draw0: int = 0,
                      tok0: int = 0, chan0: int = 0) -> np.ndarray:
    """act(y[t] + sigma a^{(draw0+k)}_{tok0+t}) for chosen (k, t) pairs: rows [m, d], fp64."""
    y = _f64(y)
    d = y.shape[1]
    k, t = _idx(k), _idx(t)
    rows = np.empty((len(k), d), dtype=np.float64)
    _load().dust_or_perturbed_rows_at(_p(y), d, chan0, sigma, seed, tag, draw0, tok0, act,
                                      _pidx(k), _pidx(t), len(k), _p(rows))
    return rows


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, as fp64."""
    f = np.vectorize(_load().dust_or_round_bf16, otypes=[np.float64])
    return f(_f64(x))


# ------------------------------------------------------------------------------ tiny model
def tiny_forward_losses(W, H, x, targets, y=None) -> np.ndarray:
    """Per-token cross-entropy of the tiny linear + fixed-head model: y = x W^T (or the given
    layer output y, any leading shape [..., T, d_out]), z = y H^T, l_t = CE(z_t, target_t)."""
    if y is None:
        y = _f64(x) @ _f64(W).T
    z = _f64(y) @ _f64(H).T
    m = z.max(axis=-1, keepdims=True)
    lse = m[..., 0] + np.log(np.exp(z - m).sum(axis=-1))
    tgt = np.asarray(targets, dtype=np.int64)
    zy = z[..., np.arange(len(tgt)), tgt]
    return lse - zy


def tiny_analytic_grad(W, H, x, targets):
    """Exact gradient of sum_t l_t for the tiny model: g_t = H^T (softmax(z_t) - e_target) is
    dL/dy_t and G_W = sum_t g_t x_t^T. Returns (g [T, d_out], G_W [d_out, d_in])."""
    x = _f64(x)
    y = x @ _f64(W).T
    z = y @ _f64(H).T
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(len(targets)), np.asarray(targets)] -= 1.0
    g = p @ _f64(H)
    return g, g.T @ x


# ------------------------------------------------------------------------------ optimizer steps
def sgd_momentum(w, g, buf, lr: float, momentum: float):
    """One SGD-with-momentum step (dust_oracle.c states the formula): returns new (w, buf)."""
    w, buf = _f64(w).copy(), _f64(buf).copy()
    gg = _f64(g)
    _load().dust_or_sgd_momentum(_p(w), _p(gg), _p(buf), w.size, lr, momentum)
    return w, buf


def adam(w, g, m, v, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
         step: int):
    """One Adam step with decoupled weight decay at step t = step >= 1 (dust_oracle.c states
    the formula): returns new (w, m, v)."""
    w, m, v = _f64(w).copy(), _f64(m).copy(), _f64(v).copy()
    gg = _f64(g)
    _load().dust_or_adam(_p(w), _p(gg), _p(m), _p(v), w.size, lr, beta1, beta2, eps,
                         weight_decay, step)
    return w, m, v
