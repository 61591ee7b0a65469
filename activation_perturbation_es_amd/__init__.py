"""Python binding of the Dust estimator's C ABI (libdust.so, HIP kernels for gfx950).

Argument marshalling only: each function has the name, arguments and meaning of the C entry
point declared in include/dust.h, and every step of the estimator runs in the library's HIP
kernels. Data arguments accept a torch tensor (its device pointer is passed), an int address,
or None (NULL). `stream` accepts None (torch's current HIP stream), a torch.cuda.Stream, or a
raw hipStream_t address. A non-zero status raises DustError with the library's message.

There is no fallback: if libdust.so is missing, importing a function raises at first use, with
the instruction to build it (python -m activation_perturbation_es_amd.build).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "DUST_OK", "DUST_ERR_INVALID", "DUST_ERR_UNSUPPORTED", "DUST_ERR_WORKSPACE", "DUST_ERR_HIP",
    "DUST_F32", "DUST_BF16", "DUST_DELTA_LOSS", "DUST_DELTA_INNER", "DUST_ACT_NONE",
    "DUST_ACT_RELU", "DUST_ACT_RELU2", "DUST_ACT_GELU_TANH", "DustError", "dust_perturbed_linear",
    "dust_noise_inject", "dust_loss_delta", "dust_reward_scan", "dust_loss_reward",
    "dust_error_estimate", "dust_error_estimate_losses", "dust_weight_grad_workspace",
    "dust_sgd_momentum", "dust_adam",
    "dust_cosine_terms", "dust_attn_value_scores", "dust_attn_row_weights",
    "dust_attn_key_scores", "dust_attn_query_scores", "dust_weight_grad",
    "dust_weight_grad_noalloc", "dust_head_ce_chunk", "dust_noise_words",
    "dust_status_string", "dust_last_error", "library", "LIB_PATH", "EXPORTED_SYMBOLS",
]

DUST_OK, DUST_ERR_INVALID, DUST_ERR_UNSUPPORTED, DUST_ERR_WORKSPACE, DUST_ERR_HIP = 0, 1, 2, 3, 4
DUST_F32, DUST_BF16 = 0, 1
DUST_DELTA_LOSS, DUST_DELTA_INNER = 0, 1
DUST_ACT_NONE, DUST_ACT_RELU, DUST_ACT_RELU2, DUST_ACT_GELU_TANH = 0, 1, 2, 3

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdust.so")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64
_f32 = ctypes.c_float
_int = ctypes.c_int

# name -> (restype, argtypes), mirroring include/dust.h
_SIGNATURES = {
    "dust_status_string": (ctypes.c_char_p, [_int]),
    "dust_last_error": (ctypes.c_char_p, []),
    "dust_noise_inject": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _f32, _u64, _u32,
                                 _u32, _u32, _vp]),
    "dust_perturbed_linear": (_int, [_vp, _vp, _vp, _int, _int, _i64, _i64, _i64, _i64, _i64,
                                     _f32, _u64, _u32, _u32, _u32, _vp]),
    "dust_loss_delta": (_int, [_int, _vp, _vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _vp]),
    "dust_reward_scan": (_int, [_vp, _vp, _i64, _i64, _i64, _f32, _vp]),
    "dust_loss_reward": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp]),
    "dust_attn_value_scores": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32,
                                      _u64, _u32, _u32, _u32, _vp]),
    "dust_attn_row_weights": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp]),
    "dust_attn_key_scores": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                    _f32, _f32, _u64, _u32, _u32, _u32, _vp]),
    "dust_attn_query_scores": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                      _i64, _f32, _f32, _u64, _u32, _u32, _u32, _vp]),
    "dust_cosine_terms": (_int, [_vp, _vp, _i64, _vp, _vp]),
    "dust_sgd_momentum": (_int, [_vp, _vp, _vp, _i64, _f32, _f32, _vp]),
    "dust_adam": (_int, [_vp, _vp, _vp, _vp, _i64, _f32, _f32, _f32, _f32, _f32, _i64, _vp]),
    "dust_error_estimate": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _u64, _u32,
                                   _u32, _u32, _int, _vp]),
    "dust_error_estimate_losses": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                          _u64, _u32, _u32, _u32, _int, _vp]),
    "dust_weight_grad_workspace": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "dust_weight_grad": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, ctypes.c_size_t, _vp]),
    "dust_weight_grad_noalloc": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "dust_head_ce_chunk": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _u64,
                                  _u32, _u32, _u32, _vp]),
    "dust_noise_words": (_int, [_vp, _i64, _i64, _i64, _u32, _u64, _u32, _u32, _u32, _vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


class DustError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library() -> ctypes.CDLL:
    """The loaded libdust.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdust.so not found at %s; build it with "
                               "`python -m activation_perturbation_es_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _call(name: str, *args) -> int:
    rc = getattr(library(), name)(*args)
    if rc != DUST_OK:
        raise DustError(rc, "%s: %s: %s" % (name, dust_status_string(rc), dust_last_error()))
    return rc


def dust_status_string(status: int) -> str:
    return library().dust_status_string(status).decode()


def dust_last_error() -> str:
    return library().dust_last_error().decode()


def dust_noise_inject(y, y_pert, dtype, T, d, ld_y, chan0, Kc, sigma, seed, tag, draw0, tok0,
                      stream=None):
    return _call("dust_noise_inject", _ptr(y), _ptr(y_pert), dtype, T, d, ld_y, chan0, Kc, sigma,
                 seed, tag, draw0, tok0, _stream(stream))


def dust_perturbed_linear(y, w, out, out_dtype, act, T, d, n_out, chan0, Kc, sigma, seed, tag,
                          draw0, tok0, stream=None):
    return _call("dust_perturbed_linear", _ptr(y), _ptr(w), _ptr(out), out_dtype, act, T, d, n_out,
                 chan0, Kc, sigma, seed, tag, draw0, tok0, _stream(stream))


def dust_loss_delta(mode, loss_clean, loss_pert, delta_o, g_o, io_dtype, c, Kc, T, d,
                    stream=None):
    return _call("dust_loss_delta", mode, _ptr(loss_clean), _ptr(loss_pert), _ptr(delta_o),
                 _ptr(g_o), io_dtype, _ptr(c), Kc, T, d, _stream(stream))


def dust_reward_scan(c, r, K, T, seg_len, gamma, stream=None):
    return _call("dust_reward_scan", _ptr(c), _ptr(r), K, T, seg_len, gamma, _stream(stream))


def dust_attn_value_scores(P, g_o, c, Kc, B, H, S, dh, chan0, sigma, seed, tag, draw0, tok0,
                           stream=None):
    return _call("dust_attn_value_scores", _ptr(P), _ptr(g_o), _ptr(c), Kc, B, H, S, dh, chan0,
                 sigma, seed, tag, draw0, tok0, _stream(stream))


def dust_attn_row_weights(P, v, g_o, W, Z, B, H, S, dh, stream=None):
    return _call("dust_attn_row_weights", _ptr(P), _ptr(v), _ptr(g_o), _ptr(W), _ptr(Z), B, H, S,
                 dh, _stream(stream))


def dust_attn_key_scores(P, q, W, Z, c, Kc, B, H, S, dh, chan0, sigma, softmax_scale, seed, tag,
                         draw0, tok0, stream=None):
    return _call("dust_attn_key_scores", _ptr(P), _ptr(q), _ptr(W), _ptr(Z), _ptr(c), Kc, B, H,
                 S, dh, chan0, sigma, softmax_scale, seed, tag, draw0, tok0, _stream(stream))


def dust_attn_query_scores(P, k, W, Z, c, Kc, B, H, S, dh, chan0, sigma, softmax_scale, seed,
                           tag, draw0, tok0, stream=None):
    return _call("dust_attn_query_scores", _ptr(P), _ptr(k), _ptr(W), _ptr(Z), _ptr(c), Kc, B,
                 H, S, dh, chan0, sigma, softmax_scale, seed, tag, draw0, tok0, _stream(stream))


def dust_cosine_terms(a, b, n, terms, stream=None):
    return _call("dust_cosine_terms", _ptr(a), _ptr(b), n, _ptr(terms), _stream(stream))


def dust_sgd_momentum(w, g, buf, n, lr, momentum, stream=None):
    return _call("dust_sgd_momentum", _ptr(w), _ptr(g), _ptr(buf), n, lr, momentum, _stream(stream))


def dust_adam(w, g, m, v, n, lr, beta1, beta2, eps, weight_decay, step, stream=None):
    return _call("dust_adam", _ptr(w), _ptr(g), _ptr(m), _ptr(v), n, lr, beta1, beta2, eps,
                 weight_decay, step, _stream(stream))


def dust_loss_reward(loss_clean, loss_pert, r, K, T, seg_len, gamma, stream=None):
    return _call("dust_loss_reward", _ptr(loss_clean), _ptr(loss_pert), _ptr(r), K, T, seg_len,
                 gamma, _stream(stream))


def dust_error_estimate(r, g_hat, g_hat_t_bf16, K, K_total, T, d, chan0, sigma, seed, tag, draw0,
                        tok0, accumulate, stream=None):
    return _call("dust_error_estimate", _ptr(r), _ptr(g_hat), _ptr(g_hat_t_bf16), K, K_total, T, d,
                 chan0, sigma, seed, tag, draw0, tok0, int(accumulate), _stream(stream))


def dust_error_estimate_losses(loss_clean, loss_pert, g_hat, g_hat_t_bf16, K, K_total, T, d, chan0,
                               sigma, seed, tag, draw0, tok0, accumulate, stream=None):
    return _call("dust_error_estimate_losses", _ptr(loss_clean), _ptr(loss_pert), _ptr(g_hat),
                 _ptr(g_hat_t_bf16), K, K_total, T, d, chan0, sigma, seed, tag, draw0, tok0,
                 int(accumulate), _stream(stream))


def dust_weight_grad_workspace(T, d_out, d_in) -> int:
    return library().dust_weight_grad_workspace(T, d_out, d_in)


def dust_weight_grad(g_hat_t_bf16, x_bf16, G, T, d_out, d_in, workspace, ws_bytes, stream=None):
    return _call("dust_weight_grad", _ptr(g_hat_t_bf16), _ptr(x_bf16), _ptr(G), T, d_out, d_in,
                 _ptr(workspace), ws_bytes, _stream(stream))


def dust_weight_grad_noalloc(g_hat_t_bf16, x_bf16, G, T, d_out, d_in, stream=None):
    return _call("dust_weight_grad_noalloc", _ptr(g_hat_t_bf16), _ptr(x_bf16), _ptr(G), T, d_out,
                 d_in, _stream(stream))


def dust_head_ce_chunk(logits, targets, loss_pert, loss_clean, T, V, v0, C, Kc, sigma, seed, tag,
                       draw0, tok0, stream=None):
    return _call("dust_head_ce_chunk", _ptr(logits), _ptr(targets), _ptr(loss_pert),
                 _ptr(loss_clean), T, V, v0, C, Kc, sigma, seed, tag, draw0, tok0, _stream(stream))


def dust_noise_words(words, Kc, T, G, group0, seed, tag, draw0, tok0, stream=None):
    return _call("dust_noise_words", _ptr(words), Kc, T, G, group0, seed, tag, draw0, tok0,
                 _stream(stream))
