// C ABI of the Dust estimator: argument validation, then one launcher call per entry point.
// Every check runs on the host before any HIP call, so a rejected call enqueues nothing and
// touches no device state. The declarations and their contracts are in include/dust.h.
#include "dust.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "dust_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return DUST_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(DUST_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMax32 = 0xFFFFFFFFll;      // counter words are 32-bit
constexpr int64_t kMaxIdx = 0x7FFFFFFFll;     // kernels index tokens / channels in 32 bits

bool elem_aligned(const void *p, size_t elem) { return ((uintptr_t)p % elem) == 0; }

dust::Key make_key(uint64_t seed, uint32_t tag) {
    dust::Key k;
    k.k0 = (uint32_t)(seed & 0xFFFFFFFFull);
    k.k1 = (uint32_t)(seed >> 32);
    k.tag = tag;
    return k;
}

// Shared checks of the noise index ranges (see "Noise" in dust.h).
int check_noise_ranges(const char *fn, int64_t T, int64_t d, int64_t chan0, int64_t K,
                       uint32_t draw0, uint32_t tok0) {
    if (chan0 < 0 || chan0 % 4 != 0)
        return fail(DUST_ERR_INVALID, "%s: chan0=%lld must be >= 0 and a multiple of 4", fn,
                    (long long)chan0);
    if ((chan0 + d + 3) / 4 > kMax32 + 1)
        return fail(DUST_ERR_INVALID, "%s: chan0 + d exceeds 2^34 channels", fn);
    if ((int64_t)tok0 + T > kMax32 + 1)
        return fail(DUST_ERR_INVALID, "%s: tok0 + T exceeds 2^32 tokens", fn);
    if ((int64_t)draw0 + K > kMax32 + 1)
        return fail(DUST_ERR_INVALID, "%s: draw0 + K exceeds 2^32 draws", fn);
    return DUST_OK;
}

// Bytes of an n0 x n1 x n2 array of es-byte elements, or -1 when that exceeds 2^62: no device
// holds such an array, and the product could overflow 64-bit size arithmetic.
int64_t span(int64_t n0, int64_t n1, int64_t n2, int64_t es) {
    const __int128 p = (__int128)n0 * n1 * n2 * es;
    return p > ((__int128)1 << 62) ? -1 : (int64_t)p;
}

bool ranges_overlap(const void *a, size_t abytes, const void *b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Shared validation of the key and query scores: x is q for keys, k for queries; S_max is the
// longest sequence the kernel supports.
int check_softmax_scores(const char *fn, const void *P, const void *x, const float *W,
                         const float *Z, float *c, int64_t Kc, int64_t B, int64_t H, int64_t S,
                         int64_t dh, int64_t chan0, float sigma, float softmax_scale,
                         uint32_t draw0, uint32_t tok0, const char *xname, bool *nothing) {
    constexpr int64_t S_max = 4096;
    *nothing = false;
    if (Kc < 0 || B < 0 || H < 0 || S < 0 || dh < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size", fn);
    if (!std::isfinite(sigma) || !std::isfinite(softmax_scale))
        return fail(DUST_ERR_INVALID, "%s: sigma and softmax_scale must be finite", fn);
    if (std::fabs((double)sigma * (double)softmax_scale) > 1048576.0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: |sigma * softmax_scale| beyond 2^20", fn);
    if (Kc > kMaxIdx || B > kMaxIdx || H > kMaxIdx || S > kMaxIdx || dh > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if (int rc = check_noise_ranges(fn, B * S, H * dh, chan0, Kc, draw0, tok0)) return rc;
    if (Kc == 0 || B == 0 || S == 0) {
        *nothing = true;
        return ok();
    }
    if (H == 0 || dh == 0) return fail(DUST_ERR_INVALID, "%s: H and dh must be >= 1", fn);
    if (S % 32 != 0 || S > S_max || dh % 16 != 0 || dh > 128)
        return fail(DUST_ERR_UNSUPPORTED,
                    "%s: S=%lld must be a multiple of 32 up to %lld and dh=%lld a multiple of 16 "
                    "up to 128", fn, (long long)S, (long long)S_max, (long long)dh);
    if (!P || !x || !W || !Z || !c) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (((uintptr_t)P & 15u) || ((uintptr_t)x & 15u) || ((uintptr_t)W & 15u) ||
        !elem_aligned(Z, 4) || !elem_aligned(c, 4))
        return fail(DUST_ERR_INVALID, "%s: P, the %s, and W must be 16-byte, Z and c 4-byte "
                    "aligned", fn, xname);
    const int64_t p_bytes = span(B * H, S, S, 2), w_bytes = span(B * H, S, S, 4);
    const int64_t x_bytes = span(B * S, H * dh, 1, 2), z_bytes = span(B * H, S, 1, 4);
    const int64_t c_bytes = span(Kc, B * S, 1, 4);
    if (p_bytes < 0 || w_bytes < 0 || x_bytes < 0 || z_bytes < 0 || c_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    // every layout puts at least 2 draws in a block
    if (B * ((Kc + 1) / 2) > kMaxIdx) return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large", fn);
    if (ranges_overlap(c, (size_t)c_bytes, P, (size_t)p_bytes) ||
        ranges_overlap(c, (size_t)c_bytes, x, (size_t)x_bytes) ||
        ranges_overlap(c, (size_t)c_bytes, W, (size_t)w_bytes) ||
        ranges_overlap(c, (size_t)c_bytes, Z, (size_t)z_bytes))
        return fail(DUST_ERR_INVALID, "%s: c overlaps an input", fn);
    return DUST_OK;
}

}  // namespace

extern "C" {

const char *dust_status_string(int status) {
    switch (status) {
        case DUST_OK: return "DUST_OK";
        case DUST_ERR_INVALID: return "DUST_ERR_INVALID";
        case DUST_ERR_UNSUPPORTED: return "DUST_ERR_UNSUPPORTED";
        case DUST_ERR_WORKSPACE: return "DUST_ERR_WORKSPACE";
        case DUST_ERR_HIP: return "DUST_ERR_HIP";
        default: return "DUST_ERR_UNKNOWN";
    }
}

const char *dust_last_error(void) { return g_last_error; }

int dust_noise_inject(const void *y, void *y_pert, int dtype, int64_t T, int64_t d,
                      int64_t ld_y, int64_t chan0, int64_t Kc, float sigma, uint64_t seed,
                      uint32_t tag, uint32_t draw0, uint32_t tok0, void *stream) {
    const char *fn = "dust_noise_inject";
    if (dtype != DUST_F32 && dtype != DUST_BF16)
        return fail(DUST_ERR_INVALID, "%s: dtype=%d is not DUST_F32 or DUST_BF16", fn, dtype);
    if (T < 0 || d < 0 || Kc < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (T=%lld d=%lld Kc=%lld)", fn,
                    (long long)T, (long long)d, (long long)Kc);
    if (ld_y < d) return fail(DUST_ERR_INVALID, "%s: ld_y=%lld < d=%lld", fn, (long long)ld_y,
                              (long long)d);
    if (!std::isfinite(sigma)) return fail(DUST_ERR_INVALID, "%s: sigma is not finite", fn);
    if (int rc = check_noise_ranges(fn, T, d, chan0, Kc, draw0, tok0)) return rc;
    if (T == 0 || d == 0 || Kc == 0) return ok();
    if (!y || !y_pert) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    const size_t es = dtype == DUST_BF16 ? 2 : 4;
    if (!elem_aligned(y, es) || !elem_aligned(y_pert, es))
        return fail(DUST_ERR_INVALID, "%s: pointers must be aligned to the element size", fn);
    if (T > kMaxIdx || d > kMaxIdx || Kc > kMaxIdx || ld_y > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if ((d + 3) / 4 >= 256 && ((d + 3) / 4 + 255) / 256 * T > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large", fn);
    const int64_t y_bytes = span(T - 1, ld_y, 1, es) + span(d, 1, 1, es);
    const int64_t out_bytes = span(Kc, T, d, es);
    if (out_bytes < 0 || y_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (ranges_overlap(y, (size_t)y_bytes, y_pert, (size_t)out_bytes))
        return fail(DUST_ERR_INVALID, "%s: y and y_pert overlap", fn);
    return hip_status(dust::launch_noise_inject(y, y_pert, dtype == DUST_BF16, T, d, ld_y, chan0,
                                                Kc, sigma, make_key(seed, tag), draw0, tok0,
                                                (hipStream_t)stream),
                      fn);
}

int dust_loss_delta(int mode, const float *loss_clean, const float *loss_pert,
                    const void *delta_o, const void *g_o, int io_dtype, float *c, int64_t Kc,
                    int64_t T, int64_t d, void *stream) {
    const char *fn = "dust_loss_delta";
    if (mode != DUST_DELTA_LOSS && mode != DUST_DELTA_INNER)
        return fail(DUST_ERR_INVALID, "%s: mode=%d is not DUST_DELTA_LOSS or DUST_DELTA_INNER",
                    fn, mode);
    if (Kc < 0 || T < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (Kc=%lld T=%lld)", fn, (long long)Kc,
                    (long long)T);
    if (Kc > kMaxIdx || T > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if (mode == DUST_DELTA_LOSS) {
        if (Kc == 0 || T == 0) return ok();
        if (!loss_clean || !loss_pert || !c) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
        if (!elem_aligned(loss_clean, 4) || !elem_aligned(loss_pert, 4) || !elem_aligned(c, 4))
            return fail(DUST_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
        if (((T + 255) / 256) * Kc > kMaxIdx)
            return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large", fn);
        const int64_t c_bytes = span(Kc, T, 1, 4);
        if (c_bytes < 0) return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
        if (ranges_overlap(loss_clean, (size_t)T * 4, c, (size_t)c_bytes))
            return fail(DUST_ERR_INVALID, "%s: loss_clean and c overlap", fn);
        if (loss_pert != c && ranges_overlap(loss_pert, (size_t)c_bytes, c, (size_t)c_bytes))
            return fail(DUST_ERR_INVALID, "%s: loss_pert and c partially overlap", fn);
        return hip_status(dust::launch_loss_delta_loss(loss_clean, loss_pert, c, Kc, T,
                                                       (hipStream_t)stream),
                          fn);
    }
    if (io_dtype != DUST_F32 && io_dtype != DUST_BF16)
        return fail(DUST_ERR_INVALID, "%s: io_dtype=%d is not DUST_F32 or DUST_BF16", fn,
                    io_dtype);
    if (d < 1) return fail(DUST_ERR_INVALID, "%s: inner mode needs d >= 1 (d=%lld)", fn,
                           (long long)d);
    if (d > kMaxIdx) return fail(DUST_ERR_UNSUPPORTED, "%s: d beyond 2^31", fn);
    if (Kc == 0 || T == 0) return ok();
    if (!delta_o || !g_o || !c) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    const size_t es = io_dtype == DUST_BF16 ? 2 : 4;
    if (!elem_aligned(delta_o, es) || !elem_aligned(g_o, es) || !elem_aligned(c, 4))
        return fail(DUST_ERR_INVALID, "%s: pointers must be aligned to the element size", fn);
    const int64_t do_bytes = span(Kc, T, d, es), go_bytes = span(T, d, 1, es);
    const int64_t c_bytes = span(Kc, T, 1, 4);
    if (do_bytes < 0 || go_bytes < 0 || c_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (ranges_overlap(delta_o, (size_t)do_bytes, c, (size_t)c_bytes) ||
        ranges_overlap(g_o, (size_t)go_bytes, c, (size_t)c_bytes))
        return fail(DUST_ERR_INVALID, "%s: inputs and c overlap", fn);
    return hip_status(dust::launch_loss_delta_inner(delta_o, g_o, io_dtype == DUST_BF16, c, Kc, T,
                                                    d, (hipStream_t)stream),
                      fn);
}

int dust_reward_scan(const float *c, float *r, int64_t K, int64_t T, int64_t seg_len,
                     float gamma, void *stream) {
    const char *fn = "dust_reward_scan";
    if (K < 0 || T < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (K=%lld T=%lld)", fn, (long long)K,
                    (long long)T);
    if (seg_len < 1) return fail(DUST_ERR_INVALID, "%s: seg_len=%lld < 1", fn, (long long)seg_len);
    if (T % seg_len != 0)
        return fail(DUST_ERR_INVALID, "%s: T=%lld is not a multiple of seg_len=%lld", fn,
                    (long long)T, (long long)seg_len);
    if (!(gamma >= 0.f && gamma <= 1.f))
        return fail(DUST_ERR_INVALID, "%s: gamma=%g outside [0, 1]", fn, (double)gamma);
    if (K == 0 || T == 0) return ok();
    if (!c || !r) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(c, 4) || !elem_aligned(r, 4))
        return fail(DUST_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
    if (K > kMaxIdx || T > kMaxIdx || K * (T / seg_len) > 4 * kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    const int64_t c_bytes = span(K, T, 1, 4);
    if (c_bytes < 0) return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (c != r && ranges_overlap(c, (size_t)c_bytes, r, (size_t)c_bytes))
        return fail(DUST_ERR_INVALID, "%s: c and r partially overlap", fn);
    return hip_status(dust::launch_reward_scan(c, r, K, T, seg_len, gamma, (hipStream_t)stream), fn);
}

int dust_loss_reward(const float *loss_clean, const float *loss_pert, float *r, int64_t K,
                     int64_t T, int64_t seg_len, float gamma, void *stream) {
    const char *fn = "dust_loss_reward";
    if (K < 0 || T < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (K=%lld T=%lld)", fn, (long long)K,
                    (long long)T);
    if (seg_len < 1) return fail(DUST_ERR_INVALID, "%s: seg_len=%lld < 1", fn, (long long)seg_len);
    if (T % seg_len != 0)
        return fail(DUST_ERR_INVALID, "%s: T=%lld is not a multiple of seg_len=%lld", fn,
                    (long long)T, (long long)seg_len);
    if (!(gamma >= 0.f && gamma <= 1.f))
        return fail(DUST_ERR_INVALID, "%s: gamma=%g outside [0, 1]", fn, (double)gamma);
    if (K == 0 || T == 0) return ok();
    if (!loss_clean || !loss_pert || !r) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(loss_clean, 4) || !elem_aligned(loss_pert, 4) || !elem_aligned(r, 4))
        return fail(DUST_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
    if (K > kMaxIdx || T > kMaxIdx || K * (T / seg_len) > 4 * kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    const int64_t r_bytes = span(K, T, 1, 4);
    if (r_bytes < 0) return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (ranges_overlap(loss_clean, (size_t)T * 4, r, (size_t)r_bytes))
        return fail(DUST_ERR_INVALID, "%s: loss_clean and r overlap", fn);
    if (loss_pert != r && ranges_overlap(loss_pert, (size_t)r_bytes, r, (size_t)r_bytes))
        return fail(DUST_ERR_INVALID, "%s: loss_pert and r partially overlap", fn);
    return hip_status(dust::launch_loss_reward(loss_clean, loss_pert, r, K, T, seg_len, gamma,
                                               (hipStream_t)stream),
                      fn);
}

}  // extern "C"

namespace {

// dust_error_estimate (lc == nullptr: r holds the rewards) and dust_error_estimate_losses (r
// holds the perturbed losses, lc the clean ones).
int error_estimate_call(const char *fn, const float *lc, const float *r, float *g_hat,
                        void *g_hat_t_bf16, int64_t K, int64_t K_total, int64_t T, int64_t d,
                        int64_t chan0, float sigma, uint64_t seed, uint32_t tag, uint32_t draw0,
                        uint32_t tok0, int accumulate, void *stream, bool losses) {
    const char *rname = losses ? "loss_pert" : "r";
    if (K < 0 || T < 0 || d < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (K=%lld T=%lld d=%lld)", fn,
                    (long long)K, (long long)T, (long long)d);
    if (K_total < 1 || K_total < K)
        return fail(DUST_ERR_INVALID, "%s: K_total=%lld must be >= max(1, K=%lld)", fn,
                    (long long)K_total, (long long)K);
    if (!(sigma > 0.f) || !std::isfinite(sigma))
        return fail(DUST_ERR_INVALID, "%s: sigma must be finite and > 0", fn);
    if (int rc = check_noise_ranges(fn, T, d, chan0, K, draw0, tok0)) return rc;
    if (T == 0 || d == 0) return ok();
    if (!g_hat || (K > 0 && !r) || (losses && K > 0 && !lc))
        return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(g_hat, 4) || (r && !elem_aligned(r, 4)) || (lc && !elem_aligned(lc, 4)) ||
        (g_hat_t_bf16 && !elem_aligned(g_hat_t_bf16, 2)))
        return fail(DUST_ERR_INVALID, "%s: pointers must be aligned to the element size", fn);
    if (T > kMaxIdx || d > kMaxIdx || K > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if ((T / 4 + 1) * ((d + 255) / 256) > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large", fn);
    const int64_t r_bytes = span(K, T, 1, 4), g_bytes = span(T, d, 1, 4);
    if (r_bytes < 0 || g_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (r && ranges_overlap(r, (size_t)r_bytes, g_hat, (size_t)g_bytes))
        return fail(DUST_ERR_INVALID, "%s: %s and g_hat overlap", fn, rname);
    if (lc && ranges_overlap(lc, (size_t)T * 4, g_hat, (size_t)g_bytes))
        return fail(DUST_ERR_INVALID, "%s: loss_clean and g_hat overlap", fn);
    if (g_hat_t_bf16 && ranges_overlap(g_hat_t_bf16, (size_t)g_bytes / 2, g_hat, (size_t)g_bytes))
        return fail(DUST_ERR_INVALID, "%s: g_hat_t_bf16 and g_hat overlap", fn);
    return hip_status(dust::launch_error_estimate_losses(losses ? lc : nullptr, r, g_hat,
                                                         (uint16_t *)g_hat_t_bf16, K, K_total, T,
                                                         d, chan0, sigma, make_key(seed, tag),
                                                         draw0, tok0, accumulate != 0,
                                                         (hipStream_t)stream),
                      fn);
}

}  // namespace

extern "C" {

int dust_error_estimate(const float *r, float *g_hat, void *g_hat_t_bf16, int64_t K,
                        int64_t K_total, int64_t T, int64_t d, int64_t chan0, float sigma,
                        uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0,
                        int accumulate, void *stream) {
    return error_estimate_call("dust_error_estimate", nullptr, r, g_hat, g_hat_t_bf16, K, K_total,
                               T, d, chan0, sigma, seed, tag, draw0, tok0, accumulate, stream,
                               false);
}

int dust_error_estimate_losses(const float *loss_clean, const float *loss_pert, float *g_hat,
                               void *g_hat_t_bf16, int64_t K, int64_t K_total, int64_t T,
                               int64_t d, int64_t chan0, float sigma, uint64_t seed, uint32_t tag,
                               uint32_t draw0, uint32_t tok0, int accumulate, void *stream) {
    return error_estimate_call("dust_error_estimate_losses", loss_clean, loss_pert, g_hat,
                               g_hat_t_bf16, K, K_total, T, d, chan0, sigma, seed, tag, draw0,
                               tok0, accumulate, stream, true);
}

size_t dust_weight_grad_workspace(int64_t T, int64_t d_out, int64_t d_in) {
    // sizes dust_weight_grad rejects need no workspace
    if (T < 0 || d_out < 0 || d_in < 0 || T > kMaxIdx || d_out > kMaxIdx || d_in > kMaxIdx ||
        d_out * d_in > 256 * kMaxIdx)
        return 0;
    return dust::weight_grad_workspace_bytes(T, d_out, d_in);
}

// Checks shared by dust_weight_grad and dust_weight_grad_noalloc (everything but the
// workspace). *nothing is set when the call has no work (d_out or d_in zero).
int check_weight_grad(const char *fn, const void *g_hat_t_bf16, const void *x_bf16, float *G,
                      int64_t T, int64_t d_out, int64_t d_in, bool *nothing) {
    *nothing = false;
    if (T < 0 || d_out < 0 || d_in < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (T=%lld d_out=%lld d_in=%lld)", fn,
                    (long long)T, (long long)d_out, (long long)d_in);
    if (d_out == 0 || d_in == 0) {
        *nothing = true;
        return ok();
    }
    if (!G || (T > 0 && (!g_hat_t_bf16 || !x_bf16)))
        return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(G, 4) || (T > 0 && (!elem_aligned(g_hat_t_bf16, 2) || !elem_aligned(x_bf16, 2))))
        return fail(DUST_ERR_INVALID, "%s: pointers must be aligned to the element size", fn);
    if (T > kMaxIdx || d_out > kMaxIdx || d_in > kMaxIdx || d_out * d_in > 256 * kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    return DUST_OK;
}

// The array-size and G-overlap checks of the weight gradient (after the workspace checks).
int check_weight_grad_arrays(const char *fn, const void *g_hat_t_bf16, const void *x_bf16,
                             float *G, int64_t T, int64_t d_out, int64_t d_in) {
    const int64_t G_bytes = span(d_out, d_in, 1, 4);
    const int64_t a_bytes = span(d_out, T, 1, 2), b_bytes = span(T, d_in, 1, 2);
    if (G_bytes < 0 || a_bytes < 0 || b_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (T > 0 && (ranges_overlap(G, (size_t)G_bytes, g_hat_t_bf16, (size_t)a_bytes) ||
                  ranges_overlap(G, (size_t)G_bytes, x_bf16, (size_t)b_bytes)))
        return fail(DUST_ERR_INVALID, "%s: G overlaps an input", fn);
    return DUST_OK;
}

int dust_weight_grad(const void *g_hat_t_bf16, const void *x_bf16, float *G, int64_t T,
                     int64_t d_out, int64_t d_in, void *workspace, size_t ws_bytes,
                     void *stream) {
    const char *fn = "dust_weight_grad";
    bool nothing;
    if (int rc = check_weight_grad(fn, g_hat_t_bf16, x_bf16, G, T, d_out, d_in, &nothing))
        return rc;
    if (nothing) return ok();
    const size_t need = dust::weight_grad_workspace_bytes(T, d_out, d_in);
    if (need > 0 && (workspace == nullptr || ws_bytes < need))
        return fail(DUST_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                    workspace ? ws_bytes : (size_t)0);
    if (need > 0 && ((uintptr_t)workspace & 15u))
        return fail(DUST_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
    if (int rc = check_weight_grad_arrays(fn, g_hat_t_bf16, x_bf16, G, T, d_out, d_in)) return rc;
    const int64_t G_bytes = span(d_out, d_in, 1, 4);
    const int64_t a_bytes = span(d_out, T, 1, 2), b_bytes = span(T, d_in, 1, 2);
    if (need > 0 && ranges_overlap(G, (size_t)G_bytes, workspace, need))
        return fail(DUST_ERR_INVALID, "%s: G overlaps the workspace", fn);
    if (need > 0 && T > 0 &&
        (ranges_overlap(workspace, need, g_hat_t_bf16, (size_t)a_bytes) ||
         ranges_overlap(workspace, need, x_bf16, (size_t)b_bytes)))
        return fail(DUST_ERR_INVALID, "%s: the workspace overlaps an input", fn);
    return hip_status(dust::launch_weight_grad((const uint16_t *)g_hat_t_bf16,
                                               (const uint16_t *)x_bf16, G, T, d_out, d_in,
                                               workspace, (hipStream_t)stream),
                      fn);
}

int dust_perturbed_linear(const void *y, const void *w, void *out, int out_dtype, int act,
                          int64_t T, int64_t d, int64_t n_out, int64_t chan0, int64_t Kc,
                          float sigma, uint64_t seed, uint32_t tag, uint32_t draw0,
                          uint32_t tok0, void *stream) {
    const char *fn = "dust_perturbed_linear";
    if (out_dtype != DUST_F32 && out_dtype != DUST_BF16)
        return fail(DUST_ERR_INVALID, "%s: out_dtype=%d is not DUST_F32 or DUST_BF16", fn,
                    out_dtype);
    if (act < DUST_ACT_NONE || act > DUST_ACT_GELU_TANH)
        return fail(DUST_ERR_INVALID, "%s: act=%d is not a dust_activation", fn, act);
    if (T < 0 || d < 0 || n_out < 0 || Kc < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size", fn);
    if (!std::isfinite(sigma)) return fail(DUST_ERR_INVALID, "%s: sigma must be finite", fn);
    if (T > kMaxIdx || d > kMaxIdx || n_out > kMaxIdx || Kc > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if (int rc = check_noise_ranges(fn, T, d, chan0, Kc, draw0, tok0)) return rc;
    if (Kc == 0 || T == 0 || n_out == 0) return ok();
    if (d == 0 || d % 64 != 0 || n_out % 32 != 0)
        return fail(DUST_ERR_UNSUPPORTED,
                    "%s: d=%lld must be a positive multiple of 64 and n_out=%lld of 32", fn,
                    (long long)d, (long long)n_out);
    if (d > ((int64_t)1 << 23))
        return fail(DUST_ERR_UNSUPPORTED, "%s: d beyond 2^23 is not supported", fn);
    if (!y || !w || !out) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    const size_t es = out_dtype == DUST_BF16 ? 2 : 4;
    if (((uintptr_t)y & 15u) || ((uintptr_t)w & 15u) || !elem_aligned(out, es))
        return fail(DUST_ERR_INVALID, "%s: y and w must be 16-byte aligned, out element-aligned",
                    fn);
    const int64_t y_bytes = span(T, d, 1, 2), w_bytes = span(n_out, d, 1, 2);
    const int64_t o_bytes = span(Kc, T, n_out, (int64_t)es);
    if (y_bytes < 0 || w_bytes < 0 || o_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    const int64_t blocks = Kc * ((T + 127) / 128) * ((n_out + 511) / 512);
    if (blocks > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large; split the draws", fn);
    if (ranges_overlap(out, (size_t)o_bytes, y, (size_t)y_bytes) ||
        ranges_overlap(out, (size_t)o_bytes, w, (size_t)w_bytes))
        return fail(DUST_ERR_INVALID, "%s: out overlaps an input", fn);
    return hip_status(dust::launch_perturbed_linear((const uint16_t *)y, (const uint16_t *)w, out,
                                                    out_dtype == DUST_BF16, act, T, d, n_out,
                                                    chan0, Kc, sigma, make_key(seed, tag), draw0,
                                                    tok0, (hipStream_t)stream),
                      fn);
}

int dust_weight_grad_noalloc(const void *g_hat_t_bf16, const void *x_bf16, float *G, int64_t T,
                             int64_t d_out, int64_t d_in, void *stream) {
    const char *fn = "dust_weight_grad_noalloc";
    bool nothing;
    if (int rc = check_weight_grad(fn, g_hat_t_bf16, x_bf16, G, T, d_out, d_in, &nothing))
        return rc;
    if (nothing) return ok();
    const size_t need = dust::weight_grad_workspace_bytes(T, d_out, d_in);
    if (need > dust::weight_grad_scratch_bytes())
        return fail(DUST_ERR_UNSUPPORTED,
                    "%s: this shape needs %zu bytes of split partial sums, beyond the %zu-byte "
                    "per-device scratch; use dust_weight_grad with a workspace", fn, need,
                    dust::weight_grad_scratch_bytes());
    if (int rc = check_weight_grad_arrays(fn, g_hat_t_bf16, x_bf16, G, T, d_out, d_in)) return rc;
    void *scratch = nullptr;
    if (need > 0) {
        const hipError_t e = dust::weight_grad_scratch(&scratch);
        if (e != hipSuccess)
            return fail(DUST_ERR_HIP, "%s: scratch address lookup failed: %s", fn,
                        hipGetErrorString(e));
    }
    return hip_status(dust::launch_weight_grad((const uint16_t *)g_hat_t_bf16,
                                               (const uint16_t *)x_bf16, G, T, d_out, d_in,
                                               scratch, (hipStream_t)stream),
                      fn);
}

int dust_attn_value_scores(const void *P, const void *g_o, float *c, int64_t Kc, int64_t B,
                           int64_t H, int64_t S, int64_t dh, int64_t chan0, float sigma,
                           uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0,
                           void *stream) {
    const char *fn = "dust_attn_value_scores";
    if (Kc < 0 || B < 0 || H < 0 || S < 0 || dh < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size", fn);
    if (!std::isfinite(sigma)) return fail(DUST_ERR_INVALID, "%s: sigma is not finite", fn);
    if (Kc > kMaxIdx || B > kMaxIdx || H > kMaxIdx || S > kMaxIdx || dh > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if (int rc = check_noise_ranges(fn, B * S, H * dh, chan0, Kc, draw0, tok0)) return rc;
    if (Kc == 0 || B == 0 || S == 0) return ok();
    if (H == 0 || dh == 0) return fail(DUST_ERR_INVALID, "%s: H and dh must be >= 1", fn);
    if (S % 32 != 0 || S > 4096 || dh % 16 != 0 || dh > 128)
        return fail(DUST_ERR_UNSUPPORTED,
                    "%s: S=%lld must be a multiple of 32 up to 4096 and dh=%lld a multiple of 16 "
                    "up to 128", fn, (long long)S, (long long)dh);
    if (!P || !g_o || !c) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (((uintptr_t)P & 7u) || ((uintptr_t)g_o & 15u) || !elem_aligned(c, 4))
        return fail(DUST_ERR_INVALID, "%s: P must be 8-byte, g_o 16-byte, c 4-byte aligned", fn);
    const int64_t p_bytes = span(B * H, S, S, 2), g_bytes = span(B * S, H * dh, 1, 2);
    const int64_t c_bytes = span(Kc, B * S, 1, 4);
    if (p_bytes < 0 || g_bytes < 0 || c_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    // every layout puts at least 2 draws in a block
    if (B * ((Kc + 1) / 2) > kMaxIdx) return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large", fn);
    if (ranges_overlap(c, (size_t)c_bytes, P, (size_t)p_bytes) ||
        ranges_overlap(c, (size_t)c_bytes, g_o, (size_t)g_bytes))
        return fail(DUST_ERR_INVALID, "%s: c overlaps P or g_o", fn);
    return hip_status(dust::launch_attn_value_scores((const uint16_t *)P, (const uint16_t *)g_o, c,
                                                     Kc, B, H, S, dh, chan0, sigma,
                                                     make_key(seed, tag), draw0, tok0,
                                                     (hipStream_t)stream),
                      fn);
}

int dust_attn_row_weights(const void *P, const void *v, const void *g_o, float *W, float *Z,
                          int64_t B, int64_t H, int64_t S, int64_t dh, void *stream) {
    const char *fn = "dust_attn_row_weights";
    if (B < 0 || H < 0 || S < 0 || dh < 0) return fail(DUST_ERR_INVALID, "%s: negative size", fn);
    if (B > kMaxIdx || H > kMaxIdx || S > kMaxIdx || dh > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if (B == 0 || S == 0) return ok();
    if (H == 0 || dh == 0) return fail(DUST_ERR_INVALID, "%s: H and dh must be >= 1", fn);
    if (S % 32 != 0 || S > 4096 || dh % 16 != 0 || dh > 128)
        return fail(DUST_ERR_UNSUPPORTED,
                    "%s: S=%lld must be a multiple of 32 up to 4096 and dh=%lld a multiple of 16 "
                    "up to 128", fn, (long long)S, (long long)dh);
    if (!P || !v || !g_o || !W || !Z) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (((uintptr_t)P & 15u) || ((uintptr_t)v & 15u) || ((uintptr_t)g_o & 15u) ||
        ((uintptr_t)W & 15u) || !elem_aligned(Z, 4))
        return fail(DUST_ERR_INVALID, "%s: P, v, g_o and W must be 16-byte, Z 4-byte aligned",
                    fn);
    if (B * H * (S / 32) > kMaxIdx || B * S > kMaxIdx || H * dh > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: grid too large", fn);
    const int64_t p_bytes = span(B * H, S, S, 2), w_bytes = span(B * H, S, S, 4);
    const int64_t x_bytes = span(B * S, H * dh, 1, 2), z_bytes = span(B * H, S, 1, 4);
    if (p_bytes < 0 || w_bytes < 0 || x_bytes < 0 || z_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (ranges_overlap(W, (size_t)w_bytes, Z, (size_t)z_bytes))
        return fail(DUST_ERR_INVALID, "%s: W overlaps Z", fn);
    const void *outs[2] = {W, Z};
    const size_t out_bytes[2] = {(size_t)w_bytes, (size_t)z_bytes};
    for (int o = 0; o < 2; ++o)
        if (ranges_overlap(outs[o], out_bytes[o], P, (size_t)p_bytes) ||
            ranges_overlap(outs[o], out_bytes[o], v, (size_t)x_bytes) ||
            ranges_overlap(outs[o], out_bytes[o], g_o, (size_t)x_bytes))
            return fail(DUST_ERR_INVALID, "%s: W or Z overlaps P, v or g_o", fn);
    return hip_status(dust::launch_attn_row_weights((const uint16_t *)P, (const uint16_t *)v,
                                                    (const uint16_t *)g_o, W, Z, B, H, S, dh,
                                                    (hipStream_t)stream),
                      fn);
}

int dust_attn_key_scores(const void *P, const void *q, const float *W, const float *Z, float *c,
                         int64_t Kc, int64_t B, int64_t H, int64_t S, int64_t dh, int64_t chan0,
                         float sigma, float softmax_scale, uint64_t seed, uint32_t tag,
                         uint32_t draw0, uint32_t tok0, void *stream) {
    const char *fn = "dust_attn_key_scores";
    bool nothing;
    if (int rc = check_softmax_scores(fn, P, q, W, Z, c, Kc, B, H, S, dh, chan0, sigma,
                                      softmax_scale, draw0, tok0, "queries", &nothing))
        return rc;
    if (nothing) return ok();
    return hip_status(dust::launch_attn_key_scores((const uint16_t *)P, (const uint16_t *)q, W, Z,
                                                   c, Kc, B, H, S, dh, chan0, sigma,
                                                   softmax_scale, make_key(seed, tag), draw0,
                                                   tok0, (hipStream_t)stream),
                      fn);
}

int dust_attn_query_scores(const void *P, const void *k, const float *W, const float *Z,
                           float *c, int64_t Kc, int64_t B, int64_t H, int64_t S, int64_t dh,
                           int64_t chan0, float sigma, float softmax_scale, uint64_t seed,
                           uint32_t tag, uint32_t draw0, uint32_t tok0, void *stream) {
    const char *fn = "dust_attn_query_scores";
    bool nothing;
    if (int rc = check_softmax_scores(fn, P, k, W, Z, c, Kc, B, H, S, dh, chan0, sigma,
                                      softmax_scale, draw0, tok0, "keys", &nothing))
        return rc;
    if (nothing) return ok();
    return hip_status(dust::launch_attn_query_scores((const uint16_t *)P, (const uint16_t *)k, W,
                                                     Z, c, Kc, B, H, S, dh, chan0, sigma,
                                                     softmax_scale, make_key(seed, tag), draw0,
                                                     tok0, (hipStream_t)stream),
                      fn);
}

int dust_cosine_terms(const float *a, const float *b, int64_t n, double *terms, void *stream) {
    const char *fn = "dust_cosine_terms";
    if (n < 0) return fail(DUST_ERR_INVALID, "%s: negative size n=%lld", fn, (long long)n);
    if (n == 0) return ok();
    if (!a || !b || !terms) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(a, 4) || !elem_aligned(b, 4) || !elem_aligned(terms, 8))
        return fail(DUST_ERR_INVALID, "%s: a and b must be 4-byte, terms 8-byte aligned", fn);
    if (n > ((int64_t)1 << 40)) return fail(DUST_ERR_UNSUPPORTED, "%s: n beyond 2^40", fn);
    const size_t nb = (size_t)n * 4;
    if (ranges_overlap(terms, 24, a, nb) || ranges_overlap(terms, 24, b, nb))
        return fail(DUST_ERR_INVALID, "%s: terms overlaps a or b", fn);
    return hip_status(dust::launch_cosine_terms(a, b, n, terms, (hipStream_t)stream), fn);
}

int dust_sgd_momentum(float *w, const float *g, float *buf, int64_t n, float lr, float momentum,
                      void *stream) {
    const char *fn = "dust_sgd_momentum";
    if (n < 0) return fail(DUST_ERR_INVALID, "%s: negative size n=%lld", fn, (long long)n);
    if (!std::isfinite(lr) || !std::isfinite(momentum) || momentum < 0.f)
        return fail(DUST_ERR_INVALID, "%s: lr and momentum must be finite, momentum >= 0", fn);
    if (n == 0) return ok();
    if (!w || !g || !buf) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(w, 4) || !elem_aligned(g, 4) || !elem_aligned(buf, 4))
        return fail(DUST_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
    if (n > ((int64_t)1 << 39)) return fail(DUST_ERR_UNSUPPORTED, "%s: n beyond 2^39", fn);
    const size_t b = (size_t)n * 4;
    if (ranges_overlap(w, b, g, b) || ranges_overlap(w, b, buf, b) || ranges_overlap(g, b, buf, b))
        return fail(DUST_ERR_INVALID, "%s: w, g and buf overlap", fn);
    return hip_status(dust::launch_sgd_momentum(w, g, buf, n, lr, momentum, (hipStream_t)stream),
                      fn);
}

int dust_adam(float *w, const float *g, float *m, float *v, int64_t n, float lr, float beta1,
              float beta2, float eps, float weight_decay, int64_t step, void *stream) {
    const char *fn = "dust_adam";
    if (n < 0) return fail(DUST_ERR_INVALID, "%s: negative size n=%lld", fn, (long long)n);
    if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
        return fail(DUST_ERR_INVALID, "%s: betas must lie in [0, 1)", fn);
    if (!(eps > 0.f) || !std::isfinite(eps) || !std::isfinite(lr) ||
        !(weight_decay >= 0.f) || !std::isfinite(weight_decay))
        return fail(DUST_ERR_INVALID, "%s: eps > 0, lr finite and weight_decay >= 0 required", fn);
    if (step < 1) return fail(DUST_ERR_INVALID, "%s: step=%lld < 1", fn, (long long)step);
    if (n == 0) return ok();
    if (!w || !g || !m || !v) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(w, 4) || !elem_aligned(g, 4) || !elem_aligned(m, 4) || !elem_aligned(v, 4))
        return fail(DUST_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
    if (n > ((int64_t)1 << 39)) return fail(DUST_ERR_UNSUPPORTED, "%s: n beyond 2^39", fn);
    const size_t b = (size_t)n * 4;
    const void *p[4] = {w, g, m, v};
    for (int a = 0; a < 4; ++a)
        for (int c = a + 1; c < 4; ++c)
            if (ranges_overlap(p[a], b, p[c], b))
                return fail(DUST_ERR_INVALID, "%s: w, g, m and v overlap", fn);
    return hip_status(dust::launch_adam(w, g, m, v, n, lr, beta1, beta2, eps, weight_decay, step,
                                        (hipStream_t)stream),
                      fn);
}

int dust_head_ce_chunk(const float *logits, const int32_t *targets, float *loss_pert,
                       float *loss_clean, int64_t T, int64_t V, int64_t v0, int64_t C,
                       int64_t Kc, float sigma, uint64_t seed, uint32_t tag, uint32_t draw0,
                       uint32_t tok0, void *stream) {
    const char *fn = "dust_head_ce_chunk";
    if (T < 0 || Kc < 0 || V < 1)
        return fail(DUST_ERR_INVALID, "%s: bad size (T=%lld V=%lld Kc=%lld)", fn, (long long)T,
                    (long long)V, (long long)Kc);
    if (v0 < 0 || C < 1 || v0 + C > V)
        return fail(DUST_ERR_INVALID, "%s: chunk [%lld, %lld) outside [0, V=%lld)", fn,
                    (long long)v0, (long long)(v0 + C), (long long)V);
    if (!std::isfinite(sigma)) return fail(DUST_ERR_INVALID, "%s: sigma is not finite", fn);
    if (int rc = check_noise_ranges(fn, T, C, v0, Kc, draw0, tok0)) return rc;
    if (C > 4096) return fail(DUST_ERR_UNSUPPORTED, "%s: chunk size C=%lld > 4096", fn, (long long)C);
    if (T > kMaxIdx || V > kMaxIdx || Kc > kMaxIdx)
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    if (T == 0) return ok();
    if (!logits || !targets || (Kc > 0 && !loss_pert))
        return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!elem_aligned(logits, 4) || !elem_aligned(targets, 4) ||
        (loss_pert && !elem_aligned(loss_pert, 4)) || (loss_clean && !elem_aligned(loss_clean, 4)))
        return fail(DUST_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
    if (Kc == 0 && loss_clean == nullptr) return ok();
    const int64_t lp_bytes = span(Kc, T, 1, 4), z_bytes = span(T, V, 1, 4);
    if (lp_bytes < 0 || z_bytes < 0)
        return fail(DUST_ERR_UNSUPPORTED, "%s: arrays beyond 2^62 bytes", fn);
    if (Kc > 0 && ranges_overlap(loss_pert, (size_t)lp_bytes, logits, (size_t)z_bytes))
        return fail(DUST_ERR_INVALID, "%s: loss_pert overlaps logits", fn);
    return hip_status(dust::launch_head_ce_chunk(logits, targets, loss_pert, loss_clean, T, V, v0, C,
                                                 Kc, sigma, make_key(seed, tag), draw0, tok0,
                                                 (hipStream_t)stream),
                      fn);
}

int dust_noise_words(uint32_t *words, int64_t Kc, int64_t T, int64_t G, uint32_t group0,
                     uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0, void *stream) {
    const char *fn = "dust_noise_words";
    if (Kc < 0 || T < 0 || G < 0)
        return fail(DUST_ERR_INVALID, "%s: negative size (Kc=%lld T=%lld G=%lld)", fn,
                    (long long)Kc, (long long)T, (long long)G);
    if ((int64_t)group0 + G > kMax32 + 1 || (int64_t)tok0 + T > kMax32 + 1 ||
        (int64_t)draw0 + Kc > kMax32 + 1)
        return fail(DUST_ERR_INVALID, "%s: counter range exceeds 2^32", fn);
    if (Kc == 0 || T == 0 || G == 0) return ok();
    if (!words) return fail(DUST_ERR_INVALID, "%s: null pointer", fn);
    if (!dust::aligned16(words)) return fail(DUST_ERR_INVALID, "%s: words must be 16-byte aligned", fn);
    if (T > kMaxIdx || G > kMaxIdx || Kc > kMaxIdx || (G >= 256 && (G + 255) / 256 * T > kMaxIdx))
        return fail(DUST_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 are not supported", fn);
    return hip_status(dust::launch_noise_words(words, Kc, T, G, group0, make_key(seed, tag), draw0,
                                               tok0, (hipStream_t)stream),
                      fn);
}

}  // extern "C"
