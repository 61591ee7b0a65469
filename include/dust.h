/*
 * dust.h -- C ABI of the Dust gradient estimator on AMD Instinct MI355X (gfx950).
 *
 * Dust estimates a linear layer's weight gradient without backpropagation: it adds per-token
 * Gaussian noise to the layer's output, scores every draw by the per-token change of the loss,
 * folds those scores into discounted rewards, averages reward-weighted noise into an estimate
 * of the output error, and contracts that estimate with the layer input. The LM-head variant
 * perturbs cached logits and recomputes the cross-entropy for one vocabulary chunk only.
 *
 * Method source: the "Dust" explainer at cnblogs.com/32bin/p/23212811 ("explainer" below),
 *   section "Credit assignment: one forward, two rewards" (信用分配：一次前向，两种奖励) and
 *   section "The real work: suppressing interference" (真正的工作量：压住干扰).
 *
 * ------------------------------------------------------------------------------------------
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller (e.g. a torch tensor). The
 *     library never allocates, frees, or synchronises; all work is enqueued on `stream`
 *     (a hipStream_t; NULL = the legacy default stream) and runs asynchronously.
 *   - Arrays are row-major and contiguous unless a leading dimension (ld_*) is given.
 *   - Sizes are element counts. A size of zero is valid and enqueues nothing (the outputs are
 *     left untouched, except where an entry point states otherwise).
 *   - All arguments are validated on the host before any HIP call. Invalid arguments return
 *     DUST_ERR_INVALID; shapes that are valid but outside what the kernels implement return
 *     DUST_ERR_UNSUPPORTED (among them any array of more than 2^62 bytes); a short workspace
 *     returns DUST_ERR_WORKSPACE; a failed launch
 *     returns DUST_ERR_HIP. dust_last_error() then holds a one-line description for the
 *     calling thread. Nothing is enqueued when a call fails validation.
 *   - Entry points are re-entrant and keep no state between calls (except the scratch array of
 *     dust_weight_grad_noalloc, which is stated there).
 *
 * Noise (shared by inject, error estimate and head chunk; regenerated, never stored).
 *   The explainer draws a_t ~ N(0, I) independently per token and per draw and adds sigma*a_t
 *   to the layer output. The generator and the index layout are this library's definition:
 *     key      = (seed mod 2^32, seed >> 32)
 *     counter  = (floor(ch / 4), token, draw, tag)         -- Philox4x32-10 (Salmon et al.,
 *                                                             SC'11) -> words w0..w3
 *     u(w)     = (floor(w / 2^9) + 1/2) * 2^-23            -- radius uniform in (0, 1)
 *     v(w)     =  floor(w / 2^9) * 2^-23                   -- angle uniform in [0, 1) turns
 *     rho(w)   = sqrt(-2 ln u(w))                          -- Box-Muller radius
 *     a[ch=4q+0] = rho(w0) cos(2 pi v(w1))   a[ch=4q+1] = rho(w0) sin(2 pi v(w1))
 *     a[ch=4q+2] = rho(w2) cos(2 pi v(w3))   a[ch=4q+3] = rho(w2) sin(2 pi v(w3))
 *   `ch` is the GLOBAL channel (chan0 + local channel; the vocabulary id for the head), `token`
 *   is tok0 + local token and `draw` is draw0 + local draw, so the noise of an element does not
 *   depend on how tokens, draws or channels are split across calls. `tag` separates
 *   independent noise streams (layer types, perturbation passes).
 *   Requirements: chan0 % 4 == 0; chan0 + d <= 2^34; tok0 + T <= 2^32; draw0 + K <= 2^32.
 * ------------------------------------------------------------------------------------------
 */
#ifndef DUST_H_
#define DUST_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DUST_OK = 0,
    DUST_ERR_INVALID = 1,      /* bad pointer, size, alignment, or parameter */
    DUST_ERR_UNSUPPORTED = 2,  /* valid, but outside what the kernels implement */
    DUST_ERR_WORKSPACE = 3,    /* workspace missing or too small */
    DUST_ERR_HIP = 4           /* a HIP launch failed */
} dust_status;

typedef enum { DUST_F32 = 0, DUST_BF16 = 1 } dust_dtype;

typedef enum { DUST_DELTA_LOSS = 0, DUST_DELTA_INNER = 1 } dust_delta_mode;

/* Elementwise activation applied to a perturbed output before the next linear layer
 * (dust_perturbed_linear). GELU is the tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
typedef enum {
    DUST_ACT_NONE = 0, DUST_ACT_RELU = 1, DUST_ACT_RELU2 = 2 /* max(x, 0)^2 */,
    DUST_ACT_GELU_TANH = 3
} dust_activation;

/* Static name of a status code ("DUST_OK", ...). Never NULL. */
const char *dust_status_string(int status);

/* Description of the last failure on the calling thread ("" if none). Valid until the next
 * call into the library from the same thread. */
const char *dust_last_error(void);

/*
 * dust_noise_inject -- perturbed layer outputs for a block of draws.
 * Explainer, "Credit assignment": the perturbed output of token t in draw i is
 *     y'^{(i)}_t = y_t + sigma * a^{(i)}_t.
 *   y       [T, ld_y] of `dtype` (the first d columns are used)         (in)
 *   y_pert  [Kc, T, d] of `dtype`: y_pert[k][t][j] for draw draw0 + k    (out)
 * Arithmetic in fp32; a bf16 output is rounded to nearest-even. dtype is DUST_F32 or DUST_BF16.
 * Requires ld_y >= d and element-aligned pointers; 16-byte-aligned pointers with d and ld_y
 * multiples of 4 take the vectorised path. sigma must be finite.
 */
int dust_noise_inject(const void *y, void *y_pert, int dtype, int64_t T, int64_t d,
                      int64_t ld_y, int64_t chan0, int64_t Kc, float sigma, uint64_t seed,
                      uint32_t tag, uint32_t draw0, uint32_t tok0, void *stream);

/*
 * dust_perturbed_linear -- the next linear layer applied to the perturbed outputs of a block of
 * draws, without writing them. Explainer, "The real work: suppressing interference" (first
 * measure): a perturbed layer is scored by re-running the network from that layer onward; the
 * first operation of that re-run, for a layer followed by an activation and a linear map
 * (e.g. an MLP up-projection followed by the down-projection), is
 *     out[k][t][n] = sum_j act(y[t][j] + sigma * a^{(draw0+k)}_{tok0+t, chan0+j}) * w[n][j]
 * with the noise of dust_noise_inject (same seed, tag, draw0, tok0, chan0 give the same
 * y'), regenerated on the fly, so the [Kc, T, d] perturbed outputs never reach memory.
 *   y       [T, d] bf16 clean layer output                                             (in)
 *   w       [n_out, d] bf16 weight of the next linear layer (row n = output n)         (in)
 *   out     [Kc, T, n_out] of out_dtype (DUST_F32 or DUST_BF16, nearest even)          (out)
 *   act     a dust_activation
 * act(y + sigma a) is formed in fp32 and rounded to bf16 (nearest even) as the matrix-core
 * operand; products accumulate in fp32. Requires d a multiple of 64 (at most 2^23), n_out a
 * multiple of 32, y and w 16-byte aligned,
 * out element-aligned, sigma finite; out must not overlap y or w. Kc == 0 or T == 0 or
 * n_out == 0 does nothing.
 */
int dust_perturbed_linear(const void *y, const void *w, void *out, int out_dtype, int act,
                          int64_t T, int64_t d, int64_t n_out, int64_t chan0, int64_t Kc,
                          float sigma, uint64_t seed, uint32_t tag, uint32_t draw0,
                          uint32_t tok0, void *stream);

/*
 * dust_loss_delta -- per-token score of every draw, c [Kc, T] fp32 (out).
 * DUST_DELTA_LOSS (explainer, "Credit assignment": the centred per-token loss change, read as
 *   clean minus perturbed so that c is the loss REDUCTION the noise caused):
 *     c[i][t] = loss_clean[t] - loss_pert[i][t]
 *   loss_clean [T] fp32, loss_pert [Kc, T] fp32 (in); delta_o, g_o, io_dtype and d unused.
 * DUST_DELTA_INNER (explainer, "The real work": attention internals are scored through the
 *   attention output by the inner product of the output change with that output's estimated
 *   error; the sign is chosen so that c is again a first-order loss reduction):
 *     c[i][s] = - sum_j delta_o[i][s][j] * g_o[s][j]
 *   delta_o [Kc, T, d] and g_o [T, d] of io_dtype (DUST_F32 or DUST_BF16) (in); products
 *   accumulate in fp32; loss_clean and loss_pert unused. d >= 1.
 */
int dust_loss_delta(int mode, const float *loss_clean, const float *loss_pert,
                    const void *delta_o, const void *g_o, int io_dtype, float *c, int64_t Kc,
                    int64_t T, int64_t d, void *stream);

/*
 * dust_reward_scan -- discounted rewards, r [K, T] fp32 (out) from c [K, T] fp32 (in).
 * Explainer, "Credit assignment": r_t = sum_{s >= t} gamma^(s-t) c_s; gamma = 0 keeps each
 * token's own score. The sum runs to the end of token t's own sequence: tokens form
 * T / seg_len sequences of seg_len consecutive tokens and no reward crosses a sequence end.
 * Requires seg_len >= 1, T % seg_len == 0, 0 <= gamma <= 1. r == c (in place) is allowed; any
 * other overlap is rejected. fp32 arithmetic (a parallel scan, so rounding order differs from
 * the sequential recursion).
 */
int dust_reward_scan(const float *c, float *r, int64_t K, int64_t T, int64_t seg_len,
                     float gamma, void *stream);

/*
 * dust_loss_reward -- dust_loss_delta (loss mode) and dust_reward_scan in one pass:
 *     r[i][t] = sum_{s >= t, s in t's sequence} gamma^(s-t) (loss_clean[s] - loss_pert[i][s])
 * (explainer, "Credit assignment": the loss reduction c of each draw and token, then its
 * discounted reward). The scores c are formed on load and never stored, so the K x T scores
 * make no round trip through memory; the result equals dust_loss_delta followed by
 * dust_reward_scan bit for bit.
 *   loss_clean  [T] fp32                                                             (in)
 *   loss_pert   [K, T] fp32                                                          (in)
 *   r           [K, T] fp32; r == loss_pert (in place) is allowed                    (out)
 * Requires seg_len >= 1, T % seg_len == 0, 0 <= gamma <= 1; r must not overlap loss_clean,
 * nor loss_pert other than exactly.
 */
int dust_loss_reward(const float *loss_clean, const float *loss_pert, float *r, int64_t K,
                     int64_t T, int64_t seg_len, float gamma, void *stream);

/*
 * dust_error_estimate -- output-error estimate g_hat [T, d] fp32 (out, or in/out).
 * Explainer, "Credit assignment":
 *     g_hat[t][j] = -(1 / (K_total * sigma)) * sum_{i < K} r[i][t] * a^{(draw0+i)}_{t, chan0+j}
 *   r           [K, T] fp32 rewards of draws draw0 .. draw0+K-1                       (in)
 *   g_hat       [T, d] fp32; with accumulate != 0 the sum is ADDED to its contents   (in/out)
 *   g_hat_t_bf16  nullable; [d, T] bf16 transpose of the resulting g_hat (round to nearest
 *               even), the operand dust_weight_grad takes                               (out)
 * K_total is the whole population when draws arrive in chunks (K <= K_total); the noise is
 * regenerated from (seed, tag) exactly as dust_noise_inject drew it. sigma > 0 and finite.
 * The draw sum accumulates in fp32. K == 0 with accumulate == 0 writes zeros.
 */
int dust_error_estimate(const float *r, float *g_hat, void *g_hat_t_bf16, int64_t K,
                        int64_t K_total, int64_t T, int64_t d, int64_t chan0, float sigma,
                        uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0,
                        int accumulate, void *stream);

/*
 * dust_error_estimate_losses -- dust_loss_delta (loss mode), dust_reward_scan with gamma = 0 and
 * dust_error_estimate in one pass (explainer, "Credit assignment": with gamma = 0 a token's
 * reward is its own loss reduction c = l_clean - l_pert):
 *     g_hat[t][j] = -(1 / (K_total * sigma)) * sum_{i < K} (loss_clean[t] - loss_pert[i][t])
 *                   * a^{(draw0+i)}_{t, chan0+j}
 * The scores are formed on load (the same fp32 subtraction as dust_loss_delta) and never
 * stored, so no [K, T] score or reward array is needed; the result equals dust_loss_delta
 * followed by dust_error_estimate bit for bit. Arguments as dust_error_estimate, with
 *   loss_clean  [T] fp32, loss_pert [K, T] fp32                                          (in)
 * in place of r. Only gamma = 0: a discounted reward needs the scan (dust_loss_reward).
 */
int dust_error_estimate_losses(const float *loss_clean, const float *loss_pert, float *g_hat,
                               void *g_hat_t_bf16, int64_t K, int64_t K_total, int64_t T,
                               int64_t d, int64_t chan0, float sigma, uint64_t seed, uint32_t tag,
                               uint32_t draw0, uint32_t tok0, int accumulate, void *stream);

/*
 * dust_weight_grad_workspace -- bytes of device workspace dust_weight_grad needs for this
 * shape (0 when none, and for shapes dust_weight_grad rejects). Host-only; never fails.
 */
size_t dust_weight_grad_workspace(int64_t T, int64_t d_out, int64_t d_in);

/*
 * dust_weight_grad -- weight-gradient estimate G [d_out, d_in] fp32 (out).
 * Explainer, "Credit assignment": G_W = sum_t g_hat_t x_t^T, the same outer product as
 * backpropagation with the estimated output error in place of the chain-rule one:
 *     G[o][i] = sum_t g_hat_t_bf16[o][t] * x_bf16[t][i]
 *   g_hat_t_bf16  [d_out, T] bf16 (as written by dust_error_estimate)                  (in)
 *   x_bf16        [T, d_in] bf16, the layer input                                      (in)
 *   workspace     device scratch of at least dust_weight_grad_workspace(T, d_out, d_in)
 *                 bytes (may be NULL when that is 0)
 * bf16 matrix-core products with fp32 accumulation; split-T partial sums are reduced in a
 * fixed order, so results are deterministic. T == 0 writes zeros.
 */
int dust_weight_grad(const void *g_hat_t_bf16, const void *x_bf16, float *G, int64_t T,
                     int64_t d_out, int64_t d_in, void *workspace, size_t ws_bytes,
                     void *stream);

/*
 * dust_weight_grad_noalloc -- dust_weight_grad without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): same arguments, result and kernels, with the split partial sums in a
 * scratch array of 64 MiB that the library holds on each GPU it runs on until the process ends.
 * The call allocates and frees nothing. Shapes whose partial sums exceed the scratch (when
 * dust_weight_grad_workspace(T, d_out, d_in) > 64 MiB) return DUST_ERR_UNSUPPORTED; the MLP
 * shapes 2048 x 512 and 4096 x 1024 over 16384 tokens need exactly 64 MiB, and shapes that need
 * no workspace (e.g. 4096 x 4096) use none. Every split partial the kernels read is written by
 * the same call first, so nothing needs clearing between calls. All calls on one GPU share its
 * scratch: two calls that overlap in time on one GPU (e.g. on two streams) race and give wrong
 * results; calls serialised on one stream are safe. DUST_ERR_HIP if the scratch's device address cannot be looked up.
 */
int dust_weight_grad_noalloc(const void *g_hat_t_bf16, const void *x_bf16, float *G, int64_t T,
                             int64_t d_out, int64_t d_in, void *stream);

/*
 * dust_attn_value_scores -- loss change of K draws that perturb an attention VALUE projection,
 * scored through the attention output (explainer, "The real work: suppressing interference":
 * the inner product of the output's change with the output's estimated error):
 *     c[i][t] = -<Delta o^{(i)}_t, g_o[t]>,  Delta o^{(i)}_t = sigma sum_{s <= t} P^h_ts a^h_s
 * per head h. With v'_s = v_s + sigma a_s and the attention weights unchanged (they come from
 * queries and keys), Delta o is exactly the change of the attention output a re-run with the
 * perturbed values gives; the call computes the scores without forming Delta o. Use them as
 * dust_loss_delta's inner-mode scores (dust_reward_scan, then dust_error_estimate with the
 * same seed, tag, draw0, tok0 and chan0 and d = H * dh).
 *   P       [B, H, S, S] bf16 attention weights of the clean forward, row t (query) over
 *           keys s; only s <= t is read                                                 (in)
 *   g_o     [B*S, H*dh] bf16 estimated error of the attention output, head h in columns
 *           h*dh .. h*dh+dh-1                                                           (in)
 *   c       [Kc, B*S] fp32 scores of draws draw0 .. draw0+Kc-1                          (out)
 * The noise a of (token s, head h, column j) is channel chan0 + h*dh + j of token tok0 + s
 * (the value projection's output channels; see "Noise"). Sequences are the B rows of S tokens.
 * Supported: S a multiple of 32 and at most 4096, dh a multiple of 16 in [16, 128]; P 8-byte
 * and g_o 16-byte aligned; sigma finite. c must not overlap P or g_o. fp32 accumulation; the
 * noise enters the bf16 matrix cores as a high part plus a remainder (16 significant bits).
 */
int dust_attn_value_scores(const void *P, const void *g_o, float *c, int64_t Kc, int64_t B,
                           int64_t H, int64_t S, int64_t dh, int64_t chan0, float sigma,
                           uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0,
                           void *stream);

/*
 * dust_attn_row_weights -- the draw-independent part of the softmax re-run that
 * dust_attn_key_scores and dust_attn_query_scores share (explainer, "The real work: suppressing
 * interference": attention internals are scored through the attention output). For head h of
 * sequence b, with u_ts = <v^h_s, g^h_t>, Z_t = sum_{s <= t} P_ts and base_t =
 * sum_{s <= t} P_ts u_ts, a re-run of the weights under logit shifts delta (each row normalised,
 * as dust_attn_key_scores states) changes <o_t, g_t> by
 *     sum_s W_ts (e^{delta_ts} - 1) / (Z_t (Z_t + sum_s P_ts (e^{delta_ts} - 1))),
 *     W_ts = P_ts (Z_t u_ts - base_t) for s <= t,  W_ts = 0 for s > t.
 * Compute W and Z once per batch of weights; every draw of the key or query scores reuses them.
 *   P       [B, H, S, S] bf16 attention weights of the clean forward, row t (query) over
 *           keys s; entries above the diagonal are ignored                              (in)
 *   v       [B*S, H*dh] bf16 values, head h in columns h*dh .. h*dh+dh-1                 (in)
 *   g_o     [B*S, H*dh] bf16 estimated error of the attention output                     (in)
 *   W       [B, H, S, S] fp32 row weights, zero above the diagonal                      (out)
 *   Z       [B, H, S] fp32 causal row sums of P                                         (out)
 * Supported: S a multiple of 32 and at most 4096, dh a multiple of 16 in [16, 128]; P, v, g_o
 * and W 16-byte, Z 4-byte aligned. W and Z must not overlap each other or the inputs. The inner
 * products u run on the bf16 matrix cores with fp32 accumulation; Z, base and W are fp32.
 * B = 0 or S = 0 does nothing.
 */
int dust_attn_row_weights(const void *P, const void *v, const void *g_o, float *W, float *Z,
                          int64_t B, int64_t H, int64_t S, int64_t dh, void *stream);

/*
 * dust_attn_key_scores -- loss change of K draws that perturb an attention KEY projection,
 * scored through the attention output (explainer, "The real work: suppressing interference":
 * the inner product of the output's change with the output's estimated error). With
 * k'_s = k_s + sigma a_s, head h's logit of query t on key s moves by
 * delta_ts = sigma * softmax_scale * <q^h_t, a^h_s>, and the re-run attention weights are the
 * softmax of the moved logits, taken relative to the given weights:
 *     P'_ts = P_ts e^{delta_ts} / sum_{s' <= t} P_ts' e^{delta_ts'},
 *     c[i][t] = -sum_h <sum_{s <= t} (P'_ts - P_ts / Z_t) v^h_s, g^h_t>,  Z_t = sum_{s <= t} P_ts
 * (each row is normalised, so bf16 weights that do not sum to one exactly still give 0 at
 * sigma = 0; a row whose weights sum to zero adds nothing). The values v and the output error
 * g_o enter through W and Z of dust_attn_row_weights(P, v, g_o), which the caller computes
 * first, once for all draws. The call computes the scores without forming the perturbed
 * outputs. Use them as dust_loss_delta's inner-mode scores (dust_reward_scan, then
 * dust_error_estimate with the same seed, tag, draw0, tok0 and chan0 and d = H * dh).
 *   P       [B, H, S, S] bf16 attention weights of the clean forward, row t (query) over
 *           keys s; entries above the diagonal are ignored                              (in)
 *   q       [B*S, H*dh] bf16 queries, head h in columns h*dh .. h*dh+dh-1                (in)
 *   W, Z    [B, H, S, S] and [B, H, S] fp32 from dust_attn_row_weights; entries of W above
 *           the diagonal are ignored                                                    (in)
 *   c       [Kc, B*S] fp32 scores of draws draw0 .. draw0+Kc-1                          (out)
 * The noise a of (token s, head h, column j) is channel chan0 + h*dh + j of token tok0 + s
 * (the key projection's output channels; see "Noise"). Sequences are the B rows of S tokens.
 * Supported: S a multiple of 32 and at most 4096 (sequences longer than 1024 run fewer draws per
 * block, 4 up to 2048 and 2 beyond), dh a multiple of 16 in [16, 128]; P, q and W
 * 16-byte, Z and c 4-byte aligned; sigma and softmax_scale finite with
 * |sigma * softmax_scale| <= 2^20. c must not overlap the inputs. fp32 accumulation; the noise
 * enters the bf16 matrix cores as a high part plus a remainder (16 significant bits). The fast
 * pass forms e^delta - 1 directly, which is accurate while the shifts leave the row's mass
 * sum_s P_ts e^delta_ts between Z_t / 2 and 2^20 Z_t (and below 10^30 / Z_t); any other query
 * (large shifts) is recomputed, in the same call, by an exact pass that subtracts its row
 * maximum and takes the noise in fp32 (one block per draw and sequence holding such a query;
 * slower, but the scores stay finite and accurate for finite inputs).
 */
int dust_attn_key_scores(const void *P, const void *q, const float *W, const float *Z, float *c,
                         int64_t Kc, int64_t B, int64_t H, int64_t S, int64_t dh, int64_t chan0,
                         float sigma, float softmax_scale, uint64_t seed, uint32_t tag,
                         uint32_t draw0, uint32_t tok0, void *stream);

/*
 * dust_attn_query_scores -- loss change of K draws that perturb an attention QUERY projection,
 * scored through the attention output as above. With q'_t = q_t + sigma a_t, head h's logit of
 * query t on key s moves by delta_ts = sigma * softmax_scale * <a^h_t, k^h_s>, and the scores
 * are those of dust_attn_key_scores with these shifts (the softmax re-run relative to the
 * given weights, each row normalised; v and g_o enter through W and Z of
 * dust_attn_row_weights).
 *   P       [B, H, S, S] bf16 attention weights of the clean forward, row t (query) over
 *           keys s; entries above the diagonal are ignored                              (in)
 *   k       [B*S, H*dh] bf16 keys, head h in columns h*dh .. h*dh+dh-1                   (in)
 *   W, Z    [B, H, S, S] and [B, H, S] fp32 from dust_attn_row_weights                   (in)
 *   c       [Kc, B*S] fp32 scores of draws draw0 .. draw0+Kc-1                          (out)
 * The noise a of (token t, head h, column j) is channel chan0 + h*dh + j of token tok0 + t
 * (the query projection's output channels; see "Noise"). Sequences are the B rows of S tokens.
 * Supported: S a multiple of 32 and at most 4096, dh a multiple of 16 in [16, 128]; P, k and W
 * 16-byte, Z and c 4-byte aligned; sigma and softmax_scale finite with
 * |sigma * softmax_scale| <= 2^20. c must not overlap the inputs. Precision, and the exact pass
 * for large logit shifts, as for dust_attn_key_scores.
 */
int dust_attn_query_scores(const void *P, const void *k, const float *W, const float *Z,
                           float *c, int64_t Kc, int64_t B, int64_t H, int64_t S, int64_t dh,
                           int64_t chan0, float sigma, float softmax_scale, uint64_t seed,
                           uint32_t tag, uint32_t draw0, uint32_t tok0, void *stream);

/*
 * dust_cosine_terms -- the three sums of the cosine between two fp32 arrays, for screening
 * hyperparameters (explainer, "The real work": candidate settings are ranked by the cosine
 * between the estimate and the backpropagation gradient on one batch, and training decides
 * among the best):
 *     terms[0] = sum_i a_i b_i,  terms[1] = sum_i a_i^2,  terms[2] = sum_i b_i^2
 * so that cos(a, b) = terms[0] / sqrt(terms[1] terms[2]).
 *   a, b    [n] fp32                                                                     (in)
 *   terms   [3] fp64, device memory                                                     (out)
 * fp64 accumulation in a fixed order (the result does not depend on scheduling); one block, so
 * it is meant for a few calls per screening, not for the estimate's inner loop. n == 0 leaves
 * terms untouched. a, b 4-byte and terms 8-byte aligned; terms must not overlap a or b;
 * n <= 2^40.
 */
int dust_cosine_terms(const float *a, const float *b, int64_t n, double *terms, void *stream);

/*
 * dust_sgd_momentum -- one SGD-with-momentum step on n fp32 weights, in place.
 * The explainer's section "Results" trains with the estimate through SGD with momentum at a
 * constant learning rate; the step is the textbook heavy ball without dampening:
 *     buf <- momentum * buf + g;   w <- w - lr * buf
 *   w    [n] fp32 weights                                                       (in/out)
 *   g    [n] fp32 gradient estimate, e.g. dust_weight_grad's G                  (in)
 *   buf  [n] fp32 momentum buffer, zero before the first step                   (in/out)
 * lr and momentum finite, momentum >= 0. w, g and buf must not overlap. fp32 arithmetic.
 */
int dust_sgd_momentum(float *w, const float *g, float *buf, int64_t n, float lr, float momentum,
                      void *stream);

/*
 * dust_adam -- one Adam step (Kingma & Ba, ICLR 2015) with decoupled weight decay
 * (Loshchilov & Hutter, ICLR 2019; weight_decay = 0 is plain Adam) on n fp32 weights, in place.
 * The explainer's section "Results" reruns a comparison of Dust with Adam. At step t >= 1:
 *     w <- w (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *     w <- w - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 *   w, g, m, v  [n] fp32: weights (in/out), gradient estimate (in), first and second moments
 *               (in/out; zero before step 1)
 * 0 <= beta1, beta2 < 1; eps > 0; lr, weight_decay finite, weight_decay >= 0; step >= 1.
 * No two arrays may overlap. fp32 arithmetic with the bias corrections formed in fp64.
 */
int dust_adam(float *w, const float *g, float *m, float *v, int64_t n, float lr, float beta1,
              float beta2, float eps, float weight_decay, int64_t step, void *stream);

/*
 * dust_head_ce_chunk -- perturbed per-token cross-entropy of the LM head for one vocabulary
 * chunk. Explainer, "The real work": the head is perturbed directly on cached logits and only
 * the cross-entropy involving one chunk of the vocabulary is recomputed. For draw i and token t
 * the logits of the chunk [v0, v0 + C) become z_j + sigma * a^{(i)}_{t, j} (global channel
 * j = vocabulary id); every other logit keeps its cached value; the loss is the full-vocabulary
 * cross-entropy  log sum_j exp(z'_j) - z'_{target}.
 *   logits      [T, V] fp32 cached clean logits                                     (in)
 *   targets     [T] int32 in [0, V); an out-of-range target yields NaN losses        (in)
 *   loss_pert   [Kc, T] fp32, draws draw0 .. draw0+Kc-1                              (out)
 *   loss_clean  nullable; [T] fp32 unperturbed cross-entropy                         (out)
 * Requires 1 <= C <= 4096, v0 % 4 == 0, v0 + C <= V. Log-sum-exp is taken online in fp32.
 */
int dust_head_ce_chunk(const float *logits, const int32_t *targets, float *loss_pert,
                       float *loss_clean, int64_t T, int64_t V, int64_t v0, int64_t C,
                       int64_t Kc, float sigma, uint64_t seed, uint32_t tag, uint32_t draw0,
                       uint32_t tok0, void *stream);

/*
 * dust_noise_words -- the raw Philox4x32-10 words behind the noise, for bit-exact checks of
 * the generator and its indexing (the same device routine every noise kernel calls).
 *   words  [Kc, T, G, 4] uint32: words[k][t][g][w] = word w of
 *          counter (group0 + g, tok0 + t, draw0 + k, tag) under key (seed lo, seed hi)  (out)
 * Requires group0 + G <= 2^32, tok0 + T <= 2^32, draw0 + Kc <= 2^32.
 */
int dust_noise_words(uint32_t *words, int64_t Kc, int64_t T, int64_t G, uint32_t group0,
                     uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DUST_H_ */
