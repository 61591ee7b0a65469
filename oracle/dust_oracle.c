/*
 * Dust gradient estimator -- CPU ORACLE. TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct fp64 statement of what the Dust estimator computes for one
 * linear layer and for one vocabulary chunk of the LM head. Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark load this library; the product path (the HIP
 * library and its Python binding) never links, imports or calls it, and shares no code with it.
 *
 * Sources (the "Dust" explainer at cnblogs.com/32bin/p/23212811, abbreviated "explainer"):
 *   - section "Credit assignment: one forward, two rewards" (信用分配：一次前向，两种奖励):
 *       noise a_t ~ N(0, I) scaled by sigma and added to the layer output y_t; the centred
 *       per-token loss change c_s; the discounted reward r_t; the output-error estimate g_t;
 *       the weight-gradient outer product G_W;
 *   - section "The real work: suppressing interference" (真正的工作量：压住干扰):
 *       attention internals scored by the inner product of the attention-output change with
 *       that output's estimated error; the LM head perturbed on cached logits with only the
 *       cross-entropy of one vocabulary chunk recomputed.
 * The random numbers are Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
 * As Easy as 1, 2, 3", SC'11) followed by the Box-Muller transform (Box & Muller, 1958). The
 * pages fix neither the generator nor the index layout; the readings used here are:
 *   key     = (seed mod 2^32, seed >> 32)
 *   counter = (floor(ch / 4), token, draw, tag)      ch = global channel (vocab id for the head)
 *   u(w)    = (floor(w / 2^9) + 1/2) * 2^-23          radius uniform, exact, in (0, 1)
 *   v(w)    =  floor(w / 2^9) * 2^-23                 angle uniform (turns), exact, in [0, 1)
 *   channel 4q+0 = rho(w0) cos(2 pi v(w1)), 4q+1 = rho(w0) sin(2 pi v(w1)),
 *   channel 4q+2 = rho(w2) cos(2 pi v(w3)), 4q+3 = rho(w2) sin(2 pi v(w3)),
 *   rho(w) = sqrt(-2 ln u(w)).
 * The radius uniform must exclude 0 (log), the angle uniform need not, so the angle takes the
 * left end of each of the 2^23 bins.
 *
 * Every loop below is the definition written out: no blocking, fusion or reordering of any
 * sum. OpenMP splits only independent output elements across threads.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* Number of threads the OpenMP loops below use. */
int dust_or_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------------- */
/* Philox4x32-10 (SC'11). One round maps (x0, x1, x2, x3) under key (k0, k1) to
 *   (hi(B*x2) ^ x1 ^ k0,  lo(B*x2),  hi(A*x0) ^ x3 ^ k1,  lo(A*x0))
 * with the multipliers A = 0xD2511F53 and B = 0xCD9E8D57; between rounds the key is advanced
 * by the Weyl constants (0x9E3779B9, 0xBB67AE85). Ten rounds, nine key advances. */
void dust_or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t pa = (uint64_t)0xD2511F53u * (uint64_t)x0;
        uint64_t pb = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
        uint32_t y0 = (uint32_t)(pb >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)pb;
        uint32_t y2 = (uint32_t)(pa >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)pa;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The four words that carry the noise of channels 4q .. 4q+3 of (draw, token). */
void dust_or_noise_words(uint64_t seed, uint32_t tag, uint32_t draw, uint32_t token, uint32_t q,
                         uint32_t out[4])
{
    uint32_t ctr[4] = {q, token, draw, tag};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    dust_or_philox4x32_10(ctr, key, out);
}

/* Radius uniform in (0, 1) from the top 23 bits of a word, centred in its bin. */
double dust_or_uniform(uint32_t w)
{
    return ((double)(w >> 9) + 0.5) * (1.0 / 8388608.0);
}

/* Angle uniform in [0, 1) (turns) from the top 23 bits of a word, left end of its bin. */
double dust_or_angle(uint32_t w)
{
    return (double)(w >> 9) * (1.0 / 8388608.0);
}

/* Box-Muller (1958): one of the two normals of the word pair (wa, wb); sine != 0 selects
 * rho sin(theta), else rho cos(theta). */
double dust_or_box_muller(uint32_t wa, uint32_t wb, int sine)
{
    double rho = sqrt(-2.0 * log(dust_or_uniform(wa)));
    double theta = 2.0 * M_PI * dust_or_angle(wb);
    return sine ? rho * sin(theta) : rho * cos(theta);
}

/* Standard normal a^{(draw)}_{token, ch}: explainer, "Credit assignment", a_t ~ N(0, I). */
double dust_or_normal(uint64_t seed, uint32_t tag, uint32_t draw, uint32_t token, uint64_t ch)
{
    uint32_t w[4];
    dust_or_noise_words(seed, tag, draw, token, (uint32_t)(ch / 4), w);
    unsigned pair = (unsigned)((ch % 4) / 2);       /* words (0,1) or (2,3) */
    return dust_or_box_muller(w[2 * pair], w[2 * pair + 1], (int)(ch % 2));
}

/* Bulk normals for (draw0 + k, token0 + t, chan0 + j): out[k][t][j], k < K, t < T, j < d. */
void dust_or_normals(uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0, int64_t chan0,
                     int64_t K, int64_t T, int64_t d, double *out)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < d; ++j)
                out[(k * T + t) * d + j] = dust_or_normal(seed, tag, (uint32_t)(draw0 + k),
                                                          (uint32_t)(tok0 + t),
                                                          (uint64_t)(chan0 + j));
}

/* Normals at n chosen (draw, token, channel) triples: out[m] = a^{(draw0+k[m])}_{tok0+t[m], chan0+j[m]}. */
void dust_or_normals_at(uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0, int64_t chan0,
                        const int64_t *k, const int64_t *t, const int64_t *j, int64_t n,
                        double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < n; ++m)
        out[m] = dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]), (uint32_t)(tok0 + t[m]),
                                (uint64_t)(chan0 + j[m]));
}

/* ---------------------------------------------------------------------------------------- */
/* Perturbed layer output y'^{(i)}_t = y_t + sigma a^{(i)}_t (explainer, "Credit assignment").
 * y is [T, ld_y] (first d columns used); y_pert is [K, T, d]. */
void dust_or_noise_inject(const double *y, int64_t T, int64_t d, int64_t ld_y, int64_t chan0,
                          int64_t K, double sigma, uint64_t seed, uint32_t tag, uint32_t draw0,
                          uint32_t tok0, double *y_pert)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < d; ++j)
                y_pert[(k * T + t) * d + j] =
                    y[t * ld_y + j] +
                    sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k), (uint32_t)(tok0 + t),
                                           (uint64_t)(chan0 + j));
}

/* ---------------------------------------------------------------------------------------- */
/* Per-token loss change, loss mode: c^{(i)}_t = l_clean,t - l^{(i)}_pert,t (explainer,
 * "Credit assignment": the centred change, read as clean minus perturbed so that c is the
 * reduction the noise produced). */
void dust_or_loss_delta_loss(const double *loss_clean, const double *loss_pert, int64_t K,
                             int64_t T, double *c)
{
    for (int64_t i = 0; i < K; ++i)
        for (int64_t t = 0; t < T; ++t)
            c[i * T + t] = loss_clean[t] - loss_pert[i * T + t];
}

/* Inner-product mode for attention internals: c^{(i)}_s = -<delta_o^{(i)}_s, g^o_s>
 * (explainer, "The real work: suppressing interference", second measure). delta_o is
 * [K, T, d], g_o is [T, d]. */
void dust_or_loss_delta_inner(const double *delta_o, const double *g_o, int64_t K, int64_t T,
                              int64_t d, double *c)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < K; ++i)
        for (int64_t s = 0; s < T; ++s) {
            double acc = 0.0;
            for (int64_t j = 0; j < d; ++j)
                acc += delta_o[(i * T + s) * d + j] * g_o[s * d + j];
            c[i * T + s] = -acc;
        }
}

/* ---------------------------------------------------------------------------------------- */
/* Inner-product scores of a perturbed attention VALUE projection (explainer, "The real work":
 * attention internals are scored through the attention output, by the inner product of the
 * output's change with the output's estimated error). Perturbing the value projection's output,
 * v'_s = v_s + sigma a_s, leaves the attention weights P of the clean forward unchanged (they
 * come from queries and keys), so re-running head h's attention changes its output at query t
 * by Delta o_t = sigma sum_{s <= t, same sequence} P^h_ts a^h_s, and the score is
 *     c_t = -<Delta o_t, g_t>
 *         = -sigma sum_h sum_{s <= t} P^h_ts sum_j a_{s, h dh + j} g_{t, h dh + j}.
 * P [B, H, S, S] holds head h's weights of query row t over keys s (only s <= t is read),
 * g [T, H dh] with T = B S; the noise of (token s, head h, column j) is channel chan0 + h dh + j
 * of token tok0 + s in draw draw0 + i. */
void dust_or_attn_value_scores(const double *P, const double *g, int64_t K, int64_t B, int64_t H,
                               int64_t S, int64_t dh, double sigma, uint64_t seed, uint32_t tag,
                               uint32_t draw0, uint32_t tok0, int64_t chan0, double *c)
{
    const int64_t T = B * S, d = H * dh;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t i = 0; i < K; ++i)
        for (int64_t t = 0; t < T; ++t) {
            const int64_t b = t / S, tl = t % S;
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h)
                for (int64_t sl = 0; sl <= tl; ++sl) {
                    const double p = P[((b * H + h) * S + tl) * S + sl];
                    double dot = 0.0;
                    for (int64_t j = 0; j < dh; ++j)
                        dot += dust_or_normal(seed, tag, (uint32_t)(draw0 + i),
                                              (uint32_t)(tok0 + b * S + sl),
                                              (uint64_t)(chan0 + h * dh + j)) *
                               g[t * d + h * dh + j];
                    acc += p * dot;
                }
            c[i * T + t] = -sigma * acc;
        }
}

/* The same scores at n chosen (draw, token) pairs: out[m] = c[k[m]][t[m]]. */
void dust_or_attn_value_scores_at(const double *P, const double *g, int64_t B, int64_t H,
                                  int64_t S, int64_t dh, double sigma, uint64_t seed,
                                  uint32_t tag, uint32_t draw0, uint32_t tok0, int64_t chan0,
                                  const int64_t *k, const int64_t *t, int64_t n, double *out)
{
    const int64_t d = H * dh;
    (void)B;
    #pragma omp parallel for schedule(dynamic)
    for (int64_t m = 0; m < n; ++m) {
        const int64_t b = t[m] / S, tl = t[m] % S;
        double acc = 0.0;
        for (int64_t h = 0; h < H; ++h)
            for (int64_t sl = 0; sl <= tl; ++sl) {
                const double p = P[((b * H + h) * S + tl) * S + sl];
                double dot = 0.0;
                for (int64_t j = 0; j < dh; ++j)
                    dot += dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]),
                                          (uint32_t)(tok0 + b * S + sl),
                                          (uint64_t)(chan0 + h * dh + j)) *
                           g[t[m] * d + h * dh + j];
                acc += p * dot;
            }
        out[m] = -sigma * acc;
    }
}

/* ---------------------------------------------------------------------------------------- */
/* Scores of draws that perturb an attention KEY projection, scored through the attention output
 * (explainer, "The real work": the inner product of the output's change with its estimated
 * error). With k'_s = k_s + sigma a_s, head h's logit of query t on key s moves by
 * delta_ts = sigma tau <q_t, a_s> (tau the softmax scale), so the re-run weights are the softmax
 * of the moved logits, P'_ts = P_ts e^{delta_ts} / sum_{s' <= t} P_ts' e^{delta_ts'}, the given
 * weights standing in for the clean softmax. The clean output is taken with the given weights
 * normalised per row, Pbar_ts = P_ts / sum_{s' <= t} P_ts', so that sigma = 0 changes nothing:
 *     Delta o_t = sum_{s <= t} (P'_ts - Pbar_ts) v_s,   c_t = -sum_h <Delta o^h_t, g^h_t>.
 * A row whose weights sum to zero adds nothing. q, v and g are [T, H dh]; the noise of
 * (token s, head h, column j) is channel chan0 + h dh + j of token tok0 + s in draw draw0 + i. */
static double key_score_one(const double *P, const double *q, const double *v, const double *g,
                            int64_t H, int64_t S, int64_t dh, double sigma, double tau,
                            uint64_t seed, uint32_t tag, uint32_t draw, uint32_t tok0,
                            int64_t chan0, int64_t t, double *dl)
{
    const int64_t b = t / S, tl = t % S, d = H * dh;
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        const double *prow = P + ((b * H + h) * S + tl) * S;
        double Z = 0.0, mx = -INFINITY;
        for (int64_t sl = 0; sl <= tl; ++sl) {
            double dot = 0.0;
            for (int64_t j = 0; j < dh; ++j)
                dot += q[t * d + h * dh + j] *
                       dust_or_normal(seed, tag, draw, (uint32_t)(tok0 + b * S + sl),
                                      (uint64_t)(chan0 + h * dh + j));
            dl[sl] = sigma * tau * dot;
            Z += prow[sl];
            if (dl[sl] > mx) mx = dl[sl];
        }
        if (Z == 0.0) continue;
        double den = 0.0;
        for (int64_t sl = 0; sl <= tl; ++sl) den += prow[sl] * exp(dl[sl] - mx);
        for (int64_t j = 0; j < dh; ++j) {
            double dO = 0.0;
            for (int64_t sl = 0; sl <= tl; ++sl)
                dO += (prow[sl] * exp(dl[sl] - mx) / den - prow[sl] / Z) *
                      v[(b * S + sl) * d + h * dh + j];
            acc += dO * g[t * d + h * dh + j];
        }
    }
    return -acc;
}

void dust_or_attn_key_scores(const double *P, const double *q, const double *v, const double *g,
                             int64_t K, int64_t B, int64_t H, int64_t S, int64_t dh, double sigma,
                             double tau, uint64_t seed, uint32_t tag, uint32_t draw0,
                             uint32_t tok0, int64_t chan0, double *c)
{
    const int64_t T = B * S;
    #pragma omp parallel
    {
        double *dl = malloc((size_t)S * sizeof(double));
        #pragma omp for collapse(2) schedule(dynamic)
        for (int64_t i = 0; i < K; ++i)
            for (int64_t t = 0; t < T; ++t)
                c[i * T + t] = key_score_one(P, q, v, g, H, S, dh, sigma, tau, seed, tag,
                                             (uint32_t)(draw0 + i), tok0, chan0, t, dl);
        free(dl);
    }
}

/* The same scores at n chosen (draw, token) pairs: out[m] = c[k[m]][t[m]]. */
void dust_or_attn_key_scores_at(const double *P, const double *q, const double *v,
                                const double *g, int64_t H, int64_t S, int64_t dh, double sigma,
                                double tau, uint64_t seed, uint32_t tag, uint32_t draw0,
                                uint32_t tok0, int64_t chan0, const int64_t *k, const int64_t *t,
                                int64_t n, double *out)
{
    #pragma omp parallel
    {
        double *dl = malloc((size_t)S * sizeof(double));
        #pragma omp for schedule(dynamic)
        for (int64_t m = 0; m < n; ++m)
            out[m] = key_score_one(P, q, v, g, H, S, dh, sigma, tau, seed, tag,
                                   (uint32_t)(draw0 + k[m]), tok0, chan0, t[m], dl);
        free(dl);
    }
}

/* Scores of draws that perturb an attention QUERY projection, scored the same way. With
 * q'_t = q_t + sigma a_t, head h's logit of query t on key s moves by
 * delta_ts = sigma tau <a_t, k_s>, and the re-run is the softmax re-run above with these shifts:
 *     P'_ts = P_ts e^{delta_ts} / sum_{s' <= t} P_ts' e^{delta_ts'},
 *     Delta o_t = sum_{s <= t} (P'_ts - Pbar_ts) v_s,   c_t = -sum_h <Delta o^h_t, g^h_t>.
 * k, v and g are [T, H dh]; the noise of (token t, head h, column j) is channel chan0 + h dh + j
 * of token tok0 + t in draw draw0 + i. */
static double query_score_one(const double *P, const double *k, const double *v,
                              const double *g, int64_t H, int64_t S, int64_t dh, double sigma,
                              double tau, uint64_t seed, uint32_t tag, uint32_t draw,
                              uint32_t tok0, int64_t chan0, int64_t t, double *dl, double *a)
{
    const int64_t b = t / S, tl = t % S, d = H * dh;
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        const double *prow = P + ((b * H + h) * S + tl) * S;
        for (int64_t j = 0; j < dh; ++j)
            a[j] = dust_or_normal(seed, tag, draw, (uint32_t)(tok0 + t),
                                  (uint64_t)(chan0 + h * dh + j));
        double Z = 0.0, mx = -INFINITY;
        for (int64_t sl = 0; sl <= tl; ++sl) {
            double dot = 0.0;
            for (int64_t j = 0; j < dh; ++j) dot += a[j] * k[(b * S + sl) * d + h * dh + j];
            dl[sl] = sigma * tau * dot;
            Z += prow[sl];
            if (dl[sl] > mx) mx = dl[sl];
        }
        if (Z == 0.0) continue;
        double den = 0.0;
        for (int64_t sl = 0; sl <= tl; ++sl) den += prow[sl] * exp(dl[sl] - mx);
        for (int64_t j = 0; j < dh; ++j) {
            double dO = 0.0;
            for (int64_t sl = 0; sl <= tl; ++sl)
                dO += (prow[sl] * exp(dl[sl] - mx) / den - prow[sl] / Z) *
                      v[(b * S + sl) * d + h * dh + j];
            acc += dO * g[t * d + h * dh + j];
        }
    }
    return -acc;
}

void dust_or_attn_query_scores(const double *P, const double *k, const double *v,
                               const double *g, int64_t K, int64_t B, int64_t H, int64_t S,
                               int64_t dh, double sigma, double tau, uint64_t seed, uint32_t tag,
                               uint32_t draw0, uint32_t tok0, int64_t chan0, double *c)
{
    const int64_t T = B * S;
    #pragma omp parallel
    {
        double *dl = malloc((size_t)S * sizeof(double));
        double *a = malloc((size_t)dh * sizeof(double));
        #pragma omp for collapse(2) schedule(dynamic)
        for (int64_t i = 0; i < K; ++i)
            for (int64_t t = 0; t < T; ++t)
                c[i * T + t] = query_score_one(P, k, v, g, H, S, dh, sigma, tau, seed, tag,
                                               (uint32_t)(draw0 + i), tok0, chan0, t, dl, a);
        free(a);
        free(dl);
    }
}

/* The same scores at n chosen (draw, token) pairs: out[m] = c[kk[m]][t[m]]. */
void dust_or_attn_query_scores_at(const double *P, const double *k, const double *v,
                                  const double *g, int64_t H, int64_t S, int64_t dh,
                                  double sigma, double tau, uint64_t seed, uint32_t tag,
                                  uint32_t draw0, uint32_t tok0, int64_t chan0,
                                  const int64_t *kk, const int64_t *t, int64_t n, double *out)
{
    #pragma omp parallel
    {
        double *dl = malloc((size_t)S * sizeof(double));
        double *a = malloc((size_t)dh * sizeof(double));
        #pragma omp for schedule(dynamic)
        for (int64_t m = 0; m < n; ++m)
            out[m] = query_score_one(P, k, v, g, H, S, dh, sigma, tau, seed, tag,
                                     (uint32_t)(draw0 + kk[m]), tok0, chan0, t[m], dl, a);
        free(a);
        free(dl);
    }
}

/* Draw-independent row weights of the softmax re-run. With u_ts = <v^h_s, g^h_t>,
 * Z_t = sum_{s <= t} P_ts and base_t = sum_{s <= t} P_ts u_ts, the re-run change of head h's
 * output inner product at query t under logit shifts delta_ts is
 *     <Delta o_t, g_t> = (base_t + N1_t) / (Z_t + N0_t) - base_t / Z_t
 *                      = sum_s W_ts (e^{delta_ts} - 1) / (Z_t (Z_t + N0_t)),
 * N0_t = sum_s P_ts (e^{delta_ts} - 1), N1_t = sum_s P_ts u_ts (e^{delta_ts} - 1), with
 *     W_ts = P_ts (Z_t u_ts - base_t)  for s <= t,   W_ts = 0 for s > t.
 * W [B, H, S, S] and Z [B, H, S]; P [B, H, S, S] (entries above the diagonal ignored), v and g
 * [B S, H dh]. Written out per element, as defined. */
void dust_or_attn_row_weights(const double *P, const double *v, const double *g, int64_t B,
                              int64_t H, int64_t S, int64_t dh, double *W, double *Z)
{
    const int64_t d = H * dh;
    #pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t t = 0; t < S; ++t) {
                const double *prow = P + ((b * H + h) * S + t) * S;
                double *wrow = W + ((b * H + h) * S + t) * S;
                double z = 0.0, base = 0.0;
                for (int64_t s = 0; s <= t; ++s) {
                    double u = 0.0;
                    for (int64_t j = 0; j < dh; ++j)
                        u += v[(b * S + s) * d + h * dh + j] * g[(b * S + t) * d + h * dh + j];
                    z += prow[s];
                    base += prow[s] * u;
                }
                for (int64_t s = 0; s < S; ++s) {
                    if (s > t) {
                        wrow[s] = 0.0;
                        continue;
                    }
                    double u = 0.0;
                    for (int64_t j = 0; j < dh; ++j)
                        u += v[(b * S + s) * d + h * dh + j] * g[(b * S + t) * d + h * dh + j];
                    wrow[s] = prow[s] * (z * u - base);
                }
                Z[(b * H + h) * S + t] = z;
            }
}

/* ---------------------------------------------------------------------------------------- */
/* Discounted reward r_t = sum_{s >= t, s in t's sequence} gamma^(s - t) c_s (explainer,
 * "Credit assignment"). Tokens are T = B * seg_len, sequence b owns [b*seg_len, (b+1)*seg_len).
 * Written as the backward recursion r_t = c_t + gamma r_{t+1}, r_last = c_last. */
void dust_or_reward_scan(const double *c, int64_t K, int64_t T, int64_t seg_len, double gamma,
                         double *r)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K; ++i)
        for (int64_t b = 0; b < T / seg_len; ++b) {
            int64_t first = b * seg_len, last = first + seg_len - 1;
            r[i * T + last] = c[i * T + last];
            for (int64_t t = last - 1; t >= first; --t)
                r[i * T + t] = c[i * T + t] + gamma * r[i * T + t + 1];
        }
}

/* ---------------------------------------------------------------------------------------- */
/* Output-error estimate g_t = -(1/(K sigma)) sum_i r^{(i)}_t a^{(i)}_t (explainer, "Credit
 * assignment"). r is [K, T] holding draws draw0 .. draw0+K-1 of a population of K_total; g is
 * [T, d] and, when accumulate != 0, the sum is added to the g passed in. */
void dust_or_error_estimate(const double *r, int64_t K, int64_t K_total, int64_t T, int64_t d,
                            int64_t chan0, double sigma, uint64_t seed, uint32_t tag,
                            uint32_t draw0, uint32_t tok0, int accumulate, double *g)
{
    double scale = -1.0 / ((double)K_total * sigma);
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < K; ++i)
                acc += r[i * T + t] * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),
                                                     (uint32_t)(tok0 + t), (uint64_t)(chan0 + j));
            double prev = accumulate ? g[t * d + j] : 0.0;
            g[t * d + j] = prev + scale * acc;
        }
}

/* The same quantity at n chosen (token, channel) pairs only: out[n] = g[tok[n], ch[n]]
 * (without any accumulate term). */
void dust_or_error_estimate_at(const double *r, int64_t K, int64_t K_total, int64_t T,
                               int64_t chan0, double sigma, uint64_t seed, uint32_t tag,
                               uint32_t draw0, uint32_t tok0, const int64_t *tok,
                               const int64_t *ch, int64_t n, double *out)
{
    double scale = -1.0 / ((double)K_total * sigma);
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < n; ++m) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i)
            acc += r[i * T + tok[m]] * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),
                                                      (uint32_t)(tok0 + tok[m]),
                                                      (uint64_t)(chan0 + ch[m]));
        out[m] = scale * acc;
    }
}

/* ---------------------------------------------------------------------------------------- */
/* LM head on cached logits (explainer, "The real work", third measure): for each draw only the
 * logits of vocabulary chunk [v0, v0 + C) are perturbed, z'_j = z_j + sigma a_j, every other
 * logit keeps its cached value, and the per-token cross-entropy over the whole vocabulary is
 * recomputed: l = log sum_j exp(z'_j) - z'_{target}. logits is [T, V], loss_pert [K, T].
 * loss_clean (may be NULL) receives the unperturbed cross-entropy. */
void dust_or_head_ce_chunk(const double *logits, const int32_t *targets, int64_t T, int64_t V,
                           int64_t v0, int64_t C, int64_t K, double sigma, uint64_t seed,
                           uint32_t tag, uint32_t draw0, uint32_t tok0, double *loss_pert,
                           double *loss_clean)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double *z = logits + t * V;
        int64_t y = targets[t];
        if (loss_clean) {
            double m = z[0];
            for (int64_t j = 1; j < V; ++j) m = z[j] > m ? z[j] : m;
            double s = 0.0;
            for (int64_t j = 0; j < V; ++j) s += exp(z[j] - m);
            loss_clean[t] = m + log(s) - z[y];
        }
        for (int64_t i = 0; i < K; ++i) {
            /* the perturbed logit of entry j, written out for this draw */
            double m = -INFINITY, zy = 0.0;
            for (int64_t j = 0; j < V; ++j) {
                double zj = z[j];
                if (j >= v0 && j < v0 + C)
                    zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),
                                                 (uint32_t)(tok0 + t), (uint64_t)j);
                if (zj > m) m = zj;
                if (j == y) zy = zj;
            }
            double s = 0.0;
            for (int64_t j = 0; j < V; ++j) {
                double zj = z[j];
                if (j >= v0 && j < v0 + C)
                    zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),
                                                 (uint32_t)(tok0 + t), (uint64_t)j);
                s += exp(zj - m);
            }
            loss_pert[i * T + t] = m + log(s) - zy;
        }
    }
}

/* The same perturbed cross-entropy at n chosen (draw, token) pairs: out[m] is loss_pert of draw
 * draw0 + k[m] at token t[m]. */
void dust_or_head_ce_at(const double *logits, const int32_t *targets, int64_t T, int64_t V,
                        int64_t v0, int64_t C, double sigma, uint64_t seed, uint32_t tag,
                        uint32_t draw0, uint32_t tok0, const int64_t *k, const int64_t *t,
                        int64_t n, double *out)
{
    (void)T;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < n; ++m) {
        const double *z = logits + t[m] * V;
        int64_t y = targets[t[m]];
        double mx = -INFINITY, zy = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            double zj = z[j];
            if (j >= v0 && j < v0 + C)
                zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]),
                                             (uint32_t)(tok0 + t[m]), (uint64_t)j);
            if (zj > mx) mx = zj;
            if (j == y) zy = zj;
        }
        double s = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            double zj = z[j];
            if (j >= v0 && j < v0 + C)
                zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]),
                                             (uint32_t)(tok0 + t[m]), (uint64_t)j);
            s += exp(zj - mx);
        }
        out[m] = mx + log(s) - zy;
    }
}

/* ---------------------------------------------------------------------------------------- */
/* Optimizer steps that turn the estimate G into a weight update. The explainer names the two
 * used with Dust in its section "Results" -- SGD with momentum at a constant learning rate
 * (the ladders of the main comparison) and Adam (the rerun of the 1M-token ladders) -- and
 * prints neither formula, so these are the textbook ones, state updated in place:
 *   SGD with momentum (heavy ball, no dampening, as torch.optim.SGD):
 *       buf <- mu buf + g;  w <- w - lr buf
 *   Adam (Kingma & Ba, ICLR 2015) with decoupled weight decay wd (Loshchilov & Hutter,
 *   ICLR 2019; wd = 0 is plain Adam), step t >= 1:
 *       w <- w (1 - lr wd)
 *       m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *       w <- w - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)                       */
void dust_or_sgd_momentum(double *w, const double *g, double *buf, int64_t n, double lr,
                          double mu)
{
    for (int64_t i = 0; i < n; ++i) {
        buf[i] = mu * buf[i] + g[i];
        w[i] = w[i] - lr * buf[i];
    }
}

void dust_or_adam(double *w, const double *g, double *m, double *v, int64_t n, double lr,
                  double b1, double b2, double eps, double wd, int64_t t)
{
    const double bc1 = 1.0 - pow(b1, (double)t), bc2 = 1.0 - pow(b2, (double)t);
    for (int64_t i = 0; i < n; ++i) {
        w[i] = w[i] * (1.0 - lr * wd);
        m[i] = b1 * m[i] + (1.0 - b1) * g[i];
        v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
        w[i] = w[i] - lr * (m[i] / bc1) / (sqrt(v[i] / bc2) + eps);
    }
}

/* ---------------------------------------------------------------------------------------- */
/* The first operation of a perturbed re-run from a layer onward (explainer, "The real work:
 * suppressing interference", first measure: the network is re-run from the perturbed layer on):
 * the next linear layer applied to the activated perturbed output,
 *     out[k][t][n] = sum_j act(y[t][j] + sigma a^{(draw0+k)}_{tok0+t, chan0+j}) w[n][j],
 * i.e. the perturbation of dust_or_noise_inject, an elementwise activation, and a matrix
 * product with the next layer's weight w [n_out, d] (row n = output n). act: 0 identity,
 * 1 ReLU max(x, 0), 2 squared ReLU max(x, 0)^2, 3 GELU in its tanh form
 * 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). The pages name no activation; these are the
 * common choices for a transformer MLP. */
double dust_or_activation(double x, int act)
{
    if (act == 1) return x > 0.0 ? x : 0.0;
    if (act == 2) return x > 0.0 ? x * x : 0.0;
    if (act == 3) {
        const double u = sqrt(2.0 / 3.14159265358979323846) * (x + 0.044715 * x * x * x);
        return 0.5 * x * (1.0 + tanh(u));
    }
    return x;
}

/* out [K, T, n_out]; y [T, d]; w [n_out, d]. */
void dust_or_perturbed_linear(const double *y, const double *w, int64_t T, int64_t d,
                              int64_t n_out, int64_t chan0, int64_t K, double sigma,
                              uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0,
                              int act, double *out)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t t = 0; t < T; ++t) {
            double *row = (double *)malloc((size_t)d * sizeof(double));
            for (int64_t j = 0; j < d; ++j)
                row[j] = dust_or_activation(
                    y[t * d + j] + sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k),
                                                          (uint32_t)(tok0 + t),
                                                          (uint64_t)(chan0 + j)),
                    act);
            for (int64_t n = 0; n < n_out; ++n) {
                double acc = 0.0;
                for (int64_t j = 0; j < d; ++j) acc += row[j] * w[n * d + j];
                out[(k * T + t) * n_out + n] = acc;
            }
            free(row);
        }
}

/* The activated perturbed rows act(y[t] + sigma a^{(draw0+k)}_t) [d] at chosen (k, t) pairs:
 * rows [m, d], for checks of the full-size product at sampled rows. */
void dust_or_perturbed_rows_at(const double *y, int64_t d, int64_t chan0, double sigma,
                               uint64_t seed, uint32_t tag, uint32_t draw0, uint32_t tok0,
                               int act, const int64_t *k, const int64_t *t, int64_t m,
                               double *rows)
{
    #pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < m; ++q)
        for (int64_t j = 0; j < d; ++j)
            rows[q * d + j] = dust_or_activation(
                y[t[q] * d + j] + sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k[q]),
                                                         (uint32_t)(tok0 + t[q]),
                                                         (uint64_t)(chan0 + j)),
                act);
}

/* ---------------------------------------------------------------------------------------- */
/* Round a double to the nearest bfloat16 value (8 significant bits, fp32 exponent range),
 * ties to even, returned as a double. Used to state what a bf16 output must hold. */
double dust_or_round_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                     /* ax = m * 2^e, 0.5 <= m < 1 */
    int qexp = e - 8;                  /* spacing of 8-bit significands in this binade */
    if (qexp < -133) qexp = -133;      /* subnormal spacing of the fp32 exponent range */
    double q = ldexp(1.0, qexp);
    double n = ax / q;                 /* exact: a power-of-two scaling */
    double fl = floor(n);
    double rem = n - fl;
    double rn = (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) ? fl + 1.0 : fl;
    double v = rn * q;
    if (v > 3.3895313892515355e38) v = INFINITY;   /* beyond the largest finite bf16 */
    return x < 0 ? -v : v;
}
