// Output-error estimate of the Dust estimator (gfx950):
//     g_hat[t][j] = -(1 / (K_total sigma)) * sum_i r[i][t] * a^{(i)}_{t, j}
// (explainer cnblogs.com/32bin/p/23212811, "Credit assignment: one forward, two rewards").
//
// The noise a is regenerated, never read: each wave owns a tile of TPW tokens x 256 channels
// (lane l holds channel group l of the tile, i.e. four channels = one Philox call per token and
// draw) and loops over the draws. The TPW rewards r[i][t0 .. t0+TPW) of a draw are the same for
// every lane, so they arrive through one scalar load and enter the FMAs as scalar operands;
// HBM traffic is the reward matrix (read once per channel tile) plus one write of g_hat. The
// kernel is bound by the generator's ALU work. The draw sum runs in fp32 in draw order per
// element; the optional bf16 transpose g_hat^T [d, T] is written from the same registers, so
// the contraction kernel reads its A operand K-contiguous.
// LOSSES (gamma = 0 only): the kernel reads the perturbed losses instead of the rewards and forms
// r = c = l_clean - l_pert on load (the same fp32 subtraction as the loss-change kernel; with
// gamma = 0 the reward is the score), so the K x T scores and rewards are never stored. gfx950
// has no scalar floating-point unit, so this costs one vector subtraction per token and draw.
#include "dust_internal.hpp"

namespace dust {
namespace {

template <int TPW, bool VEC, bool LOSSES>
__global__ __launch_bounds__(256) void error_estimate_kernel(
    const float *__restrict__ r, const float *__restrict__ lc, float *__restrict__ g,
    uint16_t *__restrict__ gt, uint32_t K,
    uint32_t T, uint32_t d, uint32_t q0, float scale, Key key, uint32_t draw0, uint32_t tok0,
    int accumulate, uint32_t n_ctiles) {
    // Consecutive logical waves share g_hat^T lines (neighbouring token tiles) and reward rows
    // (the channel tiles of one token tile), so they are kept on one XCD.
    const uint32_t w = xcd_logical_block(blockIdx.x, gridDim.x) * 4u + wave_in_block();
    const uint32_t ttile = w / n_ctiles;
    const uint32_t ctile = w % n_ctiles;
    const uint32_t t0 = ttile * TPW;
    if (t0 >= T) return;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t grp = ctile * 64u + lane;   // local channel group
    const uint32_t j0 = grp * 4u;              // first local channel of the group
    const uint32_t q = q0 + grp;
    const uint32_t ntok = min((uint32_t)TPW, T - t0);

    float acc[TPW][4];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tt][e] = 0.f;

    // one draw: r a = kNormalScale (r rho) (cos, sin); kNormalScale is folded into the final scale
    auto accumulate_draw = [&](uint32_t draw, const float (&rv)[TPW]) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            Polar p[2];
            noise4_polar<true>(key, q, tok0 + t0 + tt, draw, p);
            const float k0 = rv[tt] * p[0].rho, k1 = rv[tt] * p[1].rho;
            acc[tt][0] = __builtin_fmaf(k0, p[0].c, acc[tt][0]);
            acc[tt][1] = __builtin_fmaf(k0, p[0].s, acc[tt][1]);
            acc[tt][2] = __builtin_fmaf(k1, p[1].c, acc[tt][2]);
            acc[tt][3] = __builtin_fmaf(k1, p[1].s, acc[tt][3]);
        }
    };
    const float *rp = r + t0;
    float lcv[TPW];   // LOSSES: the clean losses of the tile's tokens
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) lcv[tt] = (LOSSES && tt < (int)ntok) ? lc[t0 + tt] : 0.f;
    if (ntok == TPW) {
        // whole tile: a draw's TPW rewards are one contiguous row piece, fetched by one scalar
        // load one draw ahead of their use
        typedef float f32xT __attribute__((ext_vector_type(TPW)));
        f32xT next = K > 0 ? *(const f32xT *)rp : f32xT{};
        for (uint32_t i = 0; i < K; ++i) {
            float rv[TPW];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) rv[tt] = LOSSES ? lcv[tt] - next[tt] : next[tt];
            if (i + 1 < K) next = *(const f32xT *)(rp + (uint64_t)(i + 1) * T);
            accumulate_draw(draw0 + i, rv);
        }
    } else {
        for (uint32_t i = 0; i < K; ++i, rp += T) {
            float rv[TPW];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
                rv[tt] = (tt < (int)ntok) ? (LOSSES ? lcv[tt] - rp[tt] : rp[tt]) : 0.f;
            accumulate_draw(draw0 + i, rv);
        }
    }

    if (j0 >= d) return;
    const uint32_t nch = min(4u, d - j0);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        if (tt < (int)ntok) {
            float *gr = g + (uint64_t)(t0 + tt) * d + j0;
            if constexpr (VEC) {
                float4 v = make_float4(scale * acc[tt][0], scale * acc[tt][1], scale * acc[tt][2],
                                       scale * acc[tt][3]);
                if (accumulate) {
                    const float4 o = *(const float4 *)gr;
                    v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
                }
                *(float4 *)gr = v;
                acc[tt][0] = v.x; acc[tt][1] = v.y; acc[tt][2] = v.z; acc[tt][3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (e < (int)nch) {
                        float v = scale * acc[tt][e];
                        if (accumulate) v += gr[e];
                        gr[e] = v;
                        acc[tt][e] = v;
                    }
                }
            }
        }
    }
    if (gt == nullptr) return;
    // g_hat^T [d, T] in bf16: this lane writes ntok consecutive tokens of each of its channels
    const bool gt_vec = VEC && (ntok == TPW) && ((T % 8u) == 0u) && ((TPW % 8) == 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < (int)nch) {
            uint16_t *row = gt + (uint64_t)(j0 + e) * T + t0;
            if (gt_vec) {
#pragma unroll
                for (int h = 0; h < TPW / 8; ++h) {
                    uint4 v;
                    v.x = pack_bf16x2(acc[8 * h + 0][e], acc[8 * h + 1][e]);
                    v.y = pack_bf16x2(acc[8 * h + 2][e], acc[8 * h + 3][e]);
                    v.z = pack_bf16x2(acc[8 * h + 4][e], acc[8 * h + 5][e]);
                    v.w = pack_bf16x2(acc[8 * h + 6][e], acc[8 * h + 7][e]);
                    *(uint4 *)(row + 8 * h) = v;
                }
            } else {
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt)
                    if (tt < (int)ntok) row[tt] = f32_to_bf16(acc[tt][e]);
            }
        }
    }
}

// K == 0 and no accumulation: the estimate is exactly zero.
__global__ __launch_bounds__(256) void zero_estimate_kernel(float *__restrict__ g,
                                                            uint16_t *__restrict__ gt,
                                                            uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    g[i] = 0.f;
    if (gt) gt[i] = 0;
}

}  // namespace

hipError_t launch_error_estimate(const float *r, float *g, uint16_t *gt, int64_t K,
                                 int64_t K_total, int64_t T, int64_t d, int64_t chan0,
                                 float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                 bool accumulate, hipStream_t s) {
    return launch_error_estimate_losses(nullptr, r, g, gt, K, K_total, T, d, chan0, sigma, key,
                                        draw0, tok0, accumulate, s);
}

hipError_t launch_error_estimate_losses(const float *lc, const float *r, float *g, uint16_t *gt,
                                        int64_t K, int64_t K_total, int64_t T, int64_t d,
                                        int64_t chan0, float sigma, Key key, uint32_t draw0,
                                        uint32_t tok0, bool accumulate, hipStream_t s) {
    if (K == 0 && !accumulate) {
        const uint64_t n = (uint64_t)T * (uint64_t)d;
        zero_estimate_kernel<<<(uint32_t)((n + 255) / 256), 256, 0, s>>>(g, gt, n);
        return hipGetLastError();
    }
    // the generator's normals come divided by kNormalScale
    const float scale = (float)(-kNormalScale / ((double)K_total * (double)sigma));
    const uint32_t n_ctiles = (uint32_t)((d + 255) / 256);
    const bool vec = (d % 4 == 0) && aligned16(g) && (gt == nullptr || aligned16(gt));
    // Largest token tile (8 or 4) that still gives every SIMD several waves. A 16-token tile
    // would need more than the registers the compiler keeps the accumulators in.
    int tpw = 8;
    while (tpw > 4 && ((T + tpw - 1) / tpw) * (int64_t)n_ctiles < 8192) tpw /= 2;
    const uint64_t waves = (uint64_t)((T + tpw - 1) / tpw) * n_ctiles;
    const uint32_t blocks = (uint32_t)((waves + 3) / 4);
    const uint32_t q0 = (uint32_t)(chan0 / 4);
#define DUST_EE(TP, V, L)                                                                      \
    error_estimate_kernel<TP, V, L><<<blocks, 256, 0, s>>>(r, lc, g, gt, (uint32_t)K,          \
                                                           (uint32_t)T, (uint32_t)d, q0, scale, \
                                                           key, draw0, tok0,                   \
                                                           accumulate ? 1 : 0, n_ctiles)
#define DUST_EE_TV(L)                                                                          \
    do {                                                                                       \
        if (vec) {                                                                             \
            if (tpw == 8) DUST_EE(8, true, L); else DUST_EE(4, true, L);                       \
        } else {                                                                               \
            if (tpw == 8) DUST_EE(8, false, L); else DUST_EE(4, false, L);                     \
        }                                                                                      \
    } while (0)
    if (lc != nullptr) DUST_EE_TV(true); else DUST_EE_TV(false);
#undef DUST_EE_TV
#undef DUST_EE
    return hipGetLastError();
}

}  // namespace dust
