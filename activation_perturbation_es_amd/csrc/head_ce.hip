// LM-head chunk cross-entropy of the Dust estimator (gfx950).
//
// Explainer cnblogs.com/32bin/p/23212811, "The real work: suppressing interference": the head
// is perturbed directly on its cached logits and only the cross-entropy involving one
// vocabulary chunk is recomputed, which makes a far larger population affordable there. For
// draw i and token t the chunk logits become z_j + sigma a_j; all other logits stay clean:
//     l'_t = log( sum_{j not in chunk} e^{z_j} + sum_{j in chunk} e^{z_j + sigma a_j} ) - z'_y.
// One wave per token. Pass 1 (once per token) reads the logit row: an online log-sum-exp over
// the entries outside the chunk (running max and rescaled sum per lane, then merged across
// lanes) and the chunk entries kept in registers as q_j = e^{z_j - M}. Pass 2 loops over the
// draws: each lane regenerates the noise of its chunk channels (four per Philox call) and forms
// its part of sum_j q_j 2^{sigma log2(e) a_j}. The parts, and the target's perturbation from
// the lane that owns the target channel, go to LDS; every 16 draws the wave sums them transposed
// and 16 lanes finish one draw's loss each, so neither the cross-lane sum nor the log and store
// cost vector instructions per draw. The loop is bound by the generator's ALU work; the logits
// are read once per token.
#include "dust_internal.hpp"

namespace dust {
namespace {

constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * LN2; }

// Draws per batch: one per lane of a 16-lane quarter of the wave. A partial-sum row holds the
// 64 lanes plus 4 words of padding, so the 16 lanes of a quarter read 16 different bank groups.
constexpr int kBatch = 16;
constexpr int kRow = 68;

template <int GPL>  // channel groups (of 4) per lane: chunk size C <= 256 * GPL
__global__ __launch_bounds__(256) void head_ce_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ targets,
    float *__restrict__ lp, float *__restrict__ lc, uint32_t T, uint32_t V, uint32_t v0,
    uint32_t C, uint32_t Kc, float sigma_log2e, Key key, uint32_t draw0,
    uint32_t tok0) {
    __shared__ __align__(16) float part_lds[4][kBatch][kRow];
    __shared__ float xsel_lds[4][kBatch];
    // tokens dealt to the XCDs in contiguous ranges, so that each 128-byte line of a draw's
    // loss row (32 tokens, 8 blocks) is written whole by one L2
    const uint32_t t = xcd_logical_block(blockIdx.x, gridDim.x) * 4u + wave_in_block();
    if (t >= T) return;
    const uint32_t lane = threadIdx.x & 63u;
    const float *z = logits + (uint64_t)t * V;
    const int32_t y = targets[t];
    const bool ybad = (y < 0) || ((uint32_t)y >= V);

    // chunk logits of this lane: channels 4*(lane + 64 m) + e of the chunk
    float q[GPL][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int m = 0; m < GPL; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t cc = 4u * (lane + 64u * m) + e;
            q[m][e] = (cc < C) ? z[v0 + cc] : -INFINITY;
            mloc = fmaxf(mloc, q[m][e]);
        }
    }
    // online log-sum-exp over the entries outside the chunk
    float mr = -INFINITY, sr = 0.f;
    for (uint32_t j = lane; j < V; j += 64u) {
        if (j - v0 < C) continue;   // inside the chunk (unsigned compare)
        const float x = z[j];
        if (x > mr) {
            sr = sr * fast_exp(mr - x) + 1.f;
            mr = x;
        } else if (x != -INFINITY) {
            // a masked (-inf) logit adds nothing; without this test one met before any finite
            // logit would form e^{-inf - (-inf)} = NaN
            sr += fast_exp(x - mr);
        }
    }
    const float M = wave_max(fmaxf(mloc, mr));
    const float s_rest = wave_sum(mr == -INFINITY ? 0.f : sr * fast_exp(mr - M));
    float qsum = 0.f;
#pragma unroll
    for (int m = 0; m < GPL; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q[m][e] = (q[m][e] == -INFINITY) ? 0.f : fast_exp(q[m][e] - M);
            qsum += q[m][e];
        }
    const float s_chunk = wave_sum(qsum);

    const float zy = ybad ? __builtin_nanf("") : z[y];
    const uint32_t cy = (uint32_t)y - v0;
    const bool y_in = !ybad && cy < C;
    const uint32_t owner = (cy >> 2) & 63u;
    const uint32_t my = cy >> 8;        // group-of-lane index of the target channel
    const uint32_t ey = cy & 3u;
    if (lc != nullptr && lane == 0) lc[t] = M + fast_log(s_rest + s_chunk) - zy;

    const uint32_t token = tok0 + t;
    const uint32_t q0 = v0 / 4u;
    // Draws go in batches of kBatch. Per draw each lane leaves its partial sum in LDS (no VALU
    // work), and the lane owning the target channel leaves x_y there; after the batch the wave
    // sums the partials transposed (lane l: draw l % kBatch, a quarter of the lanes) and lanes
    // 0 .. kBatch-1 finish one draw's loss each, so the log and the store run once per batch.
    float(&part)[kBatch][kRow] = part_lds[wave_in_block()];
    float(&xsel)[kBatch] = xsel_lds[wave_in_block()];
    const float base = M;                        // l' = M + ln(s_rest + tot) - z_y - ln2 x_y
    for (uint32_t ib = 0; ib < Kc; ib += kBatch) {
        const uint32_t nb = __builtin_amdgcn_readfirstlane(min((uint32_t)kBatch, Kc - ib));
        for (uint32_t b = 0; b < nb; ++b) {
            const uint32_t draw = draw0 + ib + b;
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < GPL; ++m) {
                const uint32_t grp = lane + 64u * m;
                if (4u * grp >= C) continue;
                Polar p[2];
                noise4_polar<true>(key, q0 + grp, token, draw, p);
                // x_j = sigma log2(e) a_j: the exponent of e^{sigma a_j} in base 2
                const float k0 = sigma_log2e * p[0].rho, k1 = sigma_log2e * p[1].rho;
                const float x0 = k0 * p[0].c, x1 = k0 * p[0].s, x2 = k1 * p[1].c,
                            x3 = k1 * p[1].s;
                s = __builtin_fmaf(q[m][0], __builtin_amdgcn_exp2f(x0), s);
                s = __builtin_fmaf(q[m][1], __builtin_amdgcn_exp2f(x1), s);
                s = __builtin_fmaf(q[m][2], __builtin_amdgcn_exp2f(x2), s);
                s = __builtin_fmaf(q[m][3], __builtin_amdgcn_exp2f(x3), s);
                if (y_in && (uint32_t)m == my && lane == owner)   // wave-uniform but for lane
                    xsel[b] = ey == 0 ? x0 : (ey == 1 ? x1 : (ey == 2 ? x2 : x3));
            }
            part[b][lane] = s;
        }
        __builtin_amdgcn_wave_barrier();
        // lane l adds the partials of draw l % kBatch from lanes 16 (l / 16) .. 16 (l / 16) + 15
        const uint32_t bl = lane % kBatch, quarter = lane / 16u;
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < 16; k += 4) {
            const float4 v = *(const float4 *)&part[bl][16u * quarter + k];
            tot += (v.x + v.y) + (v.z + v.w);
        }
        tot += __shfl_xor(tot, 16);
        tot += __shfl_xor(tot, 32);
        if (lane < nb) {
            const float xy = y_in ? xsel[lane] : 0.f;
            // the perturbed target logit is z_y + sigma a_y = z_y + ln(2) x_y
            lp[(uint64_t)(ib + lane) * T + t] =
                base + fast_log(s_rest + tot) - __builtin_fmaf(LN2, xy, zy);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

hipError_t launch_head_ce_chunk(const float *logits, const int32_t *targets, float *loss_pert,
                                float *loss_clean, int64_t T, int64_t V, int64_t v0, int64_t C,
                                int64_t Kc, float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                hipStream_t s) {
    const uint32_t blocks = (uint32_t)((T + 3) / 4);
    // the generator's polar form leaves out kNormalScale: the coefficient carries it
    const float sl2e = (float)((double)sigma * 1.44269504088896340736 * kNormalScale);
#define DUST_HEAD(G)                                                                           \
    head_ce_kernel<G><<<blocks, 256, 0, s>>>(logits, targets, loss_pert, loss_clean,           \
                                             (uint32_t)T, (uint32_t)V, (uint32_t)v0,           \
                                             (uint32_t)C, (uint32_t)Kc, sl2e, key,             \
                                             draw0, tok0)
    if (C <= 256) DUST_HEAD(1);
    else if (C <= 512) DUST_HEAD(2);
    else if (C <= 1024) DUST_HEAD(4);
    else if (C <= 2048) DUST_HEAD(8);
    else DUST_HEAD(16);
#undef DUST_HEAD
    return hipGetLastError();
}

}  // namespace dust
