// Inner-product scores of a perturbed attention value projection (gfx950).
//
// Explainer cnblogs.com/32bin/p/23212811, "The real work: suppressing interference": attention
// internals are scored through the attention output, by the inner product of the output's
// change with the output's estimated error g. When the value projection's output is perturbed,
// v'_s = v_s + sigma a_s, the attention weights P of the clean forward stay as they are (they
// come from queries and keys), so the re-run changes head h's output at query t by
// Delta o_t = sigma sum_{s <= t} P^h_ts a^h_s, exactly, and
//     c_t = -<Delta o_t, g_t> = -sigma sum_h sum_{s <= t} P^h_ts <a^h_s, g^h_t>.
// The kernel never forms Delta o (K x T x d values): per draw it regenerates the noise of one
// tile of 32 keys once, and for every later tile of 32 queries forms the 32 x 32 key-query inner
// products E_st = <a^h_s, g^h_t> on the matrix cores (v_mfma_f32_32x32x16_bf16, the noise split
// into a bf16 high part and a bf16 remainder so that it keeps 16 significant bits), weights
// them by P and sums over the keys into the query's score.
//
// Work layout: a block of 4 waves owns one sequence and 4 draws, one draw per wave; a wave walks
// heads, then key tiles, then the query tiles at or after the key tile (causal order), keeping
// its S running scores in LDS. The MFMA operands come straight from registers: a lane generates
// the 8 consecutive head columns of its own key row (A operand) and loads the 8 matching columns
// of its own query's g row (B operand); the output tile's layout (lane l holds query l % 32 and
// 16 of the key rows) lets each lane weight and sum its keys, and one exchange between the lanes
// l and l ^ 32 completes the sum over the 32 keys.
#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// KS k-slices of 16 head columns: head width dh = 16 KS.
template <int KS>
__global__ __launch_bounds__(256) void attn_value_scores_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ g, float *__restrict__ c,
    uint32_t Kc, uint32_t T, uint32_t H, uint32_t S, uint32_t chan0, float scale, Key key,
    uint32_t draw0, uint32_t tok0, uint32_t ndg) {
    extern __shared__ float c_lds[];   // [4][S] running scores, one row per wave
    const uint32_t wave = wave_in_block();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t b = blockIdx.x / ndg;
    const uint32_t i = (blockIdx.x % ndg) * 4u + wave;   // this wave's draw (local index)
    if (i >= Kc) return;
    float *cw = c_lds + (uint64_t)wave * S;
    for (uint32_t t = lane; t < S; t += 64u) cw[t] = 0.f;

    constexpr uint32_t DH = 16u * KS;
    const uint32_t d = H * DH;
    const uint32_t col = lane & 31u, half = lane >> 5;
    const uint32_t draw = draw0 + i;
    const uint32_t nt = S / 32u;
    for (uint32_t h = 0; h < H; ++h) {
        const uint16_t *Ph = P + ((uint64_t)b * H + h) * S * S;
        for (uint32_t kt = 0; kt < nt; ++kt) {
            // A operand: the noise of key 32 kt + col at head columns 16 ks + 8 half .. + 7,
            // as a bf16 high part and a bf16 remainder (scaled by kNormalScale in the end)
            bf16x8 ahi[KS], alo[KS];
            const uint32_t token = tok0 + b * S + kt * 32u + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint32_t q = (chan0 + h * DH + 16u * ks + 8u * half) / 4u;
                Polar pa[2], pb[2];   // channels 4q .. 4q+3 and 4q+4 .. 4q+7
                noise4_polar<false>(key, q, token, draw, pa);
                noise4_polar<false>(key, q + 1u, token, draw, pb);
                const Polar *pp[4] = {&pa[0], &pa[1], &pb[0], &pb[1]};
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = pp[e]->rho * pp[e]->c, x1 = pp[e]->rho * pp[e]->s;
                    hw[e] = pack_bf16x2(x0, x1);
                    lw[e] = pack_bf16x2(x0 - __uint_as_float(hw[e] << 16),
                                        x1 - __uint_as_float(hw[e] & 0xFFFF0000u));
                }
                ahi[ks] = as_bf16x8(hw);
                alo[ks] = as_bf16x8(lw);
            }
            for (uint32_t ct = kt; ct < nt; ++ct) {
                const uint32_t t = ct * 32u + col;   // this lane's query (within the sequence)
                // B operand: g of query t at the same head columns
                const uint16_t *grow = g + ((uint64_t)b * S + t) * d + h * DH + 8u * half;
                f32x16 e = {};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 gb = *(const bf16x8 *)(grow + 16u * ks);
                    e = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], gb, e, 0, 0, 0);
                    e = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[ks], gb, e, 0, 0, 0);
                }
                // e[4 q + r] is key row 8 q + 4 half + r of the tile; weight by P and sum
                const uint16_t *prow = Ph + (uint64_t)t * S + kt * 32u + 4u * half;
                float part = 0.f;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const uint2 pw = *(const uint2 *)(prow + 8u * qd);
                    const float pv[4] = {__uint_as_float(pw.x << 16),
                                         __uint_as_float(pw.x & 0xFFFF0000u),
                                         __uint_as_float(pw.y << 16),
                                         __uint_as_float(pw.y & 0xFFFF0000u)};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t krow = 8u * qd + 4u * half + r;
                        const float wgt = (ct == kt && krow > col) ? 0.f : pv[r];   // keys after t
                        part = __builtin_fmaf(wgt, e[4 * qd + r], part);
                    }
                }
                part += __shfl_xor(part, 32);
                if (half == 0) cw[t] += part;
            }
        }
    }
    float *cr = c + (uint64_t)i * T + (uint64_t)b * S;
    for (uint32_t t = lane; t < S; t += 64u) cr[t] = scale * cw[t];
}

}  // namespace

hipError_t launch_attn_value_scores(const uint16_t *P, const uint16_t *g, float *c, int64_t Kc,
                                    int64_t B, int64_t H, int64_t S, int64_t dh, int64_t chan0,
                                    float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                    hipStream_t s) {
    const uint32_t ndg = (uint32_t)((Kc + 3) / 4);
    const uint32_t blocks = (uint32_t)(B * ndg);
    const size_t lds = (size_t)4 * S * sizeof(float);
    // the noise comes divided by kNormalScale; the score carries -sigma
    const float scale = (float)(-(double)sigma * kNormalScale);
#define DUST_AVS(KS)                                                                           \
    attn_value_scores_kernel<KS><<<blocks, 256, lds, s>>>(                                     \
        P, g, c, (uint32_t)Kc, (uint32_t)(B * S), (uint32_t)H, (uint32_t)S, (uint32_t)chan0,   \
        scale, key, draw0, tok0, ndg)
    switch (dh / 16) {
        case 1: DUST_AVS(1); break;
        case 2: DUST_AVS(2); break;
        case 3: DUST_AVS(3); break;
        case 4: DUST_AVS(4); break;
        case 5: DUST_AVS(5); break;
        case 6: DUST_AVS(6); break;
        case 7: DUST_AVS(7); break;
        default: DUST_AVS(8); break;
    }
#undef DUST_AVS
    return hipGetLastError();
}

}  // namespace dust
