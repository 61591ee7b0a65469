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

// LDS row pitches (bytes): 32 keys of P as fp32 plus 16 bytes and DH bf16 columns of g plus
// 16 bytes, so that the 16-byte fragment reads of 16 consecutive rows fall into distinct banks.
constexpr uint32_t kPPitch = 144;
__host__ __device__ constexpr uint32_t g_pitch(int KS) { return 32u * KS + 16u; }
__host__ __device__ constexpr uint32_t stage_bytes(int KS) { return 32u * (kPPitch + g_pitch(KS)); }

// KS k-slices of 16 head columns: head width dh = 16 KS.
template <int KS>
__global__ __launch_bounds__(256) void attn_value_scores_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ g, float *__restrict__ c,
    uint32_t Kc, uint32_t T, uint32_t H, uint32_t S, uint32_t chan0, float scale, Key key,
    uint32_t draw0, uint32_t tok0, uint32_t ndg) {
    // LDS: two stages of one step's operands (P tile [32 queries][32 keys], g tile
    // [32 queries][DH]), then per wave two rows of S running scores (lanes 0-31 and 32-63 hold
    // different key rows of a tile, so each half keeps its own partial sums).
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr uint32_t DH = 16u * KS;
    constexpr uint32_t GP = g_pitch(KS), SB = stage_bytes(KS);
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = wave_in_block();
    const uint32_t lane = tid & 63u;
    const uint32_t b = blockIdx.x / ndg;
    // this wave's two draws (local indices i0, i0 + 1); a draw past the last one is computed
    // with the last draw's noise and not written, so every wave loads and synchronises
    const uint32_t i0 = (blockIdx.x % ndg) * 8u + wave * 2u;
    const uint32_t drawA = draw0 + min(i0, Kc - 1u), drawB = draw0 + min(i0 + 1u, Kc - 1u);
    const uint32_t col = lane & 31u, half = lane >> 5;
    // running scores of the two draws: lanes 0-31 add draw i0's, lanes 32-63 draw i0 + 1's
    float *cw = (float *)(lds + 2u * SB) + (uint64_t)wave * 2u * S;
    for (uint32_t t = lane; t < 2u * S; t += 64u) cw[t] = 0.f;
    float *cwh = cw + half * S;

    const uint32_t d = H * DH;
    const uint32_t nt = S / 32u;

    // Global -> registers -> LDS staging of one step's tiles, coalesced: P rows are 64 bytes
    // (4 pieces of 16), g rows DH * 2 bytes (2 KS pieces).
    constexpr uint32_t NPC = 128u + 64u * KS;            // 16-byte pieces per step
    constexpr uint32_t PPT = (NPC + 255u) / 256u;        // pieces per thread
    u32x4 stg[PPT];
    auto gload = [&](uint32_t h, uint32_t kt, uint32_t ct) {
#pragma unroll
        for (uint32_t j = 0; j < PPT; ++j) {
            const uint32_t pc = tid + 256u * j;
            if (pc < 128u) {
                const uint32_t row = pc >> 2, seg = pc & 3u;
                stg[j] = *(const u32x4 *)(P + (((uint64_t)b * H + h) * S + ct * 32u + row) * S +
                                          kt * 32u + 8u * seg);
            } else if (pc < NPC) {
                const uint32_t q = pc - 128u, row = q / (2u * KS), seg = q % (2u * KS);
                stg[j] = *(const u32x4 *)(g + ((uint64_t)b * S + ct * 32u + row) * d + h * DH +
                                          8u * seg);
            }
        }
    };
    auto lstore = [&](uint32_t st) {
        unsigned char *base = lds + st * SB;
#pragma unroll
        for (uint32_t j = 0; j < PPT; ++j) {
            const uint32_t pc = tid + 256u * j;
            if (pc < 128u) {   // 8 weights, widened to fp32 once here for all four draws
                const uint32_t row = pc >> 2, seg = pc & 3u;
                f32x4 *dst = (f32x4 *)(base + row * kPPitch + 32u * seg);
                const u32x4 w = stg[j];
                dst[0] = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
                dst[1] = f32x4{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u),
                               __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xFFFF0000u)};
            } else if (pc < NPC) {
                const uint32_t q = pc - 128u, row = q / (2u * KS), seg = q % (2u * KS);
                *(u32x4 *)(base + 32u * kPPitch + row * GP + 16u * seg) = stg[j];
            }
        }
    };

    // A operand: the noise of key 32 kt + col at head columns 16 ks + 8 half .. + 7, as a bf16
    // high part and a bf16 remainder (kNormalScale is applied to the final score)
    bf16x8 ahiA[KS], aloA[KS], ahiB[KS], aloB[KS];
    auto noise = [&](uint32_t h, uint32_t kt, uint32_t draw, bf16x8 (&ahi)[KS],
                     bf16x8 (&alo)[KS]) {
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
    };

    // Steps in the order head, key tile, query tile >= key tile. Step n's tiles are in LDS
    // stage n % 2; step n + 1's are fetched into registers at the start of step n and stored
    // to the other stage at its end, before the one barrier per step.
    uint32_t h = 0, kt = 0, ct = 0;
    gload(0, 0, 0);
    lstore(0);
    noise(0, 0, drawA, ahiA, aloA);
    noise(0, 0, drawB, ahiB, aloB);
    __syncthreads();
    for (uint32_t st = 0;; st ^= 1u) {
        uint32_t nh = h, nk = kt, nc = ct + 1u;
        if (nc == nt) {
            nk = kt + 1u;
            nc = nk;
            if (nk == nt) { nh = h + 1u; nk = 0; nc = 0; }
        }
        const bool more = nh < H;   // uniform across the block
        if (more) gload(nh, nk, nc);

        const unsigned char *base = lds + st * SB;
        const unsigned char *grow = base + 32u * kPPitch + col * GP + 16u * half;
        bf16x8 gb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) gb[ks] = *(const bf16x8 *)(grow + 32u * ks);
        // two independent accumulation chains, one per draw
        f32x16 eA = {}, eB = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            eA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahiA[ks], gb[ks], eA, 0, 0, 0);
            eB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahiB[ks], gb[ks], eB, 0, 0, 0);
            eA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aloA[ks], gb[ks], eA, 0, 0, 0);
            eB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aloB[ks], gb[ks], eB, 0, 0, 0);
        }
        // e[4 qd + r] is key row 8 qd + 4 half + r of the tile: weight by P and sum
        const unsigned char *prow = base + col * kPPitch + 16u * half;
        float partA = 0.f, partB = 0.f;
        if (ct != kt) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const f32x4 w = *(const f32x4 *)(prow + 32u * qd);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    partA = __builtin_fmaf(w[r], eA[4 * qd + r], partA);
                    partB = __builtin_fmaf(w[r], eB[4 * qd + r], partB);
                }
            }
        } else {   // diagonal tile: keys after the lane's query do not count
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const f32x4 w = *(const f32x4 *)(prow + 32u * qd);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t krow = 8u * qd + 4u * half + r;
                    const float wr = krow <= col ? w[r] : 0.f;
                    partA = __builtin_fmaf(wr, eA[4 * qd + r], partA);
                    partB = __builtin_fmaf(wr, eB[4 * qd + r], partB);
                }
            }
        }
        // Swap the upper half of partA with the lower half of partB: afterwards lanes 0-31
        // hold both halves of draw A's key rows, lanes 32-63 both halves of draw B's.
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(partA),
                                                         __float_as_uint(partB), false, false);
        cwh[ct * 32u + col] += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (!more) break;
        lstore(st ^ 1u);
        if (nk != kt || nh != h) {
            noise(nh, nk, drawA, ahiA, aloA);
            noise(nh, nk, drawB, ahiB, aloB);
        }
        __syncthreads();
        h = nh;
        kt = nk;
        ct = nc;
    }
#pragma unroll
    for (uint32_t k = 0; k < 2u; ++k) {
        if (i0 + k >= Kc) break;
        float *cr = c + (uint64_t)(i0 + k) * T + (uint64_t)b * S;
        for (uint32_t t = lane; t < S; t += 64u) cr[t] = scale * cw[k * S + t];
    }
}

}  // namespace

hipError_t launch_attn_value_scores(const uint16_t *P, const uint16_t *g, float *c, int64_t Kc,
                                    int64_t B, int64_t H, int64_t S, int64_t dh, int64_t chan0,
                                    float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                    hipStream_t s) {
    const uint32_t ndg = (uint32_t)((Kc + 7) / 8);   // blocks of 8 draws, 2 per wave
    const uint32_t blocks = (uint32_t)(B * ndg);
    const size_t cbytes = (size_t)8 * S * sizeof(float);   // 4 waves x 2 draws x S scores
    // the noise comes divided by kNormalScale; the score carries -sigma
    const float scale = (float)(-(double)sigma * kNormalScale);
#define DUST_AVS(KS)                                                                           \
    attn_value_scores_kernel<KS><<<blocks, 256, 2 * stage_bytes(KS) + cbytes, s>>>(           \
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
