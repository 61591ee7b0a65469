// Inner-product scores of a perturbed attention value or key projection (gfx950).
//
// Explainer cnblogs.com/32bin/p/23212811, "The real work: suppressing interference": attention
// internals are scored through the attention output, by the inner product of the output's
// change with the output's estimated error g. Neither kernel forms Delta o (K x T x d values).
//
// Values. When the value projection's output is perturbed, v'_s = v_s + sigma a_s, the attention
// weights P of the clean forward stay as they are (they come from queries and keys), so the
// re-run changes head h's output at query t by Delta o_t = sigma sum_{s <= t} P^h_ts a^h_s,
// exactly, and
//     c_t = -<Delta o_t, g_t> = -sigma sum_h sum_{s <= t} P^h_ts <a^h_s, g^h_t>.
//
// Keys. When the key projection's output is perturbed, k'_s = k_s + sigma a_s, the logit of
// query t on key s moves by delta_ts = sigma tau <q_t, a_s> (tau the softmax scale), and the
// re-run weights are the softmax of the moved logits, P'_ts = P_ts e^delta_ts / sum P_ts' e^..,
// with the clean output taken with each row normalised (Pbar = P / Z, Z_t = sum_s P_ts). With
// u_ts = <v_s, g_t>, base_t = sum_s P_ts u_ts, N0_t = sum_s P_ts (e^delta_ts - 1) and
// N1_t = sum_s P_ts (e^delta_ts - 1) u_ts, the change of the output's inner product is
//     <Delta o_t, g_t> = (base + N1) / (Z + N0) - base / Z = (Z N1 - base N0) / (Z (Z + N0)),
// a form whose terms are all O(sigma), so nothing cancels at the O(1) level.
//
// Both kernels regenerate the noise of one tile of 32 keys once per draw, and for every later
// tile of 32 queries form the 32 x 32 key-query inner products on the matrix cores
// (v_mfma_f32_32x32x16_bf16; the noise split into a bf16 high part and a bf16 remainder so that
// it keeps 16 significant bits): E_st = <a_s, g_t> for values, D_st = <a_s, q_t> for keys. The
// output tile's layout (lane l holds query l % 32 and 16 of the key rows) lets each lane weight
// and sum its keys; one lane-half swap (v_permlane32_swap) completes the sum over the 32 keys
// of two draws at once.
//
// Work layout: a block of 4 waves owns one sequence and 8 draws, two per wave; the block walks
// heads, then key tiles, then the query tiles at or after the key tile (causal order). Each
// step's weight tile (widened to fp32) and the query-side bf16 tiles are staged in LDS by the
// whole block, double-buffered with one barrier per step; the key-side operands (noise, and the
// values for keys) stay in registers for the whole key tile.
#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// LDS row pitches (bytes): 32 keys of P as fp32 plus 16 bytes and DH bf16 columns of a
// query-side tile plus 16 bytes, so that the 16-byte fragment reads of 16 consecutive rows fall
// into distinct banks.
constexpr uint32_t kPPitch = 144;
__host__ __device__ constexpr uint32_t g_pitch(int KS) { return 32u * KS + 16u; }
// one step's operands: P tile and NQ query-side tiles of 32 rows
__host__ __device__ constexpr uint32_t stage_bytes(int KS, int NQ) {
    return 32u * (kPPitch + NQ * g_pitch(KS));
}

// The A operand of one key row: the noise of key `token` at channels 4 q0 + 16 ks + 8 half ..
// + 7 of every k-slice ks (q0 = the head's first channel / 4), as a bf16 high part and a bf16
// remainder. The values are the normals divided by kNormalScale; callers fold it into their
// scale.
template <int KS>
__device__ __forceinline__ void noise_fragments(const Key &key, uint32_t q0, uint32_t half,
                                                uint32_t token, uint32_t draw, bf16x8 (&ahi)[KS],
                                                bf16x8 (&alo)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint32_t q = q0 + 4u * ks + 2u * half;
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
}

// Staging of one step: 16-byte pieces, P rows first (4 per query row), then the NQ query-side
// tiles (2 KS per row each); loads into registers, stores to LDS after the step's compute.
template <int KS, int NQ>
struct Stager {
    static constexpr uint32_t kPieces = 128u + 64u * KS * NQ;
    static constexpr uint32_t kPerThread = (kPieces + 255u) / 256u;
    u32x4 r[kPerThread];

    // P [B, H, S, S]; the query-side arrays [T, H DH], tile ct of sequence b, head h
    __device__ __forceinline__ void load(uint32_t tid, const uint16_t *P,
                                         const uint16_t *const (&qs)[NQ], uint32_t b, uint32_t H,
                                         uint32_t S, uint32_t d, uint32_t h, uint32_t kt,
                                         uint32_t ct) {
        constexpr uint32_t DH = 16u * KS;
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t pc = tid + 256u * j;
            if (pc < 128u) {
                const uint32_t row = pc >> 2, seg = pc & 3u;
                r[j] = *(const u32x4 *)(P + (((uint64_t)b * H + h) * S + ct * 32u + row) * S +
                                        kt * 32u + 8u * seg);
            } else if (pc < kPieces) {
                const uint32_t x = pc - 128u, m = x / (64u * KS), y = x % (64u * KS);
                const uint32_t row = y / (2u * KS), seg = y % (2u * KS);
#pragma unroll
                for (int n = 0; n < NQ; ++n)
                    if (m == (uint32_t)n)
                        r[j] = *(const u32x4 *)(qs[n] + ((uint64_t)b * S + ct * 32u + row) * d +
                                                h * DH + 8u * seg);
            }
        }
    }

    // P widened to fp32 once here for all draws; on a diagonal tile (mask) the keys after the
    // row's query become 0, so later arithmetic needs no causal test
    __device__ __forceinline__ void store(uint32_t tid, unsigned char *base, bool mask) const {
        constexpr uint32_t GP = g_pitch(KS);
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t pc = tid + 256u * j;
            if (pc < 128u) {
                const uint32_t row = pc >> 2, seg = pc & 3u;
                f32x4 *dst = (f32x4 *)(base + row * kPPitch + 32u * seg);
                const u32x4 w = r[j];
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[2 * e] = __uint_as_float(w[e] << 16);
                    f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
                if (mask) {
#pragma unroll
                    for (uint32_t e = 0; e < 8u; ++e) f[e] = 8u * seg + e <= row ? f[e] : 0.f;
                }
                dst[0] = f32x4{f[0], f[1], f[2], f[3]};
                dst[1] = f32x4{f[4], f[5], f[6], f[7]};
            } else if (pc < kPieces) {
                const uint32_t x = pc - 128u, m = x / (64u * KS), y = x % (64u * KS);
                const uint32_t row = y / (2u * KS), seg = y % (2u * KS);
                *(u32x4 *)(base + 32u * kPPitch + (m * 32u + row) * GP + 16u * seg) = r[j];
            }
        }
    }
};

// Steps in the order head, key tile, query tile >= key tile.
struct StepOrder {
    uint32_t h = 0, kt = 0, ct = 0;
    __device__ __forceinline__ StepOrder next(uint32_t nt) const {
        StepOrder n = *this;
        n.ct = ct + 1u;
        if (n.ct == nt) {
            n.kt = kt + 1u;
            n.ct = n.kt;
            if (n.kt == nt) { n.h = h + 1u; n.kt = 0; n.ct = 0; }
        }
        return n;
    }
};

// KS k-slices of 16 head columns: head width dh = 16 KS.
template <int KS>
__global__ __launch_bounds__(256) void attn_value_scores_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ g, float *__restrict__ c,
    uint32_t Kc, uint32_t T, uint32_t H, uint32_t S, uint32_t q0, float scale, Key key,
    uint32_t draw0, uint32_t tok0, uint32_t ndg) {
    // LDS: two stages of one step's operands (P tile [32 queries][32 keys], g tile
    // [32 queries][DH]), then per wave two rows of S running scores (lanes 0-31 sum draw i0's
    // keys, lanes 32-63 draw i0 + 1's).
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr uint32_t DH = 16u * KS;
    constexpr uint32_t GP = g_pitch(KS), SB = stage_bytes(KS, 1);
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = wave_in_block();
    const uint32_t lane = tid & 63u;
    const uint32_t b = blockIdx.x / ndg;
    // this wave's two draws (local indices i0, i0 + 1); a draw past the last one is computed
    // with the last draw's noise and not written, so every wave loads and synchronises
    const uint32_t i0 = (blockIdx.x % ndg) * 8u + wave * 2u;
    const uint32_t drawA = draw0 + min(i0, Kc - 1u), drawB = draw0 + min(i0 + 1u, Kc - 1u);
    const uint32_t col = lane & 31u, half = lane >> 5;
    float *cw = (float *)(lds + 2u * SB) + (uint64_t)wave * 2u * S;
    for (uint32_t t = lane; t < 2u * S; t += 64u) cw[t] = 0.f;
    float *cwh = cw + half * S;

    const uint32_t d = H * DH;
    const uint32_t nt = S / 32u;
    const uint16_t *const qs[1] = {g};
    Stager<KS, 1> stg;

    bf16x8 ahiA[KS], aloA[KS], ahiB[KS], aloB[KS];
    auto noise = [&](uint32_t h, uint32_t kt) {
        const uint32_t token = tok0 + b * S + kt * 32u + col;
        noise_fragments<KS>(key, q0 + h * (DH / 4u), half, token, drawA, ahiA, aloA);
        noise_fragments<KS>(key, q0 + h * (DH / 4u), half, token, drawB, ahiB, aloB);
    };

    // Step n's tiles are in LDS stage n % 2; step n + 1's are fetched into registers at the
    // start of step n and stored to the other stage at its end, before the one barrier per step.
    StepOrder cur;
    stg.load(tid, P, qs, b, H, S, d, 0, 0, 0);
    stg.store(tid, lds, true);
    noise(0, 0);
    __syncthreads();
    for (uint32_t st = 0;; st ^= 1u) {
        const StepOrder nx = cur.next(nt);
        const bool more = nx.h < H;   // uniform across the block
        if (more) stg.load(tid, P, qs, b, H, S, d, nx.h, nx.kt, nx.ct);

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
        // e[4 qd + r] is key row 8 qd + 4 half + r of the tile: weight by P and sum (the
        // diagonal tile's later keys were zeroed when staged)
        const unsigned char *prow = base + col * kPPitch + 16u * half;
        float partA = 0.f, partB = 0.f;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const f32x4 w = *(const f32x4 *)(prow + 32u * qd);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                partA = __builtin_fmaf(w[r], eA[4 * qd + r], partA);
                partB = __builtin_fmaf(w[r], eB[4 * qd + r], partB);
            }
        }
        // Swap the upper half of partA with the lower half of partB: afterwards lanes 0-31
        // hold both halves of draw A's key rows, lanes 32-63 both halves of draw B's.
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(partA),
                                                         __float_as_uint(partB), false, false);
        cwh[cur.ct * 32u + col] += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (!more) break;
        stg.store(tid, lds + (st ^ 1u) * SB, nx.kt == nx.ct);
        if (nx.kt != cur.kt || nx.h != cur.h) noise(nx.h, nx.kt);
        __syncthreads();
        cur = nx;
    }
#pragma unroll
    for (uint32_t k = 0; k < 2u; ++k) {
        if (i0 + k >= Kc) break;
        float *cr = c + (uint64_t)(i0 + k) * T + (uint64_t)b * S;
        for (uint32_t t = lane; t < S; t += 64u) cr[t] = scale * cw[k * S + t];
    }
}

// e^x - 1 with x = s1 D: a degree-5 Taylor polynomial in D (coefficients s_k = s1^k / k!) for
// |x| <= kPolyRange, where its error is below 1e-7 of the result; beyond, exp(x) - 1, whose
// relative error there is below 1e-6.
constexpr float kPolyRange = 0.2f;
struct Expm1Coef {
    float s1, s2, s3, s4, s5;
    float lim;   // kPolyRange / |s1|: |D| up to lim takes the polynomial
};

__device__ __forceinline__ float expm1_poly(float D, const Expm1Coef &e) {
    float p = __builtin_fmaf(D, e.s5, e.s4);
    p = __builtin_fmaf(D, p, e.s3);
    p = __builtin_fmaf(D, p, e.s2);
    p = __builtin_fmaf(D, p, e.s1);
    return D * p;
}

__device__ __forceinline__ float expm1_any(float D, const Expm1Coef &e) {
    const float x = e.s1 * D;
    return fabsf(x) <= kPolyRange ? expm1_poly(D, e) : expf(x) - 1.f;
}

template <int KS>
__global__ __launch_bounds__(256) void attn_key_scores_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ qm,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g, float *__restrict__ c,
    uint32_t Kc, uint32_t T, uint32_t H, uint32_t S, uint32_t q0, Expm1Coef ec, Key key,
    uint32_t draw0, uint32_t tok0, uint32_t ndg) {
    // LDS: two stages of one step's operands (P tile [32 queries][32 keys], q and g tiles
    // [32 queries][DH]); then per wave the head's running sums N1 and N0 of its two draws
    // ([N1 of A, N1 of B, N0 of A, N0 of B][S]); then per wave the partial row sums Z and base
    // over the 8 key rows of each tile that the wave owns ([Z, base][S]).
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr uint32_t DH = 16u * KS;
    constexpr uint32_t GP = g_pitch(KS), SB = stage_bytes(KS, 2);
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = wave_in_block();
    const uint32_t lane = tid & 63u;
    const uint32_t b = blockIdx.x / ndg;
    const uint32_t i0 = (blockIdx.x % ndg) * 8u + wave * 2u;
    const uint32_t drawA = draw0 + min(i0, Kc - 1u), drawB = draw0 + min(i0 + 1u, Kc - 1u);
    const uint32_t col = lane & 31u, half = lane >> 5;
    float *NN = (float *)(lds + 2u * SB);
    float *ZB = NN + 16u * S;
    float *n1w = NN + (wave * 4u + half) * S, *n0w = NN + (wave * 4u + 2u + half) * S;
    float *zbw = ZB + (wave * 2u + half) * S;

    const uint32_t d = H * DH;
    const uint32_t nt = S / 32u;
    const uint16_t *const qs[2] = {qm, g};
    Stager<KS, 2> stg;

    // key-side operands of the current key tile: both draws' noise and the values
    bf16x8 ahiA[KS], aloA[KS], ahiB[KS], aloB[KS], vb[KS];
    auto key_tile = [&](uint32_t h, uint32_t kt) {
        const uint32_t row = b * S + kt * 32u + col;
        const uint16_t *vrow = v + (uint64_t)row * d + h * DH + 8u * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            vb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(vrow + 16u * ks));
        noise_fragments<KS>(key, q0 + h * (DH / 4u), half, tok0 + row, drawA, ahiA, aloA);
        noise_fragments<KS>(key, q0 + h * (DH / 4u), half, tok0 + row, drawB, ahiB, aloB);
    };

    // A head is complete: fold its sums into the scores of this wave's draws. The first head
    // stores, later heads add; each lane rereads only what it wrote itself.
    auto fold_head = [&](bool first) {
#pragma unroll
        for (uint32_t k = 0; k < 2u; ++k) {
            if (i0 + k >= Kc) break;
            float *cr = c + (uint64_t)(i0 + k) * T + (uint64_t)b * S;
            const float *n1 = NN + (wave * 4u + k) * S, *n0 = NN + (wave * 4u + 2u + k) * S;
            for (uint32_t t = lane; t < S; t += 64u) {
                float Z = 0.f, bs = 0.f;
#pragma unroll
                for (uint32_t w = 0; w < 4u; ++w) {
                    Z += ZB[(2u * w) * S + t];
                    bs += ZB[(2u * w + 1u) * S + t];
                }
                const float val = Z > 0.f ? (Z * n1[t] - bs * n0[t]) / (Z * (Z + n0[t])) : 0.f;
                cr[t] = first ? -val : cr[t] - val;
            }
        }
    };

    StepOrder cur;
    stg.load(tid, P, qs, b, H, S, d, 0, 0, 0);
    stg.store(tid, lds, true);
    key_tile(0, 0);
    __syncthreads();
    for (uint32_t st = 0;; st ^= 1u) {
        if (cur.kt == 0 && cur.ct == 0 && cur.h > 0) {   // uniform across the block
            fold_head(cur.h == 1u);
            __syncthreads();   // every wave has read Z and base before they are overwritten
        }
        const StepOrder nx = cur.next(nt);
        const bool more = nx.h < H;
        if (more) stg.load(tid, P, qs, b, H, S, d, nx.h, nx.kt, nx.ct);

        const unsigned char *base = lds + st * SB;
        const unsigned char *qrow = base + 32u * kPPitch + col * GP + 16u * half;
        const unsigned char *grow = qrow + 32u * GP;
        f32x16 dA = {}, dB = {}, u = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 qb = *(const bf16x8 *)(qrow + 32u * ks);
            const bf16x8 gb = *(const bf16x8 *)(grow + 32u * ks);
            dA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahiA[ks], qb, dA, 0, 0, 0);
            dB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahiB[ks], qb, dB, 0, 0, 0);
            u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[ks], gb, u, 0, 0, 0);
            dA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aloA[ks], qb, dA, 0, 0, 0);
            dB = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aloB[ks], qb, dB, 0, 0, 0);
        }
        // element 4 qd + r is key row 8 qd + 4 half + r of the tile, query column col
        const unsigned char *prow = base + col * kPPitch + 16u * half;
        float w[16];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const f32x4 x = *(const f32x4 *)(prow + 32u * qd);
#pragma unroll
            for (int r = 0; r < 4; ++r) w[4 * qd + r] = x[r];
        }
        float mx = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(fabsf(dA[r]), fabsf(dB[r])));
        float n1A = 0.f, n0A = 0.f, n1B = 0.f, n0B = 0.f;
        if (__builtin_amdgcn_ballot_w64(!(mx <= ec.lim)) == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pu = w[r] * u[r];
                const float eA = expm1_poly(dA[r], ec), eB = expm1_poly(dB[r], ec);
                n1A = __builtin_fmaf(pu, eA, n1A);
                n0A = __builtin_fmaf(w[r], eA, n0A);
                n1B = __builtin_fmaf(pu, eB, n1B);
                n0B = __builtin_fmaf(w[r], eB, n0B);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pu = w[r] * u[r];
                const float eA = expm1_any(dA[r], ec), eB = expm1_any(dB[r], ec);
                n1A = __builtin_fmaf(pu, eA, n1A);
                n0A = __builtin_fmaf(w[r], eA, n0A);
                n1B = __builtin_fmaf(pu, eB, n1B);
                n0B = __builtin_fmaf(w[r], eB, n0B);
            }
        }
        // the draw-independent row sums: wave w takes key rows 8 w .. 8 w + 7 (its qd = w)
        float zs = 0.f, bs = 0.f;
#pragma unroll
        for (uint32_t qd = 0; qd < 4u; ++qd)
            if (qd == wave) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    zs += w[4 * qd + r];
                    bs = __builtin_fmaf(w[4 * qd + r], u[4 * qd + r], bs);
                }
            }
        // lane-half swaps: lanes 0-31 end with draw A's N1 / N0 and Z, lanes 32-63 with draw
        // B's N1 / N0 and base
        const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(n1A),
                                                         __float_as_uint(n1B), false, false);
        const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(n0A),
                                                         __float_as_uint(n0B), false, false);
        const auto sz = __builtin_amdgcn_permlane32_swap(__float_as_uint(zs), __float_as_uint(bs),
                                                         false, false);
        const float n1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
        const float n0 = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
        const float zb = __uint_as_float(sz[0]) + __uint_as_float(sz[1]);
        const uint32_t tq = cur.ct * 32u + col;
        if (cur.kt == 0) {   // a query tile's first key tile of the head starts its sums
            n1w[tq] = n1;
            n0w[tq] = n0;
            zbw[tq] = zb;
        } else {
            n1w[tq] += n1;
            n0w[tq] += n0;
            zbw[tq] += zb;
        }
        if (!more) break;
        stg.store(tid, lds + (st ^ 1u) * SB, nx.kt == nx.ct);
        if (nx.kt != cur.kt || nx.h != cur.h) key_tile(nx.h, nx.kt);
        __syncthreads();
        cur = nx;
    }
    __syncthreads();
    fold_head(H == 1u);
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
    const uint32_t q0 = (uint32_t)(chan0 / 4);   // chan0 % 4 == 0 and chan0 / 4 < 2^32
#define DUST_AVS(KS)                                                                           \
    attn_value_scores_kernel<KS><<<blocks, 256, 2 * stage_bytes(KS, 1) + cbytes, s>>>(        \
        P, g, c, (uint32_t)Kc, (uint32_t)(B * S), (uint32_t)H, (uint32_t)S, q0, scale, key,    \
        draw0, tok0, ndg)
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

size_t attn_key_scores_lds_bytes(int64_t S, int64_t dh) {
    // two stages, then 4 waves x (4 running sums + 2 row sums) x S floats
    return 2 * (size_t)stage_bytes((int)(dh / 16), 2) + (size_t)24 * S * sizeof(float);
}

hipError_t launch_attn_key_scores(const uint16_t *P, const uint16_t *q, const uint16_t *v,
                                  const uint16_t *g, float *c, int64_t Kc, int64_t B, int64_t H,
                                  int64_t S, int64_t dh, int64_t chan0, float sigma,
                                  float softmax_scale, Key key, uint32_t draw0, uint32_t tok0,
                                  hipStream_t s) {
    const uint32_t ndg = (uint32_t)((Kc + 7) / 8);
    const uint32_t blocks = (uint32_t)(B * ndg);
    // the logit shift is sigma tau <q, a> and the noise comes divided by kNormalScale
    const double s1 = (double)sigma * (double)softmax_scale * kNormalScale;
    Expm1Coef ec;
    ec.s1 = (float)s1;
    ec.s2 = (float)(s1 * s1 / 2.0);
    ec.s3 = (float)(s1 * s1 * s1 / 6.0);
    ec.s4 = (float)(s1 * s1 * s1 * s1 / 24.0);
    ec.s5 = (float)(s1 * s1 * s1 * s1 * s1 / 120.0);
    ec.lim = s1 == 0.0 ? __builtin_huge_valf() : (float)((double)kPolyRange / fabs(s1));
    const uint32_t q0 = (uint32_t)(chan0 / 4);
    const size_t lds = attn_key_scores_lds_bytes(S, dh);
#define DUST_AKS(KS)                                                                           \
    attn_key_scores_kernel<KS><<<blocks, 256, lds, s>>>(P, q, v, g, c, (uint32_t)Kc,           \
                                                        (uint32_t)(B * S), (uint32_t)H,        \
                                                        (uint32_t)S, q0, ec, key, draw0, tok0, \
                                                        ndg)
    switch (dh / 16) {
        case 1: DUST_AKS(1); break;
        case 2: DUST_AKS(2); break;
        case 3: DUST_AKS(3); break;
        case 4: DUST_AKS(4); break;
        case 5: DUST_AKS(5); break;
        case 6: DUST_AKS(6); break;
        case 7: DUST_AKS(7); break;
        default: DUST_AKS(8); break;
    }
#undef DUST_AKS
    return hipGetLastError();
}

}  // namespace dust
