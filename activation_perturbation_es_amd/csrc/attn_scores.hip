// Inner-product scores of a perturbed attention value, key or query projection (gfx950).
//
// Explainer cnblogs.com/32bin/p/23212811, "The real work: suppressing interference": attention
// internals are scored through the attention output, by the inner product of the output's
// change with the output's estimated error g. No kernel forms Delta o (K x T x d values).
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
// a form whose terms are all O(sigma), so nothing cancels at the O(1) level. Its numerator is
// sum_s W_ts (e^delta_ts - 1) with W_ts = P_ts (Z_t u_ts - base_t), which does not depend on the
// draw: the row-weights kernel forms W and Z once, and per draw and element the scorers need
// only e^delta - 1 and two fused multiply-adds. Queries (q'_t = q_t + sigma a_t) are the same
// re-run with delta_ts = sigma tau <a_t, k_s>.
//
// The scorers regenerate the noise of one tile of 32 tokens once per draw, and for every tile
// of 32 tokens it meets form the 32 x 32 inner products on the matrix cores
// (v_mfma_f32_32x32x16_bf16; the noise split into a bf16 high part and a bf16 remainder so that
// it keeps 16 significant bits): E_st = <a_s, g_t> for values, D_st = <a_s, q_t> for keys,
// D_ts = <a_t, k_s> for queries. The output tile's layout (lane l holds column l % 32 and 16 of
// the rows) lets each lane weight and sum its elements; lane-half swaps (v_permlane32_swap) or
// DPP row exchanges complete the sums over the tile.
//
// Work layout: a block owns one sequence and several draws (values: 4 waves, two draws each;
// keys and queries: 12 waves of one draw where the registers allow, else 8, and for queries 8
// waves of two draws when that grid ends sooner; long sequences take fewer key draws per block,
// as the key scores' running sums fill the LDS); the block walks heads, then tiles in causal
// order. Each step's weight tiles (widened to fp32, the causal mask applied) and bf16 side tiles
// are staged in LDS by the whole block, double-buffered with one barrier per step; the operands
// of the outer tile (noise) stay in registers across its inner tiles.
#include <atomic>

#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// LDS row pitches (bytes): 32 keys of P (or W) as fp32 plus 16 bytes and DH bf16 columns of a
// query-side tile plus 16 bytes, so that the 16-byte fragment reads of 16 consecutive rows fall
// into distinct banks.
constexpr uint32_t kPPitch = 144;
__host__ __device__ constexpr uint32_t g_pitch(int KS) { return 32u * KS + 16u; }
// one step's operands: the P tile, with HW the W tile, and NQ side tiles of 32 rows
__host__ __device__ constexpr uint32_t stage_bytes(int KS, int NQ, bool HW = false) {
    return 32u * ((HW ? 2u : 1u) * kPPitch + NQ * g_pitch(KS));
}

// The A operand of one key row: the noise of key `token` at channels 4 q0 + 16 ks + 8 half ..
// + 7 of every k-slice ks (q0 = the head's first channel / 4), as a bf16 high part and a bf16
// remainder. The values are the normals divided by kNormalScale; callers fold it into their
// scale.
template <int KS>
__device__ __forceinline__ void noise_fragments(const Key &key, uint32_t q0, uint32_t half,
                                                uint32_t token, uint32_t draw, bf16x8 (&ahi)[KS],
                                                bf16x8 (&alo)[KS], float *norm2 = nullptr) {
    float n2 = 0.f;
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
            if (norm2) n2 = __builtin_fmaf(x1, x1, __builtin_fmaf(x0, x0, n2));
            hw[e] = pack_bf16x2(x0, x1);
            lw[e] = pack_bf16x2(x0 - __uint_as_float(hw[e] << 16),
                                x1 - __uint_as_float(hw[e] & 0xFFFF0000u));
        }
        ahi[ks] = as_bf16x8(hw);
        alo[ks] = as_bf16x8(lw);
    }
    if (norm2) *norm2 = n2;
}

// The value of another lane of the same DPP row (CTRL: a DPP row or quad pattern; no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_shuffled(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sums over the 32 lanes of each half of the wave of 32 values per lane, transposed: afterwards
// lane l holds the total of v[l & 31] over its half. Each stage pairs every lane with a lane of
// the other class and halves the slots: the lane keeps the slot of its class, sends the other
// and adds what its partner sends for the same slot. Classes and exchanges: lane bit 4 (rows 16
// apart, v_permlane16_swap, which exchanges and sums a pair of slots in two instructions), then
// within each row of 16 the mirror (bit 3), the half mirror (bit 2) and the quad exchanges
// (bits 1 and 0), all DPP.
__device__ __forceinline__ float half_wave_transpose_sum(const float (&v)[32], uint32_t lane) {
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                         __float_as_uint(v[i + 16]), false, false);
        a[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const bool c3 = (lane & 8u) != 0, c2 = (lane & 4u) != 0, c1 = (lane & 2u) != 0,
               c0 = (lane & 1u) != 0;
    float b8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float keep = c3 ? a[i + 8] : a[i], send = c3 ? a[i] : a[i + 8];
        b8[i] = keep + dpp_shuffled<0x140>(send);   // row_mirror: lane 15 - p of the row
    }
    float b4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = c2 ? b8[i + 4] : b8[i], send = c2 ? b8[i] : b8[i + 4];
        b4[i] = keep + dpp_shuffled<0x141>(send);   // row_half_mirror: lane 7 - p of the half row
    }
    float b2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = c1 ? b4[i + 2] : b4[i], send = c1 ? b4[i] : b4[i + 2];
        b2[i] = keep + dpp_shuffled<0x4E>(send);    // quad_perm [2, 3, 0, 1]
    }
    const float keep = c0 ? b2[1] : b2[0], send = c0 ? b2[0] : b2[1];
    return keep + dpp_shuffled<0xB1>(send);         // quad_perm [1, 0, 3, 2]
}

// Staging of one step as 16-byte pieces: the P tile's rows first (4 per row of 32 bf16), then
// with HW the W tile's rows (8 per row of 32 fp32), then the NQ side tiles (2 KS per row each);
// loads into registers, stores to LDS after the step's compute. A stage in LDS holds P
// [32][kPPitch], with HW W [32][kPPitch], then the side tiles [NQ][32][g_pitch].
template <int KS, int NQ, uint32_t NT = 256, bool TP = false, bool HW = false>
struct Stager {
    static constexpr uint32_t kW = HW ? 256u : 0u;
    static constexpr uint32_t kPieces = 128u + kW + 64u * KS * NQ;
    static constexpr uint32_t kPerThread = (kPieces + NT - 1u) / NT;
    static constexpr uint32_t kSide = (HW ? 64u : 32u) * kPPitch;   // bytes before the side tiles
    u32x4 r[kPerThread];

    const unsigned char *src[kPerThread];   // this thread's piece at tile offset zero

    // The per-thread part of every step's addresses, once per block. P [B, H, S, S] and
    // W [B, H, S, S] of sequence b; the side arrays [T, H DH] from the sequence's first row.
    __device__ __forceinline__ void init(uint32_t tid, const uint16_t *P, const float *Wm,
                                         const uint16_t *const (&qs)[NQ], uint32_t b, uint32_t H,
                                         uint32_t S, uint32_t d) {
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t pc = tid + NT * j;
            src[j] = (const unsigned char *)P;
            if (pc >= kPieces) continue;
            if (pc < 128u) {
                const uint32_t row = pc >> 2, seg = pc & 3u;
                src[j] = (const unsigned char *)(P + ((uint64_t)b * H * S + row) * S + 8u * seg);
            } else if (HW && pc < 128u + kW) {
                const uint32_t x = pc - 128u, row = x >> 3, seg = x & 7u;
                src[j] = (const unsigned char *)(Wm + ((uint64_t)b * H * S + row) * S + 4u * seg);
            } else {
                const uint32_t x = pc - 128u - kW, m = x / (64u * KS), y = x % (64u * KS);
                const uint32_t row = y / (2u * KS), seg = y % (2u * KS);
#pragma unroll
                for (int n = 0; n < NQ; ++n)
                    if (m == (uint32_t)n)
                        src[j] = (const unsigned char *)(qs[n] + ((uint64_t)b * S + row) * d +
                                                         8u * seg);
            }
        }
    }

    // One step's pieces into registers: query tile ct over key tile kt of head h for P and W,
    // row tile xt of the side arrays (the query tile for value and key scores, the key tile for
    // query scores). The kind of piece is the same across a wave (P, W and the side tiles start
    // at multiples of 64 pieces), so the tile offset is chosen on the scalar unit.
    __device__ __forceinline__ void load(uint32_t tid, uint32_t S, uint32_t d, uint32_t h,
                                         uint32_t kt, uint32_t ct, uint32_t xt) {
        constexpr uint32_t DH = 16u * KS;
        const uint64_t tile = ((uint64_t)h * S + ct * 32u) * S + kt * 32u;   // elements
        const uint64_t side = 2u * ((uint64_t)xt * 32u * d + h * DH);         // bytes
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(tid & ~63u);
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t pc0 = w0 + NT * j;
            if (pc0 >= kPieces) continue;
            const uint64_t off = pc0 < 128u ? 2u * tile : (HW && pc0 < 128u + kW) ? 4u * tile
                                                                                   : side;
            r[j] = *(const u32x4 *)(src[j] + off);
        }
    }

    // P widened to fp32 once here for all draws; on a diagonal tile (mask) the keys after the
    // row's query become 0 in P and W, so later arithmetic needs no causal test. TP stores the
    // P and W tiles transposed, [32 keys][32 queries].
    __device__ __forceinline__ void store(uint32_t tid, unsigned char *tb, bool mask) const {
        constexpr uint32_t GP = g_pitch(KS);
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; ++j) {
            const uint32_t pc = tid + NT * j;
            if (pc >= kPieces) continue;
            if (pc < 128u) {
                const uint32_t row = pc >> 2, seg = pc & 3u;
                f32x4 *dst = (f32x4 *)(tb + row * kPPitch + 32u * seg);
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
                if (TP) {
#pragma unroll
                    for (uint32_t e = 0; e < 8u; ++e)
                        *(float *)(tb + (8u * seg + e) * kPPitch + 4u * row) = f[e];
                } else {
                    dst[0] = f32x4{f[0], f[1], f[2], f[3]};
                    dst[1] = f32x4{f[4], f[5], f[6], f[7]};
                }
            } else if (HW && pc < 128u + kW) {
                const uint32_t x = pc - 128u, row = x >> 3, seg = x & 7u;
                unsigned char *wt = tb + 32u * kPPitch;
                const u32x4 w = r[j];
                float f[4];
#pragma unroll
                for (uint32_t e = 0; e < 4u; ++e) {
                    f[e] = __uint_as_float(w[e]);
                    if (mask) f[e] = 4u * seg + e <= row ? f[e] : 0.f;
                }
                if (TP) {
#pragma unroll
                    for (uint32_t e = 0; e < 4u; ++e)
                        *(float *)(wt + (4u * seg + e) * kPPitch + 4u * row) = f[e];
                } else {
                    *(f32x4 *)(wt + row * kPPitch + 16u * seg) = f32x4{f[0], f[1], f[2], f[3]};
                }
            } else {
                const uint32_t x = pc - 128u - kW, m = x / (64u * KS), y = x % (64u * KS);
                const uint32_t row = y / (2u * KS), seg = y % (2u * KS);
                *(u32x4 *)(tb + kSide + (m * 32u + row) * GP + 16u * seg) = r[j];
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
    stg.init(tid, P, nullptr, qs, b, H, S, d);
    stg.load(tid, S, d, 0, 0, 0, 0);
    stg.store(tid, lds, true);
    noise(0, 0);
    __syncthreads();
    for (uint32_t st = 0;; st ^= 1u) {
        const StepOrder nx = cur.next(nt);
        const bool more = nx.h < H;   // uniform across the block
        if (more) stg.load(tid, S, d, nx.h, nx.kt, nx.ct, nx.ct);

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

// e^x - 1 with x = s1 D: for |x| <= kPolyRange, x + x^2 q(x), the leading term exact and q the
// quadratic that minimises the largest relative error over the range (fitted by linear
// programming on a dense grid); evaluated in D by Horner's rule, three fused multiply-adds and a
// multiply, it stays within 8.5e-7 of e^x - 1 in fp32 (the fit alone 7.0e-7), and its error falls
// like x^4 towards 0. Beyond, exp(x) - 1, within about 1e-6 of the result there.
constexpr float kPolyRange = 0.15f;
constexpr double kExpm1Q0 = 0.50000103352597824, kExpm1Q1 = 0.16682308873996046,
                 kExpm1Q2 = 0.0416364346995442;
struct Expm1Coef {
    float s1, a2, a3, a4;    // s1 and s1^k q_{k-2}: the polynomial in D
    float lim;               // kPolyRange / |s1|: |D| up to lim takes the polynomial
};

__device__ __forceinline__ float expm1_poly(float D, const Expm1Coef &e) {
    float p = __builtin_fmaf(D, e.a4, e.a3);
    p = __builtin_fmaf(D, p, e.a2);
    p = __builtin_fmaf(D, p, e.s1);
    return D * p;
}

__device__ __forceinline__ float expm1_any(float D, const Expm1Coef &e) {
    const float x = e.s1 * D;
    return fabsf(x) <= kPolyRange ? expm1_poly(D, e) : expf(x) - 1.f;
}

// Row weights of the softmax re-run, shared by the key and query scores. With u_ts = <v_s, g_t>,
// Z_t = sum_{s <= t} P_ts and base_t = sum_{s <= t} P_ts u_ts, a re-run under logit shifts
// delta changes the output's inner product at query t by
//     (Z N1 - base N0) / (Z (Z + N0)) = sum_s W_ts (e^delta_ts - 1) / (Z_t (Z_t + N0_t)),
//     W_ts = P_ts (Z_t u_ts - base_t),  N0_t = sum_s P_ts (e^delta_ts - 1),
// and W, Z do not depend on the draw. One wave per tile of 32 queries of one (sequence, head):
// u on the matrix cores (value rows as the A operand, g rows as B; element r of a lane is key
// 8 (r / 4) + 4 half + r % 4 of the tile, its query the lane's column), a first pass over the
// key tiles at or before the query tile sums Z and base, a second writes W; tiles above the
// diagonal are written as zeros.
template <int KS>
__global__ __launch_bounds__(256) void attn_row_weights_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ g, float *__restrict__ W, float *__restrict__ Z, uint32_t H,
    uint32_t S, uint32_t ntiles) {
    constexpr uint32_t DH = 16u * KS;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t gt = blockIdx.x * 4u + wave_in_block();   // query tile over (b, h, ct)
    if (gt >= ntiles) return;
    const uint32_t nt = S / 32u, ct = gt % nt, bh = gt / nt, h = bh % H, b = bh / H;
    const uint32_t col = lane & 31u, half = lane >> 5;
    const uint32_t d = H * DH;
    const uint32_t t = ct * 32u + col;   // this lane's query
    bf16x8 gb[KS];
    const uint16_t *grow = g + ((uint64_t)b * S + t) * d + h * DH + 8u * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        gb[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(grow + 16u * ks));
    const uint64_t rowoff = (((uint64_t)b * H + h) * S + t) * S;
    const uint16_t *prow = P + rowoff;
    float *wrow = W + rowoff;

    auto u_tile = [&](uint32_t kt) {
        const uint16_t *vrow = v + ((uint64_t)b * S + kt * 32u + col) * d + h * DH + 8u * half;
        f32x16 u = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *(const u32x4 *)(vrow + 16u * ks)), gb[ks], u, 0, 0, 0);
        return u;
    };
    // the lane's weights over its 16 keys of tile kt, 0 past its query
    auto p_tile = [&](uint32_t kt, float (&p)[16]) {
#pragma unroll
        for (uint32_t qd = 0; qd < 4u; ++qd) {
            const uint2 w = *(const uint2 *)(prow + kt * 32u + 8u * qd + 4u * half);
            p[4 * qd + 0] = __uint_as_float(w.x << 16);
            p[4 * qd + 1] = __uint_as_float(w.x & 0xFFFF0000u);
            p[4 * qd + 2] = __uint_as_float(w.y << 16);
            p[4 * qd + 3] = __uint_as_float(w.y & 0xFFFF0000u);
#pragma unroll
            for (uint32_t r = 0; r < 4u; ++r)
                p[4 * qd + r] = kt * 32u + 8u * qd + 4u * half + r <= t ? p[4 * qd + r] : 0.f;
        }
    };

    float z = 0.f, bs = 0.f;
    for (uint32_t kt = 0; kt <= ct; ++kt) {
        const f32x16 u = u_tile(kt);
        float p[16];
        p_tile(kt, p);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            z += p[r];
            bs = __builtin_fmaf(p[r], u[r], bs);
        }
    }
    z += __shfl_xor(z, 32);
    bs += __shfl_xor(bs, 32);
    if (half == 0) Z[((uint64_t)b * H + h) * S + t] = z;
    for (uint32_t kt = 0; kt < nt; ++kt) {
        float w[16];
        if (kt <= ct) {
            const f32x16 u = u_tile(kt);
            float p[16];
            p_tile(kt, p);
#pragma unroll
            for (int r = 0; r < 16; ++r) w[r] = p[r] * __builtin_fmaf(z, u[r], -bs);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) w[r] = 0.f;
        }
#pragma unroll
        for (uint32_t qd = 0; qd < 4u; ++qd)
            *(f32x4 *)(wrow + kt * 32u + 8u * qd + 4u * half) =
                f32x4{w[4 * qd], w[4 * qd + 1], w[4 * qd + 2], w[4 * qd + 3]};
    }
}

// Key scores: NW waves per block (three per SIMD where the registers allow, so that fp32 FMAs
// of two waves can issue together), one draw per wave, one sequence per
// block. Per step each wave forms D = a q^T on the matrix cores, then per element
// e = e^{s D} - 1 and M += W e, N0 += P e over the tile's keys (one lane-half swap completes
// both sums) into running sums in LDS; at each head's end every wave folds M / (Z (Z + N0))
// into its draw's scores.
template <int KS, int NW>
__global__ __launch_bounds__(NW * 64) void attn_key_scores_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ qm,
    const float *__restrict__ Wm, const float *__restrict__ Zm, float *__restrict__ c,
    uint32_t Kc, uint32_t T, uint32_t H, uint32_t S, uint32_t q0, Expm1Coef ec, Key key,
    uint32_t draw0, uint32_t tok0, uint32_t ndg) {
    // LDS: two stages of one step's operands (P and W tiles [32 queries][32 keys] in fp32, the
    // q tile [32 queries][DH]); per wave the head's running sums of its draw, [M, N0][S]; the
    // head's query norms |q_t|, [S].
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr uint32_t DH = 16u * KS;
    constexpr uint32_t GP = g_pitch(KS), SB = stage_bytes(KS, 1, true);
    using Stg = Stager<KS, 1, NW * 64, false, true>;
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = wave_in_block();
    const uint32_t lane = tid & 63u;
    const uint32_t b = blockIdx.x / ndg;
    // this wave's draw; a draw past the last one is computed with the last draw's noise and
    // not written, so every wave loads and synchronises
    const uint32_t i = (blockIdx.x % ndg) * (uint32_t)NW + wave;
    const uint32_t draw = draw0 + min(i, Kc - 1u);
    const uint32_t col = lane & 31u, half = lane >> 5;
    float *NN = (float *)(lds + 2u * SB);
    float *QN = NN + 2u * NW * S;
    float *nnw = NN + (wave * 2u + half) * S;   // lanes 0-31 keep M, lanes 32-63 N0

    const uint32_t d = H * DH;
    const uint32_t nt = S / 32u;
    const uint16_t *const qs[1] = {qm};
    Stg stg;

    // key-side operands of the current key tile: the draw's noise and the largest noise norm
    // over the tile's 32 keys (for the range test of e^x - 1)
    bf16x8 ahi[KS], alo[KS];
    float amax = 0.f;
    auto key_tile = [&](uint32_t h, uint32_t kt) {
        const uint32_t row = b * S + kt * 32u + col;
        float n2;
        noise_fragments<KS>(key, q0 + h * (DH / 4u), half, tok0 + row, draw, ahi, alo, &n2);
        n2 += __shfl_xor(n2, 32);
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) n2 = fmaxf(n2, __shfl_xor(n2, m));
        amax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_sqrtf(n2))));
    };
    // |q_t| of head h for every query of the sequence
    auto query_norms = [&](uint32_t h) {
        for (uint32_t t = tid; t < S; t += NW * 64u) {
            const uint16_t *qrow = qm + ((uint64_t)b * S + t) * d + h * DH;
            float n2 = 0.f;
#pragma unroll
            for (uint32_t p = 0; p < 2u * KS; ++p) {
                const u32x4 w = *(const u32x4 *)(qrow + 8u * p);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(w[e] << 16);
                    const float hi = __uint_as_float(w[e] & 0xFFFF0000u);
                    n2 = __builtin_fmaf(hi, hi, __builtin_fmaf(lo, lo, n2));
                }
            }
            QN[t] = __builtin_sqrtf(n2);
        }
    };

    // Head hd is complete: fold its sums into the score of this wave's draw. Head 0 stores,
    // later heads add; each lane rereads only what it wrote itself.
    auto fold_head = [&](uint32_t hd) {
        if (i >= Kc) return;
        float *cr = c + (uint64_t)i * T + (uint64_t)b * S;
        const float *zr = Zm + ((uint64_t)b * H + hd) * S;
        const float *m1 = NN + (wave * 2u) * S, *n0 = m1 + S;
        for (uint32_t t = lane; t < S; t += 64u) {
            const float Z = zr[t];
            // The form loses precision where the shifts move the row's mass far: Z + N0 below
            // Z / 2 comes from cancellation; above 2^20 Z the shifts are large enough for the
            // noise's 16 significant bits to show in e^delta, and near 1e30 they approach its
            // range. Such a query is left NaN, and the repair pass recomputes it.
            const float zn = Z + n0[t], den = Z * zn;
            const bool exact = zn >= 0.5f * Z && zn <= 1048576.f * Z && den < 1e30f;
            const float val = !(Z > 0.f) ? 0.f : exact ? m1[t] / den : __builtin_nanf("");
            cr[t] = hd == 0 ? -val : cr[t] - val;
        }
    };

    // |D| <= lim keeps e^x - 1 on the polynomial. Cauchy-Schwarz bounds |D| by |q_t| amax; the
    // margin covers the rounding of the norms and of the matrix-core sums.
    const float lim_cs = ec.lim * 0.999f;
    const uint32_t lim_bits = __float_as_uint(ec.lim) << 1;   // |x| bits shifted past the sign

    // One query tile's vector work: e^x - 1 of the products, weighted sums over the tile's keys
    // into the running sums of query tile qt.
    auto tile_sums = [&](const f32x16 &dd, const unsigned char *tb, uint32_t qt, bool first) {
        const uint32_t tq = qt * 32u + col;
        const float qn = QN[tq];
        // element 4 qd + r is key row 8 qd + 4 half + r of the tile, query column col
        const unsigned char *prow = tb + col * kPPitch + 16u * half;
        const unsigned char *wrow = prow + 32u * kPPitch;
        float p[16], w[16];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const f32x4 x = *(const f32x4 *)(prow + 32u * qd);
            const f32x4 y = *(const f32x4 *)(wrow + 32u * qd);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[4 * qd + r] = x[r];
                w[4 * qd + r] = y[r];
            }
        }
        bool poly = __builtin_amdgcn_ballot_w64(!(qn * amax <= lim_cs)) == 0;
        if (!poly) {   // the bound is loose: test the products themselves
            uint32_t m = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) m = max(m, __float_as_uint(dd[r]) << 1);
            poly = __builtin_amdgcn_ballot_w64(!(m <= lim_bits)) == 0;
        }
        // e^x - 1 first, the sums after, so that both forms feed the same accumulators
        float e[16];
        if (poly) {
#pragma unroll
            for (int r = 0; r < 16; ++r) e[r] = expm1_poly(dd[r], ec);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) e[r] = expm1_any(dd[r], ec);
        }
        float m1 = 0.f, n0 = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            m1 = __builtin_fmaf(w[r], e[r], m1);
            n0 = __builtin_fmaf(p[r], e[r], n0);
        }
        // lane-half swap: lanes 0-31 end with M over the tile's 32 keys, lanes 32-63 with N0
        const auto sn = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1), __float_as_uint(n0),
                                                         false, false);
        const float nn = __uint_as_float(sn[0]) + __uint_as_float(sn[1]);
        if (first)   // a query tile's first key tile of the head starts its sums
            nnw[tq] = nn;
        else
            nnw[tq] += nn;
    };

    StepOrder cur;
    stg.init(tid, P, Wm, qs, b, H, S, d);
    stg.load(tid, S, d, 0, 0, 0, 0);
    stg.store(tid, lds, true);
    query_norms(0);
    key_tile(0, 0);
    __syncthreads();
    for (uint32_t st = 0;; st ^= 1u) {
        if (cur.kt == 0 && cur.ct == 0 && cur.h > 0) {   // uniform across the block
            fold_head(cur.h - 1u);
            query_norms(cur.h);
            __syncthreads();   // query norms written before they are used
        }
        const StepOrder nx = cur.next(nt);
        const bool more = nx.h < H;
        if (more) stg.load(tid, S, d, nx.h, nx.kt, nx.ct, nx.ct);

        const unsigned char *base = lds + st * SB;
        const unsigned char *qrow = base + Stg::kSide + col * GP + 16u * half;
        f32x16 dd = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 qb = *(const bf16x8 *)(qrow + 32u * ks);
            dd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], qb, dd, 0, 0, 0);
            dd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[ks], qb, dd, 0, 0, 0);
        }
        tile_sums(dd, base, cur.ct, cur.kt == 0);
        if (!more) break;
        stg.store(tid, lds + (st ^ 1u) * SB, nx.kt == nx.ct);
        if (nx.kt != cur.kt || nx.h != cur.h) key_tile(nx.h, nx.kt);
        __syncthreads();
        cur = nx;
    }
    fold_head(H - 1u);
}

// Query scores: the transpose of the key scores. The noise sits on the query side, so a block
// walks heads, then query tiles, then the key tiles at or before the query tile, generating the
// noise of a query tile once; the product D^T = a k^T comes out with the query tile's rows in
// each lane's registers and its key in the lane's column, so every lane keeps the running sums
// M, N0 of its 16 query rows in registers over the key tiles and one lane reduction per query
// tile completes them. NW waves, DPW draws per wave (two read each step's k, P and W tiles from
// LDS once for both draws).
template <int KS, int NW, int DPW>
__global__ __launch_bounds__(NW * 64) void attn_query_scores_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ km,
    const float *__restrict__ Wm, const float *__restrict__ Zm, float *__restrict__ c,
    uint32_t Kc, uint32_t T, uint32_t H, uint32_t S, uint32_t q0, Expm1Coef ec, Key key,
    uint32_t draw0, uint32_t tok0, uint32_t ndg) {
    // LDS: two stages of one step's operands (P and W tiles transposed, [32 keys][32 queries]
    // in fp32, the k tile [32 keys][DH]); the key norms |k_s|, double-buffered by head, [2][S].
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr uint32_t DH = 16u * KS;
    constexpr uint32_t GP = g_pitch(KS), SB = stage_bytes(KS, 1, true);
    using Stg = Stager<KS, 1, NW * 64, true, true>;
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = wave_in_block();
    const uint32_t lane = tid & 63u;
    const uint32_t b = blockIdx.x / ndg;
    const uint32_t i0 = ((blockIdx.x % ndg) * (uint32_t)NW + wave) * (uint32_t)DPW;
    const uint32_t col = lane & 31u, half = lane >> 5;
    float *KN = (float *)(lds + 2u * SB);

    const uint32_t d = H * DH;
    const uint32_t nt = S / 32u;
    const uint16_t *const ks_[1] = {km};
    Stg stg;

    // query-side operands of the current query tile, per draw: the noise and the largest noise
    // norm over the tile's 32 queries
    bf16x8 ahi[DPW][KS], alo[DPW][KS];
    float amax[DPW];
    auto query_tile = [&](uint32_t h, uint32_t ct) {
        const uint32_t row = b * S + ct * 32u + col;
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
            const uint32_t draw = draw0 + min(i0 + (uint32_t)j, Kc - 1u);
            float n2;
            noise_fragments<KS>(key, q0 + h * (DH / 4u), half, tok0 + row, draw, ahi[j], alo[j],
                                &n2);
            n2 += __shfl_xor(n2, 32);
#pragma unroll
            for (int m = 16; m >= 1; m >>= 1) n2 = fmaxf(n2, __shfl_xor(n2, m));
            amax[j] = __uint_as_float(
                __builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_sqrtf(n2))));
        }
    };
    // |k_s| of head h for every key of the sequence
    auto key_norms = [&](uint32_t h) {
        float *kn = KN + (h & 1u) * S;
        for (uint32_t t = tid; t < S; t += NW * 64u) {
            const uint16_t *krow = km + ((uint64_t)b * S + t) * d + h * DH;
            float n2 = 0.f;
#pragma unroll
            for (uint32_t p = 0; p < 2u * KS; ++p) {
                const u32x4 w = *(const u32x4 *)(krow + 8u * p);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(w[e] << 16);
                    const float hi = __uint_as_float(w[e] & 0xFFFF0000u);
                    n2 = __builtin_fmaf(hi, hi, __builtin_fmaf(lo, lo, n2));
                }
            }
            kn[t] = __builtin_sqrtf(n2);
        }
    };

    const float lim_cs = ec.lim * 0.999f;
    const uint32_t lim_bits = __float_as_uint(ec.lim) << 1;

    // running sums of the current query tile, per draw: element r is query row
    // 8 (r / 4) + 4 half + r % 4, summed over this lane's key column
    float m1[DPW][16], n0[DPW][16];
    auto reset = [&]() {
#pragma unroll
        for (int j = 0; j < DPW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) m1[j][r] = n0[j][r] = 0.f;
    };
    // Query tile ct of head h is complete: sum the running sums of draw j over the 32 key
    // columns (lanes of one half); lane l then takes the totals of row m(l) = 8 ((l & 15) >> 2) +
    // 4 (l >> 5) + (l & 3) when (l & 31) < 16 and folds M / (Z (Z + N0)) into the draw's score.
    // Head 0 stores, later heads add.
    auto finish_tile = [&](uint32_t h, uint32_t ct, int j) {
        // transposed sum over the 32 lanes of each half: lane l ends with the total of slot
        // l & 31 of v = (M of rows 0..15, N0 of rows 0..15)
        float v[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            v[r] = m1[j][r];
            v[16 + r] = n0[j][r];
        }
        const float x = half_wave_transpose_sum(v, lane);
        // M and N0 of row lane & 15 sit in lanes 16 apart
        const float other = __shfl_xor(x, 16);
        const bool hi16 = (lane & 16u) != 0;
        const float t1 = hi16 ? other : x, t0 = hi16 ? x : other;
        const uint32_t i = i0 + (uint32_t)j;
        if (i >= Kc || (lane & 31u) >= 16u) return;
        const uint32_t m = 8u * ((lane & 15u) >> 2) + 4u * half + (lane & 3u);
        const float Z = Zm[((uint64_t)b * H + h) * S + ct * 32u + m];
        // far-moved rows: repaired as in the key scores
        const float zn = Z + t0, den = Z * zn;
        const bool exact = zn >= 0.5f * Z && zn <= 1048576.f * Z && den < 1e30f;
        const float val = !(Z > 0.f) ? 0.f : exact ? t1 / den : __builtin_nanf("");
        float *cr = c + (uint64_t)i * T + (uint64_t)b * S + ct * 32u + m;
        *cr = h == 0 ? -val : *cr - val;
    };

    // steps: head, query tile ct, key tile kt <= ct
    uint32_t h = 0, ct = 0, kt = 0;
    stg.init(tid, P, Wm, ks_, b, H, S, d);
    stg.load(tid, S, d, 0, 0, 0, 0);
    stg.store(tid, lds, true);
    key_norms(0);
    query_tile(0, 0);
    reset();
    __syncthreads();
    for (uint32_t st = 0;; st ^= 1u) {
        uint32_t nh = h, nc = ct, nk = kt + 1u;
        if (nk > ct) {
            nk = 0;
            nc = ct + 1u;
            if (nc == nt) { nc = 0; nh = h + 1u; }
        }
        const bool more = nh < H;
        // the staged key tile is kt; the P and W tiles are (query tile ct, key tile kt)
        if (more) stg.load(tid, S, d, nh, nk, nc, nk);   // k of key tile nk

        const unsigned char *base = lds + st * SB;
        const unsigned char *krow = base + Stg::kSide + col * GP + 16u * half;
        f32x16 dd[DPW];
#pragma unroll
        for (int j = 0; j < DPW; ++j) dd[j] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kb = *(const bf16x8 *)(krow + 32u * ks);
#pragma unroll
            for (int j = 0; j < DPW; ++j)
                dd[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[j][ks], kb, dd[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < DPW; ++j)
                dd[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[j][ks], kb, dd[j], 0, 0, 0);
        }
        const float kn = KN[(h & 1u) * S + kt * 32u + col];
        const unsigned char *prow = base + col * kPPitch + 16u * half;
        const unsigned char *wrow = prow + 32u * kPPitch;
        float p[16], w[16];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const f32x4 x = *(const f32x4 *)(prow + 32u * qd);
            const f32x4 y = *(const f32x4 *)(wrow + 32u * qd);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[4 * qd + r] = x[r];
                w[4 * qd + r] = y[r];
            }
        }
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
            bool poly = __builtin_amdgcn_ballot_w64(!(kn * amax[j] <= lim_cs)) == 0;
            if (!poly) {
                uint32_t mb = 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) mb = max(mb, __float_as_uint(dd[j][r]) << 1);
                poly = __builtin_amdgcn_ballot_w64(!(mb <= lim_bits)) == 0;
            }
            // e^x - 1 first, the sums after, so that both forms feed the same accumulators
            float e[16];
            if (poly) {
#pragma unroll
                for (int r = 0; r < 16; ++r) e[r] = expm1_poly(dd[j][r], ec);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) e[r] = expm1_any(dd[j][r], ec);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                m1[j][r] = __builtin_fmaf(w[r], e[r], m1[j][r]);
                n0[j][r] = __builtin_fmaf(p[r], e[r], n0[j][r]);
            }
        }
        if (kt == ct) {   // the query tile is complete
#pragma unroll
            for (int j = 0; j < DPW; ++j) finish_tile(h, ct, j);
            reset();
        }
        if (!more) break;
        stg.store(tid, lds + (st ^ 1u) * SB, nk == nc);
        if (nh != h) key_norms(nh);
        if (nc != ct || nh != h) query_tile(nh, nc);
        __syncthreads();
        h = nh;
        ct = nc;
        kt = nk;
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

hipError_t launch_attn_row_weights(const uint16_t *P, const uint16_t *v, const uint16_t *g,
                                   float *W, float *Z, int64_t B, int64_t H, int64_t S,
                                   int64_t dh, hipStream_t s) {
    const uint32_t ntiles = (uint32_t)(B * H * (S / 32));   // one wave per query tile
    const uint32_t blocks = (ntiles + 3u) / 4u;
#define DUST_ARW(KS)                                                                           \
    attn_row_weights_kernel<KS><<<blocks, 256, 0, s>>>(P, v, g, W, Z, (uint32_t)H, (uint32_t)S, \
                                                       ntiles)
    switch (dh / 16) {
        case 1: DUST_ARW(1); break;
        case 2: DUST_ARW(2); break;
        case 3: DUST_ARW(3); break;
        case 4: DUST_ARW(4); break;
        case 5: DUST_ARW(5); break;
        case 6: DUST_ARW(6); break;
        case 7: DUST_ARW(7); break;
        default: DUST_ARW(8); break;
    }
#undef DUST_ARW
    return hipGetLastError();
}

namespace {

// e^x - 1 coefficients for logit shifts sigma tau <., .> of noise divided by kNormalScale
// Repair pass of the key and query scores. The fast pass's form is exact only while the shifts
// keep the row's perturbed mass sum_s P_ts e^delta_ts near Z_t: far below it, Z + N0 comes from
// cancellation; far above it, the noise's 16 significant bits show in e^delta, and shifts
// beyond about 88 overflow it. The fast pass leaves such queries
// NaN (as any non-finite input would), and here one block per (draw, sequence) finds them
// (nothing else is touched) and recomputes their scores from the definition with the row
// maximum subtracted, head by head:
//     <Delta o_t, g_t> = sum_s W_ts e^{delta_ts - m} / (Z_t sum_s P_ts e^{delta_ts - m}),
// m the running maximum of delta_ts over the keys with P_ts > 0 (the sum of W_ts over a row is
// zero, which makes this equal to the fast pass's form), rescaling both sums when m grows. A
// thread owns one query of a group of 256 and holds its query-side vector (q_t for keys, the
// noise a_t for queries) in registers; the block stages the key-side vectors of one 32-key tile
// (the noise a_s for keys, k_s for queries) in LDS. The noise is taken in fp32 (the fast pass
// rounds it to 16 significant bits). KEYS: the noise is on the keys.
template <int KS, bool KEYS>
__global__ __launch_bounds__(256) void attn_softmax_repair_kernel(
    const uint16_t *__restrict__ P, const uint16_t *__restrict__ xm, const float *__restrict__ Wm,
    const float *__restrict__ Zm, float *__restrict__ c, uint32_t Kc, uint32_t B, uint32_t H,
    uint32_t S, uint32_t q0, float s1, Key key, uint32_t draw0, uint32_t tok0) {
    constexpr uint32_t DH = 16u * KS;
    __shared__ float tile[32][DH + 1];
    __shared__ uint8_t bad[4096];
    __shared__ float total[4096];
    const uint32_t tid = threadIdx.x;
    const uint32_t T = B * S, d = H * DH;
    const uint64_t pairs = (uint64_t)Kc * B;
    for (uint64_t pr = blockIdx.x; pr < pairs; pr += gridDim.x) {
        const uint32_t i = (uint32_t)(pr % Kc), b = (uint32_t)(pr / Kc);
        float *cr = c + (uint64_t)i * T + (uint64_t)b * S;
        int found = 0;
        for (uint32_t t = tid; t < S; t += 256u) {
            const bool nf = !__builtin_isfinite(cr[t]);
            bad[t] = nf ? 1 : 0;
            total[t] = 0.f;
            found |= nf ? 1 : 0;
        }
        if (!__syncthreads_or(found)) continue;   // uniform: the pair is fine
        const uint32_t draw = draw0 + i;
        for (uint32_t h = 0; h < H; ++h) {
            const uint32_t qh = q0 + h * (DH / 4u);
            for (uint32_t g0 = 0; g0 < S; g0 += 256u) {
                const uint32_t t = g0 + tid;
                const bool mine = t < S && bad[t];
                if (!__syncthreads_or(mine ? 1 : 0)) continue;
                float qv[DH];
                if (mine) {
                    if constexpr (KEYS) {
                        const uint16_t *row = xm + ((uint64_t)b * S + t) * d + h * DH;
#pragma unroll
                        for (uint32_t j = 0; j < DH; ++j) qv[j] = bf16_to_f32(row[j]);
                    } else {
#pragma unroll
                        for (uint32_t j = 0; j < DH; j += 4u) {
                            Polar pp[2];
                            noise4_polar<false>(key, qh + j / 4u, tok0 + b * S + t, draw, pp);
                            qv[j] = pp[0].rho * pp[0].c;
                            qv[j + 1] = pp[0].rho * pp[0].s;
                            qv[j + 2] = pp[1].rho * pp[1].c;
                            qv[j + 3] = pp[1].rho * pp[1].s;
                        }
                    }
                }
                float m = -__builtin_huge_valf(), num = 0.f, den = 0.f;
                const uint32_t tlast = min(S, g0 + 256u) - 1u;
                const uint64_t rbase = (((uint64_t)b * H + h) * S + t) * S;
                for (uint32_t k0 = 0; k0 <= tlast; k0 += 32u) {
                    __syncthreads();   // the previous tile is no longer read
                    for (uint32_t e = tid; e < 32u * (DH / 4u); e += 256u) {
                        const uint32_t r = e / (DH / 4u), j = 4u * (e % (DH / 4u));
                        const uint32_t sk = k0 + r;
                        if constexpr (KEYS) {
                            Polar pp[2];
                            noise4_polar<false>(key, qh + j / 4u, tok0 + b * S + sk, draw, pp);
                            tile[r][j] = pp[0].rho * pp[0].c;
                            tile[r][j + 1] = pp[0].rho * pp[0].s;
                            tile[r][j + 2] = pp[1].rho * pp[1].c;
                            tile[r][j + 3] = pp[1].rho * pp[1].s;
                        } else {
                            const uint16_t *row = xm + ((uint64_t)b * S + sk) * d + h * DH + j;
#pragma unroll
                            for (uint32_t u = 0; u < 4u; ++u) tile[r][j + u] = bf16_to_f32(row[u]);
                        }
                    }
                    __syncthreads();
                    if (!mine || k0 > t) continue;
                    const uint32_t rend = min(32u, t - k0 + 1u);
                    for (uint32_t r = 0; r < rend; ++r) {
                        const uint32_t sk = k0 + r;
                        const float pw = bf16_to_f32(P[rbase + sk]);
                        if (!(pw > 0.f)) continue;   // adds nothing to either sum
                        float dot = 0.f;
#pragma unroll
                        for (uint32_t j = 0; j < DH; ++j) dot = __builtin_fmaf(qv[j], tile[r][j], dot);
                        const float delta = s1 * dot;
                        if (delta > m) {
                            const float sc = __expf(m - delta);
                            num *= sc;
                            den *= sc;
                            m = delta;
                        }
                        const float e = __expf(delta - m);
                        num = __builtin_fmaf(Wm[rbase + sk], e, num);
                        den = __builtin_fmaf(pw, e, den);
                    }
                }
                if (mine) {
                    const float Z = Zm[((uint64_t)b * H + h) * S + t];
                    total[t] -= (Z > 0.f && den > 0.f) ? num / (Z * den) : 0.f;
                }
            }
        }
        __syncthreads();
        for (uint32_t t = tid; t < S; t += 256u)
            if (bad[t]) cr[t] = total[t];
        __syncthreads();   // bad and total are reused by the next pair
    }
}

Expm1Coef expm1_coef(float sigma, float softmax_scale) {
    const double s1 = (double)sigma * (double)softmax_scale * kNormalScale;
    Expm1Coef ec;
    ec.s1 = (float)s1;
    ec.a2 = (float)(s1 * s1 * kExpm1Q0);
    ec.a3 = (float)(s1 * s1 * s1 * kExpm1Q1);
    ec.a4 = (float)(s1 * s1 * s1 * s1 * kExpm1Q2);
    ec.lim = s1 == 0.0 ? __builtin_huge_valf() : (float)((double)kPolyRange / fabs(s1));
    return ec;
}

// Layout of a key or query scores launch: nw waves per block, dpw draws per wave. One draw per
// wave keeps three waves on each SIMD (12 per block) where the registers allow it (key heads up
// to 80 wide, query heads up to 64), else 8 waves; the key kernel keeps two running sums per draw
// and query position in LDS, so its longer sequences take fewer draws per block: 4 waves up to
// S = 2048, 2 up to 4096. For query heads up to 64 wide 8 waves of two draws each are the
// alternative: each step's operands, read from LDS once, serve two draws, but with
// two waves per SIMD a draw costs about 5 % more (measured with all 16384 draws of the attention
// workload in one launch). A launch takes the layout whose grid, in whole rounds of one block
// per CU (the LDS or registers admit one), ends sooner: 512 draws over 16 sequences fill 256 CUs
// in 2 rounds of 16 draws per block, against 2.7 of 12.
struct ScoreLayout {
    uint32_t nw, dpw;
};

// Compute units of the current device, asked once per device (a lost race stores the same
// value twice); 256 if the runtime cannot tell.
uint32_t device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<uint32_t> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256u;
    if (dev >= 0 && dev < kMaxDevices) {
        const uint32_t c = cached[dev].load(std::memory_order_relaxed);
        if (c != 0u) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store((uint32_t)n, std::memory_order_relaxed);
    return (uint32_t)n;
}

// Rounds x draws per block, in twentieths of one-draw-per-wave time.
uint64_t layout_cost(int64_t B, int64_t Kc, uint32_t draws_per_block, uint32_t cus,
                     uint32_t per_draw) {
    const uint64_t blocks = (uint64_t)B * (uint64_t)((Kc + draws_per_block - 1) / draws_per_block);
    return (blocks + cus - 1) / cus * draws_per_block * per_draw;
}

ScoreLayout choose_layout(ScoreLayout one, bool two_ok, int64_t B, int64_t Kc) {
    if (!two_ok) return one;
    const uint32_t cus = device_cus();
    const ScoreLayout two = {8u, 2u};
    return layout_cost(B, Kc, two.nw * two.dpw, cus, 21u) <
                   layout_cost(B, Kc, one.nw * one.dpw, cus, 20u)
               ? two
               : one;
}

ScoreLayout key_layout(int64_t S, int64_t dh) {
    if (S > 2048) return {2u, 1u};
    if (S > 1024) return {4u, 1u};
    return {dh <= 80 ? 12u : 8u, 1u};
}

ScoreLayout query_layout(int64_t B, int64_t Kc, int64_t dh) {
    return choose_layout({dh <= 64 ? 12u : 8u, 1u}, dh <= 64, B, Kc);
}

}  // namespace

// The repair pass after a key or query scores launch (see attn_softmax_repair_kernel): one block
// per (draw, sequence), at most 4096 blocks walking the pairs.
template <bool KEYS>
static hipError_t launch_softmax_repair(const uint16_t *P, const uint16_t *x, const float *W,
                                 const float *Z, float *c, int64_t Kc, int64_t B, int64_t H,
                                 int64_t S, int64_t dh, uint32_t q0, float s1, Key key,
                                 uint32_t draw0, uint32_t tok0, hipStream_t s) {
    const uint64_t pairs = (uint64_t)Kc * (uint64_t)B;
    const uint32_t blocks = (uint32_t)(pairs < 4096u ? pairs : 4096u);
#define DUST_REP(KS)                                                                           \
    attn_softmax_repair_kernel<KS, KEYS><<<blocks, 256, 0, s>>>(                               \
        P, x, W, Z, c, (uint32_t)Kc, (uint32_t)B, (uint32_t)H, (uint32_t)S, q0, s1, key, draw0, \
        tok0)
    switch (dh / 16) {
        case 1: DUST_REP(1); break;
        case 2: DUST_REP(2); break;
        case 3: DUST_REP(3); break;
        case 4: DUST_REP(4); break;
        case 5: DUST_REP(5); break;
        case 6: DUST_REP(6); break;
        case 7: DUST_REP(7); break;
        default: DUST_REP(8); break;
    }
#undef DUST_REP
    return hipGetLastError();
}

hipError_t launch_attn_key_scores(const uint16_t *P, const uint16_t *q, const float *W,
                                  const float *Z, float *c, int64_t Kc, int64_t B, int64_t H,
                                  int64_t S, int64_t dh, int64_t chan0, float sigma,
                                  float softmax_scale, Key key, uint32_t draw0, uint32_t tok0,
                                  hipStream_t s) {
    const ScoreLayout ly = key_layout(S, dh);
    const uint32_t ndg = (uint32_t)((Kc + ly.nw - 1) / ly.nw);
    const uint32_t blocks = (uint32_t)(B * ndg);
    const Expm1Coef ec = expm1_coef(sigma, softmax_scale);
    const uint32_t q0 = (uint32_t)(chan0 / 4);
    // two stages, then (waves x 2 running sums + the query norms) x S
    const size_t lds = 2 * (size_t)stage_bytes((int)(dh / 16), 1, true) +
                       (size_t)(2 * ly.nw + 1) * S * sizeof(float);
#define DUST_AKS(KS, NW)                                                                       \
    attn_key_scores_kernel<KS, NW><<<blocks, NW * 64, lds, s>>>(                               \
        P, q, W, Z, c, (uint32_t)Kc, (uint32_t)(B * S), (uint32_t)H, (uint32_t)S, q0, ec, key,  \
        draw0, tok0, ndg)
#define DUST_AKS_NW(KS, NW0)                                                                   \
    do {                                                                                       \
        if (ly.nw == 2u) DUST_AKS(KS, 2);                                                      \
        else if (ly.nw == 4u) DUST_AKS(KS, 4);                                                 \
        else DUST_AKS(KS, NW0);                                                                \
    } while (0)
    switch (dh / 16) {
        case 1: DUST_AKS_NW(1, 12); break;
        case 2: DUST_AKS_NW(2, 12); break;
        case 3: DUST_AKS_NW(3, 12); break;
        case 4: DUST_AKS_NW(4, 12); break;
        case 5: DUST_AKS_NW(5, 12); break;
        case 6: DUST_AKS_NW(6, 8); break;
        case 7: DUST_AKS_NW(7, 8); break;
        default: DUST_AKS_NW(8, 8); break;
    }
#undef DUST_AKS_NW
#undef DUST_AKS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_softmax_repair<true>(P, q, W, Z, c, Kc, B, H, S, dh, q0, ec.s1, key, draw0,
                                       tok0, s);
}

hipError_t launch_attn_query_scores(const uint16_t *P, const uint16_t *k, const float *W,
                                    const float *Z, float *c, int64_t Kc, int64_t B, int64_t H,
                                    int64_t S, int64_t dh, int64_t chan0, float sigma,
                                    float softmax_scale, Key key, uint32_t draw0, uint32_t tok0,
                                    hipStream_t s) {
    const ScoreLayout ly = query_layout(B, Kc, dh);
    const uint32_t ndg = (uint32_t)((Kc + ly.nw * ly.dpw - 1) / (ly.nw * ly.dpw));
    const uint32_t blocks = (uint32_t)(B * ndg);
    const Expm1Coef ec = expm1_coef(sigma, softmax_scale);
    const uint32_t q0 = (uint32_t)(chan0 / 4);
    // two stages and the key norms [2][S]
    const size_t lds = 2 * (size_t)stage_bytes((int)(dh / 16), 1, true) + 2 * (size_t)S * 4;
#define DUST_AQS(KS, NW, DPW)                                                                  \
    attn_query_scores_kernel<KS, NW, DPW><<<blocks, NW * 64, lds, s>>>(                        \
        P, k, W, Z, c, (uint32_t)Kc, (uint32_t)(B * S), (uint32_t)H, (uint32_t)S, q0, ec, key,  \
        draw0, tok0, ndg)
#define DUST_AQS2(KS)                                                                          \
    do {                                                                                       \
        if (ly.dpw == 2u) DUST_AQS(KS, 8, 2);                                                  \
        else DUST_AQS(KS, 12, 1);                                                              \
    } while (0)
    switch (dh / 16) {
        case 1: DUST_AQS2(1); break;
        case 2: DUST_AQS2(2); break;
        case 3: DUST_AQS2(3); break;
        case 4: DUST_AQS2(4); break;
        case 5: DUST_AQS(5, 8, 1); break;
        case 6: DUST_AQS(6, 8, 1); break;
        case 7: DUST_AQS(7, 8, 1); break;
        default: DUST_AQS(8, 8, 1); break;
    }
#undef DUST_AQS2
#undef DUST_AQS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_softmax_repair<false>(P, k, W, Z, c, Kc, B, H, S, dh, q0, ec.s1, key, draw0,
                                        tok0, s);
}

}  // namespace dust
