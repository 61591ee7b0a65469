// Device-side noise generator of the Dust estimator (gfx950).
//
// The explainer (cnblogs.com/32bin/p/23212811, "Credit assignment: one forward, two rewards")
// draws a_t ~ N(0, I) independently per token and per draw. Storing that noise would cost
// K x T x d values; instead every kernel that needs a^{(i)}_{t, ch} regenerates it from a
// counter-based generator:
//   Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) of counter (ch/4, token, draw, tag) under
//   key (seed lo, seed hi) -> four 32-bit words -> two Box-Muller pairs -> channels 4q..4q+3:
//   channel 4q+0 = rho(w0) cos(2 pi v(w1)), 4q+1 = rho(w0) sin(2 pi v(w1)), likewise (w2, w3),
//   rho(w) = sqrt(-2 ln u(w)), radius uniform u(w) = (floor(w / 2^9) + 1/2) 2^-23 in (0, 1),
//   angle uniform v(w) = floor(w / 2^9) 2^-23 in [0, 1) (turns). Both are exact in fp32.
// Box-Muller uses the hardware transcendentals: v_log_f32 (log2), v_sqrt_f32, and
// v_sin_f32 / v_cos_f32, whose argument is in turns, so sin(2 pi v) costs one op; the angle
// needs no subtraction (see box_muller_polar). The generator returns each pair in polar form,
// rho = sqrt(-log2 u) and (cos, sin) of the angle, since sqrt(-2 ln u) = kNormalScale
// sqrt(-log2 u) with kNormalScale = sqrt(2 ln 2): every caller folds the constant into a
// coefficient it applies anyway and multiplies rho by it once per pair.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dust {

struct Key {
    uint32_t k0, k1;  // seed lo, seed hi
    uint32_t tag;
};

// 32x32 -> 64-bit product; lowers to one v_mad_u64_u32.
__device__ __forceinline__ uint64_t mul_wide(uint32_t a, uint32_t b) {
    return (uint64_t)a * (uint64_t)b;
}

// Three-input XOR in one VALU op: gfx950's v_bitop3_b32 with the parity truth table 0x96.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Ten Philox rounds on (c0, c1, c2, c3) under (k0, k1); results in place. Round r maps
//   (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0_r, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1_r, lo(M0 c0)).
// UNIFORM: the caller's token and draw are the same across the wave. Then the first rounds see
// scalar operands, and the XORs are grouped so that two scalar operands are combined on the
// scalar unit first (a VALU instruction reads at most one scalar); otherwise, and from round 3 on,
// one three-input XOR does each pair.
template <bool UNIFORM>
__device__ __forceinline__ void philox4x32_10(uint32_t &c0, uint32_t &c1, uint32_t &c2,
                                              uint32_t &c3, uint32_t k0, uint32_t k1) {
    {   // round 0: plain XORs keep wave-uniform words on the scalar unit
        const uint64_t pa = mul_wide(0xD2511F53u, c0);
        const uint64_t pb = mul_wide(0xCD9E8D57u, c2);
        const uint32_t n0 = ((uint32_t)(pb >> 32) ^ k0) ^ c1;
        const uint32_t n2 = (uint32_t)(pa >> 32) ^ (c3 ^ k1);
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
    }
#pragma unroll
    for (int round = 1; round < 10; ++round) {
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
        const uint64_t pa = mul_wide(0xD2511F53u, c0);
        const uint64_t pb = mul_wide(0xCD9E8D57u, c2);
        uint32_t n0, n2;
        if (UNIFORM && round == 1) {
            // c1 = lo(M1 draw) and hi(M0 c0) (c0 from the uniform token and draw) are scalar
            n0 = (uint32_t)(pb >> 32) ^ (c1 ^ k0);
            n2 = c3 ^ ((uint32_t)(pa >> 32) ^ k1);
        } else if (UNIFORM && round == 2) {
            // c3 = lo(M0 c0) of round 1 is scalar
            n0 = xor3((uint32_t)(pb >> 32), c1, k0);
            n2 = (uint32_t)(pa >> 32) ^ (c3 ^ k1);
        } else {
            n0 = xor3((uint32_t)(pb >> 32), c1, k0);
            n2 = xor3((uint32_t)(pa >> 32), c3, k1);
        }
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
    }
}

// Words of channel group q (channels 4q..4q+3) for (draw, token). UNIFORM: see philox4x32_10.
template <bool UNIFORM = false>
__device__ __forceinline__ uint4 noise_words(const Key &key, uint32_t q, uint32_t token,
                                             uint32_t draw) {
    uint32_t c0 = q, c1 = token, c2 = draw, c3 = key.tag;
    philox4x32_10<UNIFORM>(c0, c1, c2, c3, key.k0, key.k1);
    return make_uint4(c0, c1, c2, c3);
}

// sqrt(2 ln 2): a normal is kNormalScale * rho * (cos or sin) of its pair's polar form.
constexpr double kNormalScale = 1.17741002251547469101;

__device__ __forceinline__ float uniform01(uint32_t w) {
    // (m + 1/2) * 2^-23 with m = w >> 9 < 2^23, exact, in [2^-24, 1 - 2^-24]. One funnel shift
    // builds the fp32 bit pattern of 1 + m 2^-23 (exponent field 0x7F above the 23 mantissa
    // bits), and subtracting 1 - 2^-24 leaves (2m + 1) 2^-24, which fp32 holds exactly.
    const float one_plus = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
    return one_plus - 0x1.fffffep-1f;
}

// Polar form of one Box-Muller pair: the pair is kNormalScale * rho * (cos, sin), with
// rho = sqrt(-log2 u(wa)). The angle is passed as 1 + v(wb) (the funnel shift alone);
// v_sin / v_cos take turns and reduce their argument modulo 1 exactly, so the whole turn costs
// nothing. Callers multiply rho by their own coefficient once and apply it to both trig values.
struct Polar {
    float rho, c, s;
};

__device__ __forceinline__ Polar box_muller_polar(uint32_t wa, uint32_t wb) {
    const float ua = uniform01(wa);
    const float turns = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, wb, 9u));
    Polar p;
    p.rho = __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(ua));   // sqrt(-log2 u)
    p.c = __builtin_amdgcn_cosf(turns);
    p.s = __builtin_amdgcn_sinf(turns);
    return p;
}

// Channels 4q..4q+3 of (draw, token) in polar form: pair 0 (channels 4q, 4q+1) and pair 1
// (4q+2, 4q+3); a^{(draw)}_{token, 4q+1} = kNormalScale * p[0].rho * p[0].s, and so on.
// UNIFORM: token and draw are the same across the wave (see philox4x32_10); the result does not
// depend on it.
template <bool UNIFORM = false>
__device__ __forceinline__ void noise4_polar(const Key &key, uint32_t q, uint32_t token,
                                             uint32_t draw, Polar (&p)[2]) {
    const uint4 w = noise_words<UNIFORM>(key, q, token, draw);
    p[0] = box_muller_polar(w.x, w.y);
    p[1] = box_muller_polar(w.z, w.w);
}

}  // namespace dust
