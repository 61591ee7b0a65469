// Device-side noise generator of the Dust estimator (gfx950).
//
// The explainer (cnblogs.com/32bin/p/23212811, "Credit assignment: one forward, two rewards")
// draws a_t ~ N(0, I) independently per token and per draw. Storing that noise would cost
// K x T x d values; instead every kernel that needs a^{(i)}_{t, ch} regenerates it from a
// counter-based generator:
//   Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) of counter (ch/4, token, draw, tag) under
//   key (seed lo, seed hi) -> four 32-bit words -> two Box-Muller pairs -> channels 4q..4q+3.
// Uniform: u(w) = (floor(w / 2^9) + 1/2) * 2^-23, exact in fp32.
// Box-Muller uses the hardware transcendentals: v_log_f32 (log2), v_sqrt_f32, and
// v_sin_f32 / v_cos_f32, whose argument is in revolutions, so sin(2 pi u) costs one op.
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

// Ten Philox rounds on (c0, c1, c2, c3) under (k0, k1); results in place. The first round keeps
// plain XORs so that wave-uniform counter words (draw, tag, often token) stay on the scalar unit.
__device__ __forceinline__ void philox4x32_10(uint32_t &c0, uint32_t &c1, uint32_t &c2,
                                              uint32_t &c3, uint32_t k0, uint32_t k1) {
    {
        const uint64_t pa = mul_wide(0xD2511F53u, c0);
        const uint64_t pb = mul_wide(0xCD9E8D57u, c2);
        const uint32_t n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
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
        const uint32_t n0 = xor3((uint32_t)(pb >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(pa >> 32), c3, k1);
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
    }
}

// Words of channel group q (channels 4q..4q+3) for (draw, token).
__device__ __forceinline__ uint4 noise_words(const Key &key, uint32_t q, uint32_t token,
                                             uint32_t draw) {
    uint32_t c0 = q, c1 = token, c2 = draw, c3 = key.tag;
    philox4x32_10(c0, c1, c2, c3, key.k0, key.k1);
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ float uniform01(uint32_t w) {
    // (m + 1/2) * 2^-23 with m = w >> 9 < 2^23, exact, in [2^-24, 1 - 2^-24]. One funnel shift
    // builds the fp32 bit pattern of 1 + m 2^-23 (exponent field 0x7F above the 23 mantissa
    // bits), and subtracting 1 - 2^-24 leaves (2m + 1) 2^-24, which fp32 holds exactly.
    const float one_plus = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
    return one_plus - 0x1.fffffep-1f;
}

// One Box-Muller pair: radius from wa, angle (in revolutions) from wb.
__device__ __forceinline__ void box_muller(uint32_t wa, uint32_t wb, float &n_cos, float &n_sin) {
    const float ua = uniform01(wa);
    const float ub = uniform01(wb);
    // -2 ln u = -2 ln(2) log2(u)
    const float rho = __builtin_amdgcn_sqrtf(-1.38629436111989061883f * __builtin_amdgcn_logf(ua));
    n_cos = rho * __builtin_amdgcn_cosf(ub);
    n_sin = rho * __builtin_amdgcn_sinf(ub);
}

// The four standard normals of channels 4q..4q+3 of (draw, token).
__device__ __forceinline__ float4 noise4(const Key &key, uint32_t q, uint32_t token,
                                         uint32_t draw) {
    const uint4 w = noise_words(key, q, token, draw);
    float4 n;
    box_muller(w.x, w.y, n.x, n.y);
    box_muller(w.z, w.w, n.z, n.w);
    return n;
}

}  // namespace dust
