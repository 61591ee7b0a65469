// Noise injection and raw-word kernels of the Dust estimator (gfx950).
//
// dust_noise_inject forms the perturbed layer outputs y'^{(i)}_t = y_t + sigma a^{(i)}_t for a
// block of draws (explainer cnblogs.com/32bin/p/23212811, "Credit assignment: one forward, two
// rewards"). One thread owns one group of four channels of one token: it loads those four y
// values once and then, for every draw, regenerates the four normals with one Philox call and
// writes the four perturbed values. A wave therefore writes 64 consecutive groups of one output
// row per draw (fully coalesced), and y is read once per call, not once per draw. The kernel is
// bound by the integer and transcendental ALU work of the generator, not by HBM.
#include "dust_internal.hpp"

namespace dust {
namespace {

// Thread -> (token, group) mapping shared by the noise kernels. When a row has fewer than 256
// groups, one block covers several tokens; otherwise a row spans several blocks.
struct RowMap {
    uint32_t ngroups;   // groups per token row
    uint32_t tpr_log2;  // log2(threads per row) when ngroups < 256, else 8
    uint32_t nblk_g;    // blocks per row when ngroups >= 256
};

__device__ __forceinline__ bool map_thread(const RowMap &m, uint32_t T, uint32_t &t, uint32_t &g) {
    if (m.tpr_log2 == 8) {
        t = blockIdx.x / m.nblk_g;
        g = (blockIdx.x % m.nblk_g) * 256u + threadIdx.x;
    } else {
        t = blockIdx.x * (256u >> m.tpr_log2) + (threadIdx.x >> m.tpr_log2);
        g = threadIdx.x & ((1u << m.tpr_log2) - 1u);
    }
    return t < T && g < m.ngroups;
}

static RowMap make_rowmap(int64_t ngroups, int64_t T, uint32_t &blocks) {
    RowMap m;
    m.ngroups = (uint32_t)ngroups;
    if (ngroups >= 256) {
        m.tpr_log2 = 8;
        m.nblk_g = (uint32_t)((ngroups + 255) / 256);
        blocks = (uint32_t)(m.nblk_g * T);
    } else {
        uint32_t l = 0;
        while ((1u << l) < (uint32_t)ngroups) ++l;
        m.tpr_log2 = l;
        m.nblk_g = 1;
        const uint32_t rows_per_block = 256u >> l;
        blocks = (uint32_t)((T + rows_per_block - 1) / rows_per_block);
    }
    return m;
}

// All draws of one (token, 4-channel group): y is read once, then each draw's four normals come
// from one Philox call and the four perturbed values are written.
template <bool BF16, bool VEC, bool UNIFORM>
__device__ __forceinline__ void inject_one(const void *__restrict__ y_, void *__restrict__ yp_,
                                           uint32_t t, uint32_t T, uint32_t d, uint64_t ld_y,
                                           uint32_t j0, uint32_t q, uint32_t Kc, float sigma,
                                           const Key &key, uint32_t draw0, uint32_t token) {
    float yv[4];
    if constexpr (BF16) {
        const uint16_t *y = (const uint16_t *)y_ + (uint64_t)t * ld_y + j0;
        if constexpr (VEC) {
            const uint2 v = *(const uint2 *)y;
            yv[0] = __uint_as_float(v.x << 16);
            yv[1] = __uint_as_float(v.x & 0xFFFF0000u);
            yv[2] = __uint_as_float(v.y << 16);
            yv[3] = __uint_as_float(v.y & 0xFFFF0000u);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) yv[e] = (j0 + e < d) ? bf16_to_f32(y[e]) : 0.f;
        }
    } else {
        const float *y = (const float *)y_ + (uint64_t)t * ld_y + j0;
        if constexpr (VEC) {
            const float4 v = *(const float4 *)y;
            yv[0] = v.x; yv[1] = v.y; yv[2] = v.z; yv[3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) yv[e] = (j0 + e < d) ? y[e] : 0.f;
        }
    }

    const uint64_t draw_stride = (uint64_t)T * d;
    const uint64_t base = (uint64_t)t * d + j0;
    uint32_t lane_off = j0 * 2u;   // byte offset of this lane's group in a bf16 row
    for (uint32_t k = 0; k < Kc; ++k) {
        Polar p[2];
        noise4_polar<UNIFORM>(key, q, token, draw0 + k, p);
        const float k0 = sigma * p[0].rho, k1 = sigma * p[1].rho;   // sigma carries kNormalScale
        const float o0 = __builtin_fmaf(k0, p[0].c, yv[0]);
        const float o1 = __builtin_fmaf(k0, p[0].s, yv[1]);
        const float o2 = __builtin_fmaf(k1, p[1].c, yv[2]);
        const float o3 = __builtin_fmaf(k1, p[1].s, yv[3]);
        const uint64_t off = (uint64_t)k * draw_stride + base;
        if constexpr (BF16 && VEC && UNIFORM) {
            // the token is wave-uniform, so the row start stays on the scalar unit and each lane
            // adds a 32-bit byte offset (no 64-bit vector address arithmetic per draw)
            char *row = (char *)((uint16_t *)yp_ + (uint64_t)k * draw_stride + (uint64_t)t * d);
            asm volatile("" : "+v"(lane_off));   // keeps the per-draw step off the lane offset
            *(uint2 *)(row + lane_off) =
                make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        } else if constexpr (BF16) {
            uint16_t *out = (uint16_t *)yp_ + off;
            if constexpr (VEC) {
                *(uint2 *)out = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
            } else {
                const float o[4] = {o0, o1, o2, o3};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j0 + e < d) out[e] = f32_to_bf16(o[e]);
            }
        } else {
            float *out = (float *)yp_ + off;
            if constexpr (VEC) {
                *(float4 *)out = make_float4(o0, o1, o2, o3);
            } else {
                const float o[4] = {o0, o1, o2, o3};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j0 + e < d) out[e] = o[e];
            }
        }
    }
}

// One thread per (token slot, 4-channel group). With few draws per call a thread's life would
// be short; a token slot then covers `nseq` adjacent tokens, handled one after the other.
// WIDE (rows of at least 256 groups): a block lies inside one row, so the token is uniform across
// the block and the compiler keeps it, and the Philox words that depend only on the token and
// the draw, on the scalar unit.
template <bool BF16, bool VEC, bool WIDE>
__global__ __launch_bounds__(256) void inject_kernel(const void *__restrict__ y_,
                                                     void *__restrict__ yp_, uint32_t T,
                                                     uint32_t d, uint64_t ld_y, uint32_t q0,
                                                     uint32_t Kc, float sigma, Key key,
                                                     uint32_t draw0, uint32_t tok0, RowMap m,
                                                     uint32_t nseq) {
    uint32_t ts, g;
    if constexpr (WIDE) {
        ts = blockIdx.x / m.nblk_g;
        g = (blockIdx.x % m.nblk_g) * 256u + threadIdx.x;
        if (ts * nseq >= T || g >= m.ngroups) return;
    } else {
        if (!map_thread(m, (T + nseq - 1) / nseq, ts, g)) return;
    }
    const uint32_t t_end = min(T, (ts + 1) * nseq);
#pragma unroll 1
    for (uint32_t t = ts * nseq; t < t_end; ++t)
        inject_one<BF16, VEC, WIDE>(y_, yp_, t, T, d, ld_y, 4u * g, q0 + g, Kc, sigma, key, draw0,
                              tok0 + t);
}

__global__ __launch_bounds__(256) void words_kernel(uint4 *__restrict__ words, uint32_t T,
                                                    uint32_t Kc, uint32_t group0, Key key,
                                                    uint32_t draw0, uint32_t tok0, RowMap m) {
    uint32_t t, g;
    if (!map_thread(m, T, t, g)) return;
    const uint64_t draw_stride = (uint64_t)T * m.ngroups;
    for (uint32_t k = 0; k < Kc; ++k)
        words[(uint64_t)k * draw_stride + (uint64_t)t * m.ngroups + g] =
            noise_words(key, group0 + g, tok0 + t, draw0 + k);
}

}  // namespace

hipError_t launch_noise_inject(const void *y, void *y_pert, bool bf16, int64_t T, int64_t d,
                               int64_t ld_y, int64_t chan0, int64_t Kc, float sigma, Key key,
                               uint32_t draw0, uint32_t tok0, hipStream_t s) {
    const int64_t ngroups = (d + 3) / 4;
    // walk 4 adjacent tokens per thread when a call carries at most 4 draws and there are
    // still >= 64k threads
    const int64_t nseq = (Kc <= 4 && ((T + 3) / 4) * ngroups >= 65536) ? 4 : 1;
    uint32_t blocks = 0;
    const RowMap m = make_rowmap(ngroups, (T + nseq - 1) / nseq, blocks);
    const bool vec = (d % 4 == 0) && (ld_y % 4 == 0) && aligned16(y) && aligned16(y_pert);
    const uint32_t q0 = (uint32_t)(chan0 / 4);
    // the generator's normals come divided by kNormalScale
    const float sig = (float)((double)sigma * kNormalScale);
#define DUST_INJECT(B, V, W)                                                                   \
    inject_kernel<B, V, W><<<blocks, 256, 0, s>>>(y, y_pert, (uint32_t)T, (uint32_t)d,         \
                                                  (uint64_t)ld_y, q0, (uint32_t)Kc, sig, key,   \
                                                  draw0, tok0, m, (uint32_t)nseq)
    const bool wide = m.tpr_log2 == 8;
    if (bf16) {
        if (vec) {
            if (wide) DUST_INJECT(true, true, true); else DUST_INJECT(true, true, false);
        } else {
            DUST_INJECT(true, false, false);
        }
    } else {
        if (vec) {
            if (wide) DUST_INJECT(false, true, true); else DUST_INJECT(false, true, false);
        } else {
            DUST_INJECT(false, false, false);
        }
    }
#undef DUST_INJECT
    return hipGetLastError();
}

hipError_t launch_noise_words(uint32_t *words, int64_t Kc, int64_t T, int64_t G, uint32_t group0,
                              Key key, uint32_t draw0, uint32_t tok0, hipStream_t s) {
    uint32_t blocks = 0;
    const RowMap m = make_rowmap(G, T, blocks);
    words_kernel<<<blocks, 256, 0, s>>>((uint4 *)words, (uint32_t)T, (uint32_t)Kc, group0, key,
                                        draw0, tok0, m);
    return hipGetLastError();
}

}  // namespace dust
