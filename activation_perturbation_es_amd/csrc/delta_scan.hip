// Loss-change scoring and the discounted reward scan of the Dust estimator (gfx950).
//
// Explainer cnblogs.com/32bin/p/23212811:
//  - "Credit assignment: one forward, two rewards": the per-token change c of the loss under
//    each draw, and the reward r_t = sum_{s >= t} gamma^(s-t) c_s that credits a token's noise
//    with its effect on later tokens;
//  - "The real work: suppressing interference": attention internals are scored through the
//    attention output by the inner product of the output change with that output's error.
// All three kernels stream HBM once; none reuses data beyond a register tile.
#include "dust_internal.hpp"

namespace dust {
namespace {

// ---------------------------------------------------------------- loss mode: c = l_clean - l_pert
// VEC: each thread handles 4 float4 pieces of one draw row, strided by the block width, so four
// loads per thread are in flight at once.
template <bool VEC>
__global__ __launch_bounds__(256) void loss_delta_loss_kernel(const float *__restrict__ lc,
                                                              const float *__restrict__ lp,
                                                              float *__restrict__ c, uint32_t T,
                                                              uint32_t nb_row) {
    const uint32_t i = blockIdx.x / nb_row;
    const uint32_t tb = blockIdx.x % nb_row;
    const uint64_t row = (uint64_t)i * T;
    if constexpr (VEC) {
        f32x4 l[4], k[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t t = (tb * 1024u + u * 256u + threadIdx.x) * 4u;
            if (t < T) {
                l[u] = __builtin_nontemporal_load((const f32x4 *)(lp + row + t));
                k[u] = *(const f32x4 *)(lc + t);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t t = (tb * 1024u + u * 256u + threadIdx.x) * 4u;
            if (t < T) *(f32x4 *)(c + row + t) = k[u] - l[u];
        }
    } else {
        const uint32_t t = tb * 256u + threadIdx.x;
        if (t >= T) return;
        c[row + t] = lc[t] - lp[row + t];
    }
}

// ---------------------------------------------------------------- inner mode: c = -<dO, gO>
// One wave per token s. The wave keeps g_o[s] in registers and streams the rows dO[i][s] of all
// draws: lane l covers 16-byte pieces l, l+64, ... of the row (8 bf16 or 4 fp32 values each, or
// single elements on the unaligned path). Each draw's 64 lane partials are summed with a
// butterfly. UNROLL draws are loaded before any is reduced to keep loads in flight.
template <bool BF16, bool VEC, int MAXM>
__global__ __launch_bounds__(256) void loss_delta_inner_kernel(const void *__restrict__ dO_,
                                                               const void *__restrict__ gO_,
                                                               float *__restrict__ c,
                                                               uint32_t Kc, uint32_t T,
                                                               uint32_t d) {
    constexpr int EPV = VEC ? (BF16 ? 8 : 4) : 1;   // elements per lane piece
    constexpr int UNROLL = 4;
    const uint32_t s = blockIdx.x * 4u + wave_in_block();
    if (s >= T) return;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nchunk = (d + 64u * EPV - 1u) / (64u * EPV);

    float gv[MAXM][EPV];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        const uint32_t e0 = (m * 64u + lane) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) gv[m][e] = 0.f;
        if (m < (int)nchunk && e0 < d) {
            if constexpr (BF16) {
                const uint16_t *g = (const uint16_t *)gO_ + (uint64_t)s * d + e0;
                if constexpr (VEC) {
                    const uint4 v = *(const uint4 *)g;
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        gv[m][2 * h] = __uint_as_float(w[h] << 16);
                        gv[m][2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
                    }
                } else {
                    gv[m][0] = bf16_to_f32(g[0]);
                }
            } else {
                const float *g = (const float *)gO_ + (uint64_t)s * d + e0;
                if constexpr (VEC) {
                    const float4 v = *(const float4 *)g;
                    gv[m][0] = v.x; gv[m][1] = v.y; gv[m][2] = v.z; gv[m][3] = v.w;
                } else {
                    gv[m][0] = g[0];
                }
            }
        }
    }

    const uint64_t draw_stride = (uint64_t)T * d;
    for (uint32_t i0 = 0; i0 < Kc; i0 += UNROLL) {
        float p[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            p[u] = 0.f;
            const uint32_t i = i0 + u;
            if (i >= Kc) continue;
            const uint64_t rowoff = (uint64_t)i * draw_stride + (uint64_t)s * d;
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                const uint32_t e0 = (m * 64u + lane) * EPV;
                if (m >= (int)nchunk || e0 >= d) continue;
                if constexpr (BF16) {
                    const uint16_t *row = (const uint16_t *)dO_ + rowoff + e0;
                    if constexpr (VEC) {
                        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)row);
                        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            p[u] = __builtin_fmaf(__uint_as_float(w[h] << 16), gv[m][2 * h], p[u]);
                            p[u] = __builtin_fmaf(__uint_as_float(w[h] & 0xFFFF0000u),
                                                  gv[m][2 * h + 1], p[u]);
                        }
                    } else {
                        p[u] = __builtin_fmaf(bf16_to_f32(row[0]), gv[m][0], p[u]);
                    }
                } else {
                    const float *row = (const float *)dO_ + rowoff + e0;
                    if constexpr (VEC) {
                        const f32x4 v = __builtin_nontemporal_load((const f32x4 *)row);
                        p[u] = __builtin_fmaf(v.x, gv[m][0], p[u]);
                        p[u] = __builtin_fmaf(v.y, gv[m][1], p[u]);
                        p[u] = __builtin_fmaf(v.z, gv[m][2], p[u]);
                        p[u] = __builtin_fmaf(v.w, gv[m][3], p[u]);
                    } else {
                        p[u] = __builtin_fmaf(row[0], gv[m][0], p[u]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const float tot = wave_sum(p[u]);
            if (lane == 0 && i0 + u < Kc) c[(uint64_t)(i0 + u) * T + s] = -tot;
        }
    }
}

// Tile version for rows of at most 64 pieces (bf16 d <= 512, fp32 d <= 256, 16-byte aligned):
// one wave per 4 consecutive tokens and one slice of the draws. Per draw the wave reads the 4
// rows dO[i][s0 .. s0+3] -- one contiguous span of 4 rows -- DRAWS draws at a time (4 x DRAWS
// loads in flight per lane). The 4 x 2 row partials of a lane are summed across the wave with a
// transposed butterfly: after the 32- and 16-lane exchanges each lane carries one row's partial
// (row = 2 * bit5 + bit4 of the lane), and four in-row DPP steps finish the sums, so 4 rows
// cost 3 LDS-crossbar shuffles and 4 DPP adds instead of 24 shuffles.
__device__ __forceinline__ float sel(bool c, float a, float b) { return c ? a : b; }

template <bool BF16, int DRAWS>
__global__ __launch_bounds__(256) void loss_delta_inner_tile_kernel(const void *__restrict__ dO_,
                                                                    const void *__restrict__ gO_,
                                                                    float *__restrict__ c,
                                                                    uint32_t Kc, uint32_t T,
                                                                    uint32_t d, uint32_t nsplit) {
    constexpr int EPV = BF16 ? 8 : 4;
    const uint32_t w = blockIdx.x * 4u + wave_in_block();
    // draw slice major, token tile minor: the waves resident at one time walk the same draws over
    // adjacent tokens, so the chip reads each draw plane as one long sequential sweep
    const uint32_t ntiles = (T + 3u) / 4u;
    const uint32_t tile = w % ntiles, part = w / ntiles;
    if (part >= nsplit) return;
    const uint32_t s0 = tile * 4u;
    if (s0 >= T) return;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t e0 = lane * EPV;
    const bool lane_in = e0 < d;
    const uint32_t i_beg = (uint32_t)(((uint64_t)Kc * part) / nsplit);
    const uint32_t i_end = (uint32_t)(((uint64_t)Kc * (part + 1)) / nsplit);

    float gv[4][EPV];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t s = s0 + r;
#pragma unroll
        for (int e = 0; e < EPV; ++e) gv[r][e] = 0.f;
        if (lane_in && s < T) {
            if constexpr (BF16) {
                const u32x4 v = *(const u32x4 *)((const uint16_t *)gO_ + (uint64_t)s * d + e0);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    gv[r][2 * h] = __uint_as_float(v[h] << 16);
                    gv[r][2 * h + 1] = __uint_as_float(v[h] & 0xFFFF0000u);
                }
            } else {
                const f32x4 v = *(const f32x4 *)((const float *)gO_ + (uint64_t)s * d + e0);
#pragma unroll
                for (int e = 0; e < 4; ++e) gv[r][e] = v[e];
            }
        }
    }
    const uint64_t draw_stride = (uint64_t)T * d;
    const bool b5 = (lane & 32u) != 0, b4 = (lane & 16u) != 0;
    const uint32_t myrow = (b5 ? 2u : 0u) + (b4 ? 1u : 0u);
    const bool writer = (lane & 15u) == 0 && s0 + myrow < T;

    for (uint32_t i = i_beg; i < i_end; i += DRAWS) {
        float p[DRAWS][4];
#pragma unroll
        for (int u = 0; u < DRAWS; ++u) {
            const bool draw_ok = i + u < i_end;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[u][r] = 0.f;
                const uint32_t s = s0 + r;
                if (!(draw_ok && lane_in && s < T)) continue;
                const uint64_t off = (uint64_t)(i + u) * draw_stride + (uint64_t)s * d + e0;
                if constexpr (BF16) {
                    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)((const uint16_t *)dO_ + off));
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        p[u][r] = __builtin_fmaf(__uint_as_float(v[h] << 16), gv[r][2 * h], p[u][r]);
                        p[u][r] = __builtin_fmaf(__uint_as_float(v[h] & 0xFFFF0000u), gv[r][2 * h + 1], p[u][r]);
                    }
                } else {
                    const f32x4 v = __builtin_nontemporal_load((const f32x4 *)((const float *)dO_ + off));
#pragma unroll
                    for (int e = 0; e < 4; ++e) p[u][r] = __builtin_fmaf(v[e], gv[r][e], p[u][r]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < DRAWS; ++u) {
            // 32-lane exchange: keep rows {0,1} (bit5 = 0) or {2,3} (bit5 = 1), send the others
            const float k0 = sel(b5, p[u][2], p[u][0]), s0v = sel(b5, p[u][0], p[u][2]);
            const float k1 = sel(b5, p[u][3], p[u][1]), s1v = sel(b5, p[u][1], p[u][3]);
            const float q0 = k0 + __shfl_xor(s0v, 32);
            const float q1 = k1 + __shfl_xor(s1v, 32);
            // 16-lane exchange: keep row (bit4) of the pair, send the other
            const float kk = sel(b4, q1, q0), ss = sel(b4, q0, q1);
            const float t = row16_sum(kk + __shfl_xor(ss, 16));
            if (writer && i + u < i_end) c[(uint64_t)(i + u) * T + s0 + myrow] = -t;
        }
    }
}

// Same as above for rows too long to keep g_o in registers: g_o is re-read per draw (L1/L2).
template <bool BF16>
__global__ __launch_bounds__(256) void loss_delta_inner_long_kernel(const void *__restrict__ dO_,
                                                                    const void *__restrict__ gO_,
                                                                    float *__restrict__ c,
                                                                    uint32_t Kc, uint32_t T,
                                                                    uint32_t d) {
    const uint32_t s = blockIdx.x * 4u + wave_in_block();
    if (s >= T) return;
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t draw_stride = (uint64_t)T * d;
    for (uint32_t i = 0; i < Kc; ++i) {
        float p = 0.f;
        const uint64_t rowoff = (uint64_t)i * draw_stride + (uint64_t)s * d;
        for (uint32_t j = lane; j < d; j += 64u) {
            float a, b;
            if constexpr (BF16) {
                a = bf16_to_f32(((const uint16_t *)dO_)[rowoff + j]);
                b = bf16_to_f32(((const uint16_t *)gO_)[(uint64_t)s * d + j]);
            } else {
                a = ((const float *)dO_)[rowoff + j];
                b = ((const float *)gO_)[(uint64_t)s * d + j];
            }
            p = __builtin_fmaf(a, b, p);
        }
        const float tot = wave_sum(p);
        if (lane == 0) c[(uint64_t)i * T + s] = -tot;
    }
}

// ---------------------------------------------------------------- reverse segmented gamma-scan
// One wave per (draw, sequence). The sequence is processed in chunks of 64*VEC elements from its
// end towards its start. Inside a chunk each lane owns VEC consecutive elements and forms their
// local suffix sums; the lanes then combine with a Hillis-Steele scan over the affine carry
// (the block of lane l+off contributes gamma^(VEC*off) times its running sum), and the value at
// the chunk's first element is carried into the next chunk. gamma powers come from repeated
// squaring: gp[b] = gamma^(VEC * 2^b).
// LOSSES: the scores are not read but formed on load from the losses, c = l_clean - l_pert
// (c then points at l_pert [K, T] and lc at l_clean [T]); the same fp32 subtraction as the
// loss-change kernel, so the fused rewards equal the two-kernel ones bit for bit.
template <int VEC, bool LOSSES>
__global__ __launch_bounds__(256) void reward_scan_kernel(const float *c, const float *lc,
                                                          float *r, uint32_t K, uint32_t T,
                                                          uint32_t seg_len, float gamma) {
    const uint32_t nseg = T / seg_len;
    const uint64_t w = (uint64_t)blockIdx.x * 4u + wave_in_block();
    if (w >= (uint64_t)K * nseg) return;
    const uint32_t i = (uint32_t)(w / nseg);
    const uint32_t b = (uint32_t)(w % nseg);
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t seg_base = (uint64_t)i * T + (uint64_t)b * seg_len;
    const float *lseg = lc + (uint64_t)b * seg_len;   // l_clean of this sequence (LOSSES)
    // the VEC scores of sequence positions pos .. pos+VEC-1
    auto load = [&](int64_t pos, float (&v)[VEC]) {
        if constexpr (VEC == 4) {
            const f32x4 x = *(const f32x4 *)(c + seg_base + pos);
            if constexpr (LOSSES) {
                const f32x4 l = *(const f32x4 *)(lseg + pos);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = l[e] - x[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = x[e];
            }
        } else {
            v[0] = LOSSES ? lseg[pos] - c[seg_base + pos] : c[seg_base + pos];
        }
    };

    float gpow[VEC + 1];  // gamma^0 .. gamma^VEC
    gpow[0] = 1.f;
#pragma unroll
    for (int e = 1; e <= VEC; ++e) gpow[e] = gpow[e - 1] * gamma;
    float gp[7];          // gamma^(VEC * 2^b), b = 0..6
    gp[0] = gpow[VEC];
#pragma unroll
    for (int k = 1; k < 7; ++k) gp[k] = gp[k - 1] * gp[k - 1];
    // gamma^(VEC * (63 - lane)): product of gp[b] over the set bits of 63 - lane
    float glane = 1.f;
    {
        const uint32_t j = 63u - lane;
#pragma unroll
        for (int k = 0; k < 6; ++k)
            if (j & (1u << k)) glane *= gp[k];
    }

    constexpr uint32_t CH = 64u * VEC;
    // Sequences of up to PRE chunks are loaded up front (all loads in flight at once); longer
    // ones stream chunk by chunk.
    constexpr uint32_t PRE = 4;
    float pre[PRE][VEC];
    const bool preload = seg_len <= PRE * CH;
    if (preload) {
#pragma unroll
        for (uint32_t ch = 0; ch < PRE; ++ch) {
            const int64_t pos = (int64_t)seg_len - (int64_t)(ch + 1) * CH + (int64_t)lane * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) pre[ch][e] = 0.f;
            if (ch * CH < seg_len && pos >= 0) load(pos, pre[ch]);
        }
    }
    float carry = 0.f;  // r at the first element after the current chunk (0 past the end)
    for (uint32_t done = 0, ch = 0; done < seg_len; done += CH, ++ch) {
        // chunk covers sequence positions [seg_len - done - CH, seg_len - done)
        const int64_t start = (int64_t)seg_len - (int64_t)done - (int64_t)CH;
        const int64_t pos = start + (int64_t)lane * VEC;   // first element of this lane
        float v[VEC];
        const bool in = pos >= 0;    // with VEC > 1, seg_len % VEC == 0, so a lane is all in or out
        if (preload) {
#pragma unroll
            for (uint32_t q = 0; q < PRE; ++q)
                if (q == ch) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[e] = pre[q][e];
                }
        } else if (in) {
            load(pos, v);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = 0.f;
        }
        // local suffix sums inside the lane
#pragma unroll
        for (int e = VEC - 2; e >= 0; --e) v[e] = __builtin_fmaf(gamma, v[e + 1], v[e]);
        // inclusive reverse scan over lanes: R_l = v0_l + gamma^VEC * R_{l+1}
        float R = v[0];
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            const uint32_t off = 1u << k;
            const float up = __shfl_down(R, off);
            if (lane + off < 64u) R = __builtin_fmaf(gp[k], up, R);
        }
        // value just after this lane's block: R_{l+1} + gamma^(VEC*(63-l)) * carry
        float after = __shfl_down(R, 1);
        if (lane == 63u) after = 0.f;
        after = __builtin_fmaf(glane, carry, after);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] = __builtin_fmaf(gpow[VEC - e], after, v[e]);
        if (in) {
            if constexpr (VEC == 4) {
                const f32x4 o = {v[0], v[1], v[2], v[3]};
                *(f32x4 *)(r + seg_base + pos) = o;
            } else {
                r[seg_base + pos] = v[0];
            }
        }
        carry = __shfl(v[0], 0);
    }
}

}  // namespace

hipError_t launch_loss_delta_loss(const float *lc, const float *lp, float *c, int64_t Kc,
                                  int64_t T, hipStream_t s) {
    const bool vec = (T % 4 == 0) && aligned16(lc) && aligned16(lp) && aligned16(c);
    const int64_t per_block = vec ? 4096 : 256;
    const uint32_t nb_row = (uint32_t)((T + per_block - 1) / per_block);
    const uint32_t blocks = (uint32_t)(nb_row * Kc);
    if (vec)
        loss_delta_loss_kernel<true><<<blocks, 256, 0, s>>>(lc, lp, c, (uint32_t)T, nb_row);
    else
        loss_delta_loss_kernel<false><<<blocks, 256, 0, s>>>(lc, lp, c, (uint32_t)T, nb_row);
    return hipGetLastError();
}

hipError_t launch_loss_delta_inner(const void *delta_o, const void *g_o, bool bf16, float *c,
                                   int64_t Kc, int64_t T, int64_t d, hipStream_t s) {
    const int epv = bf16 ? 8 : 4;
    const bool vec = (d % epv == 0) && aligned16(delta_o) && aligned16(g_o);
    if (vec && d <= 64 * epv) {
        // tiles of 4 tokens; split the draws until there are >= 32768 waves (four rounds of
        // 8 waves per SIMD: shorter work units keep the concurrently read rows closer together)
        const int64_t tiles = (T + 3) / 4;
        int64_t nsplit = 1;
        while (tiles * nsplit < 32768 && nsplit * 16 <= Kc) nsplit *= 2;
        const uint32_t blocks = (uint32_t)((tiles * nsplit + 3) / 4);
        if (bf16)
            loss_delta_inner_tile_kernel<true, 2><<<blocks, 256, 0, s>>>(delta_o, g_o, c, (uint32_t)Kc,
                                                                      (uint32_t)T, (uint32_t)d,
                                                                      (uint32_t)nsplit);
        else
            loss_delta_inner_tile_kernel<false, 2><<<blocks, 256, 0, s>>>(delta_o, g_o, c, (uint32_t)Kc,
                                                                       (uint32_t)T, (uint32_t)d,
                                                                       (uint32_t)nsplit);
        return hipGetLastError();
    }
    const uint32_t blocks = (uint32_t)((T + 3) / 4);
    const int64_t piece = vec ? 64 * epv : 64;
    const int64_t nchunk = (d + piece - 1) / piece;
#define DUST_INNER(B, V, M)                                                                    \
    loss_delta_inner_kernel<B, V, M><<<blocks, 256, 0, s>>>(delta_o, g_o, c, (uint32_t)Kc,     \
                                                            (uint32_t)T, (uint32_t)d)
#define DUST_INNER_M(B, V)                                                                     \
    do {                                                                                       \
        if (nchunk <= 1) DUST_INNER(B, V, 1);                                                  \
        else if (nchunk <= 2) DUST_INNER(B, V, 2);                                             \
        else if (nchunk <= 4) DUST_INNER(B, V, 4);                                             \
        else DUST_INNER(B, V, 8);                                                              \
    } while (0)
    if (nchunk > 8) {
        if (bf16)
            loss_delta_inner_long_kernel<true><<<blocks, 256, 0, s>>>(delta_o, g_o, c, (uint32_t)Kc,
                                                                      (uint32_t)T, (uint32_t)d);
        else
            loss_delta_inner_long_kernel<false><<<blocks, 256, 0, s>>>(delta_o, g_o, c, (uint32_t)Kc,
                                                                       (uint32_t)T, (uint32_t)d);
    } else if (bf16) {
        if (vec) DUST_INNER_M(true, true); else DUST_INNER_M(true, false);
    } else {
        if (vec) DUST_INNER_M(false, true); else DUST_INNER_M(false, false);
    }
#undef DUST_INNER_M
#undef DUST_INNER
    return hipGetLastError();
}

hipError_t launch_reward_scan(const float *c, float *r, int64_t K, int64_t T, int64_t seg_len,
                              float gamma, hipStream_t s) {
    return launch_loss_reward(nullptr, c, r, K, T, seg_len, gamma, s);
}

hipError_t launch_loss_reward(const float *lc, const float *c, float *r, int64_t K, int64_t T,
                              int64_t seg_len, float gamma, hipStream_t s) {
    const int64_t waves = K * (T / seg_len);
    const uint32_t blocks = (uint32_t)((waves + 3) / 4);
    const bool vec = (seg_len % 4 == 0) && aligned16(c) && aligned16(r) &&
                     (lc == nullptr || aligned16(lc));
#define DUST_SCAN(V, L)                                                                        \
    reward_scan_kernel<V, L><<<blocks, 256, 0, s>>>(c, lc, r, (uint32_t)K, (uint32_t)T,        \
                                                    (uint32_t)seg_len, gamma)
    if (lc != nullptr) {
        if (vec) DUST_SCAN(4, true); else DUST_SCAN(1, true);
    } else {
        if (vec) DUST_SCAN(4, false); else DUST_SCAN(1, false);
    }
#undef DUST_SCAN
    return hipGetLastError();
}

}  // namespace dust
