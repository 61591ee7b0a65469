// Perturbed downstream product of the Dust estimator (gfx950):
//     out[k][t][n] = sum_j act(y[t][j] + sigma a^{(draw0+k)}_{tok0+t, chan0+j}) * w[n][j]
// Explainer cnblogs.com/32bin/p/23212811, "The real work: suppressing interference", first
// measure: a perturbed layer's effect is measured by re-running the network from that layer
// onward, and those perturbed forwards are where the method's cost lies. The first operation of
// that re-run is the next linear layer applied to the (activated) perturbed output y + sigma a.
// This kernel performs it on the bf16 matrix cores with the noise regenerated inside the operand
// path, so the perturbed outputs [Kc, T, d] are never written to memory.
//
// Tiling. One 512-thread block (two waves per SIMD) computes a 128-token x 512-output tile of
// one draw; wave w owns tokens 64 (w & 1) .. + 63 and outputs 128 (w >> 1) .. + 127 (2 x 4
// accumulators of 32 x 32, v_mfma_f32_32x32x16_bf16, fp32). The channel axis is walked in steps
// of 32. For every step all 512 threads regenerate the 128 x 32 slice of act(y + sigma a) --
// thread t owns token row t / 4 and 8 channels, two Philox calls -- round it to bf16 and write
// it into one of two LDS buffers, while the matrix
// cores multiply the slice of the previous step. w and y move by direct-to-LDS loads
// (global_load_lds_dwordx4, 1 KB per instruction) into rings of three stages of one step each
// (w: 512 rows x 32 channels = 32 KB; y: 128 rows x 32 channels = 8 KB), issued two steps
// before their use, so that one wait (vmcnt) and one barrier per step publish them. (Loading w
// fragments straight into registers, 32 rows x 32 bytes per instruction, moved four times the
// bytes through the L2; a single stage in flight exposed the load latency every step.)
// A slice is regenerated once per 512 outputs (twice for a 1024-wide next layer), y is read
// once per 512 outputs, w once per 128 tokens.
//
// Two waves per SIMD (256 registers each: 128 accumulators) hide each other's LDS and issue
// latencies; within a wave the generation is cut into 16 units of about 8 vector instructions
// and one unit is placed after each of the step's 16 MFMAs, the order pinned with sched_barrier,
// so that the vector ALU works while the matrix core multiplies.
//
// LDS layouts. An A slice and a w stage: row r (token or output) holds 32 channels = four
// 16-byte chunks; rows 4L..4L+3 share a 256-byte line and chunk c of row r sits in slot
// 4 (r & 3) + (c ^ ((r >> 2) & 3)), so that 16 lanes reading one chunk of 16 consecutive rows
// touch 16 different slots (all 64 banks). A y stage is plain row-major (64 bytes per token).
#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t PBM = 128, PBN = 512, PBK = 32;
constexpr uint32_t WSTAGE = PBN * PBK * 2;       // bytes of a w stage: 512 rows x 32 channels
constexpr uint32_t YSTAGE = PBM * PBK * 2;       // bytes of a y stage: 128 rows x 32 channels

#define DUST_LDS __attribute__((address_space(3)))

__device__ __forceinline__ uint32_t slot_byte(uint32_t r, uint32_t c) {
    return (r >> 2) * 256u + (4u * (r & 3u) + (c ^ ((r >> 2) & 3u))) * 16u;
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(DUST_LDS const void *)p;
}

// One direct-to-LDS load: lane l's 16 bytes at sbase + voff land at LDS byte m0 + 16 l. Inline
// asm, so that the compiler does not wait for it before every LDS read; the kernel waits for it
// (vmcnt) before the barrier that publishes the stage. The kernel issues no other vector-memory
// loads in its main loop, so vmcnt counts these alone.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// act(x) in fp32. ACT: 0 identity, 1 ReLU, 2 squared ReLU, 3 GELU (tanh form,
// 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) = x - x / (1 + e^{2u})).
template <int ACT>
__device__ __forceinline__ float activate(float x) {
    if constexpr (ACT == 1) {
        return fmaxf(x, 0.f);
    } else if constexpr (ACT == 2) {
        const float r = fmaxf(x, 0.f);
        return r * r;
    } else if constexpr (ACT == 3) {
        // 2 u log2(e) = x (c1 + c3 x^2), c1 = 2 sqrt(2/pi) log2(e), c3 = 0.044715 c1
        constexpr float c1 = 2.302208198842566f, c3 = 0.10294324041977871f;
        const float x2 = x * x;
        const float e = __builtin_amdgcn_exp2f(x * __builtin_fmaf(c3, x2, c1));
        return __builtin_fmaf(-x, __builtin_amdgcn_rcpf(1.f + e), x);
    } else {
        return x;
    }
}

// Grid: blocks in the logical order (draw, n-tile, m-tile), dealt to the XCDs in contiguous
// eighths, so the blocks of one draw and one 512-wide slab of w share an L2.
template <int ACT, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void perturbed_linear_kernel(
    const uint16_t *__restrict__ y, const uint16_t *__restrict__ w, void *__restrict__ out,
    uint32_t T, uint32_t d, uint32_t n_out, uint32_t mtiles, uint32_t ntiles, uint32_t q0,
    float coef, Key key, uint32_t draw0, uint32_t tok0) {
    __shared__ __attribute__((aligned(1024))) uint8_t Ws[3][WSTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t Ys[3][YSTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t As[2][PBM * PBK * 2];

    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const uint32_t per_draw = mtiles * ntiles;
    const uint32_t kd = lb / per_draw;
    const uint32_t nt_blk = (lb % per_draw) / mtiles;
    const uint32_t mt_blk = lb % mtiles;
    const uint32_t m0 = mt_blk * PBM;
    const uint32_t n0 = nt_blk * PBN;
    const uint32_t draw = draw0 + kd;
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = wave_in_block();
    const uint32_t nsteps = d / PBK;

    const uint32_t wm = wave & 1u, wn = wave >> 1;

    // generation: thread -> token row gr, channels 8 gq .. 8 gq + 7 of the step (chunk gq)
    const uint32_t gr = tid >> 2, gq = tid & 3u;
    const uint32_t token = tok0 + m0 + gr;
    const uint32_t woff = slot_byte(gr, gq);

    // Direct loads. w stage: instruction i fills LDS bytes 1024 i .. 1024 i + 1023 = stage rows
    // 16 i .. 16 i + 15; lane l takes row 16 i + l / 4 and logical chunk (l & 3) ^ ((l >> 4) & 3),
    // inverting slot_byte. Wave w issues instructions 4 w .. 4 w + 3. n_out % 32 == 0, so a group
    // of 16 rows is wholly inside or wholly past the outputs; one past them reloads the last group
    // (its products are never stored). y stage: instruction i covers tokens 16 i .. 16 i + 15,
    // lane l token 16 i + l / 4, bytes 16 (l & 3) of its 64; wave w issues instruction w;
    // tokens past T reload token T - 1 (never stored).
    const uint32_t w_voff = ((lane >> 2) * d + 8u * ((lane & 3u) ^ ((lane >> 4) & 3u))) * 2u;
    auto dma_w = [&](uint32_t s, uint8_t *stage) {
        const uint32_t sc = min(s, nsteps - 1u);
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
            const uint32_t inst = 4u * wave + q;
            const uint32_t row16 = min(n0 + 16u * inst, n_out - 16u);
            dma16(w + (uint64_t)row16 * d + PBK * sc, w_voff, lds_addr(stage + 1024u * inst));
        }
    };
    auto dma_y = [&](uint32_t s, uint8_t *stage) {
        const uint32_t sc = min(s, nsteps - 1u);
        const uint32_t inst = wave;
        const uint32_t tokr = min(m0 + 16u * inst + (lane >> 2), T - 1u);
        const uint32_t voff = (tokr - m0) * d * 2u + 16u * (lane & 3u);
        dma16(y + (uint64_t)m0 * d + PBK * sc, voff, lds_addr(stage + 1024u * inst));
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Generation of one slice, in 16 units of about 8 vector instructions each, so that one unit
    // can follow each of a step's 16 MFMAs. The thread's two channel groups are run through
    // Philox4x32-10 round by round (units 0-9: one round of both groups), then Box-Muller
    // (10-13: one pair of one group), then perturbation, activation and bf16 rounding (14-15: one
    // group). The words equal those of noise_words() (Philox, SC'11): counter (q, token, draw,
    // tag), key (k0, k1) bumped by the Weyl constants after every round.
    uint32_t c0[2], c1[2], c2[2], c3[2];
    Polar pol[2][2];
    uint32_t packed[4];
    auto gen_init = [&](uint32_t s) {
        const uint32_t qs = q0 + (min(s, nsteps - 1u) * PBK + 8u * gq) / 4u;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            c0[g] = qs + g;
            c1[g] = token;
            c2[g] = draw;
            c3[g] = key.tag;
        }
    };
    auto gen_round = [&](int r, int g) {
        const uint32_t k0 = key.k0 + (uint32_t)r * 0x9E3779B9u;
        const uint32_t k1 = key.k1 + (uint32_t)r * 0xBB67AE85u;
        const uint64_t pa = mul_wide(0xD2511F53u, c0[g]);
        const uint64_t pb = mul_wide(0xCD9E8D57u, c2[g]);
        const uint32_t n0 = xor3((uint32_t)(pb >> 32), c1[g], k0);
        const uint32_t n2 = xor3((uint32_t)(pa >> 32), c3[g], k1);
        c1[g] = (uint32_t)pb;
        c3[g] = (uint32_t)pa;
        c0[g] = n0;
        c2[g] = n2;
    };
    auto gen_polar = [&](int g, int pr) {
        pol[g][pr] = pr == 0 ? box_muller_polar(c0[g], c1[g]) : box_muller_polar(c2[g], c3[g]);
    };
    // yv: the thread's 8 y values of the step (bf16 pairs)
    auto gen_finish = [&](int g, const u32x4 &yv) {
        const uint32_t y01 = yv[2 * g], y23 = yv[2 * g + 1];
        const float k0 = coef * pol[g][0].rho, k1 = coef * pol[g][1].rho;
        const float v0 = __builtin_fmaf(k0, pol[g][0].c, __uint_as_float(y01 << 16));
        const float v1 = __builtin_fmaf(k0, pol[g][0].s, __uint_as_float(y01 & 0xFFFF0000u));
        const float v2 = __builtin_fmaf(k1, pol[g][1].c, __uint_as_float(y23 << 16));
        const float v3 = __builtin_fmaf(k1, pol[g][1].s, __uint_as_float(y23 & 0xFFFF0000u));
        packed[2 * g] = pack_bf16x2(activate<ACT>(v0), activate<ACT>(v1));
        packed[2 * g + 1] = pack_bf16x2(activate<ACT>(v2), activate<ACT>(v3));
    };
    auto gen_unit = [&](int u, const u32x4 &yv) {
        if (u < 10) {
            gen_round(u, 0);
            gen_round(u, 1);
        } else if (u < 14) {
            gen_polar((u - 10) >> 1, (u - 10) & 1);
        } else {
            gen_finish(u - 14, yv);
        }
    };
    auto gen_store = [&](uint8_t *buf) {
        const u32x4 v = {packed[0], packed[1], packed[2], packed[3]};
        *(u32x4 *)(buf + woff) = v;
    };
    // A operand of m-tile i, 16-channel slice kk: lane -> token row 64 wm + 32 i + lane % 32,
    // chunk 2 kk + lane / 32. B operand of n-tile j: lane -> stage row 128 wn + 32 j + lane % 32,
    // the same chunk.
    auto read_a = [&](const uint8_t *buf, uint32_t i, uint32_t kk) {
        return *(const bf16x8 *)(buf + slot_byte(64u * wm + 32u * i + (lane & 31u),
                                                 2u * kk + (lane >> 5)));
    };
    auto read_b = [&](const uint8_t *stage, uint32_t j, uint32_t kk) {
        return *(const bf16x8 *)(stage + slot_byte(128u * wn + 32u * j + (lane & 31u),
                                                   2u * kk + (lane >> 5)));
    };
    // One step: multiply slice s (A buffer cur, w stage ws) while generating slice s + 1 from
    // its y stage ys into buffer nxt; the order below is pinned with sched_barrier.
    auto step = [&](const uint8_t *cur, uint8_t *nxt, const uint8_t *ws, const uint8_t *ys,
                    uint32_t s) {
        bf16x8 a[2][2], b[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < 2; ++i) a[kk][i] = read_a(cur, i, kk);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[kk][j] = read_b(ws, j, kk);
        }
        const u32x4 yv = *(const u32x4 *)(ys + 64u * gr + 16u * gq);
        gen_init(s + 1u);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int kk = u >> 3, i = (u >> 2) & 1, j = u & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk][i], b[kk][j], acc[i][j], 0,
                                                                0, 0);
            __builtin_amdgcn_sched_barrier(0);
            gen_unit(u, yv);
            __builtin_amdgcn_sched_barrier(0);
        }
        gen_store(nxt);
    };

    // Step s reads w stage s % 3 and y stage (s + 1) % 3 and issues the loads of w for step s + 2
    // (into stage (s + 2) % 3, last read in step s - 1) and of y for step s + 3 (into stage s % 3,
    // last read in step s - 1). Before the step's barrier each wave waits until at most the 5
    // loads it issued in this step are outstanding, so w of step s + 1 and y of step s + 2 are in
    // LDS for the next step. Loads past the last step are clamped into stages nothing reads, and
    // the last step generates a clamped slice into a buffer nothing reads.
    dma_w(0, Ws[0]);
    dma_w(1, Ws[1]);
    dma_y(0, Ys[0]);
    dma_y(1, Ys[1]);
    dma_y(2, Ys[2]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
        const u32x4 yv = *(const u32x4 *)(Ys[0] + 64u * gr + 16u * gq);
        gen_init(0);
#pragma unroll
        for (int u = 0; u < 16; ++u) gen_unit(u, yv);
        gen_store(As[0]);
    }
    __syncthreads();
    uint32_t sw = 0, sy = 1;   // s % 3 and (s + 1) % 3
    for (uint32_t s = 0; s < nsteps; ++s) {
        const uint32_t sw2 = sw == 0 ? 2u : sw - 1u;   // (s + 2) % 3
        dma_w(s + 2u, Ws[sw2]);
        dma_y(s + 3u, Ys[sw]);
        step(As[s & 1u], As[(s + 1u) & 1u], Ws[sw], Ys[sy], s);
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        __syncthreads();
        sw = sy;
        sy = sw2;
    }

    // D layout of the 32x32 MFMA: lane l, register r -> row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32. Tiles wholly inside the token range store without per-row tests.
    const uint64_t plane = (uint64_t)kd * T;
    auto store = [&](uint64_t at, float v) {
        if constexpr (OUT_BF16)
            ((uint16_t *)out)[at] = f32_to_bf16(v);
        else
            ((float *)out)[at] = v;
    };
    const uint32_t rbase = m0 + 64u * wm + 4u * (lane >> 5);
    const uint32_t cbase = n0 + 128u * wn + (lane & 31u);
    if (m0 + PBM <= T) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t col = cbase + 32u * j;
            if (col >= n_out) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    store((plane + rbase + 32u * i + 8u * (r >> 2) + (r & 3)) * n_out + col,
                          acc[i][j][r]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t col = cbase + 32u * j;
            if (col >= n_out) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t row = rbase + 32u * i + 8u * (r >> 2) + (r & 3);
                    if (row < T) store((plane + row) * n_out + col, acc[i][j][r]);
                }
        }
    }
}

}  // namespace

hipError_t launch_perturbed_linear(const uint16_t *y, const uint16_t *w, void *out, bool out_bf16,
                                   int act, int64_t T, int64_t d, int64_t n_out, int64_t chan0,
                                   int64_t Kc, float sigma, Key key, uint32_t draw0,
                                   uint32_t tok0, hipStream_t s) {
    const uint32_t mtiles = (uint32_t)((T + PBM - 1) / PBM);
    const uint32_t ntiles = (uint32_t)((n_out + PBN - 1) / PBN);
    const uint32_t blocks = (uint32_t)Kc * mtiles * ntiles;
    // the generator's polar form leaves out kNormalScale: the coefficient carries it
    const float coef = (float)((double)sigma * kNormalScale);
    const uint32_t q0 = (uint32_t)(chan0 / 4);
#define DUST_PL(A, B)                                                                          \
    perturbed_linear_kernel<A, B><<<blocks, 512, 0, s>>>(y, w, out, (uint32_t)T, (uint32_t)d,  \
                                                         (uint32_t)n_out, mtiles, ntiles, q0,  \
                                                         coef, key, draw0, tok0)
#define DUST_PL_ACT(B)                                                                         \
    do {                                                                                       \
        if (act == 1) DUST_PL(1, B);                                                           \
        else if (act == 2) DUST_PL(2, B);                                                      \
        else if (act == 3) DUST_PL(3, B);                                                      \
        else DUST_PL(0, B);                                                                    \
    } while (0)
    if (out_bf16) DUST_PL_ACT(true); else DUST_PL_ACT(false);
#undef DUST_PL_ACT
#undef DUST_PL
#undef DUST_LDS
    return hipGetLastError();
}

}  // namespace dust
