// Weight-gradient contraction of the Dust estimator (gfx950):
//     G[o][i] = sum_t g_hat^T[o][t] * x[t][i]
// (explainer cnblogs.com/32bin/p/23212811, "Credit assignment: one forward, two rewards": the
// estimate forms the same outer product over tokens as backpropagation, only the output error
// differs). This is the one dense contraction on the path, so it runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Operands: A = g_hat^T [M = d_out][K = T] is K-contiguous (the error-estimate kernel writes it
// that way). B = x [K][N = d_in] is N-contiguous, the wrong way round for an MFMA B operand,
// which wants 8 consecutive k per lane.
//
// Two tilings. Outputs of at least 2^19 elements with T a multiple of 32 take the large-tile
// kernel: 256 x 256 output tile per 256-thread block (one block per CU), 2 x 2 waves of 128 x 128,
// both operands moved by direct-to-LDS loads through four stages of 32 tokens, A fragments read
// with ds_read_b128 and B fragments with the transposing ds_read_b64_tr_b16, so x needs no
// register transpose. Other shapes take the small-tile kernel: 128 x 128 output tile, 2 x 2 waves
// of 64 x 64, k-step 64 staged through two LDS buffers, global loads two k-steps ahead, x
// transposed 4 x 8 in registers. Both split the token axis across blocks so that the 256 CUs fill;
// the split partial sums go to a workspace and are added in split order by a second kernel, so
// results are deterministic.
#include <mutex>

#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_PITCH = BK + 8;   // bf16 elements per LDS row (144 B: 16-byte aligned rows)

struct SplitPlan {
    uint32_t mtiles, ntiles, splits, kchunk;
};

SplitPlan plan_split(int64_t T, int64_t M, int64_t N) {
    SplitPlan p;
    p.mtiles = (uint32_t)((M + BM - 1) / BM);
    p.ntiles = (uint32_t)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)p.mtiles * p.ntiles;
    int64_t splits = (512 + tiles - 1) / tiles;             // aim for >= 512 blocks
    const int64_t max_by_k = (T + 511) / 512;                 // keep >= 512 tokens per split
    if (splits > max_by_k) splits = max_by_k;
    if (splits < 1) splits = 1;
    int64_t kchunk = (T + splits - 1) / splits;
    kchunk = (kchunk + BK - 1) / BK * BK;
    splits = (T + kchunk - 1) / kchunk;
    if (splits < 1) splits = 1;
    p.splits = (uint32_t)splits;
    p.kchunk = (uint32_t)kchunk;
    return p;
}

// Block -> (split, m-tile, n-tile) in the logical order (split, m, n), n fastest, dealt out to
// the XCDs in contiguous eighths (xcd_logical_block): the n-tiles that share an A row-block run
// side by side on one XCD, and with 8 splits each XCD owns exactly one split, whose slice of x
// all of its blocks read.
__global__ __launch_bounds__(256, 2) void wgrad_mfma_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B,
                                                         float *__restrict__ out, uint32_t M,
                                                         uint32_t N, uint32_t K, SplitPlan p,
                                                         uint64_t split_stride) {
    // two LDS stages: the next k-step is written while the current one feeds the MFMAs
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_PITCH];

    const uint32_t ntile_all = p.mtiles * p.ntiles;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const uint32_t split = lb / ntile_all;
    const uint32_t tile = lb % ntile_all;
    const uint32_t m0 = (tile / p.ntiles) * BM;
    const uint32_t n0 = (tile % p.ntiles) * BN;
    const uint32_t kbeg = split * p.kchunk;
    const uint32_t kend = min(K, kbeg + p.kchunk);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t wm = wave >> 1, wn = wave & 1u;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // A: 128 rows x 8 pieces of 16 B; thread takes pieces tid, tid+256, tid+512, tid+768.
    // B: 16 x 16 blocks of 4 k-rows x 8 n-columns; thread takes block (kb, nb).
    const uint32_t kb = tid & 15u, nb = tid >> 4;
    // native clang vectors: a select on HIP's struct vector types goes through scratch
    typedef u32x4 piece4[4];
    u32x4 ra0[4], rb0[4], ra1[4], rb1[4];
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // Out-of-range pieces read a clamped in-range address and are zeroed by a value select (a
    // select between a global pointer and a private zero would put the zero in scratch).
    // K, kend and N are multiples of 8, so a piece is either wholly inside or wholly outside.
    auto gload = [&](uint32_t k0, piece4 &ra, piece4 &rb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t piece = tid + 256u * j;
            const uint32_t row = piece >> 3, kc = piece & 7u;
            const uint32_t gm = m0 + row, gk = k0 + 8u * kc;
            const bool in = gm < M && gk < kend;
            const u32x4 v = *(const u32x4 *)(A + (uint64_t)min(gm, M - 1u) * K + min(gk, kend - 8u));
            ra[j] = in ? v : zero4;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t gk = k0 + 4u * kb + r, gn = n0 + 8u * nb;
            const bool in = gk < kend && gn < N;
            const u32x4 v = *(const u32x4 *)(B + (uint64_t)min(gk, kend - 1u) * N + min(gn, N - 8u));
            rb[r] = in ? v : zero4;
        }
    };
    auto lstore = [&](int st, const piece4 &ra, const piece4 &rb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t piece = tid + 256u * j;
            const uint32_t row = piece >> 3, kc = piece & 7u;
            *(u32x4 *)(As[st] + row * LDS_PITCH + 8u * kc) = ra[j];
        }
        // rb[r] holds x[k = 4kb + r][n = 8nb .. 8nb+7]; dword h packs columns 2h (low half)
        // and 2h+1 (high half). Column n gets its four k values as two dwords.
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint2 lo, hi;
            lo.x = (rb[0][h] & 0xFFFFu) | (rb[1][h] << 16);
            lo.y = (rb[2][h] & 0xFFFFu) | (rb[3][h] << 16);
            hi.x = (rb[0][h] >> 16) | (rb[1][h] & 0xFFFF0000u);
            hi.y = (rb[2][h] >> 16) | (rb[3][h] & 0xFFFF0000u);
            *(uint2 *)(Bs[st] + (8u * nb + 2u * h) * LDS_PITCH + 4u * kb) = lo;
            *(uint2 *)(Bs[st] + (8u * nb + 2u * h + 1u) * LDS_PITCH + 4u * kb) = hi;
        }
    };
    auto mfma_step = [&](int st) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const uint32_t koff = kk * 16u + 8u * (lane >> 5);
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *(const bf16x8 *)(As[st] + (wm * 64u + i * 32u + (lane & 31u)) * LDS_PITCH + koff);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *(const bf16x8 *)(Bs[st] + (wn * 64u + j * 32u + (lane & 31u)) * LDS_PITCH + koff);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // Global loads run two k-steps ahead of the MFMAs: step s is loaded into register set s % 2
    // during step s - 2, written to LDS stage s % 2 at the end of step s - 1, and multiplied in
    // step s. The loop body covers two steps so that the register sets stay static.
    const uint32_t nsteps = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    if (nsteps > 0) {
        gload(kbeg, ra0, rb0);
        if (nsteps > 1) gload(kbeg + BK, ra1, rb1);
        lstore(0, ra0, rb0);
    }
    __syncthreads();
    for (uint32_t s = 0; s < nsteps; s += 2) {
        // step s: stage 0, registers of step s + 1 in set 1
        if (s + 2 < nsteps) gload(kbeg + (s + 2) * BK, ra0, rb0);
        mfma_step(0);
        if (s + 1 < nsteps) lstore(1, ra1, rb1);
        __syncthreads();
        // step s + 1: stage 1, registers of step s + 2 in set 0
        if (s + 1 < nsteps) {
            if (s + 3 < nsteps) gload(kbeg + (s + 3) * BK, ra1, rb1);
            mfma_step(1);
            if (s + 2 < nsteps) lstore(0, ra0, rb0);
        }
        __syncthreads();
    }

    // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32.
    float *o = out + (uint64_t)split * split_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t col = n0 + wn * 64u + j * 32u + (lane & 31u);
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t row = m0 + wm * 64u + i * 32u + 8u * (r >> 2) + 4u * (lane >> 5) + (r & 3);
                if (row < M) o[(uint64_t)row * N + col] = acc[i][j][r];
            }
        }
}

// ------------------------------------------------------------------------------------------
// Large-tile kernel.
namespace big {

constexpr uint32_t BM = 256, BN = 256, BK = 32, NST = 4;
constexpr uint32_t STAGE = 256u * BK * 2u;   // bytes per operand stage (16 KB)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
#define DUST_LDS __attribute__((address_space(3)))

struct Plan {
    uint32_t mtiles, ntiles, splits, kchunk;
};

// Aim for one block per CU (256 blocks), each split at least 256 tokens long.
Plan plan_split(int64_t T, int64_t M, int64_t N) {
    Plan p;
    p.mtiles = (uint32_t)((M + BM - 1) / BM);
    p.ntiles = (uint32_t)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)p.mtiles * p.ntiles;
    int64_t splits = (256 + tiles - 1) / tiles;
    const int64_t max_by_k = (T + 255) / 256;
    if (splits > max_by_k) splits = max_by_k;
    if (splits < 1) splits = 1;
    int64_t kchunk = (T + splits - 1) / splits;
    kchunk = (kchunk + BK - 1) / BK * BK;
    splits = (T + kchunk - 1) / kchunk;
    p.splits = (uint32_t)splits;
    p.kchunk = (uint32_t)kchunk;
    return p;
}

// LDS layouts, chosen so that the fragment reads hit all 64 banks (measured free of bank
// conflicts on gfx950). A stage: row m holds 32 k = four 16-byte chunks; rows 4L..4L+3 share a
// 256-byte line and chunk c of row r sits in slot 4 (r & 3) + (c ^ ((r >> 2) & 3)), so that 16
// lanes reading one chunk of 16 consecutive rows hit 16 different slots.
__device__ __forceinline__ uint32_t a_byte(uint32_t r, uint32_t c) {
    return (r >> 2) * 256u + (4u * (r & 3u) + (c ^ ((r >> 2) & 3u))) * 16u;
}
// B stage: row k holds 256 n (sixteen 32-byte pieces); piece p of row k sits at
// (p & ~7) | ((p & 7) ^ 2 (k & 3)), so that the 32 lanes of one transposing read (four rows x two
// adjacent pieces) hit eight different pieces of a 256-byte line.
__device__ __forceinline__ uint32_t b_byte(uint32_t k, uint32_t n) {
    const uint32_t p = n >> 4;
    const uint32_t ps = (p & ~7u) | ((p & 7u) ^ ((k & 3u) << 1));
    return k * 512u + ps * 32u + (n & 15u) * 2u;
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(DUST_LDS const void *)p;
}

// One direct-to-LDS load: lane l's 16 bytes at sbase + voff land at LDS byte m0 + 16 l. Written
// as inline asm so that the compiler, which would otherwise wait for every pending direct load
// before each LDS read, leaves the waiting to the kernel (explicit vmcnt before each barrier).
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Requires T % 32 == 0 (every split is a whole number of 32-token steps), N % 8 == 0, 16-byte
// aligned operands, 256 * T * 2 < 2^32 and 32 * N * 2 < 2^32 (32-bit lane offsets).
__global__ __launch_bounds__(256, 1) void wgrad_mfma256_kernel(const uint16_t *__restrict__ A,
                                                               const uint16_t *__restrict__ B,
                                                               float *__restrict__ out, uint32_t M,
                                                               uint32_t N, uint32_t K, Plan p,
                                                               uint64_t split_stride) {
    __shared__ __attribute__((aligned(1024))) uint8_t As[NST][STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t Bs[NST][STAGE];

    // logical block order (split, m-tile, n-tile), dealt to the XCDs in contiguous eighths:
    // the blocks of one split share an XCD and its L2
    const uint32_t tiles = p.mtiles * p.ntiles;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const uint32_t split = lb / tiles, tile = lb % tiles;
    const uint32_t m0 = (tile / p.ntiles) * BM;
    const uint32_t n0 = (tile % p.ntiles) * BN;
    const uint32_t kbeg = split * p.kchunk;
    const uint32_t kend = min(K, kbeg + p.kchunk);
    const uint32_t nsteps = (kend - kbeg) / BK;   // >= 1
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = wave_in_block();
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    const uint32_t g16 = lane >> 4, i16 = lane & 15u;

    // Each wave moves 4 KB of each operand's 16 KB stage per step as four 1 KB direct loads.
    // Per-lane byte offsets are fixed for the block; rows past M and columns past N read clamped
    // in-range data that only feeds output elements that are never stored.
    uint32_t offa[4], offb[4];
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
        const uint32_t inst = 4u * j + wave;
        // A: 16-byte unit P of the stage -> (row, chunk), inverting a_byte
        const uint32_t P = inst * 64u + lane;
        const uint32_t L = P >> 4, sl = P & 15u;
        const uint32_t r = 4u * L + (sl >> 2), ch = (sl & 3u) ^ (L & 3u);
        offa[j] = (min(m0 + r, M - 1u) - m0) * K * 2u + ch * 16u;
        // B: the instruction covers rows 2 inst, 2 inst + 1; lane -> row, stored 16-byte chunk,
        // logical column (the piece swizzle is its own inverse)
        const uint32_t k = 2u * inst + (lane >> 5);
        const uint32_t cs = lane & 31u;
        const uint32_t ps = cs >> 1;
        const uint32_t pl = (ps & ~7u) | ((ps & 7u) ^ ((k & 3u) << 1));
        const uint32_t n = pl * 16u + (cs & 1u) * 8u;
        offb[j] = k * N * 2u + (min(n0 + n, N - 8u) - n0) * 2u;
    }
    const uint16_t *abase = A + (uint64_t)m0 * K + kbeg;
    const uint16_t *bbase = B + (uint64_t)kbeg * N + n0;

    // Loads of step s go to stage s % 4. Steps past the split's end reload its last step into a
    // stage that is never read, so that every step issues the same number of loads.
    auto dma_one = [&](uint32_t s, uint32_t q) {   // q = 0..7: A (even) or B (odd), part q / 2
        const uint32_t sc = min(s, nsteps - 1u);
        const uint32_t j = q >> 1, inst = 4u * j + wave;
        if (q & 1u)
            dma16(bbase + (uint64_t)sc * BK * N, offb[j], lds_addr(Bs[s % NST] + inst * 1024u));
        else
            dma16(abase + sc * BK, offa[j], lds_addr(As[s % NST] + inst * 1024u));
    };
    // MFMA 32x32x16 operands: lane l holds row (A) or column (B) l % 32, k = 8 (l / 32) .. + 7.
    auto read_a = [&](const uint8_t *as, uint32_t kk, uint32_t i) {
        const uint32_t ch = 2u * kk + (lane >> 5);
        return *(const bf16x8 *)(as + a_byte(128u * wm + 32u * i + (lane & 31u), ch));
    };
    // ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 r + c names 4 columns of row r; lane
    // i receives column i of the 4 rows. Two reads give a lane its 8 consecutive k.
    auto read_b = [&](const uint8_t *bs, uint32_t kk, uint32_t j) {
        const uint32_t kb = 16u * kk + 8u * (g16 >> 1) + (i16 >> 2);
        const uint32_t n = 128u * wn + 32u * j + 16u * (g16 & 1u) + 4u * (i16 & 3u);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (DUST_LDS i16x4 *)(DUST_LDS void *)(bs + b_byte(kb, n)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (DUST_LDS i16x4 *)(DUST_LDS void *)(bs + b_byte(kb + 4u, n)));
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, both);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (uint32_t q = 0; q < 8; ++q) dma_one(0, q);
    for (uint32_t q = 0; q < 8; ++q) dma_one(1, q);
    for (uint32_t q = 0; q < 8; ++q) dma_one(2, q);
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");   // stage 0 complete
    bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) a0[i] = read_a(As[0], 0, i);
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) b0[j] = read_b(Bs[0], 0, j);
    // No scalar load may be pending in the loop: with one in flight the compiler could wait for
    // LDS results only with lgkmcnt(0).
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)

    // Software pipeline, scheduled by hand (sched_barrier pins the order): each half step issues
    // its 16 multiplies one by one and slips the other work between them, so that the wave never
    // stalls on a full load queue while the matrix core idles. First half of step st: multiplies
    // of k slice 0 (read during the previous half), reads of slice 1, direct loads of step st + 3
    // into the stage read last in step st - 1. Barrier: stage st + 1 complete in every wave.
    // Second half: multiplies of slice 1, reads of slice 0 of step st + 1.
#define DUST_MMA(Q, A_, B_)                                                                     \
    acc[(Q) >> 2][(Q) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_[(Q) >> 2], B_[(Q) & 3],  \
                                                                     acc[(Q) >> 2][(Q) & 3], 0, 0, 0)
#define DUST_SB __builtin_amdgcn_sched_barrier(0)
    for (uint32_t st = 0; st < nsteps; ++st) {
        const uint8_t *as = As[st % NST], *bs = Bs[st % NST];
        DUST_MMA(0, a0, b0); a1[0] = read_a(as, 1, 0); a1[1] = read_a(as, 1, 1); DUST_SB;
        DUST_MMA(1, a0, b0); a1[2] = read_a(as, 1, 2); a1[3] = read_a(as, 1, 3); DUST_SB;
        DUST_MMA(2, a0, b0); b1[0] = read_b(bs, 1, 0); DUST_SB;
        DUST_MMA(3, a0, b0); b1[1] = read_b(bs, 1, 1); DUST_SB;
        DUST_MMA(4, a0, b0); b1[2] = read_b(bs, 1, 2); DUST_SB;
        DUST_MMA(5, a0, b0); b1[3] = read_b(bs, 1, 3); DUST_SB;
        DUST_MMA(6, a0, b0); dma_one(st + 3u, 0); DUST_SB;
        DUST_MMA(7, a0, b0); dma_one(st + 3u, 1); DUST_SB;
        DUST_MMA(8, a0, b0); dma_one(st + 3u, 2); DUST_SB;
        DUST_MMA(9, a0, b0); dma_one(st + 3u, 3); DUST_SB;
        DUST_MMA(10, a0, b0); dma_one(st + 3u, 4); DUST_SB;
        DUST_MMA(11, a0, b0); dma_one(st + 3u, 5); DUST_SB;
        DUST_MMA(12, a0, b0); dma_one(st + 3u, 6); DUST_SB;
        DUST_MMA(13, a0, b0); dma_one(st + 3u, 7); DUST_SB;
        DUST_MMA(14, a0, b0); DUST_SB;
        DUST_MMA(15, a0, b0); DUST_SB;
        // This wave's loads of step st + 1 are complete once at most those of steps st + 2 and
        // st + 3 (16 instructions; loads complete in issue order) are in flight; its reads of
        // slice 1 are complete, so after the barrier stage st % 4 may be overwritten. After the
        // last step the barrier and the reads below are redundant but harmless; keeping them
        // unconditional keeps the compiler's wait counts exact.
        __builtin_amdgcn_s_waitcnt(0x4070);   // vmcnt(16) lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        const uint8_t *an = As[(st + 1u) % NST], *bn = Bs[(st + 1u) % NST];
        DUST_MMA(0, a1, b1); a0[0] = read_a(an, 0, 0); a0[1] = read_a(an, 0, 1); DUST_SB;
        DUST_MMA(1, a1, b1); a0[2] = read_a(an, 0, 2); a0[3] = read_a(an, 0, 3); DUST_SB;
        DUST_MMA(2, a1, b1); b0[0] = read_b(bn, 0, 0); DUST_SB;
        DUST_MMA(3, a1, b1); b0[1] = read_b(bn, 0, 1); DUST_SB;
        DUST_MMA(4, a1, b1); b0[2] = read_b(bn, 0, 2); DUST_SB;
        DUST_MMA(5, a1, b1); b0[3] = read_b(bn, 0, 3); DUST_SB;
        DUST_MMA(6, a1, b1); DUST_SB;
        DUST_MMA(7, a1, b1); DUST_SB;
        DUST_MMA(8, a1, b1); DUST_SB;
        DUST_MMA(9, a1, b1); DUST_SB;
        DUST_MMA(10, a1, b1); DUST_SB;
        DUST_MMA(11, a1, b1); DUST_SB;
        DUST_MMA(12, a1, b1); DUST_SB;
        DUST_MMA(13, a1, b1); DUST_SB;
        DUST_MMA(14, a1, b1); DUST_SB;
        DUST_MMA(15, a1, b1); DUST_SB;
    }
#undef DUST_MMA
#undef DUST_SB
    // no direct load may still be writing LDS when the block ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    float *o = out + (uint64_t)split * split_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t col = n0 + wn * 128u + j * 32u + (lane & 31u);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t row = m0 + wm * 128u + i * 32u + 8u * (r >> 2) + 4u * (lane >> 5) + (r & 3);
                if (row < M && col < N) o[(uint64_t)row * N + col] = acc[i][j][r];
            }
        }
}
#undef DUST_LDS

bool usable(int64_t T, int64_t M, int64_t N) {
    return T % 32 == 0 && N % 8 == 0 && M * N >= (int64_t)1 << 19 && T < ((int64_t)1 << 23) &&
           N < ((int64_t)1 << 26);
}

}  // namespace big

// Sum of the split partial sums in split order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws,
                                                            float *__restrict__ G, uint64_t n4,
                                                            uint32_t splits) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i >= n4) return;
    float4 s = ((const float4 *)ws)[i];
    for (uint32_t k = 1; k < splits; ++k) {
        const float4 v = ((const float4 *)ws)[(uint64_t)k * n4 + i];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    ((float4 *)G)[i] = s;
}

// Plain path for shapes the tiled kernel does not take (T or d_in not a multiple of 8, or
// unaligned operands): one thread per output element, tokens summed in order in fp32.
__global__ __launch_bounds__(256) void wgrad_plain_kernel(const uint16_t *__restrict__ A,
                                                          const uint16_t *__restrict__ B,
                                                          float *__restrict__ G, uint32_t M,
                                                          uint32_t N, uint32_t K) {
    const uint64_t e = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (e >= (uint64_t)M * N) return;
    const uint32_t o = (uint32_t)(e / N), i = (uint32_t)(e % N);
    float s = 0.f;
    for (uint32_t t = 0; t < K; ++t)
        s = __builtin_fmaf(bf16_to_f32(A[(uint64_t)o * K + t]), bf16_to_f32(B[(uint64_t)t * N + i]), s);
    G[e] = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ G, uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i < n) G[i] = 0.f;
}

bool tiled_ok(int64_t T, int64_t d_in) { return (T % 8 == 0) && (d_in % 8 == 0); }

}  // namespace

size_t weight_grad_workspace_bytes(int64_t T, int64_t d_out, int64_t d_in) {
    if (T <= 0 || d_out <= 0 || d_in <= 0 || !tiled_ok(T, d_in)) return 0;
    if (big::usable(T, d_out, d_in)) {
        const big::Plan q = big::plan_split(T, d_out, d_in);
        return q.splits <= 1 ? 0 : (size_t)q.splits * (size_t)d_out * (size_t)d_in * sizeof(float);
    }
    const SplitPlan p = plan_split(T, d_out, d_in);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)d_out * (size_t)d_in * sizeof(float);
}

// Split partial sums of dust_weight_grad_noalloc, for callers that cannot allocate: one array
// per GPU, loaded with the code object and held until the process ends. Host code never passes
// the array's name to a kernel (on the host it names a stand-in, not device memory): the device
// address of each GPU's copy is looked up once per device and used instead.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t weight_grad_scratch_bytes() { return kScratchBytes; }

hipError_t weight_grad_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_weight_grad(const uint16_t *gt, const uint16_t *x, float *G, int64_t T,
                              int64_t d_out, int64_t d_in, void *workspace, hipStream_t s) {
    const uint64_t n = (uint64_t)d_out * (uint64_t)d_in;
    if (T == 0) {
        fill_zero_kernel<<<(uint32_t)((n + 255) / 256), 256, 0, s>>>(G, n);
        return hipGetLastError();
    }
    if (!tiled_ok(T, d_in) || !aligned16(gt) || !aligned16(x) || !aligned16(G)) {
        wgrad_plain_kernel<<<(uint32_t)((n + 255) / 256), 256, 0, s>>>(gt, x, G, (uint32_t)d_out,
                                                                      (uint32_t)d_in, (uint32_t)T);
        return hipGetLastError();
    }
    uint32_t splits;
    if (big::usable(T, d_out, d_in)) {
        const big::Plan q = big::plan_split(T, d_out, d_in);
        splits = q.splits;
        float *dst = splits > 1 ? (float *)workspace : G;
        big::wgrad_mfma256_kernel<<<q.mtiles * q.ntiles * q.splits, 256, 0, s>>>(
            gt, x, dst, (uint32_t)d_out, (uint32_t)d_in, (uint32_t)T, q, (uint64_t)n);
    } else {
        const SplitPlan p = plan_split(T, d_out, d_in);
        splits = p.splits;
        float *dst = splits > 1 ? (float *)workspace : G;
        wgrad_mfma_kernel<<<p.mtiles * p.ntiles * p.splits, 256, 0, s>>>(
            gt, x, dst, (uint32_t)d_out, (uint32_t)d_in, (uint32_t)T, p, (uint64_t)n);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits <= 1) return e;
    const uint64_t n4 = n / 4;   // d_in % 8 == 0, so n is a multiple of 4
    splitk_reduce_kernel<<<(uint32_t)((n4 + 255) / 256), 256, 0, s>>>((const float *)workspace, G,
                                                                      n4, splits);
    return hipGetLastError();
}

}  // namespace dust
