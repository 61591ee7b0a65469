// Weight-gradient contraction of the Dust estimator (gfx950):
//     G[o][i] = sum_t g_hat^T[o][t] * x[t][i]
// (explainer cnblogs.com/32bin/p/23212811, "Credit assignment: one forward, two rewards": the
// estimate forms the same outer product over tokens as backpropagation, only the output error
// differs). This is the one dense contraction on the path, so it runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Operands: A = g_hat^T [M = d_out][K = T] is K-contiguous (the error-estimate kernel writes it
// that way). B = x [K][N = d_in] is N-contiguous, the wrong way round for an MFMA B operand,
// which wants 8 consecutive k per lane; each thread therefore loads a 4 (k) x 8 (n) block of x
// and transposes it in registers before writing it to LDS as [n][k].
// Tiling: 128 x 128 output tile per 256-thread block, 2 x 2 waves of 64 x 64, k-step 64 staged
// through two LDS buffers, with global loads issued two k-steps ahead of the MFMAs. The token axis is
// split across blocks so that small outputs still fill the 256 CUs; the split partial sums go to
// a workspace and are added in split order by a second kernel, so results are deterministic.
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
    const SplitPlan p = plan_split(T, d_out, d_in);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)d_out * (size_t)d_in * sizeof(float);
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
    const SplitPlan p = plan_split(T, d_out, d_in);
    const uint32_t blocks = p.mtiles * p.ntiles * p.splits;
    float *dst = p.splits > 1 ? (float *)workspace : G;
    wgrad_mfma_kernel<<<blocks, 256, 0, s>>>(gt, x, dst, (uint32_t)d_out, (uint32_t)d_in,
                                             (uint32_t)T, p, (uint64_t)n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits <= 1) return e;
    const uint64_t n4 = n / 4;   // d_in % 8 == 0, so n is a multiple of 4
    splitk_reduce_kernel<<<(uint32_t)((n4 + 255) / 256), 256, 0, s>>>((const float *)workspace, G,
                                                                      n4, p.splits);
    return hipGetLastError();
}

}  // namespace dust
