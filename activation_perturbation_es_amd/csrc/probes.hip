// Ceiling probes for the roofline denominators (not part of the estimator; built into
// libdust_probes.so, which only bench.py --ceilings loads).
//
//  - generator peak: the library's device noise generator (Philox4x32-10 + Box-Muller in polar
//    form, noise4_polar) with token and draw uniform across the wave, every normal summed into a
//    register and one store per thread at the end: the rate at which this part can draw normals
//    when nothing else is done with them;
//  - matrix-core peak: back-to-back v_mfma_f32_32x32x16_bf16 on 16 independent accumulators per
//    wave, operands loaded once from memory (random data draws more power than constants);
//    one wave per SIMD;
//  - clock under load: four waves per CU issue back-to-back MFMAs while the other four read LDS
//    (ds_read_b128 or the transposing ds_read_b64_tr_b16) or idle, or all eight read LDS; every
//    wave records its shader-clock cycles (s_memtime) and wall-clock ticks (s_memrealtime) over
//    its loop, so the clock the part holds under each mix, and the LDS bytes per clock, follow.
#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define DUST_LDS __attribute__((address_space(3)))

// Thread: channel group = lane, token = wave index; loops over `draws` draws.
__global__ __launch_bounds__(256) void generator_peak_kernel(float *__restrict__ out,
                                                             uint32_t draws, Key key) {
    const uint32_t token = blockIdx.x * 4u + wave_in_block();
    const uint32_t q = threadIdx.x & 63u;
    float s = 0.f;
    for (uint32_t i = 0; i < draws; ++i) {
        Polar p[2];
        noise4_polar<true>(key, q, token, i, p);
        s += p[0].rho * (p[0].c + p[0].s) + p[1].rho * (p[1].c + p[1].s);
    }
    out[(uint64_t)blockIdx.x * 256u + threadIdx.x] = s;
}

__global__ __launch_bounds__(256, 1) void mfma_peak_kernel(const uint16_t *__restrict__ src,
                                                          float *__restrict__ out,
                                                          uint32_t iters) {
    const uint64_t base = ((uint64_t)blockIdx.x * 256u + threadIdx.x) * 16u;
    const bf16x8 a = *(const bf16x8 *)(src + base), b = *(const bf16x8 *)(src + base + 8u);
    f32x16 acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
    for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[k][r];
    out[(uint64_t)blockIdx.x * 256u + threadIdx.x] = s;
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return x;
}

// MODE 0: waves 0-3 MFMA, waves 4-7 idle; 1: waves 4-7 read 16 KB of LDS per iteration with
// ds_read_b128; 2: the same with ds_read_b64_tr_b16; 3: all 8 waves ds_read_b128, 8 KB per
// iteration; 4: all 8 waves ds_read_b64_tr_b16, 8 KB per iteration; 5: waves 0-3 MFMA, waves
// 4-7 run the noise generator (two Philox calls = 8 normals per lane per iteration); 6: the
// generator waves alone (waves 0-3 idle). MFMA waves issue 16
// v_mfma_f32_32x32x16_bf16 per iteration on 8 accumulators (512 cycles at full rate). LDS
// reads: 16 consecutive bytes (b128) or 8 (tr) per lane, every wave in its own 8 KB window
// shifted by 16 bytes per iteration, so that the reads are free of bank conflicts.
template <int MODE>
__global__ __launch_bounds__(512, 1) void clock_probe_kernel(unsigned long long *__restrict__ out,
                                                             float *__restrict__ sink,
                                                             uint32_t iters) {
    __shared__ __attribute__((aligned(1024))) uint8_t buf[96u * 1024u];   // one block per CU
    const uint32_t lane = threadIdx.x & 63u, wave = wave_in_block();
    for (uint32_t i = threadIdx.x; i < 96u * 256u; i += 512u) ((uint32_t *)buf)[i] = mix32(i);
    __syncthreads();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    if ((MODE <= 2 || MODE == 5) && wave < 4u) {
        u32x4 ua, ub;
        for (uint32_t k = 0; k < 4u; ++k) {   // random finite bf16 pairs
            ua[k] = mix32(blockIdx.x * 4096u + threadIdx.x * 8u + k) & 0xBFFFBFFFu;
            ub[k] = mix32(blockIdx.x * 4096u + threadIdx.x * 8u + 4u + k) & 0xBFFFBFFFu;
        }
        const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
        f32x16 acc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
        for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int rep = 0; rep < 2; ++rep)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[k][r];
    } else if (MODE == 1 || MODE == 3) {
        constexpr uint32_t per = MODE == 1 ? 16u : 8u;
        u32x4 x[per];
#pragma unroll
        for (uint32_t j = 0; j < per; ++j) x[j] = u32x4{0u, 0u, 0u, 0u};
        const uint32_t base = wave * 8192u + lane * 16u;
        for (uint32_t it = 0; it < iters; ++it) {
            const uint32_t sh = (it & 7u) * 16u;
#pragma unroll
            for (uint32_t j = 0; j < per; ++j)
                x[j] ^= *(const DUST_LDS u32x4 *)(DUST_LDS void *)(buf + base + sh + j * 1024u);
        }
        u32x4 y = x[0];
#pragma unroll
        for (uint32_t j = 1; j < per; ++j) y ^= x[j];
        s = (float)(y[0] ^ y[1] ^ y[2] ^ y[3]);
    } else if (MODE == 2 || MODE == 4) {
        constexpr uint32_t per = MODE == 2 ? 32u : 16u;
        i16x4 x[per];
#pragma unroll
        for (uint32_t j = 0; j < per; ++j) x[j] = i16x4{0, 0, 0, 0};
        const uint32_t base = wave * 8192u + lane * 8u;
        for (uint32_t it = 0; it < iters; ++it) {
            const uint32_t sh = (it & 7u) * 16u;
#pragma unroll
            for (uint32_t j = 0; j < per; ++j)
                x[j] ^= __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DUST_LDS i16x4 *)(DUST_LDS void *)(buf + base + sh + j * 512u));
        }
        i16x4 y = x[0];
#pragma unroll
        for (uint32_t j = 1; j < per; ++j) y ^= x[j];
        s = (float)(y[0] ^ y[1] ^ y[2] ^ y[3]);
    } else if ((MODE == 5 || MODE == 6) && wave >= 4u) {
        const Key key{0x0D057005u, 0u, 1u};
        const uint32_t token = blockIdx.x * 4u + (wave - 4u);
        for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
            for (uint32_t h = 0; h < 2u; ++h) {
                Polar p[2];
                noise4_polar<true>(key, lane + 64u * h, token, it, p);
                s += p[0].rho * (p[0].c + p[0].s) + p[1].rho * (p[1].c + p[1].s);
            }
        }
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0u) {
        out[(blockIdx.x * 8u + wave) * 2u] = c1 - c0;
        out[(blockIdx.x * 8u + wave) * 2u + 1u] = r1 - r0;
    }
    sink[(uint64_t)blockIdx.x * 512u + threadIdx.x] = s;
}

}  // namespace
}  // namespace dust

extern "C" {

// normals drawn = blocks * 4 waves * 64 lanes * 4 normals * draws; out holds blocks * 256 floats
int dust_probe_generator(float *out, uint32_t blocks, uint32_t draws, void *stream) {
    dust::Key key{0x0D057005u, 0u, 1u};
    dust::generator_peak_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(out, draws, key);
    return (int)hipGetLastError();
}

// flops = blocks * 4 waves * iters * 16 * 32768; src holds blocks * 256 * 16 bf16, out
// blocks * 256 floats
int dust_probe_mfma(const uint16_t *src, float *out, uint32_t blocks, uint32_t iters,
                    void *stream) {
    dust::mfma_peak_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(src, out, iters);
    return (int)hipGetLastError();
}

// mode as in clock_probe_kernel; out holds blocks * 8 waves * (cycles, wall-clock ticks), sink
// blocks * 512 floats
int dust_probe_clock(int mode, unsigned long long *out, float *sink, uint32_t blocks,
                     uint32_t iters, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    switch (mode) {
    case 0: dust::clock_probe_kernel<0><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    case 1: dust::clock_probe_kernel<1><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    case 2: dust::clock_probe_kernel<2><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    case 3: dust::clock_probe_kernel<3><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    case 4: dust::clock_probe_kernel<4><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    case 5: dust::clock_probe_kernel<5><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    case 6: dust::clock_probe_kernel<6><<<blocks, 512, 0, s>>>(out, sink, iters); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// rate of the wall-clock counter read by s_memrealtime, in kHz (0 on error)
int dust_probe_wallclock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

}  // extern "C"
