// Ceiling probes for the roofline denominators (not part of the estimator; built into
// libdust_probes.so, which only bench.py --ceilings loads).
//
//  - generator peak: the library's device noise generator (Philox4x32-10 + Box-Muller in polar
//    form, noise4_polar) with token and draw uniform across the wave, every normal summed into a
//    register and one store per thread at the end: the rate at which this part can draw normals
//    when nothing else is done with them;
//  - matrix-core peak: back-to-back v_mfma_f32_32x32x16_bf16 on 16 independent accumulators per
//    wave, operands loaded once from memory (random data draws more power than constants);
//    one wave per SIMD.
#include "dust_internal.hpp"

namespace dust {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

}  // extern "C"
