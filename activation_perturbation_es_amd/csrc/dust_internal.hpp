// Internal launcher interface between the C ABI (dust_api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dust_noise.hpp"

namespace dust {

// Native clang vectors (the nontemporal builtins take these, not HIP's struct vector types).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 storage is raw 16-bit words; conversions are explicit.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    // round to nearest even via the compiler's bf16 conversion (v_cvt_pk_bf16_f32 on gfx950)
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 values -> packed bf16 pair (lo in bits 0..15), nearest-even, one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

hipError_t launch_noise_inject(const void *y, void *y_pert, bool bf16, int64_t T, int64_t d,
                               int64_t ld_y, int64_t chan0, int64_t Kc, float sigma, Key key,
                               uint32_t draw0, uint32_t tok0, hipStream_t s);

hipError_t launch_noise_words(uint32_t *words, int64_t Kc, int64_t T, int64_t G, uint32_t group0,
                              Key key, uint32_t draw0, uint32_t tok0, hipStream_t s);

hipError_t launch_loss_delta_loss(const float *lc, const float *lp, float *c, int64_t Kc,
                                  int64_t T, hipStream_t s);

hipError_t launch_loss_delta_inner(const void *delta_o, const void *g_o, bool bf16, float *c,
                                   int64_t Kc, int64_t T, int64_t d, hipStream_t s);

hipError_t launch_reward_scan(const float *c, float *r, int64_t K, int64_t T, int64_t seg_len,
                              float gamma, hipStream_t s);

// The scan with its scores formed on load as lc[t] - lp[i][t]; lc == nullptr reads c = lp as
// the scores themselves (launch_reward_scan).
hipError_t launch_loss_reward(const float *lc, const float *lp, float *r, int64_t K, int64_t T,
                              int64_t seg_len, float gamma, hipStream_t s);

hipError_t launch_error_estimate(const float *r, float *g, uint16_t *gt, int64_t K,
                                 int64_t K_total, int64_t T, int64_t d, int64_t chan0,
                                 float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                 bool accumulate, hipStream_t s);

// The estimate with the rewards of gamma = 0 formed on load as lc[t] - lp[i][t] (lp in place of
// r); lc == nullptr reads the rewards r themselves (launch_error_estimate).
hipError_t launch_error_estimate_losses(const float *lc, const float *lp, float *g, uint16_t *gt,
                                        int64_t K, int64_t K_total, int64_t T, int64_t d,
                                        int64_t chan0, float sigma, Key key, uint32_t draw0,
                                        uint32_t tok0, bool accumulate, hipStream_t s);

size_t weight_grad_workspace_bytes(int64_t T, int64_t d_out, int64_t d_in);

hipError_t launch_attn_value_scores(const uint16_t *P, const uint16_t *g, float *c, int64_t Kc,
                                    int64_t B, int64_t H, int64_t S, int64_t dh, int64_t chan0,
                                    float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                    hipStream_t s);

hipError_t launch_attn_row_weights(const uint16_t *P, const uint16_t *v, const uint16_t *g,
                                   float *W, float *Z, int64_t B, int64_t H, int64_t S,
                                   int64_t dh, hipStream_t s);

hipError_t launch_attn_key_scores(const uint16_t *P, const uint16_t *q, const float *W,
                                  const float *Z, float *c, int64_t Kc, int64_t B, int64_t H,
                                  int64_t S, int64_t dh, int64_t chan0, float sigma,
                                  float softmax_scale, Key key, uint32_t draw0, uint32_t tok0,
                                  hipStream_t s);

hipError_t launch_attn_query_scores(const uint16_t *P, const uint16_t *k, const float *W,
                                    const float *Z, float *c, int64_t Kc, int64_t B, int64_t H,
                                    int64_t S, int64_t dh, int64_t chan0, float sigma,
                                    float softmax_scale, Key key, uint32_t draw0, uint32_t tok0,
                                    hipStream_t s);

hipError_t launch_cosine_terms(const float *a, const float *b, int64_t n, double *out,
                               hipStream_t s);

hipError_t launch_sgd_momentum(float *w, const float *g, float *buf, int64_t n, float lr,
                               float momentum, hipStream_t s);

hipError_t launch_adam(float *w, const float *g, float *m, float *v, int64_t n, float lr,
                       float beta1, float beta2, float eps, float weight_decay, int64_t step,
                       hipStream_t s);

hipError_t launch_weight_grad(const uint16_t *gt, const uint16_t *x, float *G, int64_t T,
                              int64_t d_out, int64_t d_in, void *workspace, hipStream_t s);

// The per-device scratch array of dust_weight_grad_noalloc: its size, and the calling thread's
// current device's address of it (looked up on the first call per device, then cached).
size_t weight_grad_scratch_bytes();
hipError_t weight_grad_scratch(void **ptr);

hipError_t launch_perturbed_linear(const uint16_t *y, const uint16_t *w, void *out, bool out_bf16,
                                   int act, int64_t T, int64_t d, int64_t n_out, int64_t chan0,
                                   int64_t Kc, float sigma, Key key, uint32_t draw0,
                                   uint32_t tok0, hipStream_t s);

hipError_t launch_head_ce_chunk(const float *logits, const int32_t *targets, float *loss_pert,
                                float *loss_clean, int64_t T, int64_t V, int64_t v0, int64_t C,
                                int64_t Kc, float sigma, Key key, uint32_t draw0, uint32_t tok0,
                                hipStream_t s);

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Butterfly sum / max over the 64 lanes of a wave; every lane receives the result.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}
// Sum over the 16 lanes of each DPP row (lanes 16k .. 16k+15); every lane of the row receives
// the row's sum. No LDS traffic: four DPP steps (swap neighbours, swap pairs, mirror halves,
// mirror the row).
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8), each with its
// own L2. This maps the hardware block index to a logical one so that each XCD receives one
// contiguous eighth of the logical order; neighbouring logical blocks then share an L2.
__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t b, uint32_t nblocks) {
    if (nblocks % 8u != 0u) return b;
    return (b % 8u) * (nblocks / 8u) + b / 8u;
}

// Index of the calling wave inside its block, as a wave-uniform (scalar) value.
__device__ __forceinline__ uint32_t wave_in_block() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace dust
