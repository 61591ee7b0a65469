// Optimizer steps that apply the weight-gradient estimate (gfx950).
//
// The explainer's section "Results" trains with the Dust estimate through SGD with momentum at a
// constant learning rate, and reruns one comparison with Adam; it prints no formula, so these
// are the textbook steps (heavy-ball momentum without dampening; Adam of Kingma & Ba with the
// decoupled weight decay of Loshchilov & Hutter), state updated in place, fp32 throughout:
//   SGD:  buf <- mu buf + g;  w <- w - lr buf
//   Adam: w <- w (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
//         w <- w - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// Both are pure streams (20 and 28 bytes per weight), so each thread moves one 16-byte piece
// of every array when the arrays allow it; the step's scalars are formed on the host in fp64.
//
// The explainer's hyperparameter screening ranks candidate settings by the cosine between the
// estimate and the backpropagation gradient on one batch; cosine_terms_kernel forms the three
// sums that cosine needs, sum a b, sum a^2, sum b^2, in fp64 and in a fixed order (one block:
// thread t takes the elements t, t + 1024, ... in turn, then a fixed pairwise tree), so the
// result does not depend on scheduling.
#include <cmath>

#include "dust_internal.hpp"

namespace dust {
namespace {

template <bool VEC>
__global__ __launch_bounds__(256) void sgd_momentum_kernel(float *__restrict__ w,
                                                           const float *__restrict__ g,
                                                           float *__restrict__ buf, uint64_t n,
                                                           float lr, float mu) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if constexpr (VEC) {
        if (4 * i >= n) return;
        f32x4 wv = ((f32x4 *)w)[i], bv = ((f32x4 *)buf)[i];
        const f32x4 gv = __builtin_nontemporal_load((const f32x4 *)g + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bv[e] = __builtin_fmaf(mu, bv[e], gv[e]);
            wv[e] = __builtin_fmaf(-lr, bv[e], wv[e]);
        }
        ((f32x4 *)w)[i] = wv;
        ((f32x4 *)buf)[i] = bv;
    } else {
        if (i >= n) return;
        const float b = __builtin_fmaf(mu, buf[i], g[i]);
        buf[i] = b;
        w[i] = __builtin_fmaf(-lr, b, w[i]);
    }
}

struct AdamStep {
    float decay;          // 1 - lr wd
    float b1, omb1;       // b1, 1 - b1
    float b2, omb2;       // b2, 1 - b2
    float step_size;      // lr / (1 - b1^t)
    float inv_sqrt_bc2;   // 1 / sqrt(1 - b2^t)
    float eps;
};

__device__ __forceinline__ void adam_one(float &w, float g, float &m, float &v,
                                         const AdamStep &s) {
    w *= s.decay;
    m = __builtin_fmaf(s.b1, m, s.omb1 * g);
    v = __builtin_fmaf(s.b2, v, s.omb2 * (g * g));
    const float denom = __builtin_fmaf(__builtin_sqrtf(v), s.inv_sqrt_bc2, s.eps);
    w = __builtin_fmaf(-s.step_size, m / denom, w);
}

template <bool VEC>
__global__ __launch_bounds__(256) void adam_kernel(float *__restrict__ w,
                                                   const float *__restrict__ g,
                                                   float *__restrict__ m, float *__restrict__ v,
                                                   uint64_t n, AdamStep s) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if constexpr (VEC) {
        if (4 * i >= n) return;
        f32x4 wv = ((f32x4 *)w)[i], mv = ((f32x4 *)m)[i], vv = ((f32x4 *)v)[i];
        const f32x4 gv = __builtin_nontemporal_load((const f32x4 *)g + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float we = wv[e], me = mv[e], ve = vv[e];
            adam_one(we, gv[e], me, ve, s);
            wv[e] = we;
            mv[e] = me;
            vv[e] = ve;
        }
        ((f32x4 *)w)[i] = wv;
        ((f32x4 *)m)[i] = mv;
        ((f32x4 *)v)[i] = vv;
    } else {
        if (i >= n) return;
        float wi = w[i], mi = m[i], vi = v[i];
        adam_one(wi, g[i], mi, vi, s);
        w[i] = wi;
        m[i] = mi;
        v[i] = vi;
    }
}

__global__ __launch_bounds__(1024) void cosine_terms_kernel(const float *__restrict__ a,
                                                            const float *__restrict__ b,
                                                            uint64_t n, double *__restrict__ out) {
    __shared__ double red[3][1024];
    const uint32_t t = threadIdx.x;
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (uint64_t i = t; i < n; i += 1024u) {
        const double x = a[i], y = b[i];   // fp32 products are exact in fp64
        ab = __builtin_fma(x, y, ab);
        aa = __builtin_fma(x, x, aa);
        bb = __builtin_fma(y, y, bb);
    }
    red[0][t] = ab;
    red[1][t] = aa;
    red[2][t] = bb;
    __syncthreads();
    for (uint32_t h = 512; h > 0; h >>= 1) {
        if (t < h) {
#pragma unroll
            for (int q = 0; q < 3; ++q) red[q][t] += red[q][t + h];
        }
        __syncthreads();
    }
    if (t < 3) out[t] = red[t][0];
}

}  // namespace

hipError_t launch_cosine_terms(const float *a, const float *b, int64_t n, double *out,
                               hipStream_t s) {
    cosine_terms_kernel<<<1, 1024, 0, s>>>(a, b, (uint64_t)n, out);
    return hipGetLastError();
}

hipError_t launch_sgd_momentum(float *w, const float *g, float *buf, int64_t n, float lr,
                               float momentum, hipStream_t s) {
    const bool vec = (n % 4 == 0) && aligned16(w) && aligned16(g) && aligned16(buf);
    const uint64_t threads = vec ? (uint64_t)n / 4 : (uint64_t)n;
    const uint32_t blocks = (uint32_t)((threads + 255) / 256);
    if (vec)
        sgd_momentum_kernel<true><<<blocks, 256, 0, s>>>(w, g, buf, (uint64_t)n, lr, momentum);
    else
        sgd_momentum_kernel<false><<<blocks, 256, 0, s>>>(w, g, buf, (uint64_t)n, lr, momentum);
    return hipGetLastError();
}

hipError_t launch_adam(float *w, const float *g, float *m, float *v, int64_t n, float lr,
                       float beta1, float beta2, float eps, float weight_decay, int64_t step,
                       hipStream_t s) {
    const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
    const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
    AdamStep a;
    a.decay = (float)(1.0 - (double)lr * (double)weight_decay);
    a.b1 = beta1;
    a.omb1 = (float)(1.0 - (double)beta1);
    a.b2 = beta2;
    a.omb2 = (float)(1.0 - (double)beta2);
    a.step_size = (float)((double)lr / bc1);
    a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    a.eps = eps;
    const bool vec = (n % 4 == 0) && aligned16(w) && aligned16(g) && aligned16(m) && aligned16(v);
    const uint64_t threads = vec ? (uint64_t)n / 4 : (uint64_t)n;
    const uint32_t blocks = (uint32_t)((threads + 255) / 256);
    if (vec)
        adam_kernel<true><<<blocks, 256, 0, s>>>(w, g, m, v, (uint64_t)n, a);
    else
        adam_kernel<false><<<blocks, 256, 0, s>>>(w, g, m, v, (uint64_t)n, a);
    return hipGetLastError();
}

}  // namespace dust
