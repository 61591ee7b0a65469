/*
 * One Dust estimate driven through the C ABI alone (include/dust.h): plain C, device memory
 * from hipMalloc, the library's entry points in the order of the explainer's "Credit
 * assignment" (perturb, loss change and reward, output error, weight gradient), no Python.
 * Test infrastructure: tests/test_gpu_c_abi.py writes the inputs, runs this program and
 * compares its output with the same estimate made through the Python binding.
 *
 * usage: estimate DIR T D_IN D_OUT K SEQ SIGMA GAMMA SEED TAG
 *   DIR/y.bin  bf16 [T, D_OUT]   DIR/x.bin  bf16 [T, D_IN]
 *   DIR/lc.bin fp32 [T]          DIR/lp.bin fp32 [K, T]
 * writes DIR/G.bin (fp32 [D_OUT, D_IN]) and DIR/yp0.bin (bf16 [T, D_OUT], draw 0 perturbed).
 * Exit status 0 on success; a failing call prints its status and message and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dust.h"

static void die(const char *what, int rc) {
    fprintf(stderr, "%s failed: %s (%s)\n", what, dust_status_string(rc), dust_last_error());
    exit(1);
}

static void hip_check(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(1); }
    void *p = malloc(bytes);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(1); }
    fclose(f);
    return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(1); }
    fclose(f);
}

static void *upload(const void *h, size_t bytes) {
    void *d = NULL;
    hip_check(hipMalloc(&d, bytes), "hipMalloc");
    if (h) hip_check(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy");
    return d;
}

int main(int argc, char **argv) {
    if (argc != 11) {
        fprintf(stderr, "usage: %s DIR T D_IN D_OUT K SEQ SIGMA GAMMA SEED TAG\n", argv[0]);
        return 2;
    }
    const char *dir = argv[1];
    const int64_t T = atoll(argv[2]), d_in = atoll(argv[3]), d_out = atoll(argv[4]);
    const int64_t K = atoll(argv[5]), seq = atoll(argv[6]);
    const float sigma = (float)atof(argv[7]), gamma = (float)atof(argv[8]);
    const uint64_t seed = strtoull(argv[9], NULL, 0);
    const uint32_t tag = (uint32_t)strtoul(argv[10], NULL, 0);

    void *y = read_file(dir, "y.bin", (size_t)T * d_out * 2);
    void *x = read_file(dir, "x.bin", (size_t)T * d_in * 2);
    void *lc = read_file(dir, "lc.bin", (size_t)T * 4);
    void *lp = read_file(dir, "lp.bin", (size_t)K * T * 4);
    void *y_d = upload(y, (size_t)T * d_out * 2), *x_d = upload(x, (size_t)T * d_in * 2);
    float *lc_d = upload(lc, (size_t)T * 4), *lp_d = upload(lp, (size_t)K * T * 4);
    void *yp_d = upload(NULL, (size_t)K * T * d_out * 2);
    float *r_d = upload(NULL, (size_t)K * T * 4);
    float *gh_d = upload(NULL, (size_t)T * d_out * 4);
    void *ght_d = upload(NULL, (size_t)d_out * T * 2);
    float *G_d = upload(NULL, (size_t)d_out * d_in * 4);
    const size_t ws_bytes = dust_weight_grad_workspace(T, d_out, d_in);
    void *ws_d = ws_bytes ? upload(NULL, ws_bytes) : NULL;

    int rc;
    if ((rc = dust_noise_inject(y_d, yp_d, DUST_BF16, T, d_out, d_out, 0, K, sigma, seed, tag, 0,
                                0, NULL)))
        die("dust_noise_inject", rc);
    /* the model's perturbed forward would turn yp into lp here; the losses are inputs */
    if ((rc = dust_loss_reward(lc_d, lp_d, r_d, K, T, seq, gamma, NULL)))
        die("dust_loss_reward", rc);
    if ((rc = dust_error_estimate(r_d, gh_d, ght_d, K, K, T, d_out, 0, sigma, seed, tag, 0, 0, 0,
                                  NULL)))
        die("dust_error_estimate", rc);
    if ((rc = dust_weight_grad(ght_d, x_d, G_d, T, d_out, d_in, ws_d, ws_bytes, NULL)))
        die("dust_weight_grad", rc);
    hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");

    float *G = malloc((size_t)d_out * d_in * 4);
    void *yp0 = malloc((size_t)T * d_out * 2);
    hip_check(hipMemcpy(G, G_d, (size_t)d_out * d_in * 4, hipMemcpyDeviceToHost), "hipMemcpy");
    hip_check(hipMemcpy(yp0, yp_d, (size_t)T * d_out * 2, hipMemcpyDeviceToHost), "hipMemcpy");
    write_file(dir, "G.bin", G, (size_t)d_out * d_in * 4);
    write_file(dir, "yp0.bin", yp0, (size_t)T * d_out * 2);
    printf("ok\n");
    return 0;
}
