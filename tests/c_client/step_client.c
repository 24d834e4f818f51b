/*
 * A C99 caller of libzero_shard with no Python or torch in the process: it
 * reads one rank's inputs from a file, runs the check -> decision -> step
 * sequence for several steps on the GPU through the C ABI (buffers from
 * hipMalloc, work on a created stream, the 4-byte flag read back each step),
 * and writes what the device computed to a second file.
 *
 * usage: step_client IN OUT
 * IN (little-endian): u64 psi, u32 n, u32 rank, u32 dtype (0 FP16, 1 BF16),
 *   u32 steps, f32 loss_scale, u32 growth_interval, f32 lr, f32 beta1,
 *   f32 beta2, f32 eps, f32 weight_decay, then steps x count 16-bit
 *   gradients, then count FP32 master weights (count from the layout).
 * OUT: per step i32 found_inf, i32 apply; then f32 loss_scale, u64 step of
 *   the scaler; then count 16-bit working weights and count FP32 master, m, v.
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_shard.h"

#define FAIL(...)                         \
    do {                                  \
        fprintf(stderr, __VA_ARGS__);     \
        fprintf(stderr, "\n");            \
        exit(1);                          \
    } while (0)

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_));            \
    } while (0)

#define ZS_OK(x)                                                                    \
    do {                                                                            \
        int rc_ = (x);                                                              \
        if (rc_ != ZERO_OK) FAIL("%s: %s", #x, zero_strerror(rc_));                 \
    } while (0)

static void read_exact(FILE *f, void *p, size_t bytes) {
    if (bytes && fread(p, 1, bytes, f) != bytes) FAIL("short read of the input file");
}

static void write_exact(FILE *f, const void *p, size_t bytes) {
    if (bytes && fwrite(p, 1, bytes, f) != bytes) FAIL("short write of the output file");
}

static void *host_alloc(size_t bytes) {
    void *p = malloc(bytes ? bytes : 1);
    if (p == NULL) FAIL("out of host memory");
    return p;
}

int main(int argc, char **argv) {
    if (argc != 3) FAIL("usage: step_client IN OUT");
    FILE *in = fopen(argv[1], "rb");
    if (in == NULL) FAIL("cannot open %s", argv[1]);
    uint64_t psi;
    uint32_t n, rank, dtype, steps, growth;
    float S, lr, beta1, beta2, eps, wd;
    read_exact(in, &psi, 8);
    read_exact(in, &n, 4);
    read_exact(in, &rank, 4);
    read_exact(in, &dtype, 4);
    read_exact(in, &steps, 4);
    read_exact(in, &S, 4);
    read_exact(in, &growth, 4);
    read_exact(in, &lr, 4);
    read_exact(in, &beta1, 4);
    read_exact(in, &beta2, 4);
    read_exact(in, &eps, 4);
    read_exact(in, &wd, 4);

    zero_layout lay;
    ZS_OK(zero_shard_layout(psi, n, rank, &lay));
    const uint64_t count = lay.count;
    uint16_t *h_g = host_alloc(steps * count * 2);
    float *h_master = host_alloc(count * 4);
    read_exact(in, h_g, steps * count * 2);
    read_exact(in, h_master, count * 4);
    fclose(in);

    const zero_dtype dt = dtype == 0 ? ZERO_F16 : ZERO_BF16;
    void *d_g16, *d_w16;
    float *d_master, *d_m, *d_v;
    int32_t *d_flag;
    HIP_OK(hipMalloc(&d_g16, count * 2 + 2));
    HIP_OK(hipMalloc(&d_w16, count * 2 + 2));
    HIP_OK(hipMalloc((void **)&d_master, count * 4 + 4));
    HIP_OK(hipMalloc((void **)&d_m, count * 4 + 4));
    HIP_OK(hipMalloc((void **)&d_v, count * 4 + 4));
    HIP_OK(hipMalloc((void **)&d_flag, 4));
    float *zeros = host_alloc(count * 4);
    memset(zeros, 0, count * 4);
    HIP_OK(hipMemcpy(d_master, h_master, count * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_m, zeros, count * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, zeros, count * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w16, zeros, count * 2, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    FILE *out = fopen(argv[2], "wb");
    if (out == NULL) FAIL("cannot open %s", argv[2]);
    zero_scaler sc;
    memset(&sc, 0, sizeof sc);
    sc.loss_scale = S;
    sc.growth_interval = growth;
    for (uint32_t s = 0; s < steps; ++s) {
        HIP_OK(hipMemcpyAsync(d_g16, h_g + (size_t)s * count, count * 2, hipMemcpyHostToDevice,
                              stream));
        const float S_used = sc.loss_scale;
        ZS_OK(zero_overflow_check(d_g16, dt, psi, n, rank, S_used, d_flag, NULL, NULL, stream));
        int32_t found = -1;
        HIP_OK(hipMemcpyAsync(&found, d_flag, 4, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));
        int32_t apply = -1;
        ZS_OK(zero_scaler_update(&sc, found, &apply));
        if (apply)
            ZS_OK(zero_adam_step(d_w16, d_g16, d_master, d_m, d_v, dt, psi, n, rank, lr, beta1,
                                 beta2, eps, wd, sc.step, S_used, d_flag, stream));
        write_exact(out, &found, 4);
        write_exact(out, &apply, 4);
    }
    /* an argument error comes back as a code, with nothing enqueued */
    if (zero_adam_step(d_w16, d_g16, d_master, d_m, d_v, dt, psi, n, rank, lr, beta1, beta2,
                       eps, wd, 0, S, NULL, stream) != ZERO_EINVAL)
        FAIL("step 0 was not rejected");
    HIP_OK(hipStreamSynchronize(stream));
    write_exact(out, &sc.loss_scale, 4);
    write_exact(out, &sc.step, 8);

    uint16_t *h_w = host_alloc(count * 2);
    float *h_m = host_alloc(count * 4), *h_v = host_alloc(count * 4);
    HIP_OK(hipMemcpy(h_w, d_w16, count * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_master, d_master, count * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_m, d_m, count * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_v, d_v, count * 4, hipMemcpyDeviceToHost));
    write_exact(out, h_w, count * 2);
    write_exact(out, h_master, count * 4);
    write_exact(out, h_m, count * 4);
    write_exact(out, h_v, count * 4);
    if (fclose(out) != 0) FAIL("cannot close the output file");

    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(d_g16));
    HIP_OK(hipFree(d_w16));
    HIP_OK(hipFree(d_master));
    HIP_OK(hipFree(d_m));
    HIP_OK(hipFree(d_v));
    HIP_OK(hipFree(d_flag));
    free(h_g);
    free(h_master);
    free(zeros);
    free(h_w);
    free(h_m);
    free(h_v);
    printf("ok %llu elements, %u steps\n", (unsigned long long)count, steps);
    return 0;
}
