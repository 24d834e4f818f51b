/*
 * Calls every function of the oracle (oracle/oracle.c) on heap buffers of
 * exactly the sizes the calls may touch, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer: a read or write past an end, a leak or
 * undefined arithmetic aborts the run.  Prints "ok" when every call returned.
 * Test infrastructure, like the oracle itself.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's declarations (it has no header). */
typedef struct {
    uint64_t psi, shard, offset, count, pad, padded_total;
    uint32_t n, rank;
    uint64_t bytes_dp, bytes_z1, bytes_z2, bytes_z3;
} oracle_layout_t;
typedef struct {
    float bc1, bc2, omb1, omb2, decay;
} oracle_scalars_t;
int oracle_layout(uint64_t psi, uint32_t n, uint32_t rank, oracle_layout_t *out);
double oracle_decode16(uint16_t h, int dtype);
uint16_t oracle_encode16(double x, int dtype);
void oracle_decode16_array(const uint16_t *in, float *out, uint64_t count, int dtype);
void oracle_encode16_array(const float *in, uint16_t *out, uint64_t count, int dtype);
void oracle_overflow_check(const uint16_t *g16, int dtype, uint64_t count, float loss_scale,
                           int32_t *found_inf, double *sumsq);
void oracle_step_scalars(float lr, float beta1, float beta2, float weight_decay, uint64_t step,
                         oracle_scalars_t *out);
void oracle_adam_step(uint16_t *w16, const uint16_t *g16, float *master, float *m, float *v,
                      int dtype, uint64_t count, float lr, float beta1, float beta2, float eps,
                      float weight_decay, uint64_t step, float loss_scale);
void oracle_grad_accumulate(float *acc, const uint16_t *g16, int dtype, uint64_t count, int first);
void oracle_overflow_check_g32(const float *g32, uint64_t count, float loss_scale,
                               int32_t *found_inf, double *sumsq);
void oracle_adam_step_g32(uint16_t *w16, const float *g32, float *master, float *m, float *v,
                          int dtype, uint64_t count, float lr, float beta1, float beta2, float eps,
                          float weight_decay, uint64_t step, float loss_scale);
void oracle_adam_step_f64(double *master, double *m, double *v, const uint16_t *g16, int dtype,
                          uint64_t count, double lr, double beta1, double beta2, double eps,
                          double weight_decay, uint64_t step, double loss_scale);
void oracle_reduce_shard(void *out, int out_fmt, const void *const *replicas, int in_fmt,
                         uint64_t psi, uint32_t n, uint32_t rank);
void oracle_gather_shards(void *full, const void *const *shards, int elem_bytes, uint64_t psi,
                          uint32_t n);

static uint64_t lcg = 88172645463325252ull;
static uint32_t next32(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 32);
}

/* exactly `bytes` bytes (at least one, so that malloc never returns NULL for 0) */
static void *alloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (p == NULL) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void fill16(uint16_t *a, uint64_t n, int dtype)
{
    /* small finite values of either format, plus an occasional inf/NaN */
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t r = next32();
        uint16_t h = dtype == 0 ? (uint16_t)(0x1000u + (r & 0x1fffu)) : (uint16_t)(0x3000u + (r & 0x7ffu));
        if ((r >> 28) == 0)
            h = dtype == 0 ? 0x7c00u : 0x7fc0u;
        a[i] = (uint16_t)(h | ((r >> 16) & 0x8000u));
    }
}

static void fill32(float *a, uint64_t n, float scale)
{
    for (uint64_t i = 0; i < n; ++i)
        a[i] = scale * ((float)(next32() >> 8) / 16777216.0f - 0.5f);
}

static int check_layouts(void)
{
    int bad = 0;
    oracle_layout_t lay;
    for (uint64_t psi = 1; psi <= 300; ++psi)
        for (uint32_t n = 1; n <= 40; ++n) {
            uint64_t total = 0;
            for (uint32_t r = 0; r < n; ++r) {
                if (oracle_layout(psi, n, r, &lay) != 0)
                    ++bad;
                total += lay.count;
            }
            bad += total != psi;
        }
    bad += oracle_layout(0, 8, 0, &lay) == 0;
    bad += oracle_layout(10, 0, 0, &lay) == 0;
    bad += oracle_layout(10, 8, 8, &lay) == 0;
    bad += oracle_layout(10, 8, 0, NULL) == 0;
    bad += oracle_layout(8810000003ull, 64, 63, &lay) != 0 || lay.count != 137656190ull;
    return bad;
}

static void conversions(void)
{
    uint16_t *h = alloc(65536 * sizeof(uint16_t));
    float *f = alloc(65536 * sizeof(float));
    for (uint32_t i = 0; i < 65536; ++i)
        h[i] = (uint16_t)i;
    for (int dt = 0; dt < 2; ++dt) {
        oracle_decode16_array(h, f, 65536, dt);
        oracle_encode16_array(f, h, 65536, dt);
    }
    const uint64_t n = 1u << 20;
    float *x = alloc(n * sizeof(float));
    uint16_t *y = alloc(n * sizeof(uint16_t));
    for (uint64_t i = 0; i < n; ++i) {
        const uint32_t bits = (uint32_t)(i * 4099u);
        memcpy(&x[i], &bits, 4);
    }
    for (int dt = 0; dt < 2; ++dt)
        oracle_encode16_array(x, y, n, dt);
    (void)oracle_encode16(1e300, 0);
    (void)oracle_encode16(-0.0, 1);
    free(x);
    free(y);
    free(h);
    free(f);
}

static void steps(uint64_t count)
{
    for (int dt = 0; dt < 2; ++dt) {
        uint16_t *g16 = alloc(count * 2), *w16 = alloc(count * 2);
        float *master = alloc(count * 4), *m = alloc(count * 4), *v = alloc(count * 4);
        float *acc = alloc(count * 4);
        double *md = alloc(count * 8), *mm = alloc(count * 8), *vd = alloc(count * 8);
        fill16(g16, count, dt);
        fill32(master, count, 0.04f);
        memset(m, 0, count * 4);
        memset(v, 0, count * 4);
        int32_t flag = -1;
        double s = -1.0;
        oracle_overflow_check(g16, dt, count, 1024.0f, &flag, &s);
        oracle_overflow_check(g16, dt, count, 3.0f, &flag, NULL);
        for (uint64_t t = 1; t <= 3; ++t)
            oracle_adam_step(w16, g16, master, m, v, dt, count, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f,
                             t, 1024.0f);
        oracle_grad_accumulate(acc, g16, dt, count, 1);
        oracle_grad_accumulate(acc, g16, dt, count, 0);
        oracle_overflow_check_g32(acc, count, 2.0f, &flag, &s);
        oracle_overflow_check_g32(acc, count, 2.0f, &flag, NULL);
        oracle_adam_step_g32(w16, acc, master, m, v, dt, count, 1e-3f, 0.0f, 0.0f, 0.0f, 0.0f, 1,
                             2.0f);
        for (uint64_t i = 0; i < count; ++i) {
            md[i] = master[i];
            mm[i] = 0.0;
            vd[i] = 0.0;
        }
        oracle_adam_step_f64(md, mm, vd, g16, dt, count, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1, 65536.0);
        free(g16);
        free(w16);
        free(master);
        free(m);
        free(v);
        free(acc);
        free(md);
        free(mm);
        free(vd);
    }
    oracle_scalars_t k;
    oracle_step_scalars(1e-3f, 0.9f, 0.999f, 0.1f, 1000000, &k);
}

static int exchanges(uint64_t psi, uint32_t n)
{
    static const int bytes_of[3] = {2, 2, 4};
    int bad = 0;
    for (int fin = 0; fin < 3; ++fin)
        for (int fout = 0; fout < 3; ++fout) {
            void **reps = alloc(n * sizeof(void *));
            for (uint32_t k = 0; k < n; ++k) {
                reps[k] = alloc(psi * bytes_of[fin]);
                if (fin == 2)
                    fill32(reps[k], psi, 0.02f);
                else
                    fill16(reps[k], psi, fin);
            }
            for (uint32_t r = 0; r < n; ++r) {
                oracle_layout_t lay;
                bad += oracle_layout(psi, n, r, &lay) != 0;
                void *out = alloc(lay.count * bytes_of[fout]);
                oracle_reduce_shard(out, fout, (const void *const *)reps, fin, psi, n, r);
                free(out);
            }
            for (uint32_t k = 0; k < n; ++k)
                free(reps[k]);
            free(reps);
        }
    for (int eb = 2; eb <= 4; eb += 2) {
        void **shards = alloc(n * sizeof(void *));
        for (uint32_t k = 0; k < n; ++k) {
            oracle_layout_t lay;
            bad += oracle_layout(psi, n, k, &lay) != 0;
            shards[k] = alloc(lay.count * eb);
            memset(shards[k], 0x5a, lay.count * eb);
        }
        void *full = alloc(psi * eb);
        oracle_gather_shards(full, (const void *const *)shards, eb, psi, n);
        for (uint32_t k = 0; k < n; ++k)
            free(shards[k]);
        free(shards);
        free(full);
    }
    return bad;
}

int main(void)
{
    int bad = check_layouts();
    conversions();
    static const uint64_t counts[] = {0, 1, 7, 1000, 4097};
    for (size_t i = 0; i < sizeof counts / sizeof counts[0]; ++i)
        steps(counts[i]);
    bad += exchanges(1001, 4);
    bad += exchanges(5, 8); /* trailing ranks own nothing */
    bad += exchanges(1, 1);
    if (bad != 0) {
        fprintf(stderr, "%d unexpected results\n", bad);
        return 1;
    }
    printf("ok\n");
    return 0;
}
