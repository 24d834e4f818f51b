/*
 * Plain, slow CPU oracle for the ZeRO-sharded mixed-precision Adam step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, link or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library; every function below is written from the definitions
 * on the pages it cites.
 *
 * Precision: the pages fix it.  The master copy and Adam's two moments are
 * FP32 and the working weights and gradients are 16-bit ("Training models too
 * big for one GPU: ZeRO & FSDP", "Mixed-precision training" and "The memory
 * bill: 16 bytes per parameter").  So the step is evaluated one IEEE binary32
 * operation at a time, each rounded to nearest-even.  Built with
 *   gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 * on x86-64 (SSE scalar arithmetic, FLT_EVAL_METHOD == 0): no contraction, no
 * excess precision, no flush-to-zero.  An FP64 evaluation of the same update
 * is kept beside it, only to bound the FP32 oracle's own rounding error.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* ------------------------------------------------------------------------ */
/* Shard layout.                                                             */
/*                                                                           */
/* Rank i owns chunk i of the flat buffer and all chunks have the same size  */
/* ("Training models too big for one GPU", "Data parallelism and the         */
/* all-reduce"; "ZeRO memory math" tm_zero_math, "Stage 1 - P_os"; "How far   */
/* does splitting the batch get you?", ring all-reduce derivation).  When N  */
/* does not divide PSI the chunk size is ceil(PSI/N) and the padding sits at */
/* the tail, so trailing ranks may own fewer (or zero) real elements.        */
/*                                                                           */
/* Per-rank model-state bytes follow the stage formulas ("ZeRO stages 1, 2   */
/* and 3" on the first page; "The three stages of ZeRO" on "Stop Replicating */
/* What You Can Shard"; "Stage 3: divide everything by N" on "ZeRO Stage 3   */
/* Math"): 2+2+12 bytes per parameter, where the /N terms become S elements  */
/* and the replicated terms are the padded flat buffer of N*S elements.      */
/* ------------------------------------------------------------------------ */

typedef struct {
    uint64_t psi;          /* parameters in the flat buffer */
    uint64_t shard;        /* S = ceil(psi / n) */
    uint64_t offset;       /* first flat index of this rank's chunk: rank * S */
    uint64_t count;        /* real elements in the chunk */
    uint64_t pad;          /* S - count */
    uint64_t padded_total; /* n * S */
    uint32_t n;
    uint32_t rank;
    uint64_t bytes_dp;     /* plain data parallel: 16 * psi */
    uint64_t bytes_z1;     /* optimizer states sharded: (2+2) * nS + 12 * S */
    uint64_t bytes_z2;     /* + gradients sharded:       2 * nS + (2+12) * S */
    uint64_t bytes_z3;     /* + weights sharded:         (2+2+12) * S */
} oracle_layout_t;

#define ORACLE_MAX_PSI (1ull << 56)

int oracle_layout(uint64_t psi, uint32_t n, uint32_t rank, oracle_layout_t *out)
{
    if (out == NULL || psi == 0 || psi > ORACLE_MAX_PSI || n == 0 || rank >= n)
        return -1;
    uint64_t S = psi / n;
    if (S * n < psi)
        S += 1;
    uint64_t first = (uint64_t)rank * S;
    uint64_t count = 0;
    if (first < psi) {
        count = psi - first;
        if (count > S)
            count = S;
    }
    out->psi = psi;
    out->shard = S;
    out->offset = first;
    out->count = count;
    out->pad = S - count;
    out->padded_total = (uint64_t)n * S;
    out->n = n;
    out->rank = rank;
    out->bytes_dp = 16u * psi;
    out->bytes_z1 = 4u * out->padded_total + 12u * S;
    out->bytes_z2 = 2u * out->padded_total + 14u * S;
    out->bytes_z3 = 16u * S;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 16-bit formats ("How a computer stores real numbers", format table):     */
/* value = (-1)^sign * 1.fraction * 2^(exponent - bias) for normal numbers, */
/* (-1)^sign * 0.fraction * 2^(1 - bias) for subnormals, all-ones exponent  */
/* for infinity (fraction 0) and NaN.                                       */
/*   FP16: 1 / 5 / 10 bits, bias 15.   BF16: 1 / 8 / 7 bits, bias 127.      */
/* dtype code: 0 = FP16, 1 = BF16.                                          */
/* ------------------------------------------------------------------------ */

static int fmt_ebits(int dtype) { return dtype == 0 ? 5 : 8; }
static int fmt_fbits(int dtype) { return dtype == 0 ? 10 : 7; }

double oracle_decode16(uint16_t h, int dtype)
{
    const int eb = fmt_ebits(dtype), fb = fmt_fbits(dtype);
    const int bias = (1 << (eb - 1)) - 1;
    const uint32_t emask = (1u << eb) - 1u;
    const uint32_t sign = h >> 15;
    const uint32_t e = (h >> fb) & emask;
    const uint32_t f = h & ((1u << fb) - 1u);
    double mag;
    if (e == emask)
        mag = (f != 0) ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, 1 - bias - fb);
    else
        mag = ldexp((double)((1u << fb) | f), (int)e - bias - fb);
    return sign ? -mag : mag;
}

/* Round a real value to the 16-bit format, to nearest with ties to even.   */
/* NaN becomes the quiet NaN of the same sign.                               */
uint16_t oracle_encode16(double x, int dtype)
{
    const int eb = fmt_ebits(dtype), fb = fmt_fbits(dtype);
    const int bias = (1 << (eb - 1)) - 1;
    const int emin = 1 - bias, emax = bias;
    const uint16_t expfield = (uint16_t)(((1u << eb) - 1u) << fb);
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | expfield | (1u << (fb - 1)));
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | expfield);

    /* Binade of a (a in [2^E, 2^(E+1))), never below the subnormal range. */
    int e2;
    int E = emin;
    if (a != 0.0) {
        frexp(a, &e2); /* a = fr * 2^e2 with fr in [0.5, 1) */
        E = e2 - 1;
        if (E < emin)
            E = emin;
    }
    const double quantum = ldexp(1.0, E - fb);  /* spacing of the format in that binade */
    const double r = nearbyint(a / quantum);    /* exact scaling; round half to even */
    const double y = r * quantum;               /* exact */
    const double maxfinite = ldexp((double)((2u << fb) - 1u), emax - fb);
    if (y > maxfinite)
        return (uint16_t)(sign | expfield);

    uint32_t bits;
    if (y < ldexp(1.0, emin)) {
        bits = (uint32_t)(y / ldexp(1.0, emin - fb)); /* subnormal or zero */
    } else {
        frexp(y, &e2);
        const int Ey = e2 - 1;
        const uint32_t frac = (uint32_t)(y / ldexp(1.0, Ey - fb)) - (1u << fb);
        bits = ((uint32_t)(Ey + bias) << fb) | frac;
    }
    return (uint16_t)(sign | bits);
}

void oracle_decode16_array(const uint16_t *in, float *out, uint64_t count, int dtype)
{
    for (uint64_t i = 0; i < count; ++i)
        out[i] = (float)oracle_decode16(in[i], dtype);
}

void oracle_encode16_array(const float *in, uint16_t *out, uint64_t count, int dtype)
{
    for (uint64_t i = 0; i < count; ++i)
        out[i] = oracle_encode16((double)in[i], dtype);
}

/* ------------------------------------------------------------------------ */
/* Unscale and overflow check.                                               */
/* The loss was multiplied by S, so the gradients are divided by S before    */
/* the update, and the step is skipped when an overflow shows up            */
/* ("Training models too big for one GPU", "Mixed-precision training",       */
/* loss scaling).  found_inf = 1 iff some unscaled gradient is +-inf or NaN. */
/* sumsq is the FP64 sum of the unscaled gradients' squares (an optional    */
/* by-product for a gradient norm).                                          */
/* ------------------------------------------------------------------------ */

void oracle_overflow_check(const uint16_t *g16, int dtype, uint64_t count, float loss_scale,
                           int32_t *found_inf, double *sumsq)
{
    int32_t flag = 0;
    double s = 0.0;
    for (uint64_t i = 0; i < count; ++i) {
        const float g = (float)oracle_decode16(g16[i], dtype) / loss_scale;
        if (!isfinite(g))
            flag = 1;
        s += (double)g * (double)g;
    }
    *found_inf = flag;
    if (sumsq)
        *sumsq = s;
}

/* ------------------------------------------------------------------------ */
/* Host scalars of one step.                                                 */
/* Bias correction 1 - beta^t is formed in FP64 and rounded once to FP32;   */
/* t counts the updates applied so far, this one included ("Adam, and why   */
/* it's expensive", bias-corrected moments).                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    float bc1, bc2;   /* 1 - beta1^t, 1 - beta2^t */
    float omb1, omb2; /* 1 - beta1, 1 - beta2 (FP32 subtractions) */
    float decay;      /* 1 - lr * weight_decay (two FP32 operations) */
} oracle_scalars_t;

void oracle_step_scalars(float lr, float beta1, float beta2, float weight_decay, uint64_t step,
                         oracle_scalars_t *out)
{
    out->bc1 = (float)(1.0 - pow((double)beta1, (double)step));
    out->bc2 = (float)(1.0 - pow((double)beta2, (double)step));
    out->omb1 = 1.0f - beta1;
    out->omb2 = 1.0f - beta2;
    out->decay = 1.0f - lr * weight_decay;
}

/* ------------------------------------------------------------------------ */
/* The Adam step on one shard, elementwise, in the pages' order:            */
/*   g  = g16 / S                              (loss scaling undone)        */
/*   p  = master * (1 - lr * wd)               (decoupled weight decay)     */
/*   m  = beta1 * m + (1 - beta1) * g                                        */
/*   v  = beta2 * v + (1 - beta2) * g^2                                      */
/*   m^ = m / (1 - beta1^t),  v^ = v / (1 - beta2^t)                         */
/*   p  = p - lr * m^ / (sqrt(v^) + eps)       (eps outside the root)       */
/*   master = p;  w16 = p rounded to the 16-bit format                       */
/* ("Adam, and why it's expensive", update equations; "Mixed-precision      */
/* training", FP32 master copy rounded for the next forward pass).  The     */
/* last line's product and quotient are taken left to right.               */
/* ------------------------------------------------------------------------ */

/* One element of the step from its unscaled-gradient input graw. */
static void update_one(float graw, float loss_scale, float lr, float beta1, float beta2, float eps,
                       const oracle_scalars_t *k, float *master, float *m, float *v,
                       uint16_t *w16, int dtype)
{
    const float g = graw / loss_scale;
    const float p = *master * k->decay;
    const float m_new = beta1 * *m + k->omb1 * g;
    const float v_new = beta2 * *v + k->omb2 * (g * g);
    const float m_hat = m_new / k->bc1;
    const float v_hat = v_new / k->bc2;
    const float denom = sqrtf(v_hat) + eps;
    const float p_new = p - lr * m_hat / denom;
    *master = p_new;
    *m = m_new;
    *v = v_new;
    *w16 = oracle_encode16((double)p_new, dtype);
}

void oracle_adam_step(uint16_t *w16, const uint16_t *g16, float *master, float *m, float *v,
                      int dtype, uint64_t count, float lr, float beta1, float beta2, float eps,
                      float weight_decay, uint64_t step, float loss_scale)
{
    oracle_scalars_t k;
    oracle_step_scalars(lr, beta1, beta2, weight_decay, step, &k);
    for (uint64_t i = 0; i < count; ++i)
        update_one((float)oracle_decode16(g16[i], dtype), loss_scale, lr, beta1, beta2, eps, &k,
                   &master[i], &m[i], &v[i], &w16[i], dtype);
}

/* ------------------------------------------------------------------------ */
/* FP32 gradients.  Accumulating many 16-bit micro-batch gradients in a     */
/* 16-bit buffer loses the small contributions, so the accumulator is FP32  */
/* ("How far does splitting the batch get you?", "What does gradient        */
/* accumulation actually buy?").  The accumulate adds each micro-batch's    */
/* 16-bit gradient in FP32 (the first one initialises it); the check and    */
/* the step then read the FP32 gradients, with the same definitions.        */
/* ------------------------------------------------------------------------ */

void oracle_grad_accumulate(float *acc, const uint16_t *g16, int dtype, uint64_t count, int first)
{
    for (uint64_t i = 0; i < count; ++i) {
        const float g = (float)oracle_decode16(g16[i], dtype);
        acc[i] = first ? g : acc[i] + g;
    }
}

void oracle_overflow_check_g32(const float *g32, uint64_t count, float loss_scale,
                               int32_t *found_inf, double *sumsq)
{
    int32_t flag = 0;
    double s = 0.0;
    for (uint64_t i = 0; i < count; ++i) {
        const float g = g32[i] / loss_scale;
        if (!isfinite(g))
            flag = 1;
        s += (double)g * (double)g;
    }
    *found_inf = flag;
    if (sumsq)
        *sumsq = s;
}

void oracle_adam_step_g32(uint16_t *w16, const float *g32, float *master, float *m, float *v,
                          int dtype, uint64_t count, float lr, float beta1, float beta2, float eps,
                          float weight_decay, uint64_t step, float loss_scale)
{
    oracle_scalars_t k;
    oracle_step_scalars(lr, beta1, beta2, weight_decay, step, &k);
    for (uint64_t i = 0; i < count; ++i)
        update_one(g32[i], loss_scale, lr, beta1, beta2, eps, &k, &master[i], &m[i], &v[i],
                   &w16[i], dtype);
}

/* The same update carried out in FP64 from the same FP32 inputs and the    */
/* same FP32 hyperparameters.  Used only to bound the FP32 oracle's error.  */
void oracle_adam_step_f64(double *master, double *m, double *v, const uint16_t *g16, int dtype,
                          uint64_t count, double lr, double beta1, double beta2, double eps,
                          double weight_decay, uint64_t step, double loss_scale)
{
    const double bc1 = 1.0 - pow(beta1, (double)step);
    const double bc2 = 1.0 - pow(beta2, (double)step);
    const double decay = 1.0 - lr * weight_decay;
    for (uint64_t i = 0; i < count; ++i) {
        const double g = oracle_decode16(g16[i], dtype) / loss_scale;
        const double p = master[i] * decay;
        const double m_new = beta1 * m[i] + (1.0 - beta1) * g;
        const double v_new = beta2 * v[i] + (1.0 - beta2) * (g * g);
        const double m_hat = m_new / bc1;
        const double v_hat = v_new / bc2;
        master[i] = p - lr * m_hat / (sqrt(v_hat) + eps);
        m[i] = m_new;
        v[i] = v_new;
    }
}

/* ------------------------------------------------------------------------ */
/* The exchanges around the step, computed on one host.                     */
/*                                                                           */
/* Reduce-scatter: after it, rank i holds the SUM over all ranks of chunk i */
/* ("Training models too big for one GPU", "Data parallelism and the        */
/* all-reduce").  Here the n replicas are n full flat buffers and the sum   */
/* of each element is taken in FP32 over ranks 0..n-1 in order, then        */
/* written as FP32 or rounded once to the 16-bit output format.             */
/* All-gather: every rank's finished chunk is copied to its place in the    */
/* full buffer.  Format codes: 0 FP16, 1 BF16, 2 FP32.                       */
/* ------------------------------------------------------------------------ */

static float load_any(const void *p, int fmt, uint64_t i)
{
    if (fmt == 2)
        return ((const float *)p)[i];
    return (float)oracle_decode16(((const uint16_t *)p)[i], fmt);
}

void oracle_reduce_shard(void *out, int out_fmt, const void *const *replicas, int in_fmt,
                         uint64_t psi, uint32_t n, uint32_t rank)
{
    oracle_layout_t lay;
    if (oracle_layout(psi, n, rank, &lay) != 0)
        return;
    for (uint64_t i = 0; i < lay.count; ++i) {
        float s = 0.0f;
        for (uint32_t k = 0; k < n; ++k)
            s = s + load_any(replicas[k], in_fmt, lay.offset + i);
        if (out_fmt == 2)
            ((float *)out)[i] = s;
        else
            ((uint16_t *)out)[i] = oracle_encode16((double)s, out_fmt);
    }
}

void oracle_gather_shards(void *full, const void *const *shards, int elem_bytes, uint64_t psi,
                          uint32_t n)
{
    for (uint32_t k = 0; k < n; ++k) {
        oracle_layout_t lay;
        if (oracle_layout(psi, n, k, &lay) != 0)
            return;
        for (uint64_t i = 0; i < lay.count; ++i) {
            if (elem_bytes == 4)
                ((float *)full)[lay.offset + i] = ((const float *)shards[k])[i];
            else
                ((uint16_t *)full)[lay.offset + i] = ((const uint16_t *)shards[k])[i];
        }
    }
}
