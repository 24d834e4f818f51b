/*
 * The quotient rule of the kernels, checked on the CPU: for a divisor d > 0
 * (the loss scale S when it is not a power of two, and the bias corrections
 * 1 - beta^t), (float)((double)a * RN64(1/d)) must equal the correctly
 * rounded float division a / d whenever the result is at least 2^-125 in
 * magnitude or a is zero (otherwise the kernels divide).  Cases:
 *   1. every FP16 and BF16 pattern a against a set of S (small integers,
 *      significands just below a power of two, seeded random positive floats);
 *   2. seeded random FP32 pairs (a any non-NaN pattern, d any positive one);
 *   3. seeded random FP32 a against bias corrections 1 - beta^t (formed in
 *      FP64, rounded once) for common and random beta and t up to 10^5;
 *   4. numerators built to put a / d next to an FP32 rounding boundary: for a
 *      random d and an odd 25-bit M, a = RN32(M * 2^k * d) and its two
 *      neighbours, so that a / d lies within an ulp of the midpoint M * 2^k
 *      (the hardest inputs for the rule).
 * x86-64 SSE arithmetic: float and double operations round to nearest even.
 * Prints the counts and exits 1 on any mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_f16(uint16_t h) {
    const uint32_t s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 1024u), (int)e - 25);
    return s ? -v : v;
}

static float from_bits(uint32_t b) {
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static uint32_t to_bits(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    return b;
}

static uint64_t state = 20261202u;
static uint32_t next32(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 32);
}

static float pick_scale(int k) {
    if (k < 100) return (float)(k + 3);                              /* 3, 4, ... (powers skipped below) */
    if (k < 200) return ldexpf(from_bits(0x3fffffffu - (uint32_t)(k - 100)), (k % 40) - 20);
    return from_bits(next32() & 0x7fffffffu);
}

static int is_pow2(float S) { return (to_bits(S) & 0x7fffffu) == 0; }

static uint64_t tried = 0, fallback = 0, bad = 0;

/* One case of the rule: a / d against the FP64 reciprocal product. */
static void check(float a, float d, double rcp) {
    if (isnan(a)) return;
    const double qq = (double)a * rcp;
    const float q = (float)qq;
    ++tried;
    if (fabsf(q) < 0x1p-125f && a != 0.0f) {
        ++fallback;
        return;
    }
    if (to_bits(q) != to_bits(a / d)) {
        if (bad < 5) printf("mismatch: a %a d %a\n", (double)a, (double)d);
        ++bad;
    }
}

static float random_beta(void) {
    static const float common[] = {0.0f, 0.5f, 0.9f, 0.95f, 0.98f, 0.99f, 0.995f, 0.999f,
                                   0.9995f, 0.9999f};
    const uint32_t k = next32() % 20u;
    if (k < 10u) return common[k];
    return (float)(next32() >> 8) * 0x1p-24f; /* [0, 1) on the FP32 grid of 2^-24 */
}

int main(int argc, char **argv) {
    const int n_scales = argc > 1 ? atoi(argv[1]) : 2000;
    const int n_random = argc > 2 ? atoi(argv[2]) : 50000000;
    const int n_bias = argc > 3 ? atoi(argv[3]) : 50000000;
    const int n_edge = argc > 4 ? atoi(argv[4]) : 20000000;
    /* 1. every 16-bit gradient against a set of loss scales */
    for (int k = 0; k < n_scales; ++k) {
        const float S = pick_scale(k);
        if (!(S > 0.0f) || !isfinite(S) || is_pow2(S)) continue;
        const double rcp = 1.0 / (double)S;
        for (int fmt = 0; fmt < 2; ++fmt)
            for (uint32_t h = 0; h < 65536u; ++h)
                check(fmt ? from_bits(h << 16) : from_f16((uint16_t)h), S, rcp);
    }
    const uint64_t after1 = tried;
    /* 2. random FP32 pairs */
    for (int i = 0; i < n_random; ++i) {
        const float d = from_bits(next32() & 0x7fffffffu);
        const float a = from_bits(next32());
        if (!(d > 0.0f) || !isfinite(d)) continue;
        check(a, d, 1.0 / (double)d);
    }
    const uint64_t after2 = tried;
    /* 3. random FP32 numerators against bias corrections */
    for (int i = 0; i < n_bias; ++i) {
        const float beta = random_beta();
        const uint64_t t = 1u + (next32() % 100000u);
        const float d = (float)(1.0 - pow((double)beta, (double)t));
        if (!(d > 0.0f)) continue;
        check(from_bits(next32()), d, 1.0 / (double)d);
    }
    const uint64_t after3 = tried;
    /* 4. numerators next to a rounding boundary of the quotient */
    for (int i = 0; i < n_edge; ++i) {
        float d;
        if (i & 1) {
            d = (float)(1.0 - pow((double)random_beta(), (double)(1u + next32() % 100000u)));
        } else {
            d = from_bits(next32() & 0x7fffffffu);
        }
        if (!(d > 0.0f) || !isfinite(d)) continue;
        const double M = (double)((1u << 24) | (next32() & 0xffffffu) | 1u); /* odd, 25 bits */
        const int k = (int)(next32() % 300u) - 170;
        /* M * d is exact in FP64 (25 + 24 bits); the scaling by 2^k may round */
        const double target = ldexp(M * (double)d, k - 24);
        const float a0 = (float)target;
        if (!isfinite(a0) || a0 == 0.0f) continue;
        const double rcp = 1.0 / (double)d;
        const float cand[3] = {nextafterf(a0, 0.0f), a0, nextafterf(a0, INFINITY)};
        for (int c = 0; c < 3; ++c) {
            const float a = (next32() & 1u) ? -cand[c] : cand[c];
            check(a, d, rcp);
        }
    }
    printf("tried %llu fallback %llu mismatches %llu (16-bit %llu, random %llu, bias %llu, "
           "boundary %llu)\n",
           (unsigned long long)tried, (unsigned long long)fallback, (unsigned long long)bad,
           (unsigned long long)after1, (unsigned long long)(after2 - after1),
           (unsigned long long)(after3 - after2), (unsigned long long)(tried - after3));
    return bad != 0;
}
