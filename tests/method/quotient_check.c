/*
 * The unscaling shortcut of the sum-of-squares kernel, checked on the CPU:
 * for S not a power of two, (float)((double)g * RN64(1/S)) must equal the
 * correctly rounded float division g / S whenever the FP64 product is at
 * least 2^-125 in magnitude (below, the kernel divides).  Every FP16 and BF16
 * pattern g against a set of S (small integers, significands just below a
 * power of two, and seeded random positive floats), then seeded random FP32 g.
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

int main(int argc, char **argv) {
    const int n_scales = argc > 1 ? atoi(argv[1]) : 2000;
    const int n_random = argc > 2 ? atoi(argv[2]) : 50000000;
    uint64_t tried = 0, fallback = 0, bad = 0;
    for (int k = 0; k < n_scales; ++k) {
        const float S = pick_scale(k);
        if (!(S > 0.0f) || !isfinite(S) || is_pow2(S)) continue;
        const double rcp = 1.0 / (double)S;
        for (int fmt = 0; fmt < 2; ++fmt)
            for (uint32_t h = 0; h < 65536u; ++h) {
                const float g = fmt ? from_bits(h << 16) : from_f16((uint16_t)h);
                if (isnan(g)) continue;
                const double qq = (double)g * rcp;
                ++tried;
                if (fabs(qq) < 0x1p-125) {
                    ++fallback;
                    continue;
                }
                if (to_bits((float)qq) != to_bits(g / S)) {
                    if (bad < 5) printf("mismatch: g %a S %a\n", (double)g, (double)S);
                    ++bad;
                }
            }
    }
    for (int i = 0; i < n_random; ++i) {
        const float S = from_bits(next32() & 0x7fffffffu);
        const float g = from_bits(next32());
        if (!(S > 0.0f) || !isfinite(S) || is_pow2(S) || isnan(g)) continue;
        const double qq = (double)g * (1.0 / (double)S);
        ++tried;
        if (fabs(qq) < 0x1p-125) {
            ++fallback;
            continue;
        }
        if (to_bits((float)qq) != to_bits(g / S)) {
            if (bad < 5) printf("mismatch: g %a S %a\n", (double)g, (double)S);
            ++bad;
        }
    }
    printf("tried %llu fallback %llu mismatches %llu\n", (unsigned long long)tried,
           (unsigned long long)fallback, (unsigned long long)bad);
    return bad != 0;
}
