/* Checks, on the host's IEEE fp32 (FMA from the C library), the three
 * identities the GPU quantizer's arithmetic rests on:
 *   1. round half away from zero: (int)(q + copysign(pred(1/2), q)) equals
 *      roundf(q) for every float with |q| <= 256 (exhaustive);
 *   2. RN(m / 7) = fma(fma(-q0, 7, m), y7, q0) with y7 = RN(1/7), q0 = RN(m y7),
 *      for every finite m >= 0 (exhaustive);
 *   3. Markstein's correction with y = RN(1/s): the code round(RN(w / s)) is
 *      the same through fma(fma(-RN(w y), s, w), y, RN(w y)) for scales
 *      s in [2^-60, 2^125] and |w / s| <= 127.5, on random pairs crowded at
 *      half-integers and integers (sampled).
 * Prints one line per check with its mismatch count; exit status 0 iff all
 * counts are zero.  Usage: quant_identities [samples for check 3]. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static inline float fb(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static inline uint32_t bf(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static inline uint64_t splitmix(uint64_t* x) {
    uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(int argc, char** argv) {
    long long samples = argc > 1 ? atoll(argv[1]) : 200000000LL;
    long long bad1 = 0, bad2 = 0, bad3 = 0, n3 = 0;
    const float h = fb(0x3EFFFFFFu);
    #pragma omp parallel for reduction(+:bad1) schedule(static)
    for (long long b = 0; b <= 0x43800000LL; ++b) {
        for (int sg = 0; sg < 2; ++sg) {
            const float q = fb((uint32_t)b | (sg ? 0x80000000u : 0u));
            volatile float hs = copysignf(h, q);
            if ((int)(q + hs) != (int)roundf(q)) bad1++;
        }
    }
    printf("round_half_away: %lld mismatches over |q| <= 256\n", bad1);
    const float y7 = 1.0f / 7.0f;
    #pragma omp parallel for reduction(+:bad2) schedule(static)
    for (long long b = 0; b < 0x7F800000LL; ++b) {
        const float m = fb((uint32_t)b);
        volatile float q0 = m * y7;
        const float r = fmaf(-q0, 7.0f, m);
        const float s = fmaf(r, y7, q0);
        volatile float ref = m / 7.0f;
        if (bf(s) != bf(ref)) bad2++;
    }
    printf("div7: %lld mismatches over all finite m >= 0\n", bad2);
    #pragma omp parallel for reduction(+:bad3, n3) schedule(static)
    for (int t = 0; t < 64; ++t) {
        uint64_t st = 0x5EEDull + 7919ull * (uint64_t)t;
        for (long long i = t; i < samples; i += 64) {
            const uint64_t a = splitmix(&st), c = splitmix(&st);
            const int ex = (int)(a % 186) - 60;
            const float s = fb(((uint32_t)(ex + 127) << 23) | ((uint32_t)(a >> 8) & 0x7fffffu));
            float w;
            const int nn = (int)((c >> 8) % 255) - 127;
            const int d = (int)((c >> 40) % 9) - 4;
            switch (c & 3) {
                case 0: w = (float)((((double)(c >> 11) / 9007199254740992.0) * 255.0 - 127.5) * s);
                        break;
                case 1: w = fb(bf((float)((nn + 0.5) * (double)s)) + d); break;
                case 2: w = fb(bf((float)(nn * (double)s)) + d); break;
                default: w = ldexpf((float)((c >> 20) & 0xffff) / 65536.0f, -(int)((c >> 8) % 40)) * s;
            }
            if (!isfinite(w) || fabs((double)w / s) > 127.5) continue;
            volatile float y = 1.0f / s;
            volatile float q0 = w * y;
            const float r = fmaf(-q0, s, w);
            const float q = fmaf(r, y, q0);
            volatile float ref = w / s;
            n3++;
            if (roundf(q) != roundf(ref)) bad3++;
        }
    }
    printf("markstein_codes: %lld mismatches over %lld sampled pairs\n", bad3, n3);
    return (bad1 || bad2 || bad3) ? 1 : 0;
}
