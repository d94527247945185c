/* Checks the division-free e4m3 quotient encoder of the FP8 page writer, as
 * plain C on the host (fmaf is correctly rounded here as on the GPU):
 * for scales s in [2^-63, 2^63], inv = fp32(1 / s) and bf16 x with
 * |x| <= 2^63, the code it gives must equal the e4m3 code (round half to
 * even, saturating at 448) of the exact quotient x / s. The exact code is
 * decided from the float64 quotient, which cannot land on an e4m3 midpoint
 * unless x / s is one (8 + 5 + 24 significant bits < 53).
 *
 * Inputs: every positive and negative bf16 pattern in range under a set of
 * fixed scales (the range ends, 1, 1/448 ...), scales fp32(amax / 448) for
 * random bf16 amax, and random scales over the whole range; then, for random
 * scales, the bf16 values nearest to M * s (and two ulps either side) for
 * every e4m3 midpoint M. Two controls must fail on the same inputs: rounding
 * the plain fp32 quotient, and the reciprocal without its Newton step.
 *
 * usage: recip_quotient_check <number of random scales>; exit status 0 when
 * the encoder never differs and both controls do.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static double MAG[127];

static void init_mag(void) {
    for (int c = 0; c < 127; ++c) {
        const int e = c >> 3, m = c & 7;
        MAG[c] = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    }
}

/* nearest e4m3 code, ties to the even code, |y| >= 448 -> 0x7E, sign ORed in */
static unsigned exact_code(double y) {
    const unsigned sign = signbit(y) ? 0x80u : 0u;
    if (y != y) return 0x7Fu | sign;
    const double a = fabs(y);
    if (a >= 448.0) return 0x7Eu | sign;
    int lo = 0, hi = 126;
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (MAG[mid] >= a) hi = mid; else lo = mid + 1;
    }
    const int h = lo, l = h > 0 ? h - 1 : 0;
    const double eh = fabs(MAG[h] - a), el = fabs(MAG[l] - a);
    int pick = el < eh ? l : h;
    if (el == eh && l != h) pick = (l % 2 == 0) ? l : h;
    return (unsigned)pick | sign;
}

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

#define S_LO 0x1p-63f
#define S_HI 0x1p63f

/* the encoder: round-to-odd magnitude of x / s from the reciprocal and one
 * Newton step, clamped to 448, sign of x, then the round-half-even convert */
static unsigned recip_code(float x, float s, float inv, int newton) {
    const float ax = fabsf(x);
    float y = ax * inv;
    if (newton) y = fmaf(fmaf(-y, s, ax), inv, y);
    const uint32_t rb = u_of(fmaf(-y, s, ax));
    uint32_t u = u_of(y) + (uint32_t)((int32_t)rb >> 31);
    u |= rb < 1u ? rb : 1u;
    u = u < 0x43E00000u ? u : 0x43E00000u;
    return exact_code((double)f_of(u | (u_of(x) & 0x80000000u)));
}

static uint64_t st = 88172645463325252ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

static float rand_scale(void) {
    for (;;) {
        const double e = -63.0 + 126.0 * (double)(rnd() >> 11) / 9007199254740992.0;
        const float s = f_of((u_of((float)exp2(e)) & 0xFF800000u) | (uint32_t)(rnd() & 0x7FFFFF));
        if (s >= S_LO && s <= S_HI) return s;
    }
}

static long n_checked, n_bad, n_plain, n_no_newton;

static void check(float x, float s) {
    if ((u_of(x) & 0x7FFFFFFFu) > 0x5F000000u) return;     /* |x| > 2^63, NaN, inf */
    const float inv = 1.0f / s;
    const unsigned want = exact_code((double)x / (double)s);
    ++n_checked;
    n_plain += exact_code((double)(x / s)) != want;
    n_no_newton += recip_code(x, s, inv, 0) != want;
    const unsigned got = recip_code(x, s, inv, 1);
    if (got != want) {
        if (n_bad < 10) printf("mismatch x=%a s=%a want=%02x got=%02x\n", x, s, want, got);
        ++n_bad;
    }
}

int main(int argc, char** argv) {
    init_mag();
    const int n_scales = argc > 1 ? atoi(argv[1]) : 200;
    const float fixed[] = {S_LO, S_HI, nextafterf(S_LO, 1.0f), nextafterf(S_HI, 0.0f),
                           1.0f, 1.0f / 448.0f, 3.0f, 0.1f};
    const int n_fixed = (int)(sizeof fixed / sizeof fixed[0]);
    for (int i = 0; i < n_fixed + n_scales; ++i) {
        float s;
        if (i < n_fixed) {
            s = fixed[i];
        } else if (i % 2) {
            uint32_t a;
            do a = (uint32_t)(rnd() & 0x7FFF); while (a >= 0x7F80u || a == 0);
            s = f_of(a << 16) / 448.0f;
            if (!(s >= S_LO && s <= S_HI)) continue;
        } else {
            s = rand_scale();
        }
        for (uint32_t b = 0; b < 65536; ++b) check(f_of(b << 16), s);
    }
    const long first = n_checked;
    for (int it = 0; it < n_scales * 50; ++it) {
        const float s = rand_scale();
        for (int c = 0; c < 126; ++c) {
            const double t = 0.5 * (MAG[c] + MAG[c + 1]) * (double)s;
            const uint32_t tb = u_of((float)t) >> 16;
            for (int d = -2; d <= 2; ++d) {
                const uint32_t b = (uint32_t)((int)tb + d);
                check(f_of(b << 16), s);
                check(f_of((b | 0x8000u) << 16), s);
            }
        }
    }
    printf("every bf16 x: %ld checked; midpoint neighbourhoods: %ld checked; mismatches %ld\n",
           first, n_checked - first, n_bad);
    printf("controls: plain fp32 quotient wrong %ld times, no Newton step wrong %ld times\n",
           n_plain, n_no_newton);
    return (n_bad == 0 && n_plain > 0 && n_no_newton > 0) ? 0 : 1;
}
