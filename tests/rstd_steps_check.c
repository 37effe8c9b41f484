/* Exhaustive host check of the exact shortcut steps the fused LayerNorm kernels use
 * for rstd (binary32, fused multiply-add as on the device).  Every mode prints one
 * line "<mode> failures <n>".
 *
 *   div  H0 H1   for every H = H0, H0+8, ..., H1 and every significand of S in [1, 2):
 *                q0 = RN(S * RN(1/H)), r = fma(-q0, H, S), q = fma(r, RN(1/H), q0)
 *                must equal RN(S / H)
 *   div0 H0 H1   the same without the correction step (a control: must fail)
 *   sqrt         for every v in [1, 4) and every start s0 within one ulp of RN(sqrt v):
 *                the neighbour fix-up must give RN(sqrt(v))
 *   rcp          for every significand of s in [1, 2) except all ones, and every
 *                faithful start y0 (RD or RU of 1/s): y0 + y0 * (1 - s * y0) with two
 *                fmas must equal RN(1/s)
 *   rcp_ones     the same for the all-ones significand (expected to fail: the kernels
 *                keep the general divide there)
 *
 * Reference values come from binary64 arithmetic rounded once to binary32, which
 * equals the correctly rounded binary32 result for divide and square root. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float div_fast(float S, float H, float rH, int correct) {
    float q = S * rH;
    if (!correct) return q;
    const float r = fmaf(-q, H, S);
    return fmaf(r, rH, q);
}

static float sqrt_fix(float v, float s0) {
    const float lo = f_of(u_of(s0) - 1u), hi = f_of(u_of(s0) + 1u);
    const float t = fmaf(-lo, s0, v) <= 0.0f ? lo : s0;
    return fmaf(-hi, s0, v) > 0.0f ? hi : t;
}

static float rcp_step(float s, float y0) {
    const float e = fmaf(-s, y0, 1.0f);
    return fmaf(e, y0, y0);
}

int main(int argc, char** argv) {
    if (argc < 2) return 2;
    const char* mode = argv[1];
    long fail = 0;
    if (!strcmp(mode, "div") || !strcmp(mode, "div0")) {
        if (argc < 4) return 2;
        const int correct = !strcmp(mode, "div");
        const int h0 = atoi(argv[2]), h1 = atoi(argv[3]);
        for (int h = h0; h <= h1; h += 8) {
            const float H = (float)h, rH = (float)(1.0 / (double)h);
            for (uint32_t m = 0; m < (1u << 23); ++m) {
                const float S = f_of(0x3F800000u | m);
                const float want = (float)((double)S / (double)h);
                if (div_fast(S, H, rH, correct) != want) ++fail;
            }
        }
    } else if (!strcmp(mode, "sqrt")) {
        for (uint32_t m = 0; m < (1u << 24); ++m) {
            const float v = f_of(0x3F800000u + m);
            const float want = (float)sqrt((double)v);
            for (int d = -1; d <= 1; ++d)
                if (sqrt_fix(v, f_of(u_of(want) + (uint32_t)d)) != want) ++fail;
        }
    } else if (!strcmp(mode, "rcp") || !strcmp(mode, "rcp_ones")) {
        const int ones = !strcmp(mode, "rcp_ones");
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            if ((m == 0x7FFFFFu) != ones) continue;
            const float s = f_of(0x3F800000u | m);
            const double exact = 1.0 / (double)s;
            const float want = (float)exact;
            /* the faithful starts: the binary32 neighbours enclosing 1/s */
            float dn = want, up = want;
            if ((double)want > exact) dn = f_of(u_of(want) - 1u);
            if ((double)want < exact) up = f_of(u_of(want) + 1u);
            if (rcp_step(s, dn) != want) ++fail;
            if (rcp_step(s, up) != want) ++fail;
        }
    } else {
        return 2;
    }
    printf("%s failures %ld\n", mode, fail);
    return 0;
}
