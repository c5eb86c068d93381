/*
 * Exhaustive check of the GPU quantiser's division (CPU only).
 *
 * FrontReorder step 2c of the pto-isa MegaMoE overview page quantises each
 * token with scale = max|x| / 127 and q = CAST_ROUND(x / scale) (TDIV, then
 * round half away from zero).  The GPU kernel does not divide: with
 * inv = 1 / scale (IEEE), it forms q0 = x * inv and corrects it once by the
 * FMA residual, q0 + inv * (x - q0 * scale) (Markstein's method).  Nor does it
 * call roundf or clamp: it adds 0.49999997 (the largest float below one half)
 * with the sign of q and truncates toward zero.  Adding exactly one half would
 * round 0.49999997 itself up to 1.  This program runs both forms, in IEEE single precision with
 * fused multiply-adds where the kernel has them and no other contraction,
 * over every finite fp16 row maximum amax > 0 and every fp16 x with
 * |x| <= amax (both signs), and counts the pairs whose int8 codes differ.
 * It prints "pairs <n> mismatches <m>" and exits non-zero if m > 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

/* fp16 bit pattern (finite) -> float, from the definition of binary16 */
static float half_to_float(uint16_t h) {
    const int e = (h >> 10) & 0x1f, m = h & 0x3ff;
    const float mag = e ? ldexpf((float)(1024 + m), e - 25) : ldexpf((float)m, -24);
    return (h & 0x8000) ? -mag : mag;
}

static int clamp127(float r) { return (int)fminf(fmaxf(r, -127.0f), 127.0f); }

/* the kernel's rounding of q: (int) truncates toward zero; no clamp */
static int round_biased(float q) { return (int)(q + copysignf(0x1.fffffep-2f, q)); }

int main(void) {
    long long pairs = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad)
    for (int a = 1; a < 0x7c00; ++a) {
        const float amax = half_to_float((uint16_t)a);
        const float scale = amax / 127.0f;
        const float inv = 1.0f / scale;
        for (int xb = 0; xb <= a; ++xb) {
            for (int sgn = 0; sgn < 2; ++sgn) {
                if (sgn && xb == 0) continue;  /* -0 quantises like +0 */
                const float x = half_to_float((uint16_t)(xb | (sgn << 15)));
                const int ref = clamp127(roundf(x / scale));
                const float q0 = fmaf(x, inv, 0.0f);
                const float q = fmaf(fmaf(-q0, scale, x), inv, q0);
                const int got = round_biased(q);
                pairs += 1;
                bad += got != ref;
            }
        }
    }
    printf("pairs %lld mismatches %lld\n", pairs, bad);
    return bad != 0;
}
