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
 *
 * Second check, for SwiGLU's re-quantisation (section 4 of the page,
 * q = CAST_RINT(y * (127 / max|y|))): the GPU kernel rounds the fp32 product p
 * to an integer by adding 1.5 * 2^23 and takes the low byte of the sum's bits
 * as the int8 code.  For every float p with |p| <= 128 (every product that
 * |y| <= max|y| allows, and more) this is compared with rintf(p) as an int8.
 * It prints "rint values <n> mismatches <m>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

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

    long long vals = 0, bad2 = 0;
    const uint32_t top = 0x43000000u; /* 128.0f */
#pragma omp parallel for schedule(static) reduction(+ : vals, bad2)
    for (long long u = 0; u <= (long long)top; ++u) {
        for (int sgn = 0; sgn < 2; ++sgn) {
            const uint32_t bits = (uint32_t)u | ((uint32_t)sgn << 31);
            float p;
            memcpy(&p, &bits, 4);
            const float sum = p + 12582912.0f;
            uint32_t sb;
            memcpy(&sb, &sum, 4);
            const int8_t got = (int8_t)(sb & 0xffu);
            const int8_t ref = (int8_t)(int)rintf(p);
            vals += 1;
            bad2 += got != ref;
        }
    }
    printf("rint values %lld mismatches %lld\n", vals, bad2);
    return bad != 0 || bad2 != 0;
}
