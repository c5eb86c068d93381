/*
 * Memory-safety driver for the C oracle (CPU only), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer.  It runs the oracle's entry points on small
 * seeded shapes, including dropped routes (ids -1 and >= E), all-zero token
 * rows, duplicate experts within a token, E = 1 and top_k = E, with every
 * buffer allocated at exactly the size the oracle's signature states, so an
 * access past any of them is reported.  It also checks two facts that need no
 * second implementation: the route permutation is a bijection between valid
 * routes and rows, and the per-token forward gives the same out bits as the
 * whole forward.  Exit status 0 means every shape ran clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_route_sort(int32_t M, int32_t top_k, int32_t E, const int32_t *expert_idx,
                       int32_t *sorted_route, int32_t *expanded_row_idx,
                       int32_t *tokens_per_expert, int32_t *expert_offsets,
                       int32_t *expert_cumsum);
int64_t orc_forward(int32_t M, int32_t K, int32_t E, int32_t top_k, int32_t I,
                    const uint16_t *x, const int32_t *expert_idx, const float *probs,
                    const int8_t *w1, const float *scale1, const int8_t *w2, const float *scale2,
                    int32_t *sorted_route, int32_t *expanded_row_idx, int32_t *tokens_per_expert,
                    int32_t *expert_offsets, int32_t *expert_cumsum, int8_t *gmA, float *pts1,
                    int32_t *acc1, uint16_t *gmC, int8_t *q2, float *pts2, int32_t *acc2,
                    uint16_t *gmm2_out, uint16_t *out, float *out_f32);
void orc_forward_token(int32_t K, int32_t E, int32_t top_k, int32_t I, const uint16_t *x_t,
                       const int32_t *expert_idx_t, const float *probs_t, const int8_t *w1,
                       const float *scale1, const int8_t *w2, const float *scale2, int8_t *qa,
                       float *pts1_out, int32_t *acc1, uint16_t *gmC, int8_t *q2, float *pts2,
                       int32_t *acc2, uint16_t *gmm2_out, uint16_t *out_t, float *out_f32_t);

static uint64_t rng_state;
static uint32_t next_u32(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static int run_shape(int32_t M, int32_t K, int32_t E, int32_t top_k, int32_t I, int drop,
                     int zero_rows, uint64_t seed) {
    rng_state = seed;
    const int64_t R = (int64_t)M * top_k;
    const int32_t N1 = 2 * I;
    uint16_t *x = xmalloc(sizeof(uint16_t) * M * K);
    int32_t *ei = xmalloc(sizeof(int32_t) * R);
    float *probs = xmalloc(sizeof(float) * R);
    int8_t *w1 = xmalloc((size_t)E * K * N1), *w2 = xmalloc((size_t)E * I * K);
    float *s1 = xmalloc(sizeof(float) * E * N1), *s2 = xmalloc(sizeof(float) * E * K);
    for (int64_t i = 0; i < (int64_t)M * K; ++i) {
        /* finite fp16 values of either sign, exponent up to 2^3 */
        uint32_t u = next_u32();
        x[i] = (uint16_t)((u & 0x8000u) | ((u >> 16) % 0x4800u));
    }
    for (int32_t t = 0; t < zero_rows && t < M; ++t) memset(x + (int64_t)t * K, 0, 2 * (size_t)K);
    for (int64_t r = 0; r < R; ++r) {
        ei[r] = (int32_t)(next_u32() % (uint32_t)E);  /* duplicates allowed */
        probs[r] = (float)(next_u32() % 1000) / 1000.0f;
        if (drop && next_u32() % 10 == 0) ei[r] = (next_u32() & 1) ? -1 : E + 3;
    }
    for (int64_t i = 0; i < (int64_t)E * K * N1; ++i) w1[i] = (int8_t)((int)(next_u32() % 255) - 127);
    for (int64_t i = 0; i < (int64_t)E * I * K; ++i) w2[i] = (int8_t)((int)(next_u32() % 255) - 127);
    for (int64_t i = 0; i < (int64_t)E * N1; ++i) s1[i] = 1e-3f + (float)(next_u32() % 9000) * 1e-6f;
    for (int64_t i = 0; i < (int64_t)E * K; ++i) s2[i] = 1e-3f + (float)(next_u32() % 9000) * 1e-6f;

    int32_t *sr = xmalloc(sizeof(int32_t) * R), *eri = xmalloc(sizeof(int32_t) * R);
    int32_t *cnt = xmalloc(sizeof(int32_t) * E), *offs = xmalloc(sizeof(int32_t) * (E + 1));
    int32_t *cum = xmalloc(sizeof(int32_t) * E);
    int8_t *gmA = xmalloc((size_t)R * K);
    float *pts1 = xmalloc(sizeof(float) * R), *pts2 = xmalloc(sizeof(float) * R);
    int32_t *acc1 = xmalloc(sizeof(int32_t) * R * N1), *acc2 = xmalloc(sizeof(int32_t) * R * K);
    uint16_t *gmC = xmalloc(2 * (size_t)R * N1), *g2 = xmalloc(2 * (size_t)R * K);
    int8_t *q2 = xmalloc((size_t)R * I);
    uint16_t *out = xmalloc(2 * (size_t)M * K);
    float *out_f = xmalloc(sizeof(float) * M * K);
    const int64_t dropped = orc_forward(M, K, E, top_k, I, x, ei, probs, w1, s1, w2, s2, sr, eri,
                                        cnt, offs, cum, gmA, pts1, acc1, gmC, q2, pts2, acc2, g2,
                                        out, out_f);
    int fail = 0;
    /* bijection between valid routes and rows [0, R - dropped) */
    const int64_t Rv = R - dropped;
    char *seen = xmalloc((size_t)R);
    memset(seen, 0, (size_t)R);
    for (int64_t r = 0; r < R; ++r) {
        const int valid = ei[r] >= 0 && ei[r] < E;
        if (!valid) { fail |= eri[r] != -1; continue; }
        if (eri[r] < 0 || eri[r] >= Rv || seen[eri[r]]) { fail = 1; continue; }
        seen[eri[r]] = 1;
        fail |= sr[eri[r]] != r;
    }
    for (int64_t d = Rv; d < R; ++d) fail |= sr[d] != -1;
    fail |= Rv > 0 ? cum[E - 1] != Rv : 0;
    /* the per-token forward agrees with the whole forward */
    int8_t *qa = xmalloc((size_t)K);
    float p1;
    int32_t *ta1 = xmalloc(sizeof(int32_t) * top_k * N1), *ta2 = xmalloc(sizeof(int32_t) * top_k * K);
    uint16_t *tc = xmalloc(2 * (size_t)top_k * N1), *tg2 = xmalloc(2 * (size_t)top_k * K);
    int8_t *tq2 = xmalloc((size_t)top_k * I);
    float *tp2 = xmalloc(sizeof(float) * top_k);
    uint16_t *tout = xmalloc(2 * (size_t)K);
    float *toutf = xmalloc(sizeof(float) * K);
    for (int32_t t = 0; t < M; ++t) {
        orc_forward_token(K, E, top_k, I, x + (int64_t)t * K, ei + (int64_t)t * top_k,
                          probs + (int64_t)t * top_k, w1, s1, w2, s2, qa, &p1, ta1, tc, tq2, tp2,
                          ta2, tg2, tout, toutf);
        fail |= memcmp(tout, out + (int64_t)t * K, 2 * (size_t)K) != 0;
    }
    printf("M=%d K=%d E=%d top_k=%d I=%d drop=%d zero_rows=%d: dropped %lld %s\n", M, K, E,
           top_k, I, drop, zero_rows, (long long)dropped, fail ? "FAIL" : "ok");
    free(x); free(ei); free(probs); free(w1); free(w2); free(s1); free(s2); free(sr); free(eri);
    free(cnt); free(offs); free(cum); free(gmA); free(pts1); free(pts2); free(acc1); free(acc2);
    free(gmC); free(g2); free(q2); free(out); free(out_f); free(seen); free(qa); free(ta1);
    free(ta2); free(tc); free(tg2); free(tq2); free(tp2); free(tout); free(toutf);
    return fail;
}

int main(void) {
    int fail = 0;
    fail |= run_shape(16, 256, 4, 2, 128, 0, 0, 1);
    fail |= run_shape(37, 128, 8, 3, 128, 1, 2, 2);   /* dropped routes, zero rows */
    fail |= run_shape(9, 128, 1, 1, 128, 0, 1, 3);    /* E = 1 */
    fail |= run_shape(12, 128, 6, 6, 256, 1, 0, 4);   /* top_k = E */
    fail |= run_shape(1, 384, 3, 2, 128, 0, 0, 5);    /* one token */
    fail |= run_shape(5, 128, 4, 2, 128, 2, 5, 6);    /* every row zero */
    return fail;
}
