/*
 * MegaMoE expert pipeline -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP path and is deliberately slow and literal: one loop per formula, in
 * the order the MegaMoE pages state them.
 *
 * Source: "pto-isa MegaMoE operator" overview page (pto-isa,
 * kernels/manual/a2a3/dispatch_mega_combine).  Section names below refer to
 * that page's seven stages: 1 FrontReorder, 2 Dispatch, 3 GMM1, 4 SwiGLU,
 * 5 GMM2, 6 Combine, 7 Unpermute.  With one rank, Dispatch is the identity
 * and Combine's remote store becomes a local dequant-and-cast.
 *
 * Precision follows the page: fp32 working type for every dequant / activation
 * / accumulation step (TCVT to fp32 before arithmetic), int32 GEMM
 * accumulators, IEEE round-to-nearest-even for every float narrowing, C
 * roundf() for CAST_ROUND and rintf() for CAST_RINT.  Build with
 * -ffp-contract=off and without -ffast-math.
 *
 * Readings where the page is silent (route tie order, output element type,
 * zero rows, invalid expert ids) are listed in the design notes; each is
 * repeated at the function it affects.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

/* ------------------------------------------------------------------------- */
/* IEEE narrow formats.  Rounding is written from the definition: find the   */
/* quantum 2^(E - p + 1) of the binade (clamped at the subnormal quantum),     */
/* divide (exact: power of two), round to nearest integer with ties to even,  */
/* multiply back.  The value is exact in double, so no double rounding.       */
/* ------------------------------------------------------------------------- */

/* Round |a| (a >= 0, finite) to a binary format with p significand bits and
 * minimum normal exponent emin.  Returns the rounded magnitude. */
static double round_to_format(double a, int p, int emin) {
    if (a == 0.0) return 0.0;
    int e2;
    frexp(a, &e2);               /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;              /* floor(log2 a) */
    if (E < emin) E = emin;      /* subnormal range: fixed quantum */
    double q = ldexp(1.0, E - (p - 1));
    double n = nearbyint(a / q); /* default rounding mode: ties to even */
    return n * q;
}

/* binary16: 11 significand bits, emin = -14, max finite 65504. */
uint16_t orc_f2h(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
    double r = round_to_format(a, 11, -14);
    if (r > 65504.0) return (uint16_t)(sign | 0x7c00u);
    if (r < ldexp(1.0, -14)) {                      /* subnormal or zero */
        return (uint16_t)(sign | (uint16_t)(r * ldexp(1.0, 24)));
    }
    int e2;
    double m = frexp(r, &e2);                        /* r = m * 2^e2, m in [0.5,1) */
    uint16_t expf_ = (uint16_t)(e2 - 1 + 15);
    uint16_t man = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (expf_ << 10) | man);
}

float orc_h2f(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)man, -24);
    else if (e == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(1024 + man), e - 25);
    return (float)(sign ? -v : v);
}

/* bfloat16: 8 significand bits, emin = -126, max finite (2 - 2^-7) * 2^127. */
uint16_t orc_f2bf(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7fc0u);
    if (isinf(f)) return (uint16_t)(sign | 0x7f80u);
    double a = fabs((double)f);
    double r = round_to_format(a, 8, -126);
    double maxf = ldexp(2.0 - ldexp(1.0, -7), 127);
    if (r > maxf) return (uint16_t)(sign | 0x7f80u);
    /* r is representable in binary32 exactly; its top 16 bits are the bf16. */
    float rf = (float)r;
    uint32_t rb;
    memcpy(&rb, &rf, 4);
    return (uint16_t)(sign | (uint16_t)(rb >> 16));
}

float orc_bf2f(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* ------------------------------------------------------------------------- */
/* Stage 1, FrontReorder: route sort and metadata.                            */
/* ------------------------------------------------------------------------- */

/*
 * Routes are numbered r = t*topK + s (Unpermute section: the expanded row of
 * route (token, slot) is expandedRowIdx[token*topK + slot]).
 *
 * FrontReorder phase 1 orders the (expertId[route], route) pairs expert-major.
 * Reading: ties inside one expert keep ascending route order (a stable sort),
 * so the destination rows are unique.
 *
 * Phase 2a counts routes per expert (localTokenPerExpert); phase 2b inverts the
 * order: expandedRowIdx[srcRoute] = dstRow.  Phase 3/4's prefix metadata with
 * one rank reduces to: exclusive prefix over experts (row where expert e's
 * group starts, the single-rank preSumBeforeRank) and the inclusive prefix
 * (running total of expertTokenNums).
 *
 * Reading for invalid ids: a route whose expert id lies outside [0, E) is
 * dropped: expandedRowIdx = -1, not counted, skipped by Unpermute (the page's
 * "if expandedRow valid").  Destination rows [valid, R) get sorted_route = -1.
 * Returns the number of dropped routes.
 */
int64_t orc_route_sort(int32_t M, int32_t top_k, int32_t E, const int32_t *expert_idx,
                       int32_t *sorted_route, int32_t *expanded_row_idx,
                       int32_t *tokens_per_expert, int32_t *expert_offsets,
                       int32_t *expert_cumsum) {
    int64_t R = (int64_t)M * top_k;
    int64_t dropped = 0;
    /* 2a: count */
    for (int32_t e = 0; e < E; ++e) tokens_per_expert[e] = 0;
    for (int64_t r = 0; r < R; ++r) {
        int32_t e = expert_idx[r];
        if (e >= 0 && e < E) tokens_per_expert[e] += 1;
        else dropped += 1;
    }
    /* prefix over experts */
    int32_t run = 0;
    for (int32_t e = 0; e < E; ++e) {
        expert_offsets[e] = run;
        run += tokens_per_expert[e];
        expert_cumsum[e] = run;
    }
    expert_offsets[E] = run;
    /* 1 + 2b: stable expert-major order and its inverse */
    for (int64_t d = 0; d < R; ++d) sorted_route[d] = -1;
    int64_t d = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int64_t r = 0; r < R; ++r) {
            if (expert_idx[r] == e) {
                sorted_route[d] = (int32_t)r;
                expanded_row_idx[r] = (int32_t)d;
                ++d;
            }
        }
    }
    for (int64_t r = 0; r < R; ++r) {
        int32_t e = expert_idx[r];
        if (!(e >= 0 && e < E)) expanded_row_idx[r] = -1;
    }
    return dropped;
}

/*
 * FrontReorder phase 2c: dynamic per-token int8 quantisation, done once per
 * token.  fp32 copy of the row, max of |x|, scale = max/127, q = x / scale
 * (true division), converted with CAST_ROUND (C roundf: half away from zero).
 * Reading for an all-zero row: scale 0 and q 0.  The int8 conversion saturates
 * at +-127 (|x/scale| never exceeds 127 by more than rounding error).
 */
void orc_quant_token(int32_t K, const uint16_t *x_row, int8_t *q, float *scale_out) {
    float amax = 0.0f;
    for (int32_t k = 0; k < K; ++k) {
        float v = fabsf(orc_h2f(x_row[k]));
        if (v > amax) amax = v;
    }
    float scale = amax / 127.0f;
    *scale_out = scale;
    for (int32_t k = 0; k < K; ++k) {
        if (amax == 0.0f) { q[k] = 0; continue; }
        float v = orc_h2f(x_row[k]);
        float r = roundf(v / scale);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
}

/*
 * GMM1 / GMM2 (sections 3 and 5) for one row of one expert group:
 *   acc[n] = sum_k a[k] * w[k, n]                (int32, exact)
 *   c[n]   = half( float(acc[n]) * scale[n] )    (per-channel FixPipe dequant)
 * w is the logical [Kred, N] slice of one expert, row-major.
 */
void orc_gmm_row(int32_t Kred, int32_t N, const int8_t *a_row, const int8_t *w,
                 const float *scale, int32_t *acc, uint16_t *c) {
    for (int32_t n = 0; n < N; ++n) acc[n] = 0;
    for (int32_t k = 0; k < Kred; ++k) {
        int32_t ak = a_row[k];
        const int8_t *wk = w + (int64_t)k * N;
        for (int32_t n = 0; n < N; ++n) acc[n] += ak * (int32_t)wk[n];
    }
    for (int32_t n = 0; n < N; ++n) {
        float prod = (float)acc[n] * scale[n];
        c[n] = orc_f2h(prod);
    }
}

/*
 * SwiGLU (section 4) for one row:
 *   dequant = float(gmC[row, :]) * perTokenScale1[row]
 *   first half u = dequant[0:I] goes through silu(u) = u / (1 + exp(-u)),
 *   the second half g = dequant[I:2I] is the gate;  y = silu(u) * g
 *   dynamic quant: maxAbs = max|y|, scale2 = maxAbs / 127,
 *   q = CAST_RINT(y * (127 / maxAbs)) via int32 -> half -> int8 (exact for
 *   |q| <= 127, so a single rintf).  Reading for maxAbs == 0: scale2 0, q 0.
 */
void orc_swiglu_quant_row(int32_t I, const uint16_t *c_row, float pts1, int8_t *q2,
                          float *pts2_out) {
    float *y = (float *)malloc(sizeof(float) * (size_t)I);
    float amax = 0.0f;
    for (int32_t i = 0; i < I; ++i) {
        float u = orc_h2f(c_row[i]) * pts1;
        float g = orc_h2f(c_row[I + i]) * pts1;
        float neg = u * -1.0f;
        float ex = expf(neg);
        float den = ex + 1.0f;
        float s = u / den;
        y[i] = s * g;
        float ay = fabsf(y[i]);
        if (ay > amax) amax = ay;
    }
    float scale2 = amax / 127.0f;
    *pts2_out = scale2;
    if (amax == 0.0f) {
        for (int32_t i = 0; i < I; ++i) q2[i] = 0;
    } else {
        float mul = 127.0f / amax;
        for (int32_t i = 0; i < I; ++i) {
            float r = rintf(y[i] * mul);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q2[i] = (int8_t)r;
        }
    }
    free(y);
}

/*
 * Combine (section 6, one rank) + Unpermute (section 7) for one token:
 *   d_s  = outType( float(gmm2Output[row_s, k]) * perTokenScale2[row_s] )
 *   acc  = sum over slots s in order of float(d_s) * probs[t, s]   (fp32,
 *          separate multiply and add, skipping invalid rows)
 *   out  = outType(acc) with CAST_RINT
 * Reading: the output element type is bfloat16 (fp16 would overflow on the
 * Combine products at these scales).  out_f32 receives acc before rounding.
 */
void orc_unpermute_token(int32_t K, int32_t top_k, const int32_t *eri_t, const float *probs_t,
                         const uint16_t *gmm2_out, const float *pts2, uint16_t *out_t,
                         float *out_f32_t) {
    for (int32_t k = 0; k < K; ++k) {
        float acc = 0.0f;
        for (int32_t s = 0; s < top_k; ++s) {
            int32_t row = eri_t[s];
            if (row < 0) continue;
            float deq = orc_h2f(gmm2_out[(int64_t)row * K + k]) * pts2[row];
            float d = orc_bf2f(orc_f2bf(deq));
            float weighted = d * probs_t[s];
            acc = acc + weighted;
        }
        if (out_f32_t) out_f32_t[k] = acc;
        out_t[k] = orc_f2bf(acc);
    }
}

/* ------------------------------------------------------------------------- */
/* The whole forward, stage by stage, with every intermediate exposed.        */
/* ------------------------------------------------------------------------- */
int64_t orc_forward(int32_t M, int32_t K, int32_t E, int32_t top_k, int32_t I,
                    const uint16_t *x, const int32_t *expert_idx, const float *probs,
                    const int8_t *w1 /*[E,K,2I]*/, const float *scale1 /*[E,2I]*/,
                    const int8_t *w2 /*[E,I,K]*/, const float *scale2 /*[E,K]*/,
                    /* outputs */
                    int32_t *sorted_route, int32_t *expanded_row_idx, int32_t *tokens_per_expert,
                    int32_t *expert_offsets, int32_t *expert_cumsum,
                    int8_t *gmA /*[R,K]*/, float *pts1 /*[R]*/,
                    int32_t *acc1 /*[R,2I]*/, uint16_t *gmC /*[R,2I]*/,
                    int8_t *q2 /*[R,I]*/, float *pts2 /*[R]*/,
                    int32_t *acc2 /*[R,K]*/, uint16_t *gmm2_out /*[R,K]*/,
                    uint16_t *out /*[M,K]*/, float *out_f32 /*[M,K]*/) {
    int64_t R = (int64_t)M * top_k;
    int32_t N1 = 2 * I;
    int64_t dropped = orc_route_sort(M, top_k, E, expert_idx, sorted_route, expanded_row_idx,
                                     tokens_per_expert, expert_offsets, expert_cumsum);
    /* FrontReorder 2c (+ Dispatch, identity on one rank): quantise each token
     * once and scatter its row to every destination row of its routes. */
    int8_t *qrow = (int8_t *)malloc((size_t)K);
    for (int32_t t = 0; t < M; ++t) {
        float sc;
        orc_quant_token(K, x + (int64_t)t * K, qrow, &sc);
        for (int32_t s = 0; s < top_k; ++s) {
            int32_t d = expanded_row_idx[(int64_t)t * top_k + s];
            if (d < 0) continue;
            memcpy(gmA + (int64_t)d * K, qrow, (size_t)K);
            pts1[d] = sc;
        }
    }
    free(qrow);
    /* GMM1 -> SwiGLU -> GMM2 per expert group */
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t d = expert_offsets[e]; d < expert_offsets[e + 1]; ++d) {
            orc_gmm_row(K, N1, gmA + (int64_t)d * K, w1 + (int64_t)e * K * N1,
                        scale1 + (int64_t)e * N1, acc1 + (int64_t)d * N1, gmC + (int64_t)d * N1);
            orc_swiglu_quant_row(I, gmC + (int64_t)d * N1, pts1[d], q2 + (int64_t)d * I, &pts2[d]);
            orc_gmm_row(I, K, q2 + (int64_t)d * I, w2 + (int64_t)e * I * K,
                        scale2 + (int64_t)e * K, acc2 + (int64_t)d * K,
                        gmm2_out + (int64_t)d * K);
        }
    }
    (void)R;
    for (int32_t t = 0; t < M; ++t) {
        orc_unpermute_token(K, top_k, expanded_row_idx + (int64_t)t * top_k,
                            probs + (int64_t)t * top_k, gmm2_out, pts2, out + (int64_t)t * K,
                            out_f32 ? out_f32 + (int64_t)t * K : NULL);
    }
    return dropped;
}

/*
 * One token's forward without any sort: quantise, and for each slot run the
 * three per-row stages against that slot's expert, then combine.  Used to
 * compute sampled outputs of large workloads one token at a time.  Slot rows
 * are written to the caller's [topK, *] scratch arrays in slot order.
 */
void orc_forward_token(int32_t K, int32_t E, int32_t top_k, int32_t I,
                       const uint16_t *x_t, const int32_t *expert_idx_t, const float *probs_t,
                       const int8_t *w1, const float *scale1, const int8_t *w2,
                       const float *scale2,
                       int8_t *qa /*[K]*/, float *pts1_out /*[1]*/,
                       int32_t *acc1 /*[topK,2I]*/, uint16_t *gmC /*[topK,2I]*/,
                       int8_t *q2 /*[topK,I]*/, float *pts2 /*[topK]*/,
                       int32_t *acc2 /*[topK,K]*/, uint16_t *gmm2_out /*[topK,K]*/,
                       uint16_t *out_t /*[K]*/, float *out_f32_t /*[K]*/) {
    int32_t N1 = 2 * I;
    orc_quant_token(K, x_t, qa, pts1_out);
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)top_k);
    for (int32_t s = 0; s < top_k; ++s) {
        int32_t e = expert_idx_t[s];
        if (e < 0 || e >= E) { rows[s] = -1; continue; }
        rows[s] = s;
        orc_gmm_row(K, N1, qa, w1 + (int64_t)e * K * N1, scale1 + (int64_t)e * N1,
                    acc1 + (int64_t)s * N1, gmC + (int64_t)s * N1);
        orc_swiglu_quant_row(I, gmC + (int64_t)s * N1, *pts1_out, q2 + (int64_t)s * I, &pts2[s]);
        orc_gmm_row(I, K, q2 + (int64_t)s * I, w2 + (int64_t)e * I * K, scale2 + (int64_t)e * K,
                    acc2 + (int64_t)s * K, gmm2_out + (int64_t)s * K);
    }
    orc_unpermute_token(K, top_k, rows, probs_t, gmm2_out, pts2, out_t, out_f32_t);
    free(rows);
}
