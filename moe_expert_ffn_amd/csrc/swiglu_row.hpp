// One row of SwiGLU with dynamic int8 re-quantisation, computed by one wave.
//
// Section 4 ("SwiGLU") of the pto-isa MegaMoE overview page: dequantise the
// GMM1 output row with the row's perTokenScale1 (fp32), apply
// silu(u) = u / (1 + exp(-u)) to the first half and multiply by the second
// half, then quantise the row again: scale2 = max|y| / 127 and
// q = CAST_RINT(y * (127 / max|y|)).
//
// Shared by the SwiGLU kernel and by the GMM1 kernel's last round (where
// workgroups without a tile run SwiGLU on rows that are already complete),
// so both produce the same bits.  Each lane keeps its 8-column chunks
// c = lane + 64 i of y in registers, so the row maximum is a wave reduction
// and the row needs a single pass over HBM.
#pragma once

#include "common.hpp"

namespace megamoe {

// silu(u) * g in fp32.
//  * exp(-u) = 2^(-u * log2(e)), from the hardware base-2 exponential
//    (v_exp_f32, about 1 ulp); rounding the scaled argument adds a relative
//    error of about |u| * 2^-24 * ln 2, a few ulp for |u| up to 10.
//  * u / d, d = 1 + exp(-u) >= 1: q = u * rcp(d) with the hardware reciprocal,
//    then one correction of the quotient, q + rcp(d) * (u - q * d), with the
//    residual from an FMA (Markstein's division method).  This gives the
//    correctly rounded quotient except next to a rounding midpoint.
//  * Non-finite cases keep IEEE results: d = inf (u < -88) gives -0, u = inf
//    gives inf, u = -inf or NaN gives NaN (the uncorrected quotient q).
// On the decode, large and skewed workloads every q2 code and every
// scale2 produced this way equals the one from the IEEE exp and division.
__device__ __forceinline__ float silu_times(float u, float g) {
    const float ex = __builtin_amdgcn_exp2f(u * -1.4426950408889634f);
    const float d = ex + 1.0f;
    const float r = __builtin_amdgcn_rcpf(d);
    const float q = u * r;
    float sl = __builtin_fmaf(__builtin_fmaf(-q, d, u), r, q);
    if (!__builtin_isfinite(sl)) sl = q;
    return sl * g;
}

// The row's fp16 chunks: u from columns [0, I), g from [I, 2I).  gmC is read
// once, so the loads carry the non-temporal hint.
template <int MAXC>
__device__ __forceinline__ void swiglu_row_load(const uint16_t *__restrict__ crow, int I, int lane,
                                                uint4 (&uraw)[MAXC], uint4 (&graw)[MAXC]) {
    const int nchunk = I >> 3;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            uraw[i] = load_nt16(crow + c * 8);
            graw[i] = load_nt16(crow + I + c * 8);
        }
    }
}

// y, its row maximum, and the row's q2 codes and scale2 (p1: perTokenScale1).
template <int MAXC>
__device__ __forceinline__ void swiglu_row_finish(const uint4 (&uraw)[MAXC],
                                                  const uint4 (&graw)[MAXC], float p1, int I,
                                                  int lane, int8_t *__restrict__ qrow,
                                                  float *__restrict__ pts2_row) {
    const int nchunk = I >> 3;
    float y[MAXC][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            const uint32_t *uw = reinterpret_cast<const uint32_t *>(&uraw[i]);
            const uint32_t *gw = reinterpret_cast<const uint32_t *>(&graw[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float u = h2f((uint16_t)((uw[j >> 1] >> ((j & 1) * 16)) & 0xffffu)) * p1;
                const float g = h2f((uint16_t)((gw[j >> 1] >> ((j & 1) * 16)) & 0xffffu)) * p1;
                const float v = silu_times(u, g);
                y[i][j] = v;
                amax = fmaxf(amax, fabsf(v));
            }
        }
    }
    amax = wave_max(amax);
    const float scale2 = amax / 127.0f;
    const float mul = 127.0f / amax;

#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = lane + i * kWave;
        if (c >= nchunk) continue;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int q = 0;
            if (amax != 0.0f) {
                float r = rintf(y[i][j] * mul);  // CAST_RINT: ties to even
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                q = (int)r;
            }
            if (j < 4) lo |= ((uint32_t)q & 0xffu) << (8 * j);
            else hi |= ((uint32_t)q & 0xffu) << (8 * (j - 4));
        }
        *reinterpret_cast<uint2 *>(qrow + c * 8) = make_uint2(lo, hi);
    }
    if (lane == 0) *pts2_row = scale2;
}

}  // namespace megamoe
