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
// The row's 64-byte K slices are stored slice_stride bytes apart from qrow
// (64: a row-major row; 128: a row of the row-paired layout).
template <int MAXC>
__device__ __forceinline__ void swiglu_row_finish(const uint4 (&uraw)[MAXC],
                                                  const uint4 (&graw)[MAXC], float p1, int I,
                                                  int lane, int8_t *__restrict__ qrow,
                                                  int slice_stride, float *__restrict__ pts2_row) {
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
                // u = fp32(u16) * p1 as an FMA with a +0 addend, so that the
                // hardware reads the fp16 value in the same instruction (the
                // product and its rounding are the same; only a -0 becomes +0,
                // which gives a zero y either way)
                const float u = __builtin_fmaf(
                    h2f((uint16_t)((uw[j >> 1] >> ((j & 1) * 16)) & 0xffffu)), p1, 0.0f);
                const float g = __builtin_fmaf(
                    h2f((uint16_t)((gw[j >> 1] >> ((j & 1) * 16)) & 0xffffu)), p1, 0.0f);
                const float v = silu_times(u, g);
                y[i][j] = v;
                amax = fmaxf(amax, fabsf(v));
            }
        }
    }
    amax = wave_max(amax);
    const float scale2 = amax / 127.0f;
    const float mul = amax != 0.0f ? 127.0f / amax : 0.0f;  // an all-zero row gives 0

    // CAST_RINT(y * mul): the product is rounded to fp32 first, then adding
    // 1.5 * 2^23 rounds it to an integer, to nearest even, in the low bits of
    // the sum (|y * mul| <= 127 * (1 + 2^-23) < 2^22, so the sum has unit
    // spacing); the low byte of those bits is the int8 code.  |y| <= max|y|
    // keeps the code within [-127, 127], so no clamp is needed.
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = lane + i * kWave;
        if (c >= nchunk) continue;
        uint32_t b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = __float_as_uint(keep_f32(y[i][j] * mul) + 12582912.0f);
        // low bytes of b0..b3 and b4..b7, gathered by byte permutes
        const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u),
                                                  0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u),
                                                  0x05040100u);
        *reinterpret_cast<uint2 *>(qrow + (c >> 3) * slice_stride + ((c & 7) << 3)) =
            make_uint2(lo, hi);
    }
    if (lane == 0) *pts2_row = scale2;
}

}  // namespace megamoe
