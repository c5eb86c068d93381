// SwiGLU with dynamic per-row int8 re-quantisation.
//
// Section 4 ("SwiGLU") of the pto-isa MegaMoE overview page: dequantise the
// GMM1 output row with the row's perTokenScale1 (fp32), apply
// silu(u) = u / (1 + exp(-u)) to the first half and multiply by the second
// half, then quantise the row again: scale2 = max|y| / 127 and
// q = CAST_RINT(y * (127 / max|y|)).
//
// One wave per row, four rows per workgroup: each lane keeps its 8-column
// chunks of y in registers, so the row maximum is a wave reduction and the
// row needs a single pass over HBM.  Every load of the row is issued before
// the validity check, so the two memory round trips overlap.
//
// At large row counts the kernel is bound by VALU issue, not HBM, so silu is
// evaluated with the hardware's base-2 exponential and reciprocal (see
// silu_times below) rather than with the IEEE-rounded library exp and
// division, which cost about three times the instructions.
#include "common.hpp"
#include "kernels.hpp"

namespace megamoe {

constexpr int kRowsPerBlock = 4;

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

template <int MAXC>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void swiglu_quant_kernel(
    const uint16_t *__restrict__ gmC, const float *__restrict__ pts1,
    const int32_t *__restrict__ expert_cumsum, int R, int E, int I, int8_t *__restrict__ q2,
    float *__restrict__ pts2) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= R) return;  // wave-uniform; gmC and pts1 hold R rows
    const int nchunk = I >> 3;
    const uint16_t *crow = gmC + (size_t)row * (2 * I);

    uint4 uraw[MAXC], graw[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            uraw[i] = load_nt16(crow + c * 8);  // gmC is read once
            graw[i] = load_nt16(crow + I + c * 8);
        }
    }
    const float p1 = pts1[row];
    if (row >= expert_cumsum[E - 1]) return;  // only valid rows carry data

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

    int8_t *qrow = q2 + (size_t)row * I;
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
    if (lane == 0) pts2[row] = scale2;
}

hipError_t launch_swiglu_quant(const uint16_t *gmC, const float *pts1,
                               const int32_t *expert_cumsum, int R, int E, int I, int8_t *q2,
                               float *pts2, hipStream_t stream) {
    const int per_lane = (I / 8 + kWave - 1) / kWave;  // I <= 16384: at most 32
    dim3 grid((R + kRowsPerBlock - 1) / kRowsPerBlock), block(kRowsPerBlock * kWave);
#define MEGAMOE_SWIGLU(C)                                                                 \
    hipLaunchKernelGGL(swiglu_quant_kernel<C>, grid, block, 0, stream, gmC, pts1, expert_cumsum, \
                       R, E, I, q2, pts2)
    if (per_lane <= 1) MEGAMOE_SWIGLU(1);
    else if (per_lane <= 2) MEGAMOE_SWIGLU(2);
    else if (per_lane <= 3) MEGAMOE_SWIGLU(3);
    else if (per_lane <= 4) MEGAMOE_SWIGLU(4);
    else if (per_lane <= 8) MEGAMOE_SWIGLU(8);
    else if (per_lane <= 16) MEGAMOE_SWIGLU(16);
    else MEGAMOE_SWIGLU(32);
#undef MEGAMOE_SWIGLU
    return hipGetLastError();
}

}  // namespace megamoe
