// SwiGLU with dynamic per-row int8 re-quantisation (section 4, "SwiGLU", of
// the pto-isa MegaMoE overview page; the row arithmetic is in swiglu_row.hpp).
//
// One wave per row, four rows per workgroup.  Every load of the row is issued
// before the validity check, so the two memory round trips overlap.
//
// At large row counts the kernel is bound by VALU issue, not HBM, so silu is
// evaluated with the hardware's base-2 exponential and reciprocal rather than
// with the IEEE-rounded library exp and division, which cost about three
// times the instructions.
//
// skip (nullable): rows whose flag is set were already done by the GMM1
// kernel's last round and are left as they are.
// prow (nullable): q2 is written in the row-paired layout that GMM2 reads
// (GmmParams::a_pair): row r goes to paired row prow[r], whose 64-byte K
// slices sit 128 bytes apart beside those of its pair.
#include "common.hpp"
#include "kernels.hpp"
#include "swiglu_row.hpp"

namespace megamoe {

constexpr int kRowsPerBlock = 4;

template <int MAXC>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void swiglu_quant_kernel(
    const uint16_t *__restrict__ gmC, const float *__restrict__ pts1,
    const int32_t *__restrict__ expert_cumsum, int R, int E, int I, int8_t *__restrict__ q2,
    float *__restrict__ pts2, const uint8_t *__restrict__ skip,
    const int32_t *__restrict__ prow) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= R) return;  // wave-uniform; gmC and pts1 hold R rows
    if (skip && skip[row]) return;
    uint4 uraw[MAXC], graw[MAXC];
    swiglu_row_load<MAXC>(gmC + (size_t)row * (2 * I), I, lane, uraw, graw);
    const float p1 = pts1[row];
    const int prow_r = prow ? prow[row] : 0;
    if (row >= expert_cumsum[E - 1]) return;  // only valid rows carry data
    int8_t *qrow = prow ? q2 + (size_t)(prow_r >> 1) * (2 * I) + (prow_r & 1) * 64
                        : q2 + (size_t)row * I;
    swiglu_row_finish<MAXC>(uraw, graw, p1, I, lane, qrow, prow ? 128 : 64, pts2 + row);
}

hipError_t launch_swiglu_quant(const uint16_t *gmC, const float *pts1,
                               const int32_t *expert_cumsum, int R, int E, int I, int8_t *q2,
                               float *pts2, hipStream_t stream, const uint8_t *skip,
                               const int32_t *prow) {
    const int per_lane = (I / 8 + kWave - 1) / kWave;  // I <= 16384: at most 32
    dim3 grid((R + kRowsPerBlock - 1) / kRowsPerBlock), block(kRowsPerBlock * kWave);
#define MEGAMOE_SWIGLU(C)                                                                 \
    hipLaunchKernelGGL(swiglu_quant_kernel<C>, grid, block, 0, stream, gmC, pts1, expert_cumsum, \
                       R, E, I, q2, pts2, skip, prow)
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
