// Matrix-core rate probe (measurement only; no part of the MegaMoE path).
//
// Every wave of a full grid (workgroups of 1024 threads, 16 waves per CU: the
// GEMM's occupancy) issues back-to-back v_mfma_i32_16x16x64_i8 on a 4 x 4 set
// of 16x16 accumulators -- the wave tile of the grouped GEMM -- with operands
// held in registers, so no memory traffic, LDS access or barrier is involved.
// Operands come from a caller buffer: random int8 values reproduce the
// switching activity of the GEMMs' data, all-zero values give the same
// instruction stream with no data toggling.  Each workgroup records its
// shader-clock cycles (s_memtime) and constant 100 MHz reference ticks
// (s_memrealtime) around the loop, from which the host derives the shader
// clock under this load.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void mfma_rate_kernel(const int32_t *__restrict__ operands,
                                                        int n_words, int iters,
                                                        int64_t *__restrict__ ticks,
                                                        int32_t *__restrict__ sink) {
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            a[i][v] = operands[(gid * 32 + i * 4 + v) % n_words];
            b[i][v] = operands[(gid * 32 + 16 + i * 4 + v) % n_words];
        }
    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    __syncthreads();
    const int64_t c0 = (int64_t)__builtin_readcyclecounter();
    const int64_t r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    const int64_t c1 = (int64_t)__builtin_readcyclecounter();
    const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s ^= acc[i][j][0] ^ acc[i][j][1] ^ acc[i][j][2] ^ acc[i][j][3];
    sink[gid] = s;
    if (threadIdx.x == 0) {
        ticks[2 * blockIdx.x] = c1 - c0;
        ticks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

// operands: n_words int32 words (device); ticks: 2 * blocks int64 (device);
// sink: blocks * 1024 int32 (device).  Each wave performs iters * 16 MFMAs of
// 32768 int8 operations.  Returns 0 or the HIP error code.
extern "C" int megamoe_probe_mfma_rate(const int32_t *operands, int n_words, int iters, int blocks,
                                       int64_t *ticks, int32_t *sink, void *stream) {
    if (!operands || n_words < 1 || iters < 1 || blocks < 1 || !ticks || !sink) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(1024), 0, (hipStream_t)stream,
                       operands, n_words, iters, ticks, sink);
    return (int)hipGetLastError();
}
