// Combine (one rank) + Unpermute.
//
// Sections 6 and 7 of the pto-isa MegaMoE overview page.  Combine dequantises
// a GMM2 output row with its perTokenScale2 and casts it to the output element
// type (bfloat16 here); Unpermute gathers, for each token, the rows of its
// top-k routes through expandedRowIdx, weights them by probs and accumulates
// in fp32 (slots in order, multiply then add), then rounds to the output type.
// With one rank the combine's store-and-reload collapses into registers.
//
// The page found fp32 atomics slower than a gather for this step; this kernel
// is a pure gather: each thread owns 8 output columns of one token and reads
// the matching 16 bytes of every slot's row.  Slots are handled in batches of
// 8: the batch's row indices, scales and row chunks are all requested before
// any is used, so a token costs two memory round trips per batch instead of
// two per slot; the sum still runs over the slots in order.
#include "common.hpp"
#include "kernels.hpp"

namespace megamoe {

constexpr int kSlotBatch = 8;

__global__ __launch_bounds__(256) void unpermute_kernel(
    const uint16_t *__restrict__ gmm2_out, const float *__restrict__ pts2,
    const int32_t *__restrict__ expanded_row_idx, const float *__restrict__ probs, int K,
    int top_k, uint16_t *__restrict__ out) {
    const int t = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;  // 8-column chunk
    if (c * 8 >= K) return;
    const int32_t *rows = expanded_row_idx + (size_t)t * top_k;
    const float *pr = probs + (size_t)t * top_k;

    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;

    for (int s0 = 0; s0 < top_k; s0 += kSlotBatch) {
        int d[kSlotBatch];
        float p[kSlotBatch], sc[kSlotBatch];
        uint4 raw[kSlotBatch];
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
            const bool in = s0 + u < top_k;
            d[u] = in ? rows[s0 + u] : -1;
            p[u] = in ? pr[s0 + u] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
            if (d[u] >= 0) {  // d < 0: dropped route or past top_k
                sc[u] = pts2[d[u]];
                // each GMM2 row is read once: non-temporal
                raw[u] = load_nt16(gmm2_out + (size_t)d[u] * K + c * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
            if (d[u] < 0) continue;
            const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[u]);
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                // fp32(g) * scale as an FMA with a +0 addend, so that the
                // hardware reads the fp16 value in the same instruction: the
                // same rounded product, except that -0 becomes +0, and the sum
                // below starts at +0, so that changes no result
                const float g0 = __builtin_fmaf(h2f((uint16_t)(w[j >> 1] & 0xffffu)), sc[u], 0.0f);
                const float g1 = __builtin_fmaf(h2f((uint16_t)(w[j >> 1] >> 16)), sc[u], 0.0f);
                // combine: cast the dequantised row to the output type
                const uint32_t deq = f2bf_pk(g0, g1);
                acc[j] = acc[j] + bf2f_lo(deq) * p[u];
                acc[j + 1] = acc[j + 1] + bf2f_hi(deq) * p[u];
            }
        }
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f2bf_pk(acc[2 * j], acc[2 * j + 1]);
    store_nt16(out + (size_t)t * K + c * 8, make_uint4(o[0], o[1], o[2], o[3]));
}

hipError_t launch_unpermute(const uint16_t *gmm2_out, const float *pts2,
                            const int32_t *expanded_row_idx, const float *probs, int M, int K,
                            int top_k, uint16_t *out, hipStream_t stream) {
    dim3 grid(M, (K / 8 + 255) / 256), block(256);
    hipLaunchKernelGGL(unpermute_kernel, grid, block, 0, stream, gmm2_out, pts2, expanded_row_idx,
                       probs, K, top_k, out);
    return hipGetLastError();
}

}  // namespace megamoe
