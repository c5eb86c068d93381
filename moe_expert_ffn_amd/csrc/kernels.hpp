// Internal launch interface between the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace megamoe {

// K-split last round of the 256-row GEMM: at most kKsMaxTiles leftover tiles
// in 4 pieces, whose int32 partial tiles take at most 256 KB each; one
// counter per tile
constexpr int kKsMaxTiles = 64;
constexpr int kKsCounters = kKsMaxTiles;
constexpr size_t kKsPartBytes = 256 * 256 * 4;
// words of the forward's sync array: 3 for SwiGLU in GMM1's last round, then
// the K-split counters; the permute zeroes them
constexpr int kSyncWords = 3 + kKsCounters;

struct GmmParams {
    const int8_t *A;          // [rows, Kred] expert-major activations
    const int8_t *B;          // packed weights [E][N][Kred]
    const float *scale;       // [E][N] per-output-channel dequant scale
    const int32_t *cumsum;    // [E] inclusive row prefix over experts
    uint16_t *C;              // [rows, N] fp16
    int32_t *acc_dbg;         // nullable [rows, N] int32 accumulators
    int E, N, Kred;
    // nullable: A row d is read from row a_route[d] / a_div of A (a token-major
    // A gathered through the sorted route list)
    const int32_t *a_route = nullptr;
    int a_div = 1;
    // GMM1 only, nullable tail_q2 = off: workgroups left without a tile in a
    // sparse last round run SwiGLU on the rows that are already complete
    // (see gmm.hip).  tail_sync and tail_done must be zero at launch.
    int8_t *tail_q2 = nullptr;        // [R, tail_I] int8
    float *tail_pts2 = nullptr;       // [R]
    const float *tail_pts1 = nullptr; // [R]
    uint32_t *tail_sync = nullptr;    // [kSyncWords]: 3 counters of the last-round SwiGLU
    uint8_t *tail_done = nullptr;     // [R] set for each row the last round did
    int tail_I = 0;
    int tail_spin = 0;                // poll limit of the wait; < 0: give up at once
    const int32_t *tail_prow = nullptr;  // nullable: q2 row-paired (see a_pair), row r at tail_prow[r]
    // GMM1 of the forward, nullable: a sparse last round's leftover
    // tiles are split over K instead of into row pieces (see gmm.hip).
    // ks_part holds kKsMaxTiles x 4 int32 partial tiles (kKsPartBytes each);
    // ks_count kKsCounters counters, zero at launch (the kernel leaves them
    // at zero).
    int32_t *ks_part = nullptr;
    uint32_t *ks_count = nullptr;
    // A in the row-paired layout (GEMMs without a_route): every expert's group
    // is padded to an even row count, and padded rows 2m and 2m + 1 share each
    // 128-byte line, [Rp / 2][Kred / 64][2][64] bytes.  A copy instruction of
    // the K loop then reads 8 whole lines instead of 16 half lines.
    int a_pair = 0;
};

// block_counts: device scratch of route_sort_workspace_bytes(R, E) bytes
size_t route_sort_workspace_bytes(int R, int E);
hipError_t launch_route_sort(const int32_t *expert_idx, int R, int E, int32_t *sorted_route,
                             int32_t *expanded_row_idx, int32_t *tokens_per_expert,
                             int32_t *expert_cumsum, int32_t *err_word, int32_t *block_counts,
                             hipStream_t stream);
// prow (nullable, forward only): prow[row] = row + the number of experts before
// the row's expert with an odd row count, the row's place in the row-paired
// layout of q2 (see GmmParams::a_pair), written with the sort.
// Route sort and quant scatter in one launch, for R <= 8192 and top_k <= 16
// (permute_fused_ok); same outputs as launch_route_sort + launch_quant_scatter.
bool permute_fused_ok(int R, int top_k);
// token_major: the quantised tokens go to gmA rows 0..M-1 (row t = token t)
// instead of to every route's row; pts1 is still written per route row.
hipError_t launch_permute_fused(const uint16_t *x, const int32_t *expert_idx, int M, int K, int E,
                                int top_k, int8_t *gmA, float *pts1, int32_t *expanded_row_idx,
                                int32_t *sorted_route, int32_t *tokens_per_expert,
                                int32_t *expert_cumsum, int32_t *err_word, bool token_major,
                                hipStream_t stream, uint8_t *tail_done = nullptr,
                                uint32_t *tail_sync = nullptr, int32_t *prow = nullptr);
// The forward's permute for route counts beyond the one-launch path: the
// route counts and the token-major quantisation in one launch (per-token
// scales to tscale [M]), then the scatter pass, which also writes pts1.
hipError_t launch_permute_tokens_2pass(const uint16_t *x, const int32_t *expert_idx, int M, int K,
                                       int E, int top_k, int8_t *qx, float *pts1,
                                       int32_t *expanded_row_idx, int32_t *sorted_route,
                                       int32_t *tokens_per_expert, int32_t *expert_cumsum,
                                       int32_t *err_word, int32_t *block_counts, float *tscale,
                                       hipStream_t stream, uint8_t *tail_done = nullptr,
                                       uint32_t *tail_sync = nullptr, int32_t *prow = nullptr);
hipError_t launch_quant_scatter(const uint16_t *x, const int32_t *expanded_row_idx, int M, int K,
                                int top_k, int8_t *gmA, float *pts1, bool token_major,
                                hipStream_t stream);
// prow (nullable): q2 in the row-paired layout, row r at paired row prow[r]
// (see GmmParams::a_pair); else q2 is [R, I] row-major.
hipError_t launch_swiglu_quant(const uint16_t *gmC, const float *pts1,
                               const int32_t *expert_cumsum, int R, int E, int I, int8_t *q2,
                               float *pts2, hipStream_t stream, const uint8_t *skip = nullptr,
                               const int32_t *prow = nullptr);
hipError_t launch_unpermute(const uint16_t *gmm2_out, const float *pts2,
                            const int32_t *expanded_row_idx, const float *probs, int M, int K,
                            int top_k, uint16_t *out, hipStream_t stream);
// Weight pack into the GEMM's K-slice-major layout; packed_weight_bytes is
// its size for E experts of a logical [Kred][N] weight.
size_t packed_weight_bytes(int E, int Kred, int N);
hipError_t launch_pack(const int8_t *w, int8_t *wp, int E, int Kred, int N, hipStream_t stream);
int gmm_pick_variant(int R, int E);
// whether GMM1 at these dims can run SwiGLU in its last round (GmmParams tail_*)
bool gmm_tail_ok(int R, int E, int I);
hipError_t launch_gmm(int variant, const GmmParams &prm, int R, int cu_count, hipStream_t stream);

}  // namespace megamoe
