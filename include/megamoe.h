/*
 * megamoe.h -- C ABI of the MI355X (gfx950) MegaMoE expert pipeline, one rank.
 *
 * The pipeline is the one described on the "pto-isa MegaMoE operator" overview
 * page (pto-isa, kernels/manual/a2a3/dispatch_mega_combine), stage overview
 * and sections 1-7: FrontReorder -> (Dispatch) -> GMM1 -> SwiGLU -> GMM2 ->
 * (Combine) -> Unpermute.  With a single rank, Dispatch is the identity (the
 * quantised rows go straight into the A operand of GMM1) and Combine's remote
 * store becomes the dequant-and-cast that Unpermute applies in registers.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronises on the forward path; all work is
 *    enqueued in order on `stream` (a hipStream_t; NULL = default stream).
 *  - Tensors are dense, row-major, and 16-byte aligned.
 *  - fp16 and bf16 tensors are passed as uint16_t bit patterns.
 *  - Routes are numbered r = t * top_k + s (token t, slot s).  R = M * top_k.
 *  - Argument errors are reported synchronously by the return code and leave
 *    nothing enqueued.  A kernel launch failure returns MEGAMOE_EHIP.
 *  - Expert ids outside [0, E) cannot be checked without a device sync: such
 *    a route is dropped (expanded_row_idx = -1, not counted, skipped by the
 *    combine) and counted in a device error word kept in the workspace, which
 *    megamoe_last_error() reads.
 *  - The library is reentrant: calls with distinct buffers may run on
 *    distinct streams concurrently.
 *
 * Shape limits (checked): 1 <= M; 1 <= top_k <= E <= 256; K % 128 == 0,
 * 128 <= K <= 32768; I % 128 == 0, 128 <= I <= 16384; R * max(K, 2I) < 2^31.
 */
#ifndef MEGAMOE_H_
#define MEGAMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MEGAMOE_OK = 0,
    MEGAMOE_EINVAL = 1,        /* bad pointer, bad dims, misaligned tensor   */
    MEGAMOE_EUNSUPPORTED = 2,  /* dims outside the supported limits          */
    MEGAMOE_EWORKSPACE = 3,    /* workspace smaller than required            */
    MEGAMOE_EHIP = 4,          /* a HIP runtime call or launch failed        */
    MEGAMOE_EDEVICE = 5        /* megamoe_last_error: the device dropped routes
                                  (expert id outside [0, E))                */
} megamoe_status;

/* M tokens, hidden size K, E local experts, top_k routes per token, and the
 * SwiGLU output width I (GMM1 produces N = 2I columns: [0, I) go through
 * silu and [I, 2I) are the gate; GMM2 reduces over I back to K). */
typedef struct {
    int32_t M, K, E, top_k, I;
} megamoe_dims;

/* Human-readable text of a status code (static storage).  Library plumbing:
 * the page defines the stages, not an API. */
const char *megamoe_strerror(int status);

/* Validates dims against the shape limits.  Returns MEGAMOE_OK or an error. */
int megamoe_check_dims(const megamoe_dims *d);

/* Bytes of workspace megamoe_forward needs: the intermediates the page's
 * stage overview passes from stage to stage (the FrontReorder metadata and
 * per-token scales of section 1, GMM1's fp16 output of section 3, SwiGLU's
 * int8 rows and scales of section 4, GMM2's output of section 5) plus the
 * device error word and GMM1's partial tiles for a last round split over K
 * (megamoe_gmm1_gather_split).  megamoe_permute needs only
 * megamoe_permute_workspace_bytes (error word, sort scratch). */
int megamoe_workspace_bytes(const megamoe_dims *d, size_t *bytes);
int megamoe_permute_workspace_bytes(const megamoe_dims *d, size_t *bytes);

/* Bytes of the packed weights.  The packed layout is private to the library;
 * callers only allocate it and pass it back. */
int megamoe_packed_weight_bytes(const megamoe_dims *d, size_t *w1p_bytes, size_t *w2p_bytes);

/* One-time weight layout transform (the pages feed GMM1/GMM2 from pre-packed
 * weights; see sections 3 and 5).
 *   w1  int8 [E, K, 2I]  logical GMM1 weight (column n of expert e = w1[e, :, n])
 *   w2  int8 [E, I, K]   logical GMM2 weight
 * Output buffers must be megamoe_packed_weight_bytes() long. */
int megamoe_prepack_w1(const megamoe_dims *d, const int8_t *w1, int8_t *w1p, void *stream);
int megamoe_prepack_w2(const megamoe_dims *d, const int8_t *w2, int8_t *w2p, void *stream);

/* The whole forward (stage overview of the page):
 *   x          fp16  [M, K]
 *   expert_idx int32 [M, top_k]
 *   probs      fp32  [M, top_k]   combine weights, used as given
 *   w1p/w2p    packed weights from megamoe_prepack_w1/_w2
 *   scale1     fp32  [E, 2I]      GMM1 per-output-channel dequant scale
 *   scale2     fp32  [E, K]       GMM2 per-output-channel dequant scale
 *   out        bf16  [M, K]
 *   workspace  >= megamoe_workspace_bytes(); the caller may not touch it while
 *              the forward runs.  Intermediates live there.
 * It runs megamoe_permute_tokens_paired, megamoe_gmm1_gather_split,
 * megamoe_swiglu_quant_paired, megamoe_gmm2_paired and megamoe_unpermute in
 * order on the workspace (SwiGLU can start inside GMM1's last round, see
 * megamoe_set_overlap); the result equals, bit for bit, that of the page's
 * five stages (megamoe_permute, megamoe_gmm1, megamoe_swiglu_quant,
 * megamoe_gmm2, megamoe_unpermute). */
int megamoe_forward(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                    const float *probs, const int8_t *w1p, const float *scale1,
                    const int8_t *w2p, const float *scale2, uint16_t *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Stage 1 FrontReorder (+ identity Dispatch), section 1 of the page:
 * stable expert-major sort of the routes (ties keep ascending route order),
 * per-expert counts, inclusive prefix over experts, inverse map, and the
 * per-token dynamic int8 quantisation scattered to every route's row.
 *   gmA               int8  [R, K]  expert-major rows; rows >= valid count unused
 *   pts1              fp32  [R]     perTokenScale1 of each row
 *   expanded_row_idx  int32 [R]     route -> row, -1 for a dropped route
 *   sorted_route      int32 [R]     row -> route, -1 past the valid rows
 *   tokens_per_expert int32 [E]
 *   expert_cumsum     int32 [E]     inclusive prefix of tokens_per_expert
 *   workspace         >= megamoe_permute_workspace_bytes() (error word) */
int megamoe_permute(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                    int8_t *gmA, float *pts1, int32_t *expanded_row_idx, int32_t *sorted_route,
                    int32_t *tokens_per_expert, int32_t *expert_cumsum, void *workspace,
                    size_t workspace_bytes, void *stream);

/* megamoe_permute for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same outputs as megamoe_permute, with no
 * workspace.  The sort's per-block count table lives in a static device array
 * of 256 KiB that the library holds per GPU until the process ends, so every
 * shape megamoe_check_dims accepts fits; a larger table would be rejected with
 * MEGAMOE_EUNSUPPORTED.  The call allocates nothing.
 *   dropped  int32 [1] (device, 16-byte aligned): the number of routes whose
 *            expert id lies outside [0, E), written by this call (the value
 *            megamoe_last_error reports for the workspace variants).
 * All calls on one GPU share that array: calls that overlap in time on one GPU
 * (concurrent streams) race and must be serialised by the caller. */
int megamoe_permute_noalloc(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                            int8_t *gmA, float *pts1, int32_t *expanded_row_idx,
                            int32_t *sorted_route, int32_t *tokens_per_expert,
                            int32_t *expert_cumsum, int32_t *dropped, void *stream);

/* Stage 1 as megamoe_forward runs it: the same sort outputs and pts1 as
 * megamoe_permute, but each token's quantised row is written once,
 * token-major, instead of to every route's row:
 *   qx  int8 [M, K]   qx[t] = the int8 row of token t; gmA[row] of
 *                     megamoe_permute equals qx[sorted_route[row] / top_k]
 * The other arguments are those of megamoe_permute. */
int megamoe_permute_tokens(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                           int8_t *qx, float *pts1, int32_t *expanded_row_idx,
                           int32_t *sorted_route, int32_t *tokens_per_expert,
                           int32_t *expert_cumsum, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Stage 3 GMM1, section 3: for every row of expert e's group,
 *   acc[row, n] = sum_k gmA[row, k] * w1[e, k, n]   (int32, exact)
 *   gmC[row, n] = fp16(fp32(acc) * scale1[e, n])
 * Groups are taken from expert_cumsum (device).  gmC fp16 [R, 2I].
 * acc_dbg (nullable) receives the int32 accumulators [R, 2I]. */
int megamoe_gmm1(const megamoe_dims *d, const int8_t *gmA, const int32_t *expert_cumsum,
                 const int8_t *w1p, const float *scale1, uint16_t *gmC, int32_t *acc_dbg,
                 void *stream);

/* GMM1 as megamoe_forward runs it: the A row of sorted row `row` is read
 * from qx[sorted_route[row] / top_k] (qx from megamoe_permute_tokens), so the
 * expert-sorted gmA is never materialised.  Results equal those of
 * megamoe_gmm1 on that gmA bit for bit.
 *   qx            int8  [M, K]
 *   sorted_route  int32 [R]    from the same permute call
 * The other arguments are those of megamoe_gmm1. */
int megamoe_gmm1_gather(const megamoe_dims *d, const int8_t *qx, const int32_t *sorted_route,
                        const int32_t *expert_cumsum, const int8_t *w1p, const float *scale1,
                        uint16_t *gmC, int32_t *acc_dbg, void *stream);

/* megamoe_gmm1_gather as megamoe_forward runs it, with a buffer for the
 * GEMM's sparse last round: when fewer tiles are left for the last round
 * than groups of four workgroups are idle, each leftover tile is multiplied
 * by four workgroups over a quarter of K each, and the last of them adds the
 * four int32 partial tiles (an exact integer sum, section 3's acc) and stores
 * the tile.  Results equal megamoe_gmm1_gather's bit for bit.
 *   megamoe_gmm1_split_workspace_bytes: size of split_ws (about 67 MB).
 *   split_ws  device, zero-filled before its first use; each call leaves it
 *             ready for the next (its counters back at zero).  Calls that
 *             overlap in time on one split_ws race; give concurrent streams
 *             a buffer each.
 * The other arguments are those of megamoe_gmm1_gather (no acc_dbg). */
int megamoe_gmm1_split_workspace_bytes(const megamoe_dims *d, size_t *bytes);
int megamoe_gmm1_gather_split(const megamoe_dims *d, const int8_t *qx,
                              const int32_t *sorted_route, const int32_t *expert_cumsum,
                              const int8_t *w1p, const float *scale1, uint16_t *gmC,
                              void *split_ws, size_t split_ws_bytes, void *stream);

/* The forward's SwiGLU -> GMM2 hand-off, as stage entry points (for timing
 * the forward stage by stage and for tests): q2 in a row-paired layout.
 * Each expert's rows are padded to an even count, and padded rows 2m and
 * 2m + 1 share every 128-byte line: row r's 64-byte K slice s sits at byte
 * ((prow[r] >> 1) * (I / 64) + s) * 128 + (prow[r] & 1) * 64 of q2p, where
 * prow[r] = r + the number of experts before r's expert with an odd row
 * count.  GMM2's A copies then read whole lines instead of half lines
 * (section 5's GMM2 reads the same values; only where they lie differs).
 *   megamoe_paired_q2_bytes: size of q2p.
 *   megamoe_permute_tokens_paired: megamoe_permute_tokens, plus prow int32 [R]
 *     (valid rows only).
 *   megamoe_swiglu_quant_paired: megamoe_swiglu_quant writing q2p.
 *   megamoe_gmm2_paired: megamoe_gmm2 reading q2p; results equal those of
 *     megamoe_gmm2 on the row-major q2 bit for bit. */
int megamoe_paired_q2_bytes(const megamoe_dims *d, size_t *bytes);
int megamoe_permute_tokens_paired(const megamoe_dims *d, const uint16_t *x,
                                  const int32_t *expert_idx, int8_t *qx, float *pts1,
                                  int32_t *expanded_row_idx, int32_t *sorted_route,
                                  int32_t *tokens_per_expert, int32_t *expert_cumsum,
                                  int32_t *prow, void *workspace, size_t workspace_bytes,
                                  void *stream);
int megamoe_swiglu_quant_paired(const megamoe_dims *d, const uint16_t *gmC, const float *pts1,
                                const int32_t *expert_cumsum, const int32_t *prow, int8_t *q2p,
                                float *pts2, void *stream);
int megamoe_gmm2_paired(const megamoe_dims *d, const int8_t *q2p, const int32_t *expert_cumsum,
                        const int8_t *w2p, const float *scale2, uint16_t *gmm2_out,
                        int32_t *acc_dbg, void *stream);

/* Stage 4 SwiGLU, section 4: per valid row,
 *   c = fp32(gmC) * pts1;  y = silu(c[0:I]) * c[I:2I];  pts2 = max|y| / 127;
 *   q2 = rint(y * (127 / max|y|))  (int8)
 * Valid rows are [0, expert_cumsum[E-1]).  q2 int8 [R, I], pts2 fp32 [R].
 * silu(u) = u / (1 + exp(-u)) is evaluated with the hardware base-2 exponential
 * and reciprocal plus one correction of the quotient, a few ulp from the IEEE
 * expression; on every row of the decode, mid, large and skewed workloads each
 * q2 code and pts2 equals the one from IEEE exp and division. */
int megamoe_swiglu_quant(const megamoe_dims *d, const uint16_t *gmC, const float *pts1,
                         const int32_t *expert_cumsum, int8_t *q2, float *pts2, void *stream);

/* Stage 5 GMM2, section 5:
 *   acc[row, k] = sum_i q2[row, i] * w2[e, i, k];  gmm2_out = fp16(fp32(acc) * scale2[e, k])
 * gmm2_out fp16 [R, K]; acc_dbg (nullable) int32 [R, K]. */
int megamoe_gmm2(const megamoe_dims *d, const int8_t *q2, const int32_t *expert_cumsum,
                 const int8_t *w2p, const float *scale2, uint16_t *gmm2_out, int32_t *acc_dbg,
                 void *stream);

/* Stages 6-7 Combine (one rank) + Unpermute, sections 6 and 7: for token t,
 *   out[t, k] = bf16( sum_s bf16(fp32(gmm2_out[row_s, k]) * pts2[row_s]) * probs[t, s] )
 * with row_s = expanded_row_idx[t * top_k + s], slots in order, fp32
 * accumulation, rows < 0 skipped.  out bf16 [M, K]. */
int megamoe_unpermute(const megamoe_dims *d, const uint16_t *gmm2_out, const float *pts2,
                      const int32_t *expanded_row_idx, const float *probs, uint16_t *out,
                      void *stream);

/* How megamoe_forward runs SwiGLU (the page's overlap of the vector stage with
 * the matrix stages, "PTO-ISA overlap scheme" and section 4's SwiGLU segments).
 *   0 (default): GMM1, then SwiGLU on every row;
 *   1: when GMM1 has at least two full rounds of tiles and a sparse last one,
 *      the workgroups left without a tile in the last round run SwiGLU on the
 *      rows whose GMM1 output was complete two rounds earlier, until the
 *      last-round tiles are done; the SwiGLU kernel does the remaining rows;
 *   2: as 1, but every workgroup that would wait for the other workgroups
 *      gives up at once, so the SwiGLU kernel does every row (that path).
 * On MI355X mode 1 is slower than mode 0 at every workload measured, hence
 * the default.  The result is bit-identical in all three modes.  The setting
 * is global to the process and read when megamoe_forward enqueues its work.
 * Returns MEGAMOE_EINVAL for any other mode. */
int megamoe_set_overlap(int mode);

/* Synchronises `stream` and reads the number of routes dropped by the last
 * megamoe_permute / megamoe_forward that used this workspace: routes whose
 * expert id lies outside [0, E).  FrontReorder (section 1) sorts them past
 * every expert's rows with expanded_row_idx = -1, and the combine of
 * section 7 skips them, as the page's unpermute combines only valid expanded
 * rows.  Returns MEGAMOE_OK when none was dropped, MEGAMOE_EDEVICE (with the
 * count written) when some were, MEGAMOE_EINVAL or MEGAMOE_EHIP otherwise. */
int megamoe_last_error(const void *workspace, void *stream, int32_t *bad_route_count);

#ifdef __cplusplus
}
#endif

#endif /* MEGAMOE_H_ */
