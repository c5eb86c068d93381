// Host side of the MegaMoE C ABI: argument checks, workspace carving and the
// launch order of the stages on one stream.  The order is the stage overview
// of the pto-isa MegaMoE overview page: FrontReorder, (Dispatch), GMM1,
// SwiGLU, GMM2, (Combine), Unpermute.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/megamoe.h"
#include "kernels.hpp"


using namespace megamoe;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kErrBytes = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The four large intermediates start on 2 MiB boundaries, as separate device
// allocations of their size would.
constexpr size_t kBigAlign = 2u << 20;
size_t align_big(size_t v) { return (v + kBigAlign - 1) / kBigAlign * kBigAlign; }

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

// CU count of the current device, queried once per device.  It only sizes the
// persistent GEMM grid, so a failed query falls back to MI355X's 256.  The
// cache is filled with relaxed atomics: concurrent first calls store the same
// value.
int cu_count_current() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Scratch of megamoe_permute_noalloc: the sort's per-block expert counts.
// The sort uses at most 256 blocks of routes and at most 256 experts, so
// 256 x 256 counts cover every shape megamoe_check_dims accepts.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name `scratch` is only a stand-in for the symbol: its device address
// comes from hipGetSymbolAddress (scratch_device_ptr below).
constexpr size_t kNoAllocScratchBytes = 256u * 256u * sizeof(int32_t);
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

// Device address of `scratch` on the current device, looked up once per
// device with that device current (concurrent first calls store the same
// value).  nullptr if the HIP calls fail.
int32_t *scratch_device_ptr() {
    static std::atomic<int32_t *> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    int32_t *p = cached[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
            return nullptr;
        p = static_cast<int32_t *>(addr);
        cached[dev].store(p, std::memory_order_release);
    }
    return p;
}

struct Layout {
    size_t err, bcnt, tscale, tsync, tdone, eri, sorted, counts, cumsum, pts1, pts2, prow, gmA,
        gmC, q2, g2, ks, total;
};

// permute workspace: error word, the sort's per-block expert counts, then the
// per-token scales of the token-major path
size_t permute_ws_bytes(const megamoe_dims &d) {
    return align_up(kErrBytes) + align_up(route_sort_workspace_bytes(d.M * d.top_k, d.E)) +
           align_up((size_t)d.M * 4);
}

// GMM1's K-split buffer (megamoe_gmm1_gather_split): the tile counters, then
// the partial tiles
constexpr size_t kSplitCountBytes = (kKsCounters * 4 + 255) / 256 * 256;
size_t split_ws_bytes() { return kSplitCountBytes + (size_t)kKsMaxTiles * 4 * kKsPartBytes; }

// bytes of q2 in the row-paired layout: each expert's rows padded to an even
// count, at most R + E rows
size_t paired_q2_bytes(const megamoe_dims &d) {
    return ((size_t)d.M * d.top_k + d.E + 1) * d.I;
}

Layout forward_layout(const megamoe_dims &d) {
    const size_t R = (size_t)d.M * d.top_k;
    Layout L;
    size_t o = 0;
    L.err = o;    o += align_up(kErrBytes);
    L.bcnt = o;   o += align_up(route_sort_workspace_bytes((int)R, d.E));
    L.tscale = o; o += align_up((size_t)d.M * 4);
    L.tsync = o;  o += align_up(kSyncWords * 4);
    L.tdone = o;  o += align_up(R);
    L.eri = o;    o += align_up(R * 4);
    L.sorted = o; o += align_up(R * 4);
    L.counts = o; o += align_up((size_t)d.E * 4);
    L.cumsum = o; o += align_up((size_t)d.E * 4);
    L.pts1 = o;   o += align_up(R * 4);
    L.pts2 = o;   o += align_up(R * 4);
    L.prow = o;   o += align_up(R * 4);
    o = align_big(o);
    L.gmA = o;    o = align_big(o + (size_t)d.M * d.K);   // token-major quantised x
    L.gmC = o;    o = align_big(o + R * 2 * d.I * 2);
    // q2, row-paired when GMM2 uses the 256-row tiles: each expert's rows are
    // padded to an even count, at most R + E rows
    L.q2 = o;     o = align_big(o + paired_q2_bytes(d));
    L.g2 = o;     o = align_big(o + R * d.K * 2);
    // GMM1's partial tiles when its sparse last round splits tiles over K
    L.ks = o;     o += (size_t)kKsMaxTiles * 4 * kKsPartBytes;
    L.total = o;
    return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MEGAMOE_OK : MEGAMOE_EHIP; }

#define MEGAMOE_TRY(expr)                         \
    do {                                          \
        const int _rc = (expr);                   \
        if (_rc != MEGAMOE_OK) return _rc;        \
    } while (0)

// token_major: gmA is [M, K] (row t = quantised token t) rather than the
// expert-sorted [R, K]; the fused forward reads it through the route list.
// tscale [M] (token_major only): scratch for the per-token scales when the
// quantisation runs beside the sort's first pass.
// tail_done / tail_sync (nullable, forward only): flags of the GMM1 that
// follows, cleared by the permute's kernels.
int run_permute(const megamoe_dims &d, const uint16_t *x, const int32_t *expert_idx, int8_t *gmA,
                float *pts1, int32_t *eri, int32_t *sorted, int32_t *counts, int32_t *cumsum,
                int32_t *err_word, int32_t *block_counts, bool token_major, hipStream_t s,
                float *tscale = nullptr, uint8_t *tail_done = nullptr,
                uint32_t *tail_sync = nullptr, int32_t *prow = nullptr) {
    const int R = d.M * d.top_k;
    if (permute_fused_ok(R, d.top_k))
        return hip_status(launch_permute_fused(x, expert_idx, d.M, d.K, d.E, d.top_k, gmA, pts1, eri,
                                               sorted, counts, cumsum, err_word, token_major, s,
                                               tail_done, tail_sync, prow));
    if (token_major && tscale)
        return hip_status(launch_permute_tokens_2pass(x, expert_idx, d.M, d.K, d.E, d.top_k, gmA,
                                                      pts1, eri, sorted, counts, cumsum, err_word,
                                                      block_counts, tscale, s, tail_done,
                                                      tail_sync, prow));
    MEGAMOE_TRY(hip_status(launch_route_sort(expert_idx, R, d.E, sorted, eri, counts, cumsum,
                                             err_word, block_counts, s)));
    return hip_status(
        launch_quant_scatter(x, eri, d.M, d.K, d.top_k, gmA, pts1, token_major, s));
}

// a_route (nullable): A row d is token a_route[d] / top_k of a token-major A.
// tail (nullable, GMM1 only): SwiGLU in GMM1's last round (tail_*) or the
// K-split last round (ks_*), see gmm.hip.
// a_pair: A is in the row-paired layout (GmmParams::a_pair).
int run_gmm(const megamoe_dims &d, const int8_t *A, const int32_t *cumsum, const int8_t *Bp,
            const float *scale, uint16_t *C, int32_t *dbg, int N, int Kred, hipStream_t s,
            const int32_t *a_route = nullptr, const GmmParams *tail = nullptr,
            bool a_pair = false) {
    const int R = d.M * d.top_k;
    GmmParams prm{A, Bp, scale, cumsum, C, dbg, d.E, N, Kred, a_route, d.top_k};
    prm.a_pair = a_pair ? 1 : 0;
    if (tail) {
        prm.tail_q2 = tail->tail_q2;
        prm.tail_pts2 = tail->tail_pts2;
        prm.tail_pts1 = tail->tail_pts1;
        prm.tail_sync = tail->tail_sync;
        prm.tail_done = tail->tail_done;
        prm.tail_I = tail->tail_I;
        prm.tail_spin = tail->tail_spin;
        prm.tail_prow = tail->tail_prow;
        prm.ks_part = tail->ks_part;
        prm.ks_count = tail->ks_count;
    }
    return hip_status(launch_gmm(gmm_pick_variant(R, d.E), prm, R, cu_count_current(), s));
}

// megamoe_set_overlap: 0 (default) GMM1 then SwiGLU; 1 SwiGLU overlaps
// GMM1's last round; 2 as 1, with every waiting workgroup giving up at once.
// Measured on MI355X the overlap is slower (the device-scope L2 write-back it
// needs, and its HBM traffic beside the last-round tiles, cost more than the
// SwiGLU time it hides), so it is off unless asked for.
std::atomic<int> g_overlap{0};
// poll limit of the wait (each poll is a device-scope load and a short
// sleep): a workgroup gives up after milliseconds, long after every resident
// workgroup has arrived (one tile takes at most a few hundred microseconds)
constexpr int kTailSpin = 8192;

int permute_entry(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                  int8_t *gmA, float *pts1, int32_t *eri, int32_t *sorted_route,
                  int32_t *tokens_per_expert, int32_t *expert_cumsum, void *ws, size_t ws_bytes,
                  bool token_major, void *stream, int32_t *prow = nullptr) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {x, expert_idx, gmA, pts1, eri, sorted_route, tokens_per_expert,
                          expert_cumsum, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (prow && !aligned16(prow)) return MEGAMOE_EINVAL;
    if (ws_bytes < permute_ws_bytes(*d)) return MEGAMOE_EWORKSPACE;
    char *w = (char *)ws;
    const size_t bcnt = align_up(kErrBytes);
    const size_t tsc = bcnt + align_up(route_sort_workspace_bytes(d->M * d->top_k, d->E));
    return run_permute(*d, x, expert_idx, gmA, pts1, eri, sorted_route, tokens_per_expert,
                       expert_cumsum, (int32_t *)w, (int32_t *)(w + bcnt), token_major,
                       (hipStream_t)stream, (float *)(w + tsc), nullptr, nullptr, prow);
}


}  // namespace

extern "C" {

const char *megamoe_strerror(int status) {
    switch (status) {
        case MEGAMOE_OK: return "ok";
        case MEGAMOE_EINVAL: return "invalid argument (null or misaligned pointer, bad dims)";
        case MEGAMOE_EUNSUPPORTED: return "dims outside the supported limits";
        case MEGAMOE_EWORKSPACE: return "workspace too small";
        case MEGAMOE_EHIP: return "HIP runtime or launch failure";
        case MEGAMOE_EDEVICE: return "routes with an expert id outside [0, E) were dropped";
        default: return "unknown status";
    }
}

int megamoe_check_dims(const megamoe_dims *d) {
    if (!d) return MEGAMOE_EINVAL;
    if (d->M < 1 || d->K < 1 || d->E < 1 || d->top_k < 1 || d->I < 1) return MEGAMOE_EINVAL;
    if (d->top_k > d->E || d->E > 256) return MEGAMOE_EUNSUPPORTED;
    if (d->K % 128 != 0 || d->K > 32768) return MEGAMOE_EUNSUPPORTED;
    if (d->I % 128 != 0 || d->I > 16384) return MEGAMOE_EUNSUPPORTED;
    const long long R = (long long)d->M * d->top_k;
    const long long wide = d->K > 2 * d->I ? d->K : 2 * d->I;
    if (R * wide >= (1ll << 31)) return MEGAMOE_EUNSUPPORTED;
    return MEGAMOE_OK;
}

int megamoe_workspace_bytes(const megamoe_dims *d, size_t *bytes) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!bytes) return MEGAMOE_EINVAL;
    *bytes = forward_layout(*d).total;
    return MEGAMOE_OK;
}

int megamoe_permute_workspace_bytes(const megamoe_dims *d, size_t *bytes) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!bytes) return MEGAMOE_EINVAL;
    *bytes = permute_ws_bytes(*d);
    return MEGAMOE_OK;
}

int megamoe_packed_weight_bytes(const megamoe_dims *d, size_t *w1p, size_t *w2p) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!w1p || !w2p) return MEGAMOE_EINVAL;
    *w1p = packed_weight_bytes(d->E, d->K, 2 * d->I);
    *w2p = packed_weight_bytes(d->E, d->I, d->K);
    return MEGAMOE_OK;
}

int megamoe_prepack_w1(const megamoe_dims *d, const int8_t *w1, int8_t *w1p, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!aligned16(w1) || !aligned16(w1p)) return MEGAMOE_EINVAL;
    return hip_status(launch_pack(w1, w1p, d->E, d->K, 2 * d->I, (hipStream_t)stream));
}

int megamoe_prepack_w2(const megamoe_dims *d, const int8_t *w2, int8_t *w2p, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!aligned16(w2) || !aligned16(w2p)) return MEGAMOE_EINVAL;
    return hip_status(launch_pack(w2, w2p, d->E, d->I, d->K, (hipStream_t)stream));
}

int megamoe_permute(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                    int8_t *gmA, float *pts1, int32_t *eri, int32_t *sorted_route,
                    int32_t *tokens_per_expert, int32_t *expert_cumsum, void *ws,
                    size_t ws_bytes, void *stream) {
    return permute_entry(d, x, expert_idx, gmA, pts1, eri, sorted_route, tokens_per_expert,
                         expert_cumsum, ws, ws_bytes, false, stream);
}

int megamoe_permute_noalloc(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                            int8_t *gmA, float *pts1, int32_t *eri, int32_t *sorted_route,
                            int32_t *tokens_per_expert, int32_t *expert_cumsum,
                            int32_t *dropped, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {x, expert_idx, gmA, pts1, eri, sorted_route, tokens_per_expert,
                          expert_cumsum, dropped};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (route_sort_workspace_bytes(d->M * d->top_k, d->E) > kNoAllocScratchBytes)
        return MEGAMOE_EUNSUPPORTED;
    int32_t *block_counts = scratch_device_ptr();
    if (block_counts == nullptr) return MEGAMOE_EHIP;
    // every count the sort reads is written by the same call first, so the
    // scratch needs no clearing between calls
    return run_permute(*d, x, expert_idx, gmA, pts1, eri, sorted_route, tokens_per_expert,
                       expert_cumsum, dropped, block_counts, false, (hipStream_t)stream);
}

int megamoe_permute_tokens(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                           int8_t *qx, float *pts1, int32_t *eri, int32_t *sorted_route,
                           int32_t *tokens_per_expert, int32_t *expert_cumsum, void *ws,
                           size_t ws_bytes, void *stream) {
    return permute_entry(d, x, expert_idx, qx, pts1, eri, sorted_route, tokens_per_expert,
                         expert_cumsum, ws, ws_bytes, true, stream);
}

int megamoe_gmm1(const megamoe_dims *d, const int8_t *gmA, const int32_t *expert_cumsum,
                 const int8_t *w1p, const float *scale1, uint16_t *gmC, int32_t *acc_dbg,
                 void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {gmA, expert_cumsum, w1p, scale1, gmC};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (acc_dbg && !aligned16(acc_dbg)) return MEGAMOE_EINVAL;
    return run_gmm(*d, gmA, expert_cumsum, w1p, scale1, gmC, acc_dbg, 2 * d->I, d->K,
                   (hipStream_t)stream);
}

int megamoe_gmm1_gather(const megamoe_dims *d, const int8_t *qx, const int32_t *sorted_route,
                        const int32_t *expert_cumsum, const int8_t *w1p, const float *scale1,
                        uint16_t *gmC, int32_t *acc_dbg, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {qx, sorted_route, expert_cumsum, w1p, scale1, gmC};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (acc_dbg && !aligned16(acc_dbg)) return MEGAMOE_EINVAL;
    return run_gmm(*d, qx, expert_cumsum, w1p, scale1, gmC, acc_dbg, 2 * d->I, d->K,
                   (hipStream_t)stream, sorted_route);
}

int megamoe_swiglu_quant(const megamoe_dims *d, const uint16_t *gmC, const float *pts1,
                         const int32_t *expert_cumsum, int8_t *q2, float *pts2, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {gmC, pts1, expert_cumsum, q2, pts2};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    return hip_status(launch_swiglu_quant(gmC, pts1, expert_cumsum, d->M * d->top_k, d->E, d->I,
                                          q2, pts2, (hipStream_t)stream));
}

int megamoe_gmm2(const megamoe_dims *d, const int8_t *q2, const int32_t *expert_cumsum,
                 const int8_t *w2p, const float *scale2, uint16_t *gmm2_out, int32_t *acc_dbg,
                 void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {q2, expert_cumsum, w2p, scale2, gmm2_out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (acc_dbg && !aligned16(acc_dbg)) return MEGAMOE_EINVAL;
    return run_gmm(*d, q2, expert_cumsum, w2p, scale2, gmm2_out, acc_dbg, d->K, d->I,
                   (hipStream_t)stream);
}

int megamoe_gmm1_split_workspace_bytes(const megamoe_dims *d, size_t *bytes) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!bytes) return MEGAMOE_EINVAL;
    *bytes = split_ws_bytes();
    return MEGAMOE_OK;
}

int megamoe_gmm1_gather_split(const megamoe_dims *d, const int8_t *qx,
                              const int32_t *sorted_route, const int32_t *expert_cumsum,
                              const int8_t *w1p, const float *scale1, uint16_t *gmC,
                              void *split_ws, size_t split_ws_bytes_, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {qx, sorted_route, expert_cumsum, w1p, scale1, gmC, split_ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (split_ws_bytes_ < split_ws_bytes()) return MEGAMOE_EWORKSPACE;
    GmmParams kp{};
    kp.ks_count = (uint32_t *)split_ws;
    kp.ks_part = (int32_t *)((char *)split_ws + kSplitCountBytes);
    return run_gmm(*d, qx, expert_cumsum, w1p, scale1, gmC, nullptr, 2 * d->I, d->K,
                   (hipStream_t)stream, sorted_route, &kp);
}

int megamoe_paired_q2_bytes(const megamoe_dims *d, size_t *bytes) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    if (!bytes) return MEGAMOE_EINVAL;
    *bytes = paired_q2_bytes(*d);
    return MEGAMOE_OK;
}

int megamoe_permute_tokens_paired(const megamoe_dims *d, const uint16_t *x,
                                  const int32_t *expert_idx, int8_t *qx, float *pts1,
                                  int32_t *eri, int32_t *sorted_route, int32_t *tokens_per_expert,
                                  int32_t *expert_cumsum, int32_t *prow, void *ws,
                                  size_t ws_bytes, void *stream) {
    if (!prow) return MEGAMOE_EINVAL;
    return permute_entry(d, x, expert_idx, qx, pts1, eri, sorted_route, tokens_per_expert,
                         expert_cumsum, ws, ws_bytes, true, stream, prow);
}

int megamoe_swiglu_quant_paired(const megamoe_dims *d, const uint16_t *gmC, const float *pts1,
                                const int32_t *expert_cumsum, const int32_t *prow, int8_t *q2p,
                                float *pts2, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {gmC, pts1, expert_cumsum, prow, q2p, pts2};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    return hip_status(launch_swiglu_quant(gmC, pts1, expert_cumsum, d->M * d->top_k, d->E, d->I,
                                          q2p, pts2, (hipStream_t)stream, nullptr, prow));
}

int megamoe_gmm2_paired(const megamoe_dims *d, const int8_t *q2p, const int32_t *expert_cumsum,
                        const int8_t *w2p, const float *scale2, uint16_t *gmm2_out,
                        int32_t *acc_dbg, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {q2p, expert_cumsum, w2p, scale2, gmm2_out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    if (acc_dbg && !aligned16(acc_dbg)) return MEGAMOE_EINVAL;
    return run_gmm(*d, q2p, expert_cumsum, w2p, scale2, gmm2_out, acc_dbg, d->K, d->I,
                   (hipStream_t)stream, nullptr, nullptr, true);
}

int megamoe_unpermute(const megamoe_dims *d, const uint16_t *gmm2_out, const float *pts2,
                      const int32_t *eri, const float *probs, uint16_t *out, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {gmm2_out, pts2, eri, probs, out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    return hip_status(launch_unpermute(gmm2_out, pts2, eri, probs, d->M, d->K, d->top_k, out,
                                       (hipStream_t)stream));
}

int megamoe_forward(const megamoe_dims *d, const uint16_t *x, const int32_t *expert_idx,
                    const float *probs, const int8_t *w1p, const float *scale1,
                    const int8_t *w2p, const float *scale2, uint16_t *out, void *ws,
                    size_t ws_bytes, void *stream) {
    MEGAMOE_TRY(megamoe_check_dims(d));
    const void *ptrs[] = {x, expert_idx, probs, w1p, scale1, w2p, scale2, out, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return MEGAMOE_EINVAL;
    const Layout L = forward_layout(*d);
    if (ws_bytes < L.total) return MEGAMOE_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *base = (char *)ws;
    int32_t *err = (int32_t *)(base + L.err);
    int32_t *eri = (int32_t *)(base + L.eri);
    int32_t *sorted = (int32_t *)(base + L.sorted);
    int32_t *counts = (int32_t *)(base + L.counts);
    int32_t *cumsum = (int32_t *)(base + L.cumsum);
    float *pts1 = (float *)(base + L.pts1);
    float *pts2 = (float *)(base + L.pts2);
    int8_t *gmA = (int8_t *)(base + L.gmA);
    uint16_t *gmC = (uint16_t *)(base + L.gmC);
    int8_t *q2 = (int8_t *)(base + L.q2);
    uint16_t *g2 = (uint16_t *)(base + L.g2);

    int32_t *bcnt = (int32_t *)(base + L.bcnt);
    uint32_t *tsync = (uint32_t *)(base + L.tsync);
    uint8_t *tdone = (uint8_t *)(base + L.tdone);
    const int R = d->M * d->top_k;
    const int overlap = g_overlap.load(std::memory_order_relaxed);
    const bool tail = overlap != 0 && gmm_tail_ok(R, d->E, d->I);
    // GMM2 reads q2 in the row-paired layout: the 64-byte K slices of two
    // rows share each 128-byte line, so its A copies read whole lines (the
    // sort writes each row's paired place to prow)
    int32_t *prow = (int32_t *)(base + L.prow);
    // the quantised tokens are written once, token-major; GMM1 gathers its
    // expert-sorted rows from them through the route list, so the top_k
    // copies of each token are never written to or re-read from HBM
    MEGAMOE_TRY(run_permute(*d, x, expert_idx, gmA, pts1, eri, sorted, counts, cumsum, err, bcnt,
                            true, s, (float *)(base + L.tscale), tail ? tdone : nullptr, tsync,
                            prow));
    // SwiGLU: the rows whose GMM1 output is complete before GMM1's last round
    // are done by the workgroups left idle in that round; the SwiGLU kernel
    // does the rest (all rows without the overlap)
    GmmParams tp{};
    tp.tail_q2 = q2;
    tp.tail_pts2 = pts2;
    tp.tail_pts1 = pts1;
    tp.tail_sync = tsync;
    tp.tail_done = tdone;
    tp.tail_I = d->I;
    tp.tail_spin = overlap == 2 ? -1 : kTailSpin;
    tp.tail_prow = prow;
    // without the overlap, GMM1's sparse last round splits its tiles over K
    // (the permute zeroes the counters after the overlap's three words)
    GmmParams kp{};
    kp.ks_part = (int32_t *)(base + L.ks);
    kp.ks_count = tsync + 3;
    MEGAMOE_TRY(run_gmm(*d, gmA, cumsum, w1p, scale1, gmC, nullptr, 2 * d->I, d->K, s, sorted,
                        tail ? &tp : &kp));
    MEGAMOE_TRY(hip_status(launch_swiglu_quant(gmC, pts1, cumsum, R, d->E, d->I, q2, pts2, s,
                                               tail ? tdone : nullptr, prow)));
    MEGAMOE_TRY(run_gmm(*d, q2, cumsum, w2p, scale2, g2, nullptr, d->K, d->I, s, nullptr, nullptr,
                        true));
    return hip_status(launch_unpermute(g2, pts2, eri, probs, d->M, d->K, d->top_k, out, s));
}

int megamoe_set_overlap(int mode) {
    if (mode < 0 || mode > 2) return MEGAMOE_EINVAL;
    g_overlap.store(mode, std::memory_order_relaxed);
    return MEGAMOE_OK;
}

int megamoe_last_error(const void *ws, void *stream, int32_t *bad_route_count) {
    if (!aligned16(ws) || !bad_route_count) return MEGAMOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    int32_t v = 0;
    if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
        return MEGAMOE_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MEGAMOE_EHIP;
    *bad_route_count = v;
    return v ? MEGAMOE_EDEVICE : MEGAMOE_OK;
}

}  // extern "C"
