// FrontReorder on one rank: route sort + per-token int8 quantisation scatter.
//
// Follows section 1 ("FrontReorder") of the pto-isa MegaMoE overview page:
// order the (expertId[route], route) pairs expert-major, count routes per
// expert, build the inverse map expandedRowIdx[route] = row, quantise each
// token once (scale = max|x| / 127, q = CAST_ROUND(x / scale)) and write that
// row to every destination row of the token's routes.  Dispatch (section 2) is
// the identity on one rank, so the rows go straight to the expert-major A
// matrix of GMM1.  In the forward (token_major) each token's row is written
// once instead, to a token-major [M, K] matrix, and GMM1 gathers its
// expert-major rows from it through the sorted route list.
//
// The page sorts with merge-sort instructions sized to its 192 KiB buffer.
// With at most 256 expert keys a counting sort reaches the same stable order
// in two passes spread over many workgroups: per-block histograms, then per
// block row bases and wave-ballot peer matching for the ranks inside a block.
#include "common.hpp"
#include "kernels.hpp"

namespace megamoe {

constexpr int kMaxExperts = 256;
constexpr int kSortBlock = 256;          // threads per sort workgroup (4 waves)
constexpr int kSortWavesB = kSortBlock / kWave;

// Lanes of the wave holding the same key as this lane (among `valid` lanes).
// key < 2^nbits.  One ballot per key bit.
__device__ __forceinline__ uint64_t match_key(int key, uint64_t valid, int nbits) {
    uint64_t m = valid;
    for (int b = 0; b < nbits; ++b) {
        const int bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

__device__ __forceinline__ int route_key(const int32_t *__restrict__ expert_idx, int r, int R,
                                         int E) {
    if (r >= R) return E;
    const int e = expert_idx[r];
    return (e >= 0 && e < E) ? e : E;  // E marks a dropped route
}

// CAST_ROUND(x / scale) for x an fp16 value of a row whose largest |x| is amax
// (also fp16), scale = amax / 127 and inv = 1 / scale (both IEEE; inv = 0 for
// an all-zero row, which gives 0 everywhere).
//  * The quotient is x * inv corrected once by its FMA residual,
//    q + inv * (x - q * scale) (Markstein's method): three instructions instead
//    of the ten of an IEEE division.  The first product is an FMA with a +0
//    addend so that the hardware reads x as fp16 in the same instruction.
//  * Half away from zero is the truncation of q + copysign(0.49999997, q), the
//    largest float below one half (adding exactly one half would take
//    0.49999997 itself to 1), and the truncation is the float -> int
//    conversion: two instructions and the conversion instead of the six of
//    roundf.  |x| <= amax keeps the sum within (-127.5, 127.5), so no clamp
//    is needed.
// For every finite fp16 amax > 0 and every fp16 x with |x| <= amax this gives
// the same integer as roundf of the IEEE quotient, clamped to [-127, 127];
// tests/csrc/quant_exhaustive.c checks all 1,007,681,535 such pairs.
__device__ __forceinline__ int quant_round(float x, float scale, float inv) {
    const float q0 = __builtin_fmaf(x, inv, 0.0f);
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, scale, x), inv, q0);
    return (int)(q + __builtin_copysignf(0x1.fffffep-2f, q));
}

// 8 fp16 values (one 16-byte word) -> 8 int8 codes.  The low bytes of four
// codes are gathered into a word by three byte permutes.
__device__ __forceinline__ uint2 quant_chunk8(const uint4 &raw, float scale, float inv) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw);
    uint32_t packed[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int q[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int idx = j * 4 + h;  // element within the 8-element chunk
            const uint16_t bits = (uint16_t)((w[idx >> 1] >> ((idx & 1) * 16)) & 0xffffu);
            q[h] = quant_round(h2f(bits), scale, inv);
        }
        // bytes [q0, q1, 0, 0] and [q2, q3, 0, 0], then [q0, q1, q2, q3]
        const uint32_t lo = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x0c0c0400u);
        packed[j] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    return make_uint2(packed[0], packed[1]);
}

// 16 fp16 values (two 16-byte words) -> 16 int8 codes.
__device__ __forceinline__ uint4 quant_chunk16(const uint4 (&raw)[2], float scale, float inv) {
    const uint2 a = quant_chunk8(raw[0], scale, inv), b = quant_chunk8(raw[1], scale, inv);
    return make_uint4(a.x, a.y, b.x, b.y);
}

// The largest |x| over 16-byte words of fp16 values, as fp16 bits.  With the
// sign bits cleared, finite fp16 values order like their bit patterns, so the
// maximum takes one packed 16-bit integer max per two values.  (The
// quantiser's inputs are finite; a NaN would be taken as the maximum.)
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t absmax_step(u16x2_t m, const uint4 &raw) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[j] & 0x7fff7fffu));
    return m;
}
// ... over a thread's 16-element chunks c = tid + 256 i < nchunk
template <int MAXC>
__device__ __forceinline__ uint32_t chunks_absmax_bits(const uint4 (&raw)[MAXC][2], int tid,
                                                       int nchunk) {
    u16x2_t m = {0, 0};
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
        if (tid + i * 256 < nchunk) m = absmax_step(absmax_step(m, raw[i][0]), raw[i][1]);
    return m[0] > m[1] ? m[0] : m[1];
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Pass 1: histogram of the expert ids of routes [b*C, (b+1)*C) of block b.
// Counting is order-free, so LDS atomics are fine here.
__device__ __forceinline__ void route_count_block(const int32_t *__restrict__ expert_idx, int R,
                                                  int E, int C, int b,
                                                  int32_t *__restrict__ block_counts) {
    __shared__ int h[kMaxExperts];
    const int tid = threadIdx.x;
    for (int i = tid; i < E; i += kSortBlock) h[i] = 0;
    __syncthreads();
    const int r0 = b * C;
    const int r1 = min(R, r0 + C);
    for (int r = r0 + tid; r < r1; r += kSortBlock) {
        const int key = route_key(expert_idx, r, R, E);
        if (key < E) atomicAdd(&h[key], 1);
    }
    __syncthreads();
    for (int i = tid; i < E; i += kSortBlock) block_counts[(size_t)b * E + i] = h[i];
}

__global__ __launch_bounds__(kSortBlock) void route_count_kernel(
    const int32_t *__restrict__ expert_idx, int R, int E, int C,
    int32_t *__restrict__ block_counts /*[B][E]*/) {
    route_count_block(expert_idx, R, E, C, blockIdx.x, block_counts);
}

// Pass 2: each block derives the first row of every expert for its routes
// (exclusive prefix over experts of the totals, plus the counts of the blocks
// before it), then ranks its routes in route order: 256 routes per round, one
// 64-route chunk per wave, ranks inside a wave from ballot peer matching, the
// waves ordered by their per-expert counts.  Block 0 also writes the counts,
// the inclusive prefix and the dropped-route word.
//
// tscale (nullable): per-token scales of a quantisation that ran before the
// sort (the forward's token-major rows); each route's row then gets its
// token's scale, pts1[row] = tscale[route / top_k].
__global__ __launch_bounds__(kSortBlock) void route_scatter_kernel(
    const int32_t *__restrict__ expert_idx, int R, int E, int C, int nbits, int B,
    const int32_t *__restrict__ block_counts, int32_t *__restrict__ sorted_route,
    int32_t *__restrict__ expanded_row_idx, int32_t *__restrict__ tokens_per_expert,
    int32_t *__restrict__ expert_cumsum, int32_t *__restrict__ err_word,
    const float *__restrict__ tscale, int top_k, float *__restrict__ pts1,
    uint8_t *__restrict__ tail_done, uint32_t *__restrict__ tail_sync,
    int32_t *__restrict__ prow) {
    __shared__ int s_base[kMaxExperts];   // next row of each expert for this block
    __shared__ int s_tot[kMaxExperts];
    __shared__ int s_odd[kMaxExperts];    // experts before e with an odd row count
    __shared__ int s_wcnt[kSortWavesB][kMaxExperts];
    __shared__ int s_valid;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int b = blockIdx.x;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    // this thread's first route key and its token's scale are requested
    // before the table is read, so the two round trips overlap
    const int r_end = min(R, (b + 1) * C);
    int key_next = E;
    float ts_next = 0.0f;
    {
        const int r = b * C + tid;
        if (r < r_end) {
            key_next = route_key(expert_idx, r, R, E);
            if (tscale) ts_next = tscale[r / top_k];
        }
    }
    for (int e = tid; e < E; e += kSortBlock) {
        s_tot[e] = 0;
        s_base[e] = 0;
    }
    __syncthreads();
    // the table's column sums (all blocks, and the blocks before this one):
    // thread (part, e) sums expert e over blocks part, part + parts, ... with
    // coalesced loads, and the partial sums meet in LDS (integer sums are
    // order-free)
    {
        const int parts = kSortBlock / E;  // >= 1 since E <= kMaxExperts = kSortBlock
        const int e = tid % E, part = tid / E;
        if (part < parts) {
            int tot = 0, pre = 0;
#pragma unroll 8
            for (int bb = part; bb < B; bb += parts) {
                const int v = block_counts[(size_t)bb * E + e];
                tot += v;
                pre += bb < b ? v : 0;
            }
            if (tot) atomicAdd(&s_tot[e], tot);
            if (pre) atomicAdd(&s_base[e], pre);
        }
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of the totals over experts, four per lane
        int v[4];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            v[j] = (e < E) ? s_tot[e] : 0;
            sum += v[j];
        }
        const int incl = wave_inclusive_scan(sum);
        int run = incl - sum;
        int odds = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) odds += v[j] & 1;
        int orun = wave_inclusive_scan(odds) - odds;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            if (e < E) {
                if (b == 0) {
                    tokens_per_expert[e] = v[j];
                    expert_cumsum[e] = run + v[j];
                }
                s_base[e] += run;
                s_odd[e] = orun;
            }
            run += v[j];
            orun += v[j] & 1;
        }
        if (lane == kWave - 1) s_valid = incl;
    }
    __syncthreads();
    const int valid_rows = s_valid;
    if (b == 0) {
        if (tid == 0) err_word[0] = R - valid_rows;
        if (tail_sync && tid < kSyncWords) tail_sync[tid] = 0;
        for (int d = valid_rows + tid; d < R; d += kSortBlock) sorted_route[d] = -1;
    }

    for (int r0 = b * C; r0 < r_end; r0 += kSortBlock) {
        for (int i = tid; i < kSortWavesB * kMaxExperts; i += kSortBlock) (&s_wcnt[0][0])[i] = 0;
        __syncthreads();
        const int r = r0 + tid;  // tid = wave * kWave + lane
        const int key = key_next;
        const float ts = ts_next;
        key_next = E;  // the next round's key and scale
        if (r + kSortBlock < r_end) {
            key_next = route_key(expert_idx, r + kSortBlock, R, E);
            if (tscale) ts_next = tscale[(r + kSortBlock) / top_k];
        }
        const bool ok = key < E;
        const uint64_t m = match_key(key, __ballot(ok), nbits);
        const int rank = __popcll(m & below);
        if (ok && rank == 0) s_wcnt[wave][key] = __popcll(m);
        __syncthreads();
        int dst = -1;
        if (ok) {
            int pre = s_base[key];
            for (int w = 0; w < wave; ++w) pre += s_wcnt[w][key];
            dst = pre + rank;
        }
        if (r < r_end) {
            if (tail_done) tail_done[r] = 0;  // R flags of the GMM1 that follows
            expanded_row_idx[r] = dst;
            if (dst >= 0) {
                sorted_route[dst] = r;
                if (tscale) pts1[dst] = ts;
                if (prow) prow[dst] = dst + s_odd[key];
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += kSortBlock) {
            int add = 0;
            for (int w = 0; w < kSortWavesB; ++w) add += s_wcnt[w][e];
            s_base[e] += add;
        }
        // the next round's zeroing is ordered after these reads by its barrier
        __syncthreads();
    }
}

// One workgroup per token.  Each thread owns 16-element chunks of the row
// (two 16-byte loads of fp16, one 16-byte int8 store per destination row).
// When the chunks do not fill every thread the same number of times, the
// lighter wave moves with the token (slot), so no SIMD always gets it.
__device__ __forceinline__ int quant_slot(int t) { return ((int)threadIdx.x + ((t & 3) << 6)) & 255; }

template <int MAXC>
__device__ __forceinline__ void quant_token_load(const uint16_t *__restrict__ x, int K, int t,
                                                 uint4 (&raw)[MAXC][2]) {
    const int slot = quant_slot(t), nchunk = K >> 4;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)t * K);
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = slot + i * 256;
        if (c < nchunk) {
            raw[i][0] = load_nt16(xr + 2 * c);  // x is read once
            raw[i][1] = load_nt16(xr + 2 * c + 1);
        }
    }
}

// tscale (nullable, token-major only): the token's scale goes to tscale[t]
// instead of to its routes' rows (the sort has not run yet).
template <int MAXC>
__device__ __forceinline__ void quant_token_finish(const uint4 (&raw)[MAXC][2],
                                                   const int32_t *__restrict__ expanded_row_idx,
                                                   int K, int top_k, int8_t *__restrict__ gmA,
                                                   float *__restrict__ pts1, bool token_major,
                                                   int t, float *__restrict__ tscale) {
    __shared__ uint32_t s_red[4];
    const int tid = threadIdx.x;
    const int slot = quant_slot(t), nchunk = K >> 4;
    const uint32_t mbits = wave_max_u32(chunks_absmax_bits<MAXC>(raw, slot, nchunk));
    if ((tid & 63) == 0) s_red[tid >> 6] = mbits;
    __syncthreads();
    const uint32_t m01 = s_red[0] > s_red[1] ? s_red[0] : s_red[1];
    const uint32_t m23 = s_red[2] > s_red[3] ? s_red[2] : s_red[3];
    const float amax = h2f((uint16_t)(m01 > m23 ? m01 : m23));
    const float scale = amax / 127.0f;  // per-token dynamic scale
    const float inv = amax != 0.0f ? 1.0f / scale : 0.0f;

    const int32_t *rows = token_major ? nullptr : expanded_row_idx + (size_t)t * top_k;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = slot + i * 256;
        if (c >= nchunk) continue;
        const uint4 out = quant_chunk16(raw[i], scale, inv);
        if (token_major) {
            *reinterpret_cast<uint4 *>(gmA + (size_t)t * K + (size_t)c * 16) = out;
        } else {
            for (int s = 0; s < top_k; ++s) {
                const int d = rows[s];
                if (d >= 0) *reinterpret_cast<uint4 *>(gmA + (size_t)d * K + (size_t)c * 16) = out;
            }
        }
    }
    if (tid == 0) {
        if (tscale) {
            tscale[t] = scale;
        } else {
            for (int s = 0; s < top_k; ++s) {
                const int d = expanded_row_idx[(size_t)t * top_k + s];
                if (d >= 0) pts1[d] = scale;
            }
        }
    }
}

template <int MAXC>
__global__ __launch_bounds__(256) void quant_scatter_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ expanded_row_idx, int K,
    int top_k, int8_t *__restrict__ gmA, float *__restrict__ pts1, bool token_major) {
    uint4 raw[MAXC][2];
    quant_token_load<MAXC>(x, K, blockIdx.x, raw);
    quant_token_finish<MAXC>(raw, expanded_row_idx, K, top_k, gmA, pts1, token_major, blockIdx.x,
                             nullptr);
}

// The forward's first launch for large route counts: workgroup b quantises
// token b (if b < M) to its token-major row and its scale to tscale, and
// counts the expert ids of route block b (if b < B; sort pass 1).  The two are
// independent, so one launch runs both; the scatter pass then writes each
// route row's pts1 from tscale.  A workgroup requests its x row before it
// counts, so the two latencies overlap.  Giving the count its own workgroups
// put M + B workgroups in the launch: at M = 2048 the last 64 no longer fit
// the GPU at once (8 per CU) and started only as others ended.  (One wave per
// token, four tokens per workgroup, was slower too: 17.1 against 14.1 us at
// M = 2048, K = 7168.)
template <int MAXC>
__global__ __launch_bounds__(256) void count_quant_kernel(
    const int32_t *__restrict__ expert_idx, int R, int E, int C, int B,
    int32_t *__restrict__ block_counts, const uint16_t *__restrict__ x, int M, int K,
    int8_t *__restrict__ qx, float *__restrict__ tscale) {
    const int b = blockIdx.x;
    uint4 raw[MAXC][2];
    if (b < M) quant_token_load<MAXC>(x, K, b, raw);
    if (b < B) route_count_block(expert_idx, R, E, C, b, block_counts);
    if (b < M) quant_token_finish<MAXC>(raw, nullptr, K, 1, qx, nullptr, true, b, tscale);
}

// Small route counts: the whole of FrontReorder in one launch, one workgroup
// per token.  Every workgroup histograms all R expert ids in LDS (all routes,
// and the routes before its own token), so it knows each expert's first row
// and, for each of its own routes r, how many routes of the same expert come
// before r -- the same stable expert-major order as the two-pass sort.  It
// then quantises its token once and writes the row to its routes' rows.
// Workgroup 0 also writes the counts, the inclusive prefix, the dropped-route
// word and the -1 tail of sorted_route.  The x row and the first 2048 expert
// ids are requested before anything else, and the token-major row is
// quantised and stored before the sort's prefix, so those latencies overlap.
constexpr int kFusedMaxR = 8192;
constexpr int kFusedMaxTopK = 16;

template <int MAXC>
__global__ __launch_bounds__(256) void permute_fused_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ expert_idx, int R, int E,
    int K, int top_k, int8_t *__restrict__ gmA, float *__restrict__ pts1,
    int32_t *__restrict__ expanded_row_idx, int32_t *__restrict__ sorted_route,
    int32_t *__restrict__ tokens_per_expert, int32_t *__restrict__ expert_cumsum,
    int32_t *__restrict__ err_word, bool token_major, uint8_t *__restrict__ tail_done,
    uint32_t *__restrict__ tail_sync, int32_t *__restrict__ prow) {
    __shared__ int h_all[kMaxExperts + 1];
    __shared__ int h_pre[kMaxExperts + 1];
    __shared__ int s_key[kFusedMaxTopK];
    __shared__ int s_dst[kFusedMaxTopK];
    __shared__ uint32_t s_red[4];
    __shared__ int s_valid;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int nchunk = K >> 4;
    const int r_own = t * top_k;
    // clear the flags of the GMM1 that follows (route r's flag is row r's)
    if (tail_done && tid < top_k) tail_done[r_own + tid] = 0;
    if (tail_sync && t == 0 && tid < kSyncWords) tail_sync[tid] = 0;

    // Every first load is issued up front: the token's row, the first 2048
    // expert ids (all of them up to R = 2048) and the token's own ids.
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)t * K);
    uint4 raw[MAXC][2];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + i * 256;
        if (c < nchunk) {
            raw[i][0] = load_nt16(xr + 2 * c);  // x is read once
            raw[i][1] = load_nt16(xr + 2 * c + 1);
        }
    }
    int key0[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) key0[u] = route_key(expert_idx, u * 256 + tid, R, E);
    if (tid < top_k) s_key[tid] = route_key(expert_idx, r_own + tid, R, E);
    for (int e = tid; e <= E; e += 256) {
        h_all[e] = 0;
        h_pre[e] = 0;
    }

    // the row's absolute maximum
    const uint32_t mbits = wave_max_u32(chunks_absmax_bits<MAXC>(raw, tid, nchunk));
    if (lane == 0) s_red[tid >> 6] = mbits;
    __syncthreads();  // counters zeroed; s_key and s_red written
    const uint32_t m01 = s_red[0] > s_red[1] ? s_red[0] : s_red[1];
    const uint32_t m23 = s_red[2] > s_red[3] ? s_red[2] : s_red[3];
    const float amax = h2f((uint16_t)(m01 > m23 ? m01 : m23));
    const float scale = amax / 127.0f;
    const float inv = amax != 0.0f ? 1.0f / scale : 0.0f;

    // histograms: every route's expert, and the routes before this token's
    // (key E, a dropped route, is counted too, in slot E)
    for (int r0 = 0; r0 < R; r0 += 8 * 256) {
        int key[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            key[u] = r0 == 0 ? key0[u] : route_key(expert_idx, r0 + u * 256 + tid, R, E);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = r0 + u * 256 + tid;
            if (r < R) {
                atomicAdd(&h_all[key[u]], 1);
                if (r < r_own) atomicAdd(&h_pre[key[u]], 1);
            }
        }
    }

    // per-token dynamic quantisation; it does not depend on the sort, so the
    // token-major row is stored while the histograms complete
    uint4 q[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + i * 256;
        if (c >= nchunk) continue;
        q[i] = quant_chunk16(raw[i], scale, inv);
        if (token_major) *reinterpret_cast<uint4 *>(gmA + (size_t)t * K + (size_t)c * 16) = q[i];
    }
    __syncthreads();  // histograms complete

    if (tid < kWave) {  // exclusive prefix of the counts over experts, four per lane
        int v[4];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            v[j] = (e < E) ? h_all[e] : 0;
            sum += v[j];
        }
        const int incl = wave_inclusive_scan(sum);
        int run = incl - sum;
        int odds = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) odds += v[j] & 1;
        int orun = wave_inclusive_scan(odds) - odds;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            if (e < E) {
                if (t == 0) {
                    tokens_per_expert[e] = v[j];
                    expert_cumsum[e] = run + v[j];
                }
                h_pre[e] += run;  // first row of expert e for this token's routes
                h_all[e] = orun;  // from here on: experts before e with an odd count
            }
            run += v[j];
            orun += v[j] & 1;
        }
        if (lane == kWave - 1) s_valid = incl;
    }
    __syncthreads();
    if (tid < top_k) {
        const int key = s_key[tid];
        int dst = -1;
        if (key < E) {
            int same = 0;  // earlier slots of this token with the same expert
            for (int u = 0; u < tid; ++u) same += s_key[u] == key;
            dst = h_pre[key] + same;
        }
        s_dst[tid] = dst;
        expanded_row_idx[r_own + tid] = dst;
        if (dst >= 0) {
            sorted_route[dst] = r_own + tid;
            pts1[dst] = scale;
            if (prow) prow[dst] = dst + h_all[key];
        }
    }
    if (t == 0) {
        const int valid_rows = s_valid;
        if (tid == 0) err_word[0] = R - valid_rows;
        for (int d = valid_rows + tid; d < R; d += 256) sorted_route[d] = -1;
    }
    if (!token_major) {  // the row goes to every route's row
        __syncthreads();  // publishes s_dst
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            const int c = tid + i * 256;
            if (c >= nchunk) continue;
            for (int s2 = 0; s2 < top_k; ++s2) {
                const int d = s_dst[s2];
                if (d >= 0) *reinterpret_cast<uint4 *>(gmA + (size_t)d * K + (size_t)c * 16) = q[i];
            }
        }
    }
}

bool permute_fused_ok(int R, int top_k) { return R <= kFusedMaxR && top_k <= kFusedMaxTopK; }

hipError_t launch_permute_fused(const uint16_t *x, const int32_t *expert_idx, int M, int K, int E,
                                int top_k, int8_t *gmA, float *pts1, int32_t *expanded_row_idx,
                                int32_t *sorted_route, int32_t *tokens_per_expert,
                                int32_t *expert_cumsum, int32_t *err_word, bool token_major,
                                hipStream_t stream, uint8_t *tail_done, uint32_t *tail_sync,
                                int32_t *prow) {
    const int R = M * top_k;
    const int per_thread = (K / 16 + 255) / 256;
    dim3 grid(M), block(256);
#define MEGAMOE_PERMUTE_FUSED(C)                                                              \
    hipLaunchKernelGGL(permute_fused_kernel<C>, grid, block, 0, stream, x, expert_idx, R, E, K, \
                       top_k, gmA, pts1, expanded_row_idx, sorted_route, tokens_per_expert,     \
                       expert_cumsum, err_word, token_major, tail_done, tail_sync, prow)
    if (per_thread <= 1) MEGAMOE_PERMUTE_FUSED(1);
    else if (per_thread <= 2) MEGAMOE_PERMUTE_FUSED(2);
    else if (per_thread <= 4) MEGAMOE_PERMUTE_FUSED(4);
    else MEGAMOE_PERMUTE_FUSED(8);
#undef MEGAMOE_PERMUTE_FUSED
    return hipGetLastError();
}

// Routes per sort block: at least 256, and at most 256 blocks so that each
// block's pass over the block-count table stays short.
int route_sort_chunk(int R) {
    const int per = (R + 255) / 256;
    return max(kSortBlock, (per + kSortBlock - 1) / kSortBlock * kSortBlock);
}

size_t route_sort_workspace_bytes(int R, int E) {
    const int C = route_sort_chunk(R);
    const int B = (R + C - 1) / C;
    return (size_t)B * E * sizeof(int32_t);
}

hipError_t launch_route_sort(const int32_t *expert_idx, int R, int E, int32_t *sorted_route,
                             int32_t *expanded_row_idx, int32_t *tokens_per_expert,
                             int32_t *expert_cumsum, int32_t *err_word, int32_t *block_counts,
                             hipStream_t stream) {
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // keys 0..E (E = dropped)
    const int C = route_sort_chunk(R);
    const int B = (R + C - 1) / C;
    hipLaunchKernelGGL(route_count_kernel, dim3(B), dim3(kSortBlock), 0, stream, expert_idx, R, E,
                       C, block_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(B), dim3(kSortBlock), 0, stream, expert_idx, R,
                       E, C, nbits, B, block_counts, sorted_route, expanded_row_idx,
                       tokens_per_expert, expert_cumsum, err_word, nullptr, 1, nullptr, nullptr,
                       nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_permute_tokens_2pass(const uint16_t *x, const int32_t *expert_idx, int M, int K,
                                       int E, int top_k, int8_t *qx, float *pts1,
                                       int32_t *expanded_row_idx, int32_t *sorted_route,
                                       int32_t *tokens_per_expert, int32_t *expert_cumsum,
                                       int32_t *err_word, int32_t *block_counts, float *tscale,
                                       hipStream_t stream, uint8_t *tail_done,
                                       uint32_t *tail_sync, int32_t *prow) {
    const int R = M * top_k;
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // keys 0..E (E = dropped)
    const int C = route_sort_chunk(R);
    const int B = (R + C - 1) / C;
    const int per_thread = (K / 16 + 255) / 256;  // K <= 32768: at most 8
    dim3 grid(max(B, M)), block(256);
#define MEGAMOE_COUNT_QUANT(MC)                                                                \
    hipLaunchKernelGGL(count_quant_kernel<MC>, grid, block, 0, stream, expert_idx, R, E, C, B, \
                       block_counts, x, M, K, qx, tscale)
    if (per_thread <= 1) MEGAMOE_COUNT_QUANT(1);
    else if (per_thread <= 2) MEGAMOE_COUNT_QUANT(2);
    else if (per_thread <= 4) MEGAMOE_COUNT_QUANT(4);
    else MEGAMOE_COUNT_QUANT(8);
#undef MEGAMOE_COUNT_QUANT
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(B), dim3(kSortBlock), 0, stream, expert_idx, R,
                       E, C, nbits, B, block_counts, sorted_route, expanded_row_idx,
                       tokens_per_expert, expert_cumsum, err_word, tscale, top_k, pts1, tail_done,
                       tail_sync, prow);
    return hipGetLastError();
}

hipError_t launch_quant_scatter(const uint16_t *x, const int32_t *expanded_row_idx, int M, int K,
                                int top_k, int8_t *gmA, float *pts1, bool token_major,
                                hipStream_t stream) {
    const int per_thread = (K / 16 + 255) / 256;  // K <= 32768: at most 8
    dim3 grid(M), block(256);
    if (per_thread <= 1)
        hipLaunchKernelGGL(quant_scatter_kernel<1>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1, token_major);
    else if (per_thread <= 2)
        hipLaunchKernelGGL(quant_scatter_kernel<2>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1, token_major);
    else if (per_thread <= 4)
        hipLaunchKernelGGL(quant_scatter_kernel<4>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1, token_major);
    else
        hipLaunchKernelGGL(quant_scatter_kernel<8>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1, token_major);
    return hipGetLastError();
}

}  // namespace megamoe
