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

// CAST_ROUND(x / scale), clamped to [-127, 127], for x an fp16 value of a row
// whose largest |x| is amax (also fp16), scale = amax / 127 and inv = 1 / scale
// (both IEEE).  The quotient is x * inv corrected once by its FMA residual,
// q + inv * (x - q * scale) (Markstein's method), three instructions instead
// of the ten of an IEEE division.  For every finite fp16 amax > 0 and every
// fp16 x with |x| <= amax it yields the same integer as roundf of the IEEE
// quotient: all 2^31 such pairs were checked on the GPU.
__device__ __forceinline__ int quant_round(float x, float scale, float inv) {
    const float q0 = x * inv;
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, scale, x), inv, q0);
    const float r = roundf(q);  // half away from zero
    return (int)fminf(fmaxf(r, -127.0f), 127.0f);
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
    uint8_t *__restrict__ tail_done, uint32_t *__restrict__ tail_sync) {
    __shared__ int s_base[kMaxExperts];   // next row of each expert for this block
    __shared__ int s_tot[kMaxExperts];
    __shared__ int s_wcnt[kSortWavesB][kMaxExperts];
    __shared__ int s_valid;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int b = blockIdx.x;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

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
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            if (e < E) {
                if (b == 0) {
                    tokens_per_expert[e] = v[j];
                    expert_cumsum[e] = run + v[j];
                }
                s_base[e] += run;
            }
            run += v[j];
        }
        if (lane == kWave - 1) s_valid = incl;
    }
    __syncthreads();
    const int valid_rows = s_valid;
    if (b == 0) {
        if (tid == 0) {
            err_word[0] = R - valid_rows;
            if (tail_sync) tail_sync[0] = tail_sync[1] = tail_sync[2] = 0;
        }
        for (int d = valid_rows + tid; d < R; d += kSortBlock) sorted_route[d] = -1;
    }

    const int r_end = min(R, (b + 1) * C);
    for (int r0 = b * C; r0 < r_end; r0 += kSortBlock) {
        for (int i = tid; i < kSortWavesB * kMaxExperts; i += kSortBlock) (&s_wcnt[0][0])[i] = 0;
        __syncthreads();
        const int r = r0 + wave * kWave + lane;
        const int key = (r < r_end) ? route_key(expert_idx, r, R, E) : E;
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
                if (tscale) pts1[dst] = tscale[r / top_k];
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
// tscale (nullable, token-major only): the token's scale goes to tscale[t]
// instead of to its routes' rows (the sort has not run yet).
template <int MAXC>
__device__ __forceinline__ void quant_token(const uint16_t *__restrict__ x,
                                            const int32_t *__restrict__ expanded_row_idx, int K,
                                            int top_k, int8_t *__restrict__ gmA,
                                            float *__restrict__ pts1, bool token_major, int t,
                                            float *__restrict__ tscale) {
    __shared__ float s_red[4];
    const int tid = threadIdx.x;
    const int nchunk = K >> 4;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)t * K);

    uint4 raw[MAXC][2];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + i * 256;
        if (c < nchunk) {
            raw[i][0] = load_nt16(xr + 2 * c);  // x is read once
            raw[i][1] = load_nt16(xr + 2 * c + 1);
            const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[i][0]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                amax = fmaxf(amax, fabsf(h2f((uint16_t)(w[j] & 0xffffu))));
                amax = fmaxf(amax, fabsf(h2f((uint16_t)(w[j] >> 16))));
            }
        }
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) s_red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float scale = amax / 127.0f;  // per-token dynamic scale
    const float inv = 1.0f / scale;

    const int32_t *rows = token_major ? nullptr : expanded_row_idx + (size_t)t * top_k;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + i * 256;
        if (c >= nchunk) continue;
        const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[i][0]);
        uint32_t packed[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t word = 0;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int idx = j * 4 + h;  // element within the 16-element chunk
                const uint16_t bits = (uint16_t)((w[idx >> 1] >> ((idx & 1) * 16)) & 0xffffu);
                const int q = amax != 0.0f ? quant_round(h2f(bits), scale, inv) : 0;
                word |= ((uint32_t)q & 0xffu) << (8 * h);
            }
            packed[j] = word;
        }
        const uint4 out = make_uint4(packed[0], packed[1], packed[2], packed[3]);
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
    quant_token<MAXC>(x, expanded_row_idx, K, top_k, gmA, pts1, token_major, blockIdx.x, nullptr);
}

// The forward's first launch for large route counts: workgroups [0, B) count
// the expert ids of their route block (sort pass 1), workgroups B.. each
// quantise one token to its token-major row and its scale to tscale.  The two
// are independent, so one launch runs both; the scatter pass then writes each
// route row's pts1 from tscale.  (One wave per token, four tokens per
// workgroup, measured slower: 17.1 against 14.1 us at M = 2048, K = 7168.)
template <int MAXC>
__global__ __launch_bounds__(256) void count_quant_kernel(
    const int32_t *__restrict__ expert_idx, int R, int E, int C, int B,
    int32_t *__restrict__ block_counts, const uint16_t *__restrict__ x, int K,
    int8_t *__restrict__ qx, float *__restrict__ tscale) {
    if ((int)blockIdx.x < B) route_count_block(expert_idx, R, E, C, blockIdx.x, block_counts);
    else quant_token<MAXC>(x, nullptr, K, 1, qx, nullptr, true, blockIdx.x - B, tscale);
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
    uint32_t *__restrict__ tail_sync) {
    __shared__ int h_all[kMaxExperts + 1];
    __shared__ int h_pre[kMaxExperts + 1];
    __shared__ int s_key[kFusedMaxTopK];
    __shared__ int s_dst[kFusedMaxTopK];
    __shared__ float s_red[4];
    __shared__ int s_valid;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int nchunk = K >> 4;
    const int r_own = t * top_k;
    // clear the flags of the GMM1 that follows (route r's flag is row r's)
    if (tail_done && tid < top_k) tail_done[r_own + tid] = 0;
    if (tail_sync && t == 0 && tid < 3) tail_sync[tid] = 0;

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
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + i * 256;
        if (c < nchunk) {
            const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[i][0]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                amax = fmaxf(amax, fabsf(h2f((uint16_t)(w[j] & 0xffffu))));
                amax = fmaxf(amax, fabsf(h2f((uint16_t)(w[j] >> 16))));
            }
        }
    }
    amax = wave_max(amax);
    if (lane == 0) s_red[tid >> 6] = amax;
    __syncthreads();  // counters zeroed; s_key and s_red written
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float scale = amax / 127.0f;
    const float inv = 1.0f / scale;

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
        const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[i][0]);
        uint32_t packed[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t word = 0;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int idx = j * 4 + h;
                const uint16_t bits = (uint16_t)((w[idx >> 1] >> ((idx & 1) * 16)) & 0xffffu);
                const int qv = amax != 0.0f ? quant_round(h2f(bits), scale, inv) : 0;
                word |= ((uint32_t)qv & 0xffu) << (8 * h);
            }
            packed[j] = word;
        }
        q[i] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
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
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            if (e < E) {
                if (t == 0) {
                    tokens_per_expert[e] = v[j];
                    expert_cumsum[e] = run + v[j];
                }
                h_pre[e] += run;  // first row of expert e for this token's routes
            }
            run += v[j];
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
                                hipStream_t stream, uint8_t *tail_done, uint32_t *tail_sync) {
    const int R = M * top_k;
    const int per_thread = (K / 16 + 255) / 256;
    dim3 grid(M), block(256);
#define MEGAMOE_PERMUTE_FUSED(C)                                                              \
    hipLaunchKernelGGL(permute_fused_kernel<C>, grid, block, 0, stream, x, expert_idx, R, E, K, \
                       top_k, gmA, pts1, expanded_row_idx, sorted_route, tokens_per_expert,     \
                       expert_cumsum, err_word, token_major, tail_done, tail_sync)
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
                       nullptr);
    return hipGetLastError();
}

hipError_t launch_permute_tokens_2pass(const uint16_t *x, const int32_t *expert_idx, int M, int K,
                                       int E, int top_k, int8_t *qx, float *pts1,
                                       int32_t *expanded_row_idx, int32_t *sorted_route,
                                       int32_t *tokens_per_expert, int32_t *expert_cumsum,
                                       int32_t *err_word, int32_t *block_counts, float *tscale,
                                       hipStream_t stream, uint8_t *tail_done,
                                       uint32_t *tail_sync) {
    const int R = M * top_k;
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // keys 0..E (E = dropped)
    const int C = route_sort_chunk(R);
    const int B = (R + C - 1) / C;
    const int per_thread = (K / 16 + 255) / 256;  // K <= 32768: at most 8
    dim3 grid(B + M), block(256);
#define MEGAMOE_COUNT_QUANT(MC)                                                                \
    hipLaunchKernelGGL(count_quant_kernel<MC>, grid, block, 0, stream, expert_idx, R, E, C, B, \
                       block_counts, x, K, qx, tscale)
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
                       tail_sync);
    return hipGetLastError();
}

hipError_t launch_quant_scatter(const uint16_t *x, const int32_t *expanded_row_idx, int M, int K,
                                int top_k, int8_t *gmA, float *pts1, bool token_major,
                                hipStream_t stream) {
    const int per_thread = (K / 16 + 255) / 256;
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
