// FrontReorder on one rank: route sort + per-token int8 quantisation scatter.
//
// Follows section 1 ("FrontReorder") of the pto-isa MegaMoE overview page:
// order the (expertId[route], route) pairs expert-major, count routes per
// expert, build the inverse map expandedRowIdx[route] = row, quantise each
// token once (scale = max|x| / 127, q = CAST_ROUND(x / scale)) and write that
// row to every destination row of the token's routes.  Dispatch (section 2) is
// the identity on one rank, so the rows go straight to the expert-major A
// matrix of GMM1.
//
// The page sorts with merge-sort instructions sized to its 192 KiB buffer.
// With at most 256 expert keys a counting sort reaches the same stable order
// with two passes over the routes: one workgroup, per-wave LDS histograms,
// wave-ballot peer matching for in-wave ranks.
#include "common.hpp"
#include "kernels.hpp"

namespace megamoe {

constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kMaxExperts = 256;

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

// One workgroup.  The expert ids are first copied to LDS in segments of up to
// kSegRoutes routes (all loads in flight at once), then every pass reads LDS.
// Within a segment, wave w owns a contiguous run of 64-route chunks, so route
// order is preserved: segment s precedes s+1, and inside a segment wave w's
// routes precede wave w+1's.
constexpr int kSegRoutes = 32768;

__device__ __forceinline__ void load_keys(const int32_t *__restrict__ expert_idx, int r0, int n,
                                          int E, int16_t *keys) {
    for (int i = threadIdx.x; i < n; i += kSortThreads) {
        const int e = expert_idx[r0 + i];
        keys[i] = (int16_t)((e >= 0 && e < E) ? e : E);  // E marks a dropped route
    }
}

// Per-wave key counts of one segment into cnt[wave][*] (zeroed by the caller).
__device__ __forceinline__ void count_segment(const int16_t *keys, int n, int E, int nbits,
                                              int (*cnt)[kMaxExperts]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int nchunks = (n + kWave - 1) / kWave;
    const int c_begin = (int)((int64_t)nchunks * wave / kSortWaves);
    const int c_end = (int)((int64_t)nchunks * (wave + 1) / kSortWaves);
    for (int c = c_begin; c < c_end; ++c) {
        const int i = c * kWave + lane;
        const int key = (i < n) ? keys[i] : E;
        const bool ok = key < E;
        const uint64_t m = match_key(key, __ballot(ok), nbits);
        if (ok && (m & below) == 0) cnt[wave][key] += __popcll(m);
    }
}

__global__ __launch_bounds__(kSortThreads) void route_sort_kernel(
    const int32_t *__restrict__ expert_idx, int R, int E, int nbits,
    int32_t *__restrict__ sorted_route, int32_t *__restrict__ expanded_row_idx,
    int32_t *__restrict__ tokens_per_expert, int32_t *__restrict__ expert_cumsum,
    int32_t *__restrict__ err_word) {
    __shared__ int cnt[kSortWaves][kMaxExperts];  // per-wave counts, then row bases
    __shared__ int s_total[kMaxExperts];
    __shared__ int s_run[kMaxExperts];            // next free row of each expert
    __shared__ int s_valid;
    __shared__ int16_t keys[kSegRoutes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int nseg = (R + kSegRoutes - 1) / kSegRoutes;

    if (tid < kMaxExperts) s_total[tid] = 0;
    // Pass A: totals per expert.
    for (int sgi = 0; sgi < nseg; ++sgi) {
        const int r0 = sgi * kSegRoutes, n = min(kSegRoutes, R - r0);
        for (int i = tid; i < kSortWaves * kMaxExperts; i += kSortThreads) (&cnt[0][0])[i] = 0;
        load_keys(expert_idx, r0, n, E, keys);
        __syncthreads();
        count_segment(keys, n, E, nbits, cnt);
        __syncthreads();
        if (tid < E) {
            int v = 0;
            for (int w = 0; w < kSortWaves; ++w) v += cnt[w][tid];
            s_total[tid] += v;
        }
        __syncthreads();
    }

    // Exclusive prefix over experts (wave 0, four experts per lane).
    if (wave == 0) {
        int v[4];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            v[j] = (e < E) ? s_total[e] : 0;
            sum += v[j];
        }
        const int incl = wave_inclusive_scan(sum);
        int run = incl - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            if (e < E) s_run[e] = run;
            run += v[j];
        }
        if (lane == kWave - 1) s_valid = incl;
    }
    __syncthreads();
    if (tid < E) {
        tokens_per_expert[tid] = s_total[tid];
        expert_cumsum[tid] = s_run[tid] + s_total[tid];
    }
    const int valid_rows = s_valid;
    if (tid == 0) err_word[0] = R - valid_rows;

    // Pass B: stable destination rows, segment by segment.
    for (int sgi = 0; sgi < nseg; ++sgi) {
        const int r0 = sgi * kSegRoutes, n = min(kSegRoutes, R - r0);
        if (nseg > 1) {  // a single segment still holds its keys and counts
            __syncthreads();
            for (int i = tid; i < kSortWaves * kMaxExperts; i += kSortThreads)
                (&cnt[0][0])[i] = 0;
            load_keys(expert_idx, r0, n, E, keys);
            __syncthreads();
            count_segment(keys, n, E, nbits, cnt);
        }
        __syncthreads();
        // per-wave row bases of this segment
        if (tid < E) {
            int run = s_run[tid];
            for (int w = 0; w < kSortWaves; ++w) {
                const int v = cnt[w][tid];
                cnt[w][tid] = run;
                run += v;
            }
            s_run[tid] = run;
        }
        __syncthreads();
        const int nchunks = (n + kWave - 1) / kWave;
        const int c_begin = (int)((int64_t)nchunks * wave / kSortWaves);
        const int c_end = (int)((int64_t)nchunks * (wave + 1) / kSortWaves);
        for (int c = c_begin; c < c_end; ++c) {
            const int i = c * kWave + lane;
            const int key = (i < n) ? keys[i] : E;
            const bool ok = key < E;
            const uint64_t m = match_key(key, __ballot(ok), nbits);
            const int rank = __popcll(m & below);
            int dst = -1, base = 0;
            if (ok) {
                base = cnt[wave][key];
                dst = base + rank;
            }
            if (ok && rank == 0) cnt[wave][key] = base + __popcll(m);
            if (i < n) {
                expanded_row_idx[r0 + i] = dst;
                if (dst >= 0) sorted_route[dst] = r0 + i;
            }
        }
    }
    for (int d = valid_rows + tid; d < R; d += kSortThreads) sorted_route[d] = -1;
}

// One workgroup per token.  Each thread owns 16-element chunks of the row
// (two 16-byte loads of fp16, one 16-byte int8 store per destination row).
template <int MAXC>
__global__ __launch_bounds__(256) void quant_scatter_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ expanded_row_idx, int K,
    int top_k, int8_t *__restrict__ gmA, float *__restrict__ pts1) {
    __shared__ float s_red[4];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nchunk = K >> 4;
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)t * K);

    uint4 raw[MAXC][2];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + i * 256;
        if (c < nchunk) {
            raw[i][0] = xr[2 * c];
            raw[i][1] = xr[2 * c + 1];
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

    const int32_t *rows = expanded_row_idx + (size_t)t * top_k;
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
                int q = 0;
                if (amax != 0.0f) {
                    float r = roundf(h2f(bits) / scale);  // CAST_ROUND: half away from zero
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    q = (int)r;
                }
                word |= ((uint32_t)q & 0xffu) << (8 * h);
            }
            packed[j] = word;
        }
        const uint4 out = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        for (int s = 0; s < top_k; ++s) {
            const int d = rows[s];
            if (d >= 0) *reinterpret_cast<uint4 *>(gmA + (size_t)d * K + (size_t)c * 16) = out;
        }
    }
    if (tid == 0) {
        for (int s = 0; s < top_k; ++s) {
            const int d = rows[s];
            if (d >= 0) pts1[d] = scale;
        }
    }
}

hipError_t launch_route_sort(const int32_t *expert_idx, int R, int E, int32_t *sorted_route,
                             int32_t *expanded_row_idx, int32_t *tokens_per_expert,
                             int32_t *expert_cumsum, int32_t *err_word, hipStream_t stream) {
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;  // keys 0..E (E = dropped)
    hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(kSortThreads), 0, stream, expert_idx, R,
                       E, nbits, sorted_route, expanded_row_idx, tokens_per_expert, expert_cumsum,
                       err_word);
    return hipGetLastError();
}

hipError_t launch_quant_scatter(const uint16_t *x, const int32_t *expanded_row_idx, int M, int K,
                                int top_k, int8_t *gmA, float *pts1, hipStream_t stream) {
    const int per_thread = (K / 16 + 255) / 256;
    dim3 grid(M), block(256);
    if (per_thread <= 1)
        hipLaunchKernelGGL(quant_scatter_kernel<1>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1);
    else if (per_thread <= 2)
        hipLaunchKernelGGL(quant_scatter_kernel<2>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1);
    else if (per_thread <= 4)
        hipLaunchKernelGGL(quant_scatter_kernel<4>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1);
    else
        hipLaunchKernelGGL(quant_scatter_kernel<8>, grid, block, 0, stream, x, expanded_row_idx, K,
                           top_k, gmA, pts1);
    return hipGetLastError();
}

}  // namespace megamoe
