// Grouped int8 x int8 GEMM with per-channel dequant to fp16 (GMM1 and GMM2).
//
// Sections 3 ("GMM1") and 5 ("GMM2") of the pto-isa MegaMoE overview page:
// for every expert group of rows, acc = A_group @ W_e in int32 and the tile is
// stored as fp16(fp32(acc) * scale[e, n]) -- the per-channel scale the page
// moves to its FixPipe.  The page's scheduler gives each expert
// ceil(rows / 128) * ceil(N / 256) output tiles and deals them to its cores
// round-robin; the same idea runs on the device here, from the per-expert
// inclusive row counts, without a host round trip:
//
//  * every workgroup rebuilds the per-expert tile prefix in LDS from
//    expert_cumsum (E <= 256 values, one wave scan), so empty experts
//    contribute no tiles and nothing is read back to the host;
//  * the grid is persistent (CUs x occupancy workgroups) and walks the
//    flattened tile list; tiles of one expert are ordered n-block-major with
//    the m-blocks innermost, so the workgroups sharing a weight block are
//    adjacent in the list;
//  * the blockIdx -> list position map is XCD-aware: the hardware deals
//    workgroups round-robin over the 8 XCDs, so positions are assigned so that
//    each XCD works on a contiguous run of the list and its own L2 sees the
//    weight and activation blocks that run shares (the page's 9-column
//    swizzle serves the same purpose on its hardware).
//
// Tile pipeline: 128-byte K slices of A (rows) and B (packed weight rows,
// K-contiguous) are staged global -> VGPR -> LDS with two LDS buffers; the
// load of slice k+1 is in flight while slice k feeds v_mfma_i32_16x16x64_i8.
// LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by (row & 7),
// so the 16 rows an MFMA fragment reads spread over all banks.
#include "common.hpp"
#include "kernels.hpp"

namespace megamoe {


constexpr int kBK = 128;       // K bytes per LDS stage
constexpr int kMaxE = 256;

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct GmmCfg {
    static constexpr int kThreads = WAVES_M * WAVES_N * kWave;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = BN / WAVES_N;
    static constexpr int TM = WM / 16;
    static constexpr int TN = WN / 16;
    static constexpr int kAChunks = BM * kBK / 16 / kThreads;
    static constexpr int kBChunks = BN * kBK / 16 / kThreads;
    static constexpr int kStageBytes = (BM + BN) * kBK;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BM * kBK / 16 % kThreads == 0 && BN * kBK / 16 % kThreads == 0, "load split");
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kBK + ((chunk ^ (row & 7)) << 4);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M *WAVES_N *kWave) void gmm_i8_kernel(GmmParams p) {
    using Cfg = GmmCfg<BM, BN, WAVES_M, WAVES_N>;
    constexpr int NT = Cfg::kThreads;
    constexpr int TM = Cfg::TM, TN = Cfg::TN;

    __shared__ __attribute__((aligned(16))) int8_t smem[2][Cfg::kStageBytes];
    __shared__ int s_tile_start[kMaxE + 1];
    __shared__ int s_row_off[kMaxE];
    __shared__ int s_rows[kMaxE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int E = p.E, N = p.N, Kred = p.Kred;
    const int NB = (N + BN - 1) / BN;

    // Per-expert tile prefix from the inclusive row counts.
    if (wave == 0) {
        int run = 0;
        for (int base = 0; base < E; base += kWave) {
            const int e = base + lane;
            int rows = 0, off = 0;
            if (e < E) {
                const int hi = p.cumsum[e];
                off = e ? p.cumsum[e - 1] : 0;
                rows = hi - off;
            }
            const int tiles = ((rows + BM - 1) / BM) * NB;
            const int incl = wave_inclusive_scan(tiles);
            if (e < E) {
                s_tile_start[e] = run + incl - tiles;
                s_row_off[e] = off;
                s_rows[e] = rows;
            }
            run += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) s_tile_start[E] = run;
    }
    __syncthreads();
    const int total = s_tile_start[E];

    const int G = gridDim.x;  // a multiple of 8
    const int vid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    const int wm0 = (wave / WAVES_N) * Cfg::WM;
    const int wn0 = (wave % WAVES_N) * Cfg::WN;

    for (int t = vid; t < total; t += G) {
        // expert owning tile t: last e with s_tile_start[e] <= t
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tile_start[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int e = lo;
        const int rows_e = s_rows[e];
        const int mb = (rows_e + BM - 1) / BM;
        const int local = t - s_tile_start[e];
        const int nblk = local / mb;
        const int mblk = local - nblk * mb;
        const int row0 = s_row_off[e] + mblk * BM;
        const int rows = min(BM, rows_e - mblk * BM);
        const int n0 = nblk * BN;

        // Per-thread global and LDS addresses of the 16-byte chunks it stages.
        const int8_t *ga[Cfg::kAChunks];
        const int8_t *gb[Cfg::kBChunks];
        int la[Cfg::kAChunks], lb[Cfg::kBChunks];
#pragma unroll
        for (int i = 0; i < Cfg::kAChunks; ++i) {
            const int q = tid + i * NT;
            const int r = q >> 3, kc = q & 7;
            const int rr = min(r, rows - 1);  // rows past the group are computed, never stored
            ga[i] = p.A + (size_t)(row0 + rr) * Kred + kc * 16;
            la[i] = lds_off(r, kc);
        }
#pragma unroll
        for (int i = 0; i < Cfg::kBChunks; ++i) {
            const int q = tid + i * NT;
            const int r = q >> 3, kc = q & 7;
            const int nn = min(n0 + r, N - 1);
            gb[i] = p.B + ((size_t)e * N + nn) * Kred + kc * 16;
            lb[i] = BM * kBK + lds_off(r, kc);
        }

        v4i ra[Cfg::kAChunks], rb[Cfg::kBChunks];
        auto gload = [&](int k0) {
#pragma unroll
            for (int i = 0; i < Cfg::kAChunks; ++i) ra[i] = *reinterpret_cast<const v4i *>(ga[i] + k0);
#pragma unroll
            for (int i = 0; i < Cfg::kBChunks; ++i) rb[i] = *reinterpret_cast<const v4i *>(gb[i] + k0);
        };
        auto swrite = [&](int buf) {
            int8_t *s = smem[buf];
#pragma unroll
            for (int i = 0; i < Cfg::kAChunks; ++i) *reinterpret_cast<v4i *>(s + la[i]) = ra[i];
#pragma unroll
            for (int i = 0; i < Cfg::kBChunks; ++i) *reinterpret_cast<v4i *>(s + lb[i]) = rb[i];
        };

        v4i acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

        const int nk = Kred / kBK;
        gload(0);
        swrite(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) gload((kt + 1) * kBK);
            const int8_t *sa = smem[kt & 1];
            const int8_t *sb = sa + BM * kBK;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int chunk = (lane >> 4) + 4 * kk;
                v4i fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int r = wm0 + 16 * i + (lane & 15);
                    fa[i] = *reinterpret_cast<const v4i *>(sa + lds_off(r, chunk));
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int r = wn0 + 16 * j + (lane & 15);
                    fb[j] = *reinterpret_cast<const v4i *>(sb + lds_off(r, chunk));
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j],
                                                                          0, 0, 0);
            }
            if (kt + 1 < nk) swrite((kt + 1) & 1);
            __syncthreads();
        }

        // Epilogue: per-channel dequant to fp16.  MFMA 16x16 result layout:
        // lane l, element v holds row 4*(l/16)+v, column l%16 of the block.
        const float *sc = p.scale + (size_t)e * N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn0 + 16 * j + (lane & 15);
            if (col >= N) continue;
            const float s = sc[col];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int rl = wm0 + 16 * i + 4 * (lane >> 4) + v;
                    if (rl < rows) {
                        const size_t idx = (size_t)(row0 + rl) * N + col;
                        const int a = acc[i][j][v];
                        p.C[idx] = f2h(keep_f32((float)a * s));
                        if (p.acc_dbg) p.acc_dbg[idx] = a;
                    }
                }
            }
        }
    }
}

// Weight pack: logical [E][Kred][N] -> [E][N][Kred] (K-contiguous rows, so a
// weight block of the GEMM is BN rows of 128 contiguous bytes per K slice).
__global__ __launch_bounds__(256) void pack_kn_to_nk_kernel(const int8_t *__restrict__ w,
                                                            int8_t *__restrict__ wp, int Kred,
                                                            int N) {
    __shared__ int8_t tile[64][65];
    const int e = blockIdx.z;
    const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int8_t *src = w + (size_t)e * Kred * N;
    int8_t *dst = wp + (size_t)e * N * Kred;
    for (int r = ty; r < 64; r += 4) {
        const int k = k0 + r, n = n0 + tx;
        tile[r][tx] = (k < Kred && n < N) ? src[(size_t)k * N + n] : 0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int n = n0 + r, k = k0 + tx;
        if (n < N && k < Kred) dst[(size_t)n * Kred + k] = tile[tx][r];
    }
}

hipError_t launch_pack(const int8_t *w, int8_t *wp, int E, int Kred, int N, hipStream_t stream) {
    dim3 grid((N + 63) / 64, (Kred + 63) / 64, E), block(256);
    hipLaunchKernelGGL(pack_kn_to_nk_kernel, grid, block, 0, stream, w, wp, Kred, N);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile configurations, chosen by the host from the mean rows per expert.
// ---------------------------------------------------------------------------
struct GmmVariant {
    int bm, bn;
    void (*kernel)(GmmParams);
    int threads;
    int occupancy;  // resident workgroups per CU, filled at first use
};

#define MEGAMOE_VARIANT(BM, BN, WMW, WNW)                                                  \
    GmmVariant {                                                                           \
        BM, BN, gmm_i8_kernel<BM, BN, WMW, WNW>, GmmCfg<BM, BN, WMW, WNW>::kThreads, 0 \
    }

static GmmVariant g_variants[] = {
    MEGAMOE_VARIANT(32, 256, 1, 4),    // decode: few rows per expert, weight streaming
    MEGAMOE_VARIANT(64, 256, 2, 2),
    MEGAMOE_VARIANT(128, 128, 2, 2),
    MEGAMOE_VARIANT(256, 128, 2, 2),   // many rows per expert: MFMA bound
};

int gmm_num_variants() { return (int)(sizeof(g_variants) / sizeof(g_variants[0])); }

int gmm_pick_variant(int R, int E) {
    const int mean = (R + E - 1) / E;
    if (mean <= 40) return 0;
    if (mean <= 96) return 1;
    if (mean <= 192) return 2;
    return 3;
}

hipError_t launch_gmm(int variant, const GmmParams &prm, int R, int cu_count,
                      hipStream_t stream) {
    GmmVariant &v = g_variants[variant];
    if (v.occupancy == 0) {
        int occ = 0;
        hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, reinterpret_cast<const void *>(v.kernel), v.threads, 0);
        if (err != hipSuccess) return err;
        v.occupancy = occ > 0 ? occ : 1;
    }
    // Upper bound on the tile count: sum_e ceil(rows_e / BM) <= R / BM + E.
    const int NB = (prm.N + v.bn - 1) / v.bn;
    const long long ub = ((long long)R / v.bm + prm.E) * NB;
    long long g = (long long)cu_count * v.occupancy;
    if (ub < g) g = ub;
    g = (g + 7) / 8 * 8;
    if (g < 8) g = 8;
    hipLaunchKernelGGL(v.kernel, dim3((unsigned)g), dim3(v.threads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace megamoe
