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
// Two tile pipelines feed v_mfma_i32_16x16x64_i8 from LDS, both in 64-byte K
// stages of A rows and B (packed weight) rows: a register-staged one with a
// D-deep prefetch and an LDS double buffer, and one whose stages are copied
// global -> LDS by DMA into an NS-deep ring.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace megamoe {


constexpr int kMaxE = 256;

// ---------------------------------------------------------------------------
// Deeper pipeline: 64-byte K stages, each thread keeps the next D stages of its
// A/B chunks in flight in registers while the LDS double buffer feeds the MFMAs.
// LDS rows are 64 bytes; 16-byte chunk c of row r sits at slot c ^ ((r >> 2) & 3)
// so the 16 rows of a fragment read cover all banks once.
// ---------------------------------------------------------------------------
constexpr int kBK64 = 64;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ int lds_off64(int row, int chunk) {
    return row * kBK64 + ((chunk ^ (((row >> 1) ^ (row >> 3)) & 3)) << 4);
}

// Builds the per-expert tile prefix in LDS (wave 0) and returns the tile count.
template <int BM>
__device__ __forceinline__ int build_tile_prefix(const GmmParams &p, int NB, int *s_tile_start,
                                                 int *s_row_off, int *s_rows) {
    const int lane = threadIdx.x & (kWave - 1);
    if ((threadIdx.x >> 6) == 0) {
        int run = 0;
        for (int base = 0; base < p.E; base += kWave) {
            const int e = base + lane;
            int rows = 0, off = 0;
            if (e < p.E) {
                const int hi = p.cumsum[e];
                off = e ? p.cumsum[e - 1] : 0;
                rows = hi - off;
            }
            const int tiles = ((rows + BM - 1) / BM) * NB;
            const int incl = wave_inclusive_scan(tiles);
            if (e < p.E) {
                s_tile_start[e] = run + incl - tiles;
                s_row_off[e] = off;
                s_rows[e] = rows;
            }
            run += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) s_tile_start[p.E] = run;
    }
    __syncthreads();
    return s_tile_start[p.E];
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int D>
__global__ __launch_bounds__(WAVES_M *WAVES_N *kWave) void gmm_i8_pipe_kernel(GmmParams p) {
    constexpr int NT = WAVES_M * WAVES_N * kWave;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int ACH = BM * 4, BCH = BN * 4;            // 16-byte chunks per stage
    constexpr int AL = (ACH + NT - 1) / NT, BL = (BCH + NT - 1) / NT;
    constexpr int kStage = (BM + BN) * kBK64;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");

    __shared__ __attribute__((aligned(16))) int8_t smem[2][kStage];
    __shared__ int s_tile_start[kMaxE + 1];
    __shared__ int s_row_off[kMaxE];
    __shared__ int s_rows[kMaxE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int N = p.N, Kred = p.Kred;
    const int NB = (N + BN - 1) / BN;
    const int total = build_tile_prefix<BM>(p, NB, s_tile_start, s_row_off, s_rows);

    const int G = gridDim.x;  // a multiple of 8
    const int vid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;

    for (int t = vid; t < total; t += G) {
        int lo = 0, hi = p.E - 1;
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

        const int8_t *ga[AL];
        const int8_t *gb[BL];
        int la[AL], lb[BL];
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int q = min(tid + i * NT, ACH - 1);
            const int r = q >> 2, kc = q & 3;
            ga[i] = p.A + (size_t)(row0 + min(r, rows - 1)) * Kred + kc * 16;
            la[i] = lds_off64(r, kc);
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const int q = min(tid + i * NT, BCH - 1);
            const int r = q >> 2, kc = q & 3;
            gb[i] = p.B + ((size_t)e * N + min(n0 + r, N - 1)) * Kred + kc * 16;
            lb[i] = BM * kBK64 + lds_off64(r, kc);
        }
        // Threads past the chunk count (only when a stage has fewer chunks than
        // threads) load a duplicate chunk and skip the LDS write.
        constexpr bool kAFull = (ACH % NT) == 0, kBFull = (BCH % NT) == 0;
        bool aw[AL], bw[BL];
#pragma unroll
        for (int i = 0; i < AL; ++i) aw[i] = kAFull || (tid + i * NT) < ACH;
#pragma unroll
        for (int i = 0; i < BL; ++i) bw[i] = kBFull || (tid + i * NT) < BCH;

        v4i ra[D][AL], rb[D][BL];
        v4i acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

        const int nk = Kred / kBK64;
        // Stage s of the K loop reads K bytes [64 s, 64 s + 64).  Prefetches past
        // the last stage re-read the last stage (never used), so the steady-state
        // loop has no data-dependent branches around its loads.
        auto kofs = [&](int s) { return min(s, nk - 1) * kBK64; };
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int k0 = kofs(u);
#pragma unroll
            for (int i = 0; i < AL; ++i) ra[u][i] = *reinterpret_cast<const v4i *>(ga[i] + k0);
#pragma unroll
            for (int i = 0; i < BL; ++i) rb[u][i] = *reinterpret_cast<const v4i *>(gb[i] + k0);
        }
        {
            int8_t *s0 = smem[0];
#pragma unroll
            for (int i = 0; i < AL; ++i)
                if (aw[i]) *reinterpret_cast<v4i *>(s0 + la[i]) = ra[0][i];
#pragma unroll
            for (int i = 0; i < BL; ++i)
                if (bw[i]) *reinterpret_cast<v4i *>(s0 + lb[i]) = rb[0][i];
        }
        __syncthreads();

        const int nk_pad = (nk + D - 1) / D * D;
        for (int kt0 = 0; kt0 < nk_pad; kt0 += D) {
            static_for<0, D>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                constexpr int nu = (u + 1) % D;  // register set holding stage kt + 1
                const int kt = kt0 + u;
                {
                    const int k0 = kofs(kt + D);
#pragma unroll
                    for (int i = 0; i < AL; ++i)
                        ra[u][i] = *reinterpret_cast<const v4i *>(ga[i] + k0);
#pragma unroll
                    for (int i = 0; i < BL; ++i)
                        rb[u][i] = *reinterpret_cast<const v4i *>(gb[i] + k0);
                }
                // stages past nk exist only in the last round; they skip the
                // MFMAs with a uniform branch
                if (kt < nk) {
                    const int8_t *sa = smem[kt & 1];
                    const int8_t *sb = sa + BM * kBK64;
                    const int chunk = lane >> 4;
                    v4i fa[TM], fb[TN];
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const int r = wm0 + 16 * i + (lane & 15);
                        fa[i] = *reinterpret_cast<const v4i *>(sa + lds_off64(r, chunk));
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int r = wn0 + 16 * j + (lane & 15);
                        fb[j] = *reinterpret_cast<const v4i *>(sb + lds_off64(r, chunk));
                    }
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j],
                                                                              acc[i][j], 0, 0, 0);
                }
                int8_t *sn = smem[(kt + 1) & 1];
#pragma unroll
                for (int i = 0; i < AL; ++i)
                    if (aw[i]) *reinterpret_cast<v4i *>(sn + la[i]) = ra[nu][i];
#pragma unroll
                for (int i = 0; i < BL; ++i)
                    if (bw[i]) *reinterpret_cast<v4i *>(sn + lb[i]) = rb[nu][i];
                __syncthreads();
            });
        }

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

// ---------------------------------------------------------------------------
// DMA pipeline: the K stages (64 bytes of A rows and B rows each) are copied
// global -> LDS by global_load_lds_dwordx4 into an NS-deep ring, so NS-1
// stages are in flight without any staging registers.  Each wave issues the
// DMA for 1 KB blocks of a stage (one 16-byte chunk per lane, lanes writing
// consecutive LDS chunks); the global address of a lane is chosen so that the
// LDS image is the swizzled layout below.  Stage kt is complete for a wave when
// at most (NS - 2) stages of its DMA are outstanding; a barrier then makes all
// waves' chunks visible.
//
// Layout: 64-byte rows; 16-byte chunk c of row r sits at slot
// c ^ (((r >> 1) ^ (r >> 3)) & 3).  Any 8 consecutive rows (one 128-byte bank
// sweep) and any 16 consecutive rows read with one chunk index hit distinct
// bank groups, for both reads and DMA writes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int lds_off64s(int row, int chunk) {
    return row * kBK64 + ((chunk ^ swz64(row)) << 4);
}

// The DMA copies are issued from inline assembly, so the compiler's wait-count
// pass does not see them and cannot serialise the ring (it would otherwise
// wait for every outstanding copy before any LDS read).  The waits on them are
// explicit.  Vector-memory operations complete in issue order, so the
// compiler's own waits for its loads stay correct (they may only over-wait).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// One 16-byte chunk per lane, global -> LDS; lane i writes LDS bytes
// [lds_base + 16 i, lds_base + 16 i + 16).  lds_base is wave-uniform (M0).
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_base), "v"(gptr)
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_cvoid;

template <int BM, int BN, int WAVES_M, int WAVES_N, int NS>
__global__ __launch_bounds__(WAVES_M *WAVES_N *kWave) void gmm_i8_dma_kernel(GmmParams p) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int kStage = (BM + BN) * kBK64;
    constexpr int kBlocks = kStage / 1024;           // 1 KB DMA blocks per stage
    constexpr int LPW = kBlocks / NW;                // DMA instructions per wave per stage
    static_assert(kStage % 1024 == 0 && kBlocks % NW == 0, "stage must split over the waves");
    static_assert((BM * kBK64) % 1024 == 0, "A region must be whole 1 KB blocks");
    static_assert(NS >= 2 && WM % 16 == 0 && WN % 16 == 0, "shape");

    __shared__ __attribute__((aligned(1024))) int8_t smem[NS][kStage];
    __shared__ int s_tile_start[kMaxE + 1];
    __shared__ int s_row_off[kMaxE];
    __shared__ int s_rows[kMaxE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int N = p.N, Kred = p.Kred;
    const int NB = (N + BN - 1) / BN;
    const int total = build_tile_prefix<BM>(p, NB, s_tile_start, s_row_off, s_rows);

    const int G = gridDim.x;  // a multiple of 8
    const int vid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    const int nk = Kred / kBK64;

    for (int t = vid; t < total; t += G) {
        int lo = 0, hi = p.E - 1;
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

        // Source of this lane's chunk in each of the wave's DMA blocks.
        const int8_t *src[LPW];
        int dst[LPW];
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int b = wave + j * NW;               // block within the stage
            const int pch = b * 64 + lane;             // LDS chunk this lane fills
            dst[j] = b * 1024;
            if (pch < BM * 4) {
                const int r = pch >> 2, kc = (pch & 3) ^ swz64(pch >> 2);
                src[j] = p.A + (size_t)(row0 + min(r, rows - 1)) * Kred + kc * 16;
            } else {
                const int q = pch - BM * 4;
                const int r = q >> 2, kc = (q & 3) ^ swz64(q >> 2);
                src[j] = p.B + ((size_t)e * N + min(n0 + r, N - 1)) * Kred + kc * 16;
            }
        }
        const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(&smem[0][0]));
        auto issue = [&](int stage) {
            const int k0 = min(stage, nk - 1) * kBK64;  // past-the-end stages re-read the last
            const uint32_t sbase = ring + (uint32_t)((stage % NS) * kStage);
#pragma unroll
            for (int j = 0; j < LPW; ++j)
                dma16(src[j] + k0, __builtin_amdgcn_readfirstlane(sbase + dst[j]));
        };

        v4i acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

#pragma unroll
        for (int s = 0; s < NS - 1; ++s) issue(s);

        for (int kt = 0; kt < nk; ++kt) {
            wait_vmcnt<(NS - 2) * LPW>();
            __syncthreads();
            issue(kt + NS - 1);
            const int8_t *sa = smem[kt % NS];
            const int8_t *sb = sa + BM * kBK64;
            const int chunk = lane >> 4;
            v4i fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm0 + 16 * i + (lane & 15);
                fa[i] = *reinterpret_cast<const v4i *>(sa + lds_off64s(r, chunk));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn0 + 16 * j + (lane & 15);
                fb[j] = *reinterpret_cast<const v4i *>(sb + lds_off64s(r, chunk));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0,
                                                                      0, 0);
        }
        // drain the prefetches past the end before the ring is reused
        wait_vmcnt<0>();
        __syncthreads();

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
// Few rows per expert: the GEMM streams weights (HBM bound), so small BM with
// wide weight blocks and a register prefetch keeps every CU pulling weights.
// Many rows per expert: MFMA bound; 256x256 tiles with the DMA ring.
// ---------------------------------------------------------------------------
struct GmmVariant {
    int bm, bn;
    void (*kernel)(GmmParams);
    int threads;
    int occupancy;  // resident workgroups per CU, filled at first use
};

static GmmVariant g_variants[] = {
    {64, 256, gmm_i8_pipe_kernel<64, 256, 1, 4, 3>, 256, 0},
    {128, 256, gmm_i8_pipe_kernel<128, 256, 2, 4, 3>, 512, 0},
    {256, 256, gmm_i8_dma_kernel<256, 256, 2, 4, 4>, 512, 0},
};

int gmm_num_variants() { return (int)(sizeof(g_variants) / sizeof(g_variants[0])); }

int gmm_pick_variant(int R, int E) {
    const int mean = (R + E - 1) / E;
    if (mean <= 96) return 0;
    if (mean <= 192) return 1;
    return 2;
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
