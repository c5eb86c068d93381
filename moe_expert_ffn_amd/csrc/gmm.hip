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
// LDS rows are 64 bytes; 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 3),
// the conflict-free pattern for the fragment reads.
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
    return row * kBK64 + ((chunk ^ ((row >> 1) & 3)) << 4);
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

// The MFMAs compute the transposed tile (weight fragment as the first operand,
// activation fragment as the second), so in the 16x16 result of fragment
// (i, j) lane l holds output row 16 i + (l & 15) and the 4 consecutive output
// columns 16 j + 4 (l >> 4) + v, v = 0..3.  The store is then one 8-byte fp16
// quad per lane (the per-channel scales one float4), and the 4 lane groups of
// a row write 32 contiguous bytes.
__device__ __forceinline__ v4i mfma_t(const v4i &b_frag, const v4i &a_frag, const v4i &acc) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(b_frag, a_frag, acc, 0, 0, 0);
}

template <int TM, int TN>
__device__ __forceinline__ void store_tile(const GmmParams &p, const v4i (&acc)[TM][TN], int e,
                                           int row0, int rows, int n0, int wm0, int wn0,
                                           int lane) {
    const int N = p.N;
    const float *sc = p.scale + (size_t)e * N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn0 + 16 * j + 4 * (lane >> 4);
        if (col >= N) continue;  // N is a multiple of 16, so col + 3 < N here
        const float4 s4 = *reinterpret_cast<const float4 *>(sc + col);
        const float s[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rl = wm0 + 16 * i + (lane & 15);
            if (rl >= rows) continue;
            const size_t idx = (size_t)(row0 + rl) * N + col;
            uint32_t h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) h[v] = f2h(keep_f32((float)acc[i][j][v] * s[v]));
            *reinterpret_cast<uint2 *>(p.C + idx) =
                make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            if (p.acc_dbg) *reinterpret_cast<v4i *>(p.acc_dbg + idx) = acc[i][j];
        }
    }
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
                            acc[i][j] = mfma_t(fb[j], fa[i], acc[i][j]);
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

        store_tile<TM, TN>(p, acc, e, row0, rows, n0, wm0, wn0, lane);
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
// Layout: 64-byte rows; 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 3).
// Measured with the LDS bank-conflict counter on gfx950, this is the pattern
// for which the fragment reads (16 consecutive rows, one chunk index per lane
// group) see no conflicts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz64(int row) { return (row >> 1) & 3; }
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
                    acc[i][j] = mfma_t(fb[j], fa[i], acc[i][j]);
        }
        // drain the prefetches past the end before the ring is reused
        wait_vmcnt<0>();
        __syncthreads();

        store_tile<TM, TN>(p, acc, e, row0, rows, n0, wm0, wn0, lane);
    }
}

// ---------------------------------------------------------------------------
// Shifted DMA pipeline with register double-buffered fragments.
//
// A stage is S sub-steps of 64 K-bytes ([S][BM + BN rows][64 B], swizzled as
// above), copied by DMA into an NS-deep ring (NS >= 3).  Fragments for the
// next sub-step are read from LDS while the MFMAs of the current one run.  The
// barrier that publishes stage kt+1 sits right before the prefetch of its first
// sub-step, i.e. at the start of the last sub-step of stage kt; the DMA of
// stage kt+NS-1 is issued right after it, into the slot of stage kt-1 (whose
// last fragments were read before that barrier).  Stage kt+1 was issued NS-2
// stages earlier, so at the barrier NS-3 stages may still be in flight.
// ---------------------------------------------------------------------------
// SKIP: waves whose rows all lie past the group's end skip their fragment
// reads and MFMAs (costs registers; off for the 128-register configuration).
template <int BM, int BN, int WAVES_M, int WAVES_N, int S, int NS, bool SKIP = true>
__global__ __launch_bounds__(WAVES_M *WAVES_N *kWave) void gmm_i8_ring_kernel(GmmParams p) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int kSub = (BM + BN) * kBK64;          // bytes of one 64-byte K slice
    constexpr int kStage = kSub * S;
    constexpr int kBlocks = kStage / 1024;
    constexpr int LPW = kBlocks / NW;
    static_assert(kSub % 1024 == 0 && kBlocks % NW == 0, "stage must split over the waves");
    static_assert((BM * kBK64) % 1024 == 0, "A region must be whole 1 KB blocks");
    static_assert(NS >= 3 && WM % 16 == 0 && WN % 16 == 0, "shape");

    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * kStage];
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
    const int nst = Kred / (kBK64 * S);              // stages; Kred is a multiple of 64 S
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(&smem[0]));

    // LDS byte offsets of this lane's fragment rows inside a 64-byte slice
    int fa_off[TM], fb_off[TN];
    {
        const int chunk = lane >> 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) fa_off[i] = lds_off64s(wm0 + 16 * i + (lane & 15), chunk);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb_off[j] = BM * kBK64 + lds_off64s(wn0 + 16 * j + (lane & 15), chunk);
    }

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
        // a wave whose rows all lie past the group's end has nothing to multiply
        const bool live = !SKIP || wm0 < rows;

        // DMA sources: block b of a stage is sub-step b / (kSub/1024), and
        // inside it the lane fills LDS chunk pch of the slice.
        const int8_t *src[LPW];
        uint32_t dst[LPW];
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int b = wave + j * NW;
            const int ss = b / (kSub / 1024);
            const int pch = (b % (kSub / 1024)) * 64 + lane;
            dst[j] = (uint32_t)(b * 1024);
            if (pch < BM * 4) {
                const int r = pch >> 2, kc = (pch & 3) ^ swz64(pch >> 2);
                src[j] = p.A + (size_t)(row0 + min(r, rows - 1)) * Kred + ss * kBK64 + kc * 16;
            } else {
                const int q = pch - BM * 4;
                const int r = q >> 2, kc = (q & 3) ^ swz64(q >> 2);
                src[j] = p.B + ((size_t)e * N + min(n0 + r, N - 1)) * Kred + ss * kBK64 + kc * 16;
            }
        }
        auto issue = [&](int stage) {
            const int k0 = min(stage, nst - 1) * (kBK64 * S);
            const uint32_t sbase = ring + (uint32_t)((stage % NS) * kStage);
#pragma unroll
            for (int j = 0; j < LPW; ++j)
                dma16(src[j] + k0, __builtin_amdgcn_readfirstlane(sbase + dst[j]));
        };
        auto frag = [&](int stage, int ss, v4i *xa, v4i *xb) {
            if (!live) return;
            const int8_t *base = smem + (stage % NS) * kStage + ss * kSub;
#pragma unroll
            for (int i = 0; i < TM; ++i) xa[i] = *reinterpret_cast<const v4i *>(base + fa_off[i]);
#pragma unroll
            for (int j = 0; j < TN; ++j) xb[j] = *reinterpret_cast<const v4i *>(base + fb_off[j]);
        };

        v4i acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
        v4i fa[2][TM], fb[2][TN];

#pragma unroll
        for (int st = 0; st < NS - 1; ++st) issue(st);
        wait_vmcnt<(NS - 2) * LPW>();
        __syncthreads();
        frag(0, 0, fa[0], fb[0]);

        // two stages per trip so that the register set of every sub-step is
        // known at compile time (set = global sub-step index & 1)
        for (int kt0 = 0; kt0 < nst; kt0 += 2) {
            static_for<0, 2 * S>([&](auto gc) {
                constexpr int g = decltype(gc)::value;   // sub-step within the trip
                constexpr int u = g / S, ss = g % S;
                constexpr int cur = g & 1, nxt = cur ^ 1;
                const int kt = kt0 + u;
                if (kt < nst) {
                    if constexpr (ss == S - 1) {
                        wait_vmcnt<(NS - 3) * LPW>();
                        __syncthreads();
                        issue(kt + NS - 1);
                        frag(kt + 1, 0, fa[nxt], fb[nxt]);
                    } else {
                        frag(kt, ss + 1, fa[nxt], fb[nxt]);
                    }
                    if (live) {
#pragma unroll
                        for (int i = 0; i < TM; ++i)
#pragma unroll
                            for (int j = 0; j < TN; ++j)
                                acc[i][j] = mfma_t(fb[cur][j], fa[cur][i], acc[i][j]);
                    }
                }
            });
        }
        // drain the prefetches past the end before the ring is reused
        wait_vmcnt<0>();
        __syncthreads();

        store_tile<TM, TN>(p, acc, e, row0, rows, n0, wm0, wn0, lane);
    }
}

// ---------------------------------------------------------------------------
// Direct pipeline: no LDS.  Each wave streams the fragments it multiplies
// straight from global memory (L1/L2) into registers: lane l loads 16 bytes of
// row (l & 15) at K chunk (l >> 4) of a 64-byte slice, which is exactly the
// MFMA operand layout, for both the activation rows and the K-contiguous
// weight rows.  Fragments shared by several waves are served by the caches.
// A ring of D+1 register sets keeps D slices in flight; there are no barriers
// and no LDS writes, the two costs that bound the LDS-staged pipelines.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, int D>
__global__ __launch_bounds__(WAVES_M *WAVES_N *kWave) void gmm_i8_direct_kernel(GmmParams p) {
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int NSET = D + 1;
    static_assert(WM % 16 == 0 && WN % 16 == 0 && D >= 1, "shape");

    __shared__ int s_tile_start[kMaxE + 1];
    __shared__ int s_row_off[kMaxE];
    __shared__ int s_rows[kMaxE];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
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

        const int8_t *pa[TM];
        const int8_t *pb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = min(wm0 + 16 * i + (lane & 15), rows - 1);
            pa[i] = p.A + (size_t)(row0 + r) * Kred + (lane >> 4) * 16;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = min(n0 + wn0 + 16 * j + (lane & 15), N - 1);
            pb[j] = p.B + ((size_t)e * N + n) * Kred + (lane >> 4) * 16;
        }

        v4i fa[NSET][TM], fb[NSET][TN];
        v4i acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

        auto load = [&](int stage, v4i *xa, v4i *xb) {
            const int k0 = min(stage, nk - 1) * kBK64;  // past-the-end slices re-read the last
#pragma unroll
            for (int i = 0; i < TM; ++i) xa[i] = *reinterpret_cast<const v4i *>(pa[i] + k0);
#pragma unroll
            for (int j = 0; j < TN; ++j) xb[j] = *reinterpret_cast<const v4i *>(pb[j] + k0);
        };
#pragma unroll
        for (int u = 0; u < D; ++u) load(u, fa[u], fb[u]);

        for (int kt0 = 0; kt0 < nk; kt0 += NSET) {
            static_for<0, NSET>([&](auto uc) {
                constexpr int u = decltype(uc)::value;          // set holding slice kt
                constexpr int ld = (u + D) % NSET;              // set for slice kt + D
                const int kt = kt0 + u;
                if (kt < nk) {
                    load(kt + D, fa[ld], fb[ld]);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = mfma_t(fb[u][j], fa[u][i], acc[i][j]);
                }
            });
        }

        store_tile<TM, TN>(p, acc, e, row0, rows, n0, wm0, wn0, lane);
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
    {64, 256, gmm_i8_ring_kernel<64, 256, 1, 4, 1, 6>, 256, 0},
    {128, 256, gmm_i8_ring_kernel<128, 256, 2, 4, 1, 4>, 512, 0},
    {256, 256, gmm_i8_ring_kernel<256, 256, 4, 4, 1, 4, false>, 1024, 0},
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
