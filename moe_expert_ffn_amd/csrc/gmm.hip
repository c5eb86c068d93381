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
//  * every workgroup rebuilds the tile numbering in LDS from expert_cumsum
//    (E <= 256 values, one wave scan per cost class), so empty experts
//    contribute no tiles and nothing is read back to the host;
//  * an expert's rows are split evenly over its m-blocks, and a tile's cost
//    class is its number of live 64-row blocks; tiles are numbered largest
//    class first, then by expert, n-block and m-block, so the m-blocks that
//    share a weight block are adjacent;
//  * the grid is persistent (CUs x occupancy workgroups) and deals the tiles
//    in rounds of one tile per workgroup, backward in odd rounds when costs
//    differ (a snake, close to a longest-first schedule); a sparse last round
//    is cut into row pieces;
//  * the blockIdx -> position map is XCD-aware: the hardware deals
//    workgroups round-robin over the 8 XCDs, so positions are assigned so that
//    each XCD works on a contiguous run of tiles and its own L2 sees the
//    weight and activation blocks that run shares (the page's 9-column
//    swizzle serves the same purpose on its hardware).
//
// Tiles are fed to v_mfma_i32_16x16x64_i8 from LDS: 64-byte K slices of A rows
// and packed weight rows are copied global -> LDS by DMA into a ring of
// stages, fragments are double-buffered in registers.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "swiglu_row.hpp"

namespace megamoe {

constexpr int kMaxE = 256;
constexpr int kMaxWorkgroups = 1024;  // GEMM grid bound (4 workgroups per CU at most)
constexpr int kBK64 = 64;  // K bytes per MFMA step (one 64-byte slice per row)
constexpr int kPackRows = 256;                 // weight rows per packed n-block (= BN)
constexpr int kPackBlock = kPackRows * kBK64;  // bytes of one packed (n-block, K slice)

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Tile schedule.  Expert e's rows are split over its m-blocks =
// ceil(rows / BM) as evenly as whole units (UNIT rows, one wave row block)
// allow -- 530 rows become 192 + 192 + 146, not 256 + 256 + 18, since a ragged
// last block would stream a full tile's weights for a fraction of the MFMA
// work.  With nu = ceil(rows / UNIT) units, the first ur = nu % mb m-blocks get
// uq + 1 units and the rest uq = nu / mb.  A tile's cost class is its unit
// count c in 1..U (U = BM / UNIT), which its MFMA time follows.
//
// Tiles are numbered cost class by cost class, the largest first; inside a
// class by expert, then n-block, then m-block, so the m-blocks that share a
// weight block stay adjacent.  s_pre[c - 1][e] counts the tiles of class c of
// the experts before e (s_pre[c - 1][E]: all of class c).  With U = 1 this is
// the plain expert / n-block / m-block order.
//
// s_pad (nullable): s_pad[e] = the experts before e with an odd row count,
// the offset of expert e's rows in the row-paired layout of A (a_pair).
template <int BM, int UNIT>
__device__ __forceinline__ int build_schedule(const GmmParams &p, int NB, int (*s_pre)[kMaxE + 1],
                                              int *s_row_off, int *s_rows, int *s_pad = nullptr) {
    constexpr int U = BM / UNIT;
    const int lane = threadIdx.x & (kWave - 1);
    if ((threadIdx.x >> 6) == 0) {
        int run[U];
        int odd_run = 0;
#pragma unroll
        for (int c = 0; c < U; ++c) run[c] = 0;
        for (int base = 0; base < p.E; base += kWave) {
            const int e = base + lane;
            int rows = 0, off = 0;
            if (e < p.E) {
                const int hi = p.cumsum[e];
                off = e ? p.cumsum[e - 1] : 0;
                rows = hi - off;
            }
            const int mb = (rows + BM - 1) / BM;
            const int nu = (rows + UNIT - 1) / UNIT;
            const int uq = mb ? nu / mb : 0, ur = mb ? nu - uq * mb : 0;
#pragma unroll
            for (int c = 1; c <= U; ++c) {
                const int blocks = (c == uq + 1 ? ur : 0) + (c == uq ? mb - ur : 0);
                const int tiles = blocks * NB;
                const int incl = wave_inclusive_scan(tiles);
                if (e < p.E) s_pre[c - 1][e] = run[c - 1] + incl - tiles;
                run[c - 1] += __shfl(incl, kWave - 1, kWave);
            }
            if (e < p.E) {
                s_row_off[e] = off;
                s_rows[e] = rows;
            }
            if (s_pad) {
                const int odd = rows & 1;
                const int incl = wave_inclusive_scan(odd);
                if (e < p.E) s_pad[e] = odd_run + incl - odd;
                odd_run += __shfl(incl, kWave - 1, kWave);
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int c = 0; c < U; ++c) s_pre[c][p.E] = run[c];
        }
    }
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int c = 0; c < U; ++c) total += s_pre[c][p.E];
    return total;
}

// Cost class of tile t (largest class first in the numbering)
template <int U>
__device__ __forceinline__ int tile_class(int t, int E, const int (*s_pre)[kMaxE + 1]) {
    int c = U;
    while (c > 1 && t >= s_pre[c - 1][E]) t -= s_pre[--c][E];
    return c;
}

struct TileRows {
    int e, row0, rows, nblk;
};
template <int BM, int UNIT>
__device__ __forceinline__ TileRows tile_rows(int t, int E, const int (*s_pre)[kMaxE + 1],
                                              const int *s_row_off, const int *s_rows) {
    constexpr int U = BM / UNIT;
    int c = U;
    while (c > 1 && t >= s_pre[c - 1][E]) t -= s_pre[--c][E];
    const int *pre = s_pre[c - 1];
    int lo = 0, hi = E - 1;  // last expert whose class-c tiles start at or before t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    const int rows_e = s_rows[lo];
    const int mb = (rows_e + BM - 1) / BM;
    const int nu = (rows_e + UNIT - 1) / UNIT;
    const int uq = nu / mb, ur = nu - uq * mb;
    const bool upper = ur > 0 && c == uq + 1;  // the first ur m-blocks
    const int m = upper ? ur : mb - ur;        // m-blocks of this class
    const int local = t - pre[lo];
    const int nblk = local / m;
    const int mblk = (upper ? 0 : ur) + (local - nblk * m);
    const int first = UNIT * (mblk * uq + min(mblk, ur));
    const int last = min(rows_e, UNIT * ((mblk + 1) * uq + min(mblk + 1, ur)));
    return TileRows{lo, s_row_off[lo] + first, last - first, nblk};
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

// LDS layout of a K slice: 64-byte rows; 16-byte chunk c of row r sits at
// slot c ^ ((r >> 1) & 3).  Measured with the LDS bank-conflict counter on
// gfx950, this is the pattern for which the fragment reads (16 consecutive
// rows, one chunk index per lane group) see no conflicts.
__device__ __forceinline__ int swz64(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int lds_off64s(int row, int chunk) {
    return row * kBK64 + ((chunk ^ swz64(row)) << 4);
}

// The DMA copies are issued from inline assembly, so the compiler's wait-count
// pass does not see them and cannot serialise the ring (it would otherwise
// wait for every outstanding copy before any LDS read).  The waits on them are
// explicit.  Vector-memory operations complete in issue order, so the
// compiler's own waits for its loads stay correct, but they also wait for
// every copy issued before those loads.  A spill reload placed between a
// tile's copies and its K loop, or inside the loop, therefore drains the
// ring; in the 256-row kernel (all 128 registers in use) the reloads sit
// after each tile's K loop, and edits that moved them cost 3-12%.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// One 16-byte chunk per lane, global -> LDS; lane i writes LDS bytes
// [lds_base + 16 i, lds_base + 16 i + 16).  lds_base is wave-uniform (M0).
// The source is a wave-uniform base (a scalar register pair) plus a 32-bit
// per-lane byte offset, so each copy stream holds one vector register.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_base), "v"(voff), "s"(sbase)
        : "memory", "m0");
}

// The same copy with the non-temporal hint (streamed data: the weights).
__device__ __forceinline__ void dma16_nt(const void *sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(lds_base), "v"(voff), "s"(sbase)
        : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One dword per lane, global -> LDS (lane i writes LDS bytes [lds_base + 4 i,
// lds_base + 4 i + 4)); used for the per-channel scales of a tile.
__device__ __forceinline__ void dma4(const void *gptr, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dword %1, off"
        :
        : "s"(lds_base), "v"(gptr)
        : "memory", "m0");
}

// ---------------------------------------------------------------------------
// Ring pipeline.  A stage is one 64-byte K slice of the tile's BM A rows and
// BN weight rows ([BM + BN rows][64 B], swizzled as above), copied by DMA
// into an NS-slot ring.  Fragments for the next slice are read from LDS while
// the MFMAs of the current one run, so the fragments of stage kt+1 are read
// during stage kt.  The barrier that publishes stage kt+1 sits at the start of
// stage kt; at that point every wave has finished reading stage kt (its
// fragments went to registers during stage kt-1), so its slot is refilled with
// stage kt+NS right after the barrier.  Stage kt+1 was issued NS-1 stages
// earlier and NS-2 younger stages may still be in flight when it is awaited.
// Copies are issued for real stages only; over the last NS-2 stages of a tile,
// where fewer younger copies exist, the wait is for all of them.
//
// Weights are read from the K-slice-major packed layout (see the pack
// kernel): one stage of a tile's weight rows is a single contiguous 16 KB
// block, and the blocks of all tiles for one K slice are adjacent.
//
// The tile's per-channel scales are copied to one of two LDS slots (by tile
// parity) when the tile starts, ahead of its stage copies in issue order, so
// the first stage wait covers them and the epilogue reads them from LDS.
//
// SKIP: a wave whose rows all lie past the group's end (ragged last m-block of
// an expert) runs a copy of the K loop without fragment reads and MFMAs; it
// still issues its share of the copies and joins every barrier.  Each SIMD
// hosts waves of every row block in the WAVES_M = 4 layout, so a tile with r
// live row blocks costs about r / WAVES_M of a full one in MFMA time.
// ---------------------------------------------------------------------------
template <int TM, int TN>
__device__ __forceinline__ void store_acc_dbg(const GmmParams &p, const v4i (&acc)[TM][TN], int row0,
                                              int rows, int n0, int wm0, int wn0, int lane) {
    const int N = p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn0 + 16 * j + 4 * (lane >> 4);
        if (col >= N) continue;  // N is a multiple of 16, so col + 3 < N here
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rl = wm0 + 16 * i + (lane & 15);
            if (rl >= rows) continue;
            *reinterpret_cast<v4i *>(p.acc_dbg + (size_t)(row0 + rl) * N + col) = acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// SwiGLU in GMM1's last round (the page's overlap of the vector stage with the
// matrix stages: its SwiGLU segments start as soon as their GMM1 rows exist).
// With F full rounds and a sparse last round F, the workgroups without a tile
// in round F run SwiGLU, while the others finish the last tiles, on the rows
// of m-blocks that have no tile in rounds F - 1 and F.
//  * Producers never wait: each workgroup, once it has stored its tile of
//    round F - 2, makes its stores visible at device scope (L2 write-back)
//    and counts itself in sync[0].  A workgroup that is free in round F has
//    finished round F - 1 itself, so by then every workgroup has normally
//    counted itself long before and the wait below ends at once.
//  * The free workgroups wait until all G have counted themselves (bounded:
//    tail_spin polls; a workgroup that gives up does no SwiGLU work), then
//    take 64-row chunks of rows from the counter sync[1], and stop taking
//    them as soon as every workgroup with a last-round tile has finished
//    (sync[2]), so that this work never makes GMM1 longer.
//  * Rows done here get tail_done[row] = 1; the SwiGLU kernel that runs after
//    GMM1 does every other row.
// The rows' arithmetic is swiglu_row.hpp, the same as the SwiGLU kernel's.
// ---------------------------------------------------------------------------
// What the last-round SwiGLU needs from GmmParams, passed by value (taking
// the kernel parameter's address would move it to memory for the K loop too).
struct TailArgs {
    const uint16_t *C;  // GMM1 output [R, 2I]
    int8_t *q2;
    float *pts2;
    const float *pts1;
    uint32_t *sync;     // [3]: arrivals, row chunks taken, last-round workgroups done
    uint8_t *done;
    const int32_t *prow;  // nullable: q2 row-paired, row r at paired row prow[r]
    int I, spin, E;
};

__device__ __forceinline__ void tail_arrive(uint32_t *sync) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's tile stores are done
    __syncthreads();
    // release at device scope (the L2 write-back covers every wave's stores),
    // then the count; the counters are accessed at system scope, so their
    // read-modify-writes from all XCDs meet in memory, not in one XCD's L2
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

__device__ __forceinline__ uint32_t tail_load(const uint32_t *c) {
    return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Waits for all G arrivals (bounded); true if they all came.
__device__ __forceinline__ bool tail_wait(const TailArgs &p, int G, int *s_go) {
    if (threadIdx.x == 0) {
        int go = 0;
        if (p.spin >= 0) {
            for (int n = 0;; ++n) {
                if (tail_load(p.sync) >= (uint32_t)G) {
                    go = 1;
                    break;
                }
                if (n >= p.spin) break;
                __builtin_amdgcn_s_sleep(8);
            }
        }
        // acquire at device scope: stale lines of other XCDs' stores are
        // dropped from this CU's L1 and this XCD's L2
        if (go) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_go = go;
    }
    __syncthreads();  // orders the other waves' loads after the acquire
    return *s_go != 0;
}

// The part of a 256-row GMM1 workgroup after its tiles.  The schedule values
// it needs are recomputed here and its arguments come from LDS, so that none
// of them is kept in registers across the kernel's K loop (the 256-row
// kernel uses every scalar register there).  The round structure repeats the
// kernel's: persistent grid of G = gridDim.x workgroups on 8 XCDs, row pieces
// for a last round of at most G / WAVES_M tiles.
template <int BM, int WAVES_M, int NW>
__device__ __forceinline__ void gmm_tail(const TailArgs &p, bool has_last_tile,
                                         const int (*s_pre)[kMaxE + 1], const int *s_row_off,
                                         const int *s_rows, int8_t *smem, int *s_go) {
    if (has_last_tile) {  // done with the last round
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(p.sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return;
    }
    constexpr int UNIT = BM / WAVES_M;
    const int G = gridDim.x, act_xcd = G >> 3;
    int total = 0;
    for (int c = 0; c < WAVES_M; ++c) total += s_pre[c][p.E];
    const int F = total / G, L = total - F * G;
    // workgroups with a last-round tile: WAVES_M per leftover tile when it is
    // cut into row pieces, else one
    const int n_work = L <= 8 * (act_xcd / WAVES_M) ? L * WAVES_M : L;
    if (!tail_wait(p, G, s_go)) return;

    uint32_t *bm = reinterpret_cast<uint32_t *>(smem);     // one bit per 64-row unit
    const int Rv = s_row_off[p.E - 1] + s_rows[p.E - 1];  // valid rows
    const int nwords = (Rv + 2047) >> 11;                   // <= 4096 (R < 2^23)
    for (int i = threadIdx.x; i < nwords; i += NW * kWave) bm[i] = 0;
    __syncthreads();
    // units holding rows of an m-block with a tile in round F - 1 or F
    for (int t = (F - 1) * G + (int)threadIdx.x; t < total; t += NW * kWave) {
        const TileRows tr = tile_rows<BM, UNIT>(t, p.E, s_pre, s_row_off, s_rows);
        if (tr.rows <= 0) continue;
        for (int u = tr.row0 >> 6; u <= (tr.row0 + tr.rows - 1) >> 6; ++u)
            atomicOr(&bm[u >> 5], 1u << (u & 31));
    }
    int *s_chunk = s_go;  // reused: the wait's flag has been read
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
    const int I = p.I;
    constexpr int kRowsPerWave = 64 / NW;
    for (;;) {
        __syncthreads();  // bitmap built / every wave has read the last chunk
        if (threadIdx.x == 0) {
            int c = -1;
            if (tail_load(p.sync + 2) < (uint32_t)n_work)
                c = (int)__hip_atomic_fetch_add(p.sync + 1, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_SYSTEM);
            *s_chunk = c;
        }
        __syncthreads();
        const int c = *s_chunk;
        if (c < 0 || c >= (Rv + 63) >> 6) break;
        for (int i = 0; i < kRowsPerWave; ++i) {  // wave-uniform rows
            const int r = c * 64 + wave * kRowsPerWave + i;
            if (r >= Rv) break;
            const int u = r >> 6;
            if ((bm[u >> 5] >> (u & 31)) & 1u) continue;
            uint4 uraw[4], graw[4];  // I <= 2048: at most 4 chunks of 8 columns per lane
            swiglu_row_load<4>(p.C + (size_t)r * (2 * I), I, lane, uraw, graw);
            const float p1 = p.pts1[r];
            int8_t *qrow = p.q2 + (size_t)r * I;
            if (p.prow) {
                const int pr = p.prow[r];
                qrow = p.q2 + (size_t)(pr >> 1) * (2 * I) + (pr & 1) * 64;
            }
            swiglu_row_finish<4>(uraw, graw, p1, I, lane, qrow, p.prow ? 128 : 64, p.pts2 + r);
            if (lane == 0) p.done[r] = 1;
        }
    }
}

// The lane index, computed afresh where it is used.  In the 256-row kernel
// every vector register is taken in the K loop, so a lane value kept from
// before it would be spilled, and its reload (a vector memory load) would
// wait for every copy and store issued before it.
__device__ __forceinline__ int fresh_lane_id() {
    int l;
    asm volatile(
        "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
        "v_mbcnt_hi_u32_b32 %0, -1, %0"
        : "=v"(l));
    return l;
}

// One row group of a wave's sub-tile (rows 16 i .. 16 i + 15), dequantised
// and stored as described at store_tile_private below, from the lane's
// accumulators a[TN] of those rows (MFMA layout).  Returns the store
// instructions issued.
template <int TN>
__device__ __forceinline__ int store_group(const GmmParams &p, const v4i (&a)[TN], int i,
                                           const float *s_sc, int row0, int n0, int wm0, int wn0,
                                           int8_t *wbuf, int r_lo, int r_hi, int lane) {
    const int rb0 = wm0 + 16 * i;  // tile row of the first row
    uint2 h[TN];  // fp16 of the lane's values of row 16 i + (lane & 15), two per word
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const float4 s4 = *reinterpret_cast<const float4 *>(s_sc + wn0 + 16 * j + 4 * (lane >> 4));
        const uint32_t h0 = f2h(keep_f32((float)a[j][0] * s4.x));
        const uint32_t h1 = f2h(keep_f32((float)a[j][1] * s4.y));
        const uint32_t h2 = f2h(keep_f32((float)a[j][2] * s4.z));
        const uint32_t h3 = f2h(keep_f32((float)a[j][3] * s4.w));
        h[j] = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    }
    int nstores = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int rb = rb0 + 8 * half;  // tile row of the chunk's first row
        if (rb + 8 <= r_lo || rb >= r_hi) continue;
        // lane l holds row 16 i + (l & 15), columns 16 j + 4 (l >> 4) .. + 3
        if (((lane >> 3) & 1) == half) {
            const int rr = lane & 7;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c = 2 * j + (lane >> 5);  // 16-byte piece of the row
                *reinterpret_cast<uint2 *>(wbuf + rr * 128 + ((c ^ rr) << 4) +
                                           (((lane >> 4) & 1) << 3)) = h[j];
            }
        }
        const int rr = lane >> 3, c = lane & 7;
        const uint4 v = *reinterpret_cast<const uint4 *>(wbuf + rr * 128 + ((c ^ rr) << 4));
        const int r = rb + rr;
        // at least one row of the chunk is stored, so the instruction issues
        if (r >= r_lo && r < r_hi) store_nt16(p.C + (size_t)(row0 + r) * p.N + n0 + wn0 + 8 * c, v);
        ++nstores;
    }
    return nstores;
}

// whether rows 16 i .. 16 i + 15 of a wave's sub-tile hold an output row
__device__ __forceinline__ bool group_live(int i, int wm0, int r_lo, int r_hi) {
    const int rb0 = wm0 + 16 * i;
    return rb0 + 16 > r_lo && rb0 < r_hi;
}

// The tile's output, dequantised to fp16 (fp32(acc) * scale, rounded to
// fp32, then to fp16), stored in whole 128-byte lines without the ring and
// without a workgroup barrier.  Each wave passes its 64 x 64 sub-tile through
// its own 1 KB of LDS, 8 rows at a time: the 32 lanes that hold a chunk's 8
// rows in the MFMA layout write them there (16-byte piece c of row rr at
// slot c ^ rr, free of bank conflicts for both the 8-byte writes and the
// row reads), then every lane reads one 16-byte piece of one row and the
// wave stores 8 whole rows with one instruction.  A wave's LDS operations
// complete in order, so no wait is needed between a chunk's writes and reads.
// Since the ring is not used, the next tile's first copies can be in flight
// while these stores go out.  Returns the number of store instructions
// issued (wave-uniform).
template <int TM, int TN>
__device__ __forceinline__ int store_tile_private(const GmmParams &p, const v4i (&acc)[TM][TN],
                                                  const float *s_sc, int row0, int n0, int wm0,
                                                  int wn0, int8_t *wbuf, int r_lo, int r_hi,
                                                  bool live) {
    static_assert(TN == 4, "a wave's sub-tile row is 64 columns, one 128-byte line of fp16");
    // N is a multiple of 128, so a sub-tile's columns are all inside N or all past it
    if (!live || n0 + wn0 >= p.N) return 0;
    const int lane = fresh_lane_id();
    int nstores = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i)
        if (group_live(i, wm0, r_lo, r_hi))
            nstores += store_group<TN>(p, acc[i], i, s_sc, row0, n0, wm0, wn0, wbuf, r_lo, r_hi,
                                       lane);
    return nstores;
}

// A K piece of a leftover tile (sparse last round, GMM1 of the forward): the
// tile's NP pieces each multiply 1 / NP of K and store their int32 partial
// tile to ks_part; the last piece to count itself adds the NP partials
// (integer sums: exact, in any order) and stores the tile as
// store_tile_private does.  No piece waits for another.
//
// The partials cross CUs (and, were the pieces dealt to different XCDs, L2
// caches) as device-scope atomic stores and loads, which the hardware makes
// coherent line by line (the sc1 policy) instead of by writing back or
// invalidating a whole L2: the fences that would do that also dropped the
// cached operands of every other workgroup on the XCD.  Each wave's partial
// stores have completed (vmcnt 0) before the workgroup barrier that precedes
// its counter increment, and the last piece issues its loads only after its
// increment has returned the count of the other pieces.  The last piece also
// puts the counter back to zero, so a buffer zeroed once serves every later
// launch.  It reads its own partial back too, so that its accumulators are
// free during the sums (the K loop leaves no register for the other pieces'
// blocks beside them).  Returns the store instructions issued.
template <int TM, int TN, int NW, int NP>
__device__ __forceinline__ int ks_store_tile(const GmmParams &p, const v4i (&acc)[TM][TN], int jj,
                                             int piece, int wave, const float *s_sc, int row0,
                                             int n0, int wm0, int wn0, int8_t *wbuf, int r_lo,
                                             int r_hi, bool live, int *s_flag) {
    constexpr int kPiece = NW * TM * TN * 4 * kWave;  // 32-bit words of one partial tile
    static_assert(kPiece * 4 <= (int)kKsPartBytes, "partial tile size");
    live = live && n0 + wn0 < p.N;
    const int lane = fresh_lane_id();
    // [piece][wave][16x16 block][accumulator c][lane]: 256 contiguous bytes
    // per instruction
    uint32_t *part = reinterpret_cast<uint32_t *>(p.ks_part) + (size_t)jj * NP * kPiece +
                     (size_t)wave * TM * TN * 4 * kWave + lane;
    // a wave without an output row neither writes nor reads
    if (live) {
        uint32_t *mine = part + (size_t)piece * kPiece;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    __hip_atomic_store(mine + ((i * TN + j) * 4 + c) * kWave,
                                       (uint32_t)acc[i][j][c], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial is stored
    __syncthreads();
    if (threadIdx.x == 0) {
        *s_flag = (int)__hip_atomic_fetch_add(p.ks_count + jj, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
        // every piece has counted: the counter is free for the next launch
        if (*s_flag == NP - 1)
            __hip_atomic_store(p.ks_count + jj, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (*s_flag != NP - 1 || !live) return 0;  // another piece of the tile stores it
    int nstores = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (!group_live(i, wm0, r_lo, r_hi)) continue;
        // one row group's loads at a time: hoisted above the previous group's
        // stores, they would not fit in the registers
        asm volatile("" ::: "memory");
        v4i t[NP][TN];  // the pieces' blocks of row group i, all requested together
#pragma unroll
        for (int q = 0; q < NP; ++q)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    t[q][j][c] = (int)__hip_atomic_load(
                        part + (size_t)q * kPiece + ((i * TN + j) * 4 + c) * kWave,
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int q = 1; q < NP; ++q)
#pragma unroll
            for (int j = 0; j < TN; ++j) t[0][j] += t[q][j];
        nstores += store_group<TN>(p, t[0], i, s_sc, row0, n0, wm0, wn0, wbuf, r_lo, r_hi, lane);
    }
    return nstores;
}

// s_waitcnt vmcnt(base + extra) for a wave-uniform extra in [0, 8]
template <int base>
__device__ __forceinline__ void wait_vmcnt_plus(int extra) {
    switch (extra) {
        case 0: wait_vmcnt<base>(); break;
        case 1: wait_vmcnt<base + 1>(); break;
        case 2: wait_vmcnt<base + 2>(); break;
        case 3: wait_vmcnt<base + 3>(); break;
        case 4: wait_vmcnt<base + 4>(); break;
        case 5: wait_vmcnt<base + 5>(); break;
        case 6: wait_vmcnt<base + 6>(); break;
        case 7: wait_vmcnt<base + 7>(); break;
        case 8: wait_vmcnt<base + 8>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

template <int BM, int WAVES_M, int WAVES_N, int NS, bool TRIM, bool SKIP = true, int PRIO = 0,
          bool NTB = TRIM>
__global__ __launch_bounds__(WAVES_M *WAVES_N *kWave) void gmm_i8_ring_kernel(GmmParams p) {
    // PRIO > 0 (two workgroups per CU that stream weights): the older of the
    // two workgroups on a CU wins the CU's arbitration, and with equal work
    // it was measured to finish up to 25% before its partner, which then
    // streams alone at half the copies in flight.  The two alternate their
    // wave priority every PRIO K steps in opposite phase; the grid's first
    // and second halves are the dispatcher's first and second workgroup on
    // each CU.
    constexpr int BN = kPackRows;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int kStage = (BM + BN) * kBK64;        // bytes of one stage
    constexpr int LPW = kStage / 1024 / NW;          // 1 KB copies per wave per stage
    constexpr int kAJ = (BM / 16) / NW;              // copies j < kAJ fill A rows
    static_assert(kStage % (1024 * NW) == 0, "stage must split over the waves");
    static_assert((BM / 16) % NW == 0, "each wave fills the same number of A blocks");
    static_assert(NS >= 3 && WM % 16 == 0 && WN % 16 == 0, "shape");
    static_assert(BN % kWave == 0, "scale copies are whole waves");

    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * kStage];
    __shared__ __attribute__((aligned(16))) float s_scale[2][BN];
    constexpr int U = WAVES_M;                       // cost classes (live row blocks)
    __shared__ int s_pre[U][kMaxE + 1];
    __shared__ int s_row_off[kMaxE];
    __shared__ int s_rows[kMaxE];
    __shared__ int s_pad[kMaxE];  // row offsets in the row-paired A layout (a_pair)
    __shared__ int s_go;
    __shared__ TailArgs s_targs;  // last-round SwiGLU (GMM1 only)
    __shared__ int s_tail_round;  // the round after which producers count themselves, or -1
    // what the epilogue needs of each tile (row0, rows, n0, first and end row
    // stored, row piece): kept in LDS by tile parity, not in registers
    // across the K loop, which uses every scalar register
    __shared__ int s_tile[2][6];
    __shared__ __attribute__((aligned(16))) int8_t s_wbuf[NW][1024];  // epilogue, per wave

    // the wave index is uniform: kept in a scalar register, so that no
    // vector register holds threadIdx across the K loop
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = __lane_id();
    const int N = p.N, Kred = p.Kred;
    const int NB = (N + BN - 1) / BN;
    const int total =
        build_schedule<BM, BM / WAVES_M>(p, NB, s_pre, s_row_off, s_rows, p.a_pair ? s_pad : nullptr);

    // TRIM (active grid, for tiles of equal cost that stream weights): with
    // k = ceil(total / gridDim) tiles for the busiest workgroup, ceil(total / k)
    // workgroups (rounded up to 8, the same number on every XCD) already finish
    // in k rounds; the rest exit, so every active workgroup streams the same
    // number of tiles and no last, partly filled round leaves HBM underused.
    // Without TRIM all workgroups stay, which suits tiles of unequal cost.
    const int per_xcd = gridDim.x >> 3;              // gridDim.x is a multiple of 8
    const int rounds = (total + gridDim.x - 1) / gridDim.x;
    const int act_xcd =
        !TRIM ? per_xcd : rounds ? min(per_xcd, ((total + rounds - 1) / rounds + 7) >> 3) : 0;
    if ((int)(blockIdx.x >> 3) >= act_xcd) return;
    const int G = act_xcd << 3;
    [[maybe_unused]] const int late = (int)blockIdx.x >= (int)(gridDim.x >> 1);
    const int vid = (blockIdx.x & 7) * act_xcd + (blockIdx.x >> 3);
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    const int nst = Kred / kBK64;                    // stages (K slices)
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(&smem[0]));

    // LDS byte offsets of this lane's fragment rows inside a stage: fragment
    // i of A starts 16 i rows after fa0 and fragment j of the weights 16 j
    // rows after fb0 (a row's swizzle depends only on its bits 1-2, which
    // steps of 16 rows keep), so the other fragments' offsets are constants
    int fa0, fb0;
    {
        const int chunk = lane >> 4, r = lane & 15;
        fa0 = lds_off64s(wm0 + r, chunk);
        fb0 = BM * kBK64 + lds_off64s(wn0 + r, chunk);
    }

    // Round k of workgroup w takes tile k G + w.  When tiles differ in cost
    // (!TRIM), odd rounds run the other way (k G + G - 1 - w): with the tiles
    // numbered largest class first, this deals them like a longest-first
    // schedule, and each workgroup's sum comes out nearly equal.  Dealt in
    // plain order, an XCD's 32 workgroups took 32 consecutive tiles of one
    // expert every round, and some XCDs finished 15% after others.
    auto pos = [&](int k, int w) { return k * G + ((!TRIM && (k & 1)) ? G - 1 - w : w); };

    // When the last round is sparse (L <= G / WAVES_M tiles), each of its tiles
    // is cut into WAVES_M row pieces, one per wave row block, so a leftover
    // tile no longer keeps one workgroup busy for a whole tile after the rest
    // are done.  Only the waves of a piece's row block multiply and store;
    // the hardware places wave w on SIMD w % 4, so those WAVES_N waves sit on
    // different SIMDs and the piece has the whole CU's matrix rate (a cut by
    // wave columns put a piece's live waves on one SIMD).  A piece copies the
    // tile's weights for its live waves, and its A copies of the other row
    // blocks all read its own boundary row, one request per copy instead of
    // sixteen.  A piece whose row block holds no rows of the tile has nothing
    // to do.  The pieces of leftover tile j go to WAVES_M workgroups of one
    // XCD (XCD j % 8), which then share the tile's weights in their L2
    // (pieces spread over several XCDs each fetched the tile from HBM).  The
    // snake order has already evened out the full rounds.  A fuller last
    // round keeps the plain order, whose adjacent tiles share L2 data.
    const int F = total / G, L = total - F * G;
    const int groups = 8 * (act_xcd / WAVES_M);  // whole groups of WAVES_M slots
    const bool ranked = !TRIM && L > 0 && L <= groups;
    int extra = pos(F, vid) < total ? pos(F, vid) : -1, piece = 0;
    if (ranked) {
        const int xcd = vid / act_xcd, slot = vid % act_xcd;
        const int j = (slot / WAVES_M) * 8 + xcd;  // leftover tile of this group
        extra = j < L ? F * G + j : -1;
        piece = slot % WAVES_M;
    }
    // With a partial-tile buffer (the forward's GMM1), the pieces of a
    // leftover tile split its K slices instead of its rows: each runs a
    // quarter of the K chain that bounds a row piece, and the last of them
    // adds the partial tiles (ks_store_tile).
    const bool ksplit = !TRIM && ranked && p.ks_part != nullptr && p.acc_dbg == nullptr &&
                        nst % (2 * WAVES_M) == 0 && L <= kKsMaxTiles;

    // SwiGLU in the last round (GMM1 of the forward; tiles of unequal cost).
    // Kept in LDS and read once per tile: the K loop has no scalar register
    // to spare.  The K loop's barriers order this write before the reads.
    if constexpr (!TRIM) {
        if (threadIdx.x == 0) {
            // the tail keeps a row's chunks in registers up to I = 2048
            const bool on = p.tail_q2 != nullptr && F >= 2 && L > 0 && p.tail_I <= 2048;
            s_tail_round = on ? F - 1 : -1;
            s_targs = TailArgs{p.C, p.tail_q2, p.tail_pts2, p.tail_pts1, p.tail_sync,
                               p.tail_done, p.tail_prow, p.tail_I, p.tail_spin, p.E};
        }
    }

    // A tile's set-up: its rows, the DMA source offsets, and the copy of its
    // scales into LDS slot par.  The set-up of tile k + 1 runs between tile
    // k's K loop and its epilogue, so that tile k's output stores and tile
    // k + 1's first copies are in flight together (vector memory operations
    // complete in issue order, so a set-up after the stores would wait for
    // them before its own loads and copies).
    struct TileSetup {
        int valid, e, row0, rows, n0;
        bool piece_tile;
        int kcnt;             // K slices of this tile (a K piece: a quarter)
        const int8_t *abase;  // A at the tile's first K slice
        const int8_t *btile;  // the tile's weights at its first K slice
        uint32_t voff[LPW];
    };
    // bytes between the A operand's K slices of one row
    const int a_stage = p.a_pair ? 2 * kBK64 : kBK64;
    // packed weights are K-slice-major: the block of (expert e, n-block
    // nblk) for K slice ks sits at ((ks * E + e) * NB + nblk) blocks
    const size_t bstep = (size_t)p.E * NB * kPackBlock;
    auto setup = [&](int kk, int par) {
        TileSetup ts{};
        const int t = kk < F ? pos(kk, vid) : (kk == F ? extra : -1);
        if (t < 0) return ts;
        const TileRows tr = tile_rows<BM, BM / WAVES_M>(t, p.E, s_pre, s_row_off, s_rows);
        ts.e = tr.e;
        ts.row0 = tr.row0;
        ts.rows = tr.rows;
        ts.n0 = tr.nblk * BN;
        // a piece of a leftover tile: rows [plo, phi] of the tile (a row
        // piece), or every row and a quarter of the K slices (a K piece)
        ts.piece_tile = ranked && kk == F;
        const bool kpiece = ts.piece_tile && ksplit;
        const bool rpiece = ts.piece_tile && !ksplit;
        const int plo = rpiece ? piece * WM : 0;
        const int phi = rpiece ? min(plo + WM, tr.rows) - 1 : min(tr.rows, BM) - 1;
        if (rpiece && plo >= tr.rows) return ts;
        ts.valid = 1;
        const int kbeg = kpiece ? piece * (nst / WAVES_M) : 0;
        ts.kcnt = kpiece ? nst / WAVES_M : nst;
        ts.abase = p.A + (size_t)kbeg * a_stage;
        if (threadIdx.x == 0) {
            s_tile[par][0] = tr.row0;
            s_tile[par][1] = tr.rows;
            s_tile[par][2] = ts.n0;
            s_tile[par][3] = plo;
            s_tile[par][4] = phi + 1;
            s_tile[par][5] = kpiece ? 2 : (rpiece ? 1 : 0);  // whole, row piece, K piece
        }

        // scales of the tile's columns (clamped: columns past N are never stored)
        for (int c = wave; c < BN / kWave; c += NW)
            dma4(p.scale + (size_t)tr.e * N + min(ts.n0 + c * kWave + lane, N - 1),
                 __builtin_amdgcn_readfirstlane(lds_addr(&s_scale[par][c * kWave])));

        // DMA sources: 1 KB block b = wave + j NW of a stage; lane l fills
        // 16-byte LDS chunk 64 b + l, taking the chunk that the swizzle puts
        // there.  A rows past the group's end repeat its last row (their
        // results are not stored).
        // per-lane 32-bit source offsets: from p.A for the A rows, from the
        // tile's first weight block for the weights
        ts.btile = p.B + ((size_t)tr.e * NB + tr.nblk) * kPackBlock + (size_t)kbeg * bstep;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int pch = (wave + j * NW) * 64 + lane;
            if (j < kAJ) {
                const int r = pch >> 2, kc = (pch & 3) ^ swz64(pch >> 2);
                const int arow =
                    tr.row0 + (rpiece ? min(max(r, plo), phi) : min(r, tr.rows - 1));
                if (p.a_pair) {  // padded row g: 64-byte K slices of rows 2m, 2m + 1 share a line
                    const int g = arow + s_pad[tr.e];
                    ts.voff[j] = (uint32_t)(g >> 1) * (uint32_t)(2 * Kred) + (g & 1) * 64 + kc * 16;
                } else {
                    const int srow = p.a_route ? p.a_route[arow] / p.a_div : arow;
                    ts.voff[j] = (uint32_t)srow * (uint32_t)Kred + kc * 16;
                }
            } else {
                const int q = pch - BM * 4;
                const int r = q >> 2, kc = (q & 3) ^ swz64(q >> 2);
                ts.voff[j] = (uint32_t)(r * kBK64 + kc * 16);
            }
        }
        return ts;
    };

    // the copies of K slice `stage` of tile t into its ring slot
    auto issue = [&](const TileSetup &t, int stage) {
        if (stage >= t.kcnt) return;
        const uint32_t sbase = ring + (uint32_t)((stage % NS) * kStage);
        const int8_t *abase = t.abase + (size_t)stage * a_stage;
        const int8_t *bbase = t.btile + (size_t)stage * bstep;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const uint32_t dst =
                __builtin_amdgcn_readfirstlane(sbase + (uint32_t)((wave + j * NW) * 1024));
            // weights that are read by one tile only (NTB) carry the non-temporal hint
            if (j < kAJ) dma16(abase, t.voff[j], dst);
            else if (NTB) dma16_nt(bbase, t.voff[j], dst);
            else dma16(bbase, t.voff[j], dst);
        }
    };
    // A tile's first NS stages fill the ring; its K loop starts once stage 0
    // has landed (stages 1 .. NS - 1 may still be in flight).  The first tile
    // issues them here, every later one between the previous tile's K loop
    // and its epilogue.
    auto issue_first = [&](const TileSetup &t) {
#pragma unroll
        for (int st = 0; st < NS; ++st) issue(t, st);
    };

    int parity = 0;
    TileSetup cur = setup(0, 0);
    if (cur.valid) {
        issue_first(cur);
        if (cur.kcnt >= NS) wait_vmcnt<(NS - 1) * LPW>();
        else wait_vmcnt<0>();
    }
    for (int k = 0; cur.valid; ++k, parity ^= 1) {
        const int rows = cur.rows;
        const bool piece_tile = cur.piece_tile;
        const int kcnt = cur.kcnt;

        v4i acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

        // the K loop, with (LIVE) or without fragment reads and MFMAs
        auto kloop = [&](auto live_c) {
            constexpr bool LIVE = decltype(live_c)::value;
            v4i fa[2][TM], fb[2][TN];
            auto frag = [&](int stage, v4i *xa, v4i *xb) {
                if constexpr (LIVE) {
                    const int8_t *base = smem + (stage % NS) * kStage;
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        xa[i] = *reinterpret_cast<const v4i *>(base + fa0 + 16 * i * kBK64);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        xb[j] = *reinterpret_cast<const v4i *>(base + fb0 + 16 * j * kBK64);
                }
            };
            auto mfmas = [&](const v4i *xa, const v4i *xb) {
                if constexpr (LIVE) {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_t(xb[j], xa[i], acc[i][j]);
                }
            };
            // stage kt+1 must have landed; stages up to kt+NS-1 were issued,
            // the NS-2 after kt+1 may be in flight (the previous tile's
            // epilogue stores are older than stage 1, so they are done too)
            auto await_next = [&](int kt) {
                if (kt + NS - 1 < kcnt) wait_vmcnt<(NS - 2) * LPW>();
                else wait_vmcnt<0>();
                __syncthreads();
            };
            __syncthreads();  // publishes stage 0 (awaited by every wave)
            frag(0, fa[0], fb[0]);

            // two stages per trip so that the register set of every stage is
            // known at compile time (set = stage & 1); kcnt is even
            for (int kt0 = 0; kt0 < kcnt; kt0 += 2) {
                static_for<0, 2>([&](auto uc) {
                    constexpr int rs = decltype(uc)::value, rn = rs ^ 1;  // register sets
                    const int kt = kt0 + rs;
                    if constexpr (PRIO > 0 && rs == 0) {
                        static_assert(PRIO % 2 == 0, "kt is even here");
                        if (kt % PRIO == 0) {
                            if (((kt / PRIO) & 1) ^ late) __builtin_amdgcn_s_setprio(2);
                            else __builtin_amdgcn_s_setprio(0);
                        }
                    }
                    await_next(kt);
                    issue(cur, kt + NS);
                    frag(kt + 1, fa[rn], fb[rn]);
                    mfmas(fa[rs], fb[rs]);
                });
            }
        };
        // a row piece of a leftover tile: only its wave row block multiplies
        // and stores (the other pieces of the tile run on other workgroups)
        const bool piece_live = !piece_tile || ksplit || wave / WAVES_N == piece;
        if ((!SKIP || wm0 < rows) && piece_live) kloop(std::true_type{});
        else kloop(std::false_type{});

        // the next tile's set-up (its scale copy goes to the other LDS slot)
        const TileSetup nxt = setup(k + 1, parity ^ 1);
        const int t_row0 = __builtin_amdgcn_readfirstlane(s_tile[parity][0]);
        const int t_rows = __builtin_amdgcn_readfirstlane(s_tile[parity][1]);
        const int t_n0 = __builtin_amdgcn_readfirstlane(s_tile[parity][2]);
        const int r_lo = __builtin_amdgcn_readfirstlane(s_tile[parity][3]);
        const int r_hi = __builtin_amdgcn_readfirstlane(s_tile[parity][4]);
        const int t_kind = __builtin_amdgcn_readfirstlane(s_tile[parity][5]);
        const bool live = (t_kind != 1 || wave / WAVES_N == piece) && wm0 < t_rows;
        // the debug int32 accumulators go straight from the registers, before
        // the next tile's copies, so the wait for its first stage covers them
        if (p.acc_dbg && live) store_acc_dbg<TM, TN>(p, acc, t_row0, t_rows, t_n0, wm0, wn0, lane);
        // The next tile's stage 0 is copied while this tile's output is stored,
        // and its stages 1 .. NS - 1 after the stores: vector memory
        // operations complete in issue order, so the K loop's waits for
        // stages 1 and later then cover the stores without counting them,
        // and only the wait for stage 0 allows for them.
        __syncthreads();  // every wave has read its last fragments: the ring is free
        if (nxt.valid) issue(nxt, 0);
        // a K piece (which has no next tile): the last of its tile's pieces stores
        int nstores;
        if (TRIM || t_kind != 2)
            nstores = store_tile_private<TM, TN>(p, acc, s_scale[parity], t_row0, t_n0, wm0, wn0,
                                                 s_wbuf[wave], r_lo, r_hi, live);
        else
            nstores = ks_store_tile<TM, TN, NW, WAVES_M>(
                p, acc, extra - F * G, piece, wave, s_scale[parity], t_row0, t_n0, wm0, wn0,
                s_wbuf[wave], r_lo, r_hi, live, &s_go);
        if (nxt.valid) {
#pragma unroll
            for (int st = 1; st < NS; ++st) issue(nxt, st);
            // stage 0 (and the tile's older scale copy) has landed
            if (nxt.kcnt >= NS) wait_vmcnt_plus<(NS - 1) * LPW>(nstores);
            else wait_vmcnt<0>();
        }
        if constexpr (!TRIM) {
            // done with round F - 2: count this workgroup for the last-round SwiGLU
            if (k + 1 == __builtin_amdgcn_readfirstlane(s_tail_round)) tail_arrive(s_targs.sync);
        }
        cur = nxt;
    }

    if constexpr (!TRIM) {
        if (__builtin_amdgcn_readfirstlane(s_tail_round) >= 0)
            gmm_tail<BM, WAVES_M, NW>(s_targs, extra >= 0, s_pre, s_row_off, s_rows, smem, &s_go);
    }
}

// Weight pack: logical [E][Kred][N] -> K-slice-major [Kred/64][E][NB][256][64]
// (NB = ceil(N / 256)): for K slice ks, expert e and n-block nb, the 256
// weight rows n = 256 nb + r hold bytes w[e][64 ks + kb][n], kb = 0..63, in
// one contiguous 16 KB block; rows n >= N are zero.  When the GEMM streams
// weights (few rows per expert), all tiles advance through K together, so at
// any moment the grid reads one window of adjacent blocks; that was measured
// 3-5% faster at decode than keeping each tile's K slices together, and
// within 1.5% either way at the larger shapes.  One 64 x 64 (k, n) tile per
// workgroup, transposed through LDS; its output is 64 rows of one block.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const int8_t *__restrict__ w,
                                                         int8_t *__restrict__ wp, int Kred,
                                                         int N, int NB, int E) {
    __shared__ int8_t tile[64][65];
    const int e = blockIdx.z;
    const int ks = blockIdx.y, n0 = blockIdx.x * 64;
    const int k0 = ks * kBK64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int8_t *src = w + (size_t)e * Kred * N;
    for (int r = ty; r < 64; r += 4) {
        const int k = k0 + r, n = n0 + tx;
        tile[r][tx] = n < N ? src[(size_t)k * N + n] : 0;
    }
    __syncthreads();
    const int nb = n0 / kPackRows, r0 = n0 % kPackRows;
    int8_t *dst = wp + (((size_t)ks * E + e) * NB + nb) * kPackBlock;
    for (int r = ty; r < 64; r += 4) dst[(size_t)(r0 + r) * kBK64 + tx] = tile[tx][r];
}

size_t packed_weight_bytes(int E, int Kred, int N) {
    const size_t NB = (size_t)(N + kPackRows - 1) / kPackRows;
    return (size_t)E * NB * kPackRows * (size_t)Kred;
}

hipError_t launch_pack(const int8_t *w, int8_t *wp, int E, int Kred, int N, hipStream_t stream) {
    const int NB = (N + kPackRows - 1) / kPackRows;
    dim3 grid(NB * kPackRows / 64, Kred / kBK64, E), block(256);
    hipLaunchKernelGGL(pack_tiles_kernel, grid, block, 0, stream, w, wp, Kred, N, NB, E);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile configurations, chosen by the host from the mean rows per expert
// (measured on MI355X over the decode, mid, large and skewed shapes with
// interleaved repetitions):
//  * few rows per expert: the GEMM streams weights (HBM bound); a 64-row tile
//    with a 3-stage ring fits twice per CU, so two workgroups per CU keep
//    twice the copies in flight, and they alternate priority every 16 K
//    steps so that neither finishes long after the other.  Once many
//    experts need a second 64-row block, whose tiles stream the weights
//    again, the 256-row tiles win: at K = 7168, E = 32, uniform routing, the
//    64-row tiles were 10% faster at 48 and 52 mean rows and up to 42% slower
//    from 56 on;
//  * more rows: MFMA bound; 256 x 256 tiles on 16 waves (64 x 64 per wave),
//    which beat 8-wave layouts of the same tile at the large shapes;
//  * up to 256 rows per expert (one m-block for most experts), the same
//    tiles with the weight copies marked non-temporal: each weight block is
//    read once, and keeping it out of the caches left them to the
//    activations (mid-size shapes 2-6% faster).  With several m-blocks per
//    expert the hint evicted the weight blocks they share (large 4-7% slower).
//  The weight-streaming 64-row tiles always carry the hint (decode GMM1
//  159 -> 139 us, GMM2 90 -> 80 us).
// ---------------------------------------------------------------------------
struct GmmVariant {
    int bm, bn;
    void (*kernel)(GmmParams);
    int threads;
    std::atomic<int> occupancy;  // resident workgroups per CU, filled at first use
};

static GmmVariant g_variants[] = {
    {64, 256, gmm_i8_ring_kernel<64, 1, 4, 3, true, true, 16>, 256, 0},
    {256, 256, gmm_i8_ring_kernel<256, 4, 4, 4, false>, 1024, 0},
    {256, 256, gmm_i8_ring_kernel<256, 4, 4, 4, false, true, 0, true>, 1024, 0},
};

int gmm_num_variants() { return (int)(sizeof(g_variants) / sizeof(g_variants[0])); }

int gmm_pick_variant(int R, int E) {
    const int mean = (R + E - 1) / E;
    if (mean <= 52) return 0;
    // up to 256 rows per expert most weight blocks are read by one tile only,
    // so their copies carry the non-temporal hint; above that, the m-blocks
    // of an expert share each weight block through L2
    return mean <= 256 ? 2 : 1;
}

bool gmm_tail_ok(int R, int E, int I) {
    // the 256-row configurations deal tiles of unequal cost (no trimmed
    // grid), and the tail keeps a row's chunks in registers up to I = 2048
    return gmm_pick_variant(R, E) != 0 && I <= 2048;
}

hipError_t launch_gmm(int variant, const GmmParams &prm, int R, int cu_count,
                      hipStream_t stream) {
    GmmVariant &v = g_variants[variant];
    int occ = v.occupancy.load(std::memory_order_relaxed);
    if (occ == 0) {  // concurrent first calls store the same value
        hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, reinterpret_cast<const void *>(v.kernel), v.threads, 0);
        if (err != hipSuccess) return err;
        occ = occ > 0 ? occ : 1;
        v.occupancy.store(occ, std::memory_order_relaxed);
    }
    // Upper bound on the tile count: sum_e ceil(rows_e / BM) <= R / BM + E.
    const int NB = (prm.N + v.bn - 1) / v.bn;
    const long long ub = ((long long)R / v.bm + prm.E) * NB;
    long long g = (long long)cu_count * occ;
    if (ub < g) g = ub;
    g = (g + 7) / 8 * 8;
    if (g < 8) g = 8;
    if (g > kMaxWorkgroups) g = kMaxWorkgroups;
    hipLaunchKernelGGL(v.kernel, dim3((unsigned)g), dim3(v.threads), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace megamoe
