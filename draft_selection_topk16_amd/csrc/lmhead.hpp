// The drafter's LM head fused with top-K.
//
// The selector starts from the drafter's own logits ("DFlash 2: Keep Drafting
// Parallel", section "A Lightweight Path Selector": the selector needs no
// extra LM-head pass), read as U_t(v) = <W_lm[v], h_t> over the vocabulary.
// Computing them here, beside the top-K, keeps the [M, V] logits out of HBM:
// the one large read is W_lm itself (V x d bf16), streamed exactly once.
//
// k_lmhead: workgroup (mt, vr) multiplies M tile mt (up to 14 m-blocks of 16
// rows of X) by the W_lm rows of vocabulary range vr on the matrix cores
// (bf16 operands, fp32 sums).  The range's 16-column blocks are cut into
// chunks of 16 blocks (the last one shorter), split evenly over the four
// waves, so every wave owns at most four blocks (64 columns) of W_lm and
// streams them from HBM straight into registers, a ring of four or six
// 64-deep k slices.  X reaches the waves through LDS, one 64-deep k slice at
// a time, staged through registers two to four slices ahead; every X load is
// issued before the W loads of its step, so that waiting for an X slice never
// waits for a W slice needed later.
// After the last slice of a chunk the waves spill their fp32 tiles to LDS
// and the columns are folded into running per-row lists of
// the best KMAX candidates, which stay in LDS until the workgroup ends.
// Tiles of up to 64 rows: every wave folds its own 64 columns into its own
// lists, with one to four lanes per row (each lane its own list over its
// share of the columns), and the lists of a row are merged at the end;
// larger tiles: the waves spill 32 columns at a time where the X slices
// were, and one thread per row folds them all.  An empty list is filled by
// sorting 16 or 32 columns at once; after that a column enters only if it
// beats the list's last entry, four such columns per sorted merge.  An entry
// is one exact double that holds value key and column.
//
// k_lmhead_merge: one workgroup per row merges the row's n_vr sorted lists
// (one list per thread, loaded whole): a bound that K words are known to
// reach (the best K-th word of any list, and the K-th best head), compaction
// of the words that reach it (a prefix of each list), and ranks by counting.
// Candidate words (key << 32 | ~index) are distinct within a row, so results
// do not depend on timing or on the launch plan.
#pragma once

#include <math.h>

#include "common.hpp"

namespace df2 {

constexpr int kLmWaveBlocks = 4;                          // 16-column blocks per wave
constexpr int kLmChunkBlocks = kWaves * kLmWaveBlocks;    // 256 columns per chunk
constexpr int kLmSliceK = 64;                             // k per X slice
// W slices held in registers per wave (also the unroll of the slice loop,
// whose body is branch-free so that the compiler's memory-counter waits stay
// exact and the loads of later slices stay in flight).  Four slices keep
// 128 KB per CU in flight; a plain stream of W in this pattern reads HBM no
// faster with more, and slower with eight.  Six for eight m-blocks.
__host__ __device__ constexpr int lm_ring(int mb) { return mb <= 4 ? 4 : (mb <= 8 ? 6 : 4); }
// X slices held in registers ahead of their store to LDS.  Memory-counter
// waits complete in order, so waiting for X slice s + 1 also waits for every
// W load issued before it: a W slice gets as many steps in flight as X is
// staged ahead, whatever the depth of the W ring.  Small tiles stage X a
// whole ring ahead (one or two 16-byte pieces per thread per slice); large
// tiles have registers for two slices only.
__host__ __device__ constexpr int lm_xahead(int mb) { return mb <= 4 ? 4 : (mb <= 8 ? 3 : 2); }
// the slice loop's unroll: W slots, X slots and the two LDS buffers all
// cycle inside it
__host__ __device__ constexpr int lm_gcd(int a, int b) { return b == 0 ? a : lm_gcd(b, a % b); }
__host__ __device__ constexpr int lm_lcm(int a, int b) { return a / lm_gcd(a, b) * b; }
__host__ __device__ constexpr int lm_unroll(int mb) { return lm_lcm(lm_lcm(lm_ring(mb), lm_xahead(mb)), 2); }
constexpr int kLmXBufs = 2;                               // X slice buffers in LDS
constexpr int kLmSlabCols = 32;                           // columns per fold
// tiles of up to four m-blocks (64 rows; two for 64-entry lists, whose four
// copies would not fit in LDS): every wave folds its own columns into its
// own lists, one lane per row; larger tiles: one thread per row folds the
// whole chunk, 32 columns at a time
__host__ __device__ constexpr bool lm_wide(int mb, int kmax) { return mb <= (kmax <= 32 ? 4 : 2); }
// small tiles, lists of up to 32: the wave's 64 lanes cover its rows several
// times over (four lanes per row for one m-block, two for two), each lane
// keeping its own list of its share of the columns (16 or 32 per chunk)
__host__ __device__ constexpr int lm_lpr(int mb, int kmax) {
    return (lm_wide(mb, kmax) && kmax <= 32) ? 64 / (16 * mb) : 1;
}
constexpr int kLmMaxLists = 256;                          // vocabulary ranges per row

struct LmArgs {
    const uint16_t* X;       // [M, d] bf16 hidden states
    const uint16_t* W;       // [V, d] bf16 LM-head weight
    uint64_t* part;          // [M, n_vr, kstride] candidate words, best first, 0 = empty
    int32_t* out_idx;        // [M, K]
    float* out_val;          // [M, K]
    int64_t M;
    int V, d, K;
    int kstride;             // words per list (the kernel's KMAX)
    int n_mt, n_vr;          // M tiles, vocabulary ranges
    int nblk;                // 16-column blocks of the vocabulary, ceil(V / 16)
};

// rows of an X slice buffer: the tile's, and at least one piece per thread
__host__ __device__ constexpr int lm_xrows(int mb) { return 16 * mb > 32 ? 16 * mb : 32; }

template <int MB, int KMAX>
struct LmLds {
    union {
        // X slice: row, 16-byte slot; piece p of row r sits in slot
        // p ^ ((r >> 1) & 7): the 16 rows one matrix-operand read touches
        // then cover all 64 banks once (odd rows start 128 bytes in)
        u32x4_t xs[kLmXBufs][lm_xrows(MB)][8];
        // large tiles: the chunk's fp32 tile, 32 columns at a time
        float slab[lm_wide(MB, KMAX) ? 1 : 16 * MB][kLmSlabCols + 1];
    };
    // small tiles: each wave's own 64 columns of the chunk and its own
    // candidate lists, lm_lpr of them per row (folded without workgroup
    // barriers)
    float wslab[lm_wide(MB, KMAX) ? kWaves : 1][lm_wide(MB, KMAX) ? 16 * MB : 1][16 * kLmWaveBlocks + 1];
    // each row's running list(s) of its best KMAX candidates, best first, as
    // lm_entry values (0 = empty); rows padded by 16 bytes so that 16-byte
    // reads of consecutive rows fall in distinct banks
    double lst[lm_wide(MB, KMAX) ? kWaves * lm_lpr(MB, KMAX) : 1][16 * MB][KMAX + 2];
};

// An even split of n items into parts: part k starts at k q + min(k, r) and
// has q + (k < r) items, q = n / parts, r = n % parts (one division, once).
struct LmSplit {
    int q, r;
    __device__ LmSplit(int n, int parts) : q(n / parts), r(n - (n / parts) * parts) {}
    __device__ int start(int k) const { return k * q + min(k, r); }
    __device__ int size(int k) const { return q + (k < r ? 1 : 0); }
};

// Wave w's blocks [cb, cb + nbw) of a chunk [c0, c0 + nb): an even split over
// the four waves (nb <= 16).
__device__ __forceinline__ void lm_wave_blocks(int c0, int nb, int w, int& cb, int& nbw) {
    cb = c0 + (nb * w) / kWaves;
    nbw = c0 + (nb * (w + 1)) / kWaves - cb;
}

// A candidate as one exact double: its value key (order-preserving, so a
// larger key is a larger value) times 2^21 plus 2^21 - 1 - its column offset
// in the workgroup's range (< 2^21).  Comparing entries compares values, and
// equal values put the lower column first; 53 bits hold both exactly.
constexpr double kLmOffScale = 2097152.0;   // 2^21
constexpr int kLmMaxRangeCols = 1 << 21;
__device__ __forceinline__ double lm_entry(uint32_t key, int off) {
    return (double)key * kLmOffScale + (double)(kLmMaxRangeCols - 1 - off);
}
__device__ __forceinline__ uint32_t lm_entry_key(double e) {
    return (uint32_t)(e * (1.0 / kLmOffScale));      // exact: drops the offset part
}

// Larger and smaller of two list entries.  Entries are never NaN (0 or a
// finite positive key), so the plain instructions are exact; fmax/fmin would
// first quiet both operands (one more double operation each) because the
// compiler cannot see that.
__device__ __forceinline__ double lm_max(double a, double b) {
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ double lm_min(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// the value a candidate must beat to enter a list whose last entry is `last`
__device__ __forceinline__ float lm_floor(double last) {
    return last > 0.0 ? value_of_key_f32(lm_entry_key(last)) : -INFINITY;
}

// Buffer resource over `bytes` bytes from `base` (raw, no stride): loads at
// offsets past the end read as zero, so ragged tiles need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lm_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4_t lm_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Sort N entries, best first (bitonic network: every compare-exchange is
// one max and one min, the exchanges of a stage independent).
template <int N>
__device__ __forceinline__ void lm_sort(double (&e)[N]) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const double hi = lm_max(e[i], e[l]), lo = lm_min(e[i], e[l]);
                    const bool desc = (i & k) == 0;
                    e[i] = desc ? hi : lo;
                    e[l] = desc ? lo : hi;
                }
            }
}

// Best KMAX of two sorted lists (best first), into a: the elementwise larger
// of a and reversed b holds them as a bitonic sequence, which a half-cleaner
// network sorts.  b is read through `bk(j)`.
template <int KMAX, typename BK>
__device__ __forceinline__ void lm_merge_top(double (&a)[KMAX], BK&& bk) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) a[j] = lm_max(a[j], bk(KMAX - 1 - j));
#pragma unroll
    for (int h = KMAX / 2; h > 0; h >>= 1)
#pragma unroll
        for (int i = 0; i < KMAX; ++i)
            if ((i & h) == 0) {
                const double hi = lm_max(a[i], a[i + h]), lo = lm_min(a[i], a[i + h]);
                a[i] = hi;
                a[i + h] = lo;
            }
}

// Merge four entries e (best first; 0 = none) into a sorted list: the last
// four entries of the list become the larger of themselves and e reversed,
// which leaves a bitonic sequence holding the best KMAX, and the half-cleaner
// network sorts it (as in lm_merge_top, without the entries that cannot
// change).
template <int KMAX>
__device__ __forceinline__ void lm_merge4(double (&a)[KMAX], const double (&e)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[KMAX - 4 + k] = lm_max(a[KMAX - 4 + k], e[3 - k]);
#pragma unroll
    for (int h = KMAX / 2; h > 0; h >>= 1)
#pragma unroll
        for (int i = 0; i < KMAX; ++i)
            if ((i & h) == 0) {
                const double hi = lm_max(a[i], a[i + h]), lo = lm_min(a[i], a[i + h]);
                a[i] = hi;
                a[i + h] = lo;
            }
}

// Fold NC consecutive columns of one row (ncols of them valid; column cc has
// offset off0 + cc in the workgroup's range) into the row's list.  An empty
// list is filled by sorting the NC at once; otherwise the columns that beat
// the list's last entry are merged in four at a time (one LDS round trip,
// one merge and one new floor per four: each step is a chain of dependent
// operations at one wave per SIMD).  Entries carry their column, so the list
// does not depend on the order of insertion.
template <int KMAX, int NC>
__device__ __forceinline__ void lm_fold(double (&lw)[KMAX], float& floor_v,
                                        const float* __restrict__ srow, int ncols, int off0) {
    float xv[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) xv[cc] = srow[cc];
    if (lw[0] == 0.0) {
        double e[NC];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
            e[cc] = cc < ncols ? lm_entry(key_f32(__float_as_uint(xv[cc])), off0 + cc) : 0.0;
        lm_sort<NC>(e);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) lw[j] = j < NC ? e[j] : 0.0;
        floor_v = lm_floor(lw[KMAX - 1]);
        return;
    }
    uint32_t flagged = 0;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
        flagged |= (cc < ncols && xv[cc] > floor_v) ? (1u << cc) : 0u;
    while (flagged) {
        int c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[k] = flagged ? __builtin_ctz(flagged) : -1;
            flagged &= flagged - 1u;
        }
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = srow[c[k] < 0 ? 0 : c[k]];
        double e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            e[k] = (c[k] >= 0 && x[k] > floor_v) ? lm_entry(key_f32(__float_as_uint(x[k])), off0 + c[k])
                                                 : 0.0;
        lm_sort<4>(e);
        lm_merge4<KMAX>(lw, e);
        floor_v = lm_floor(lw[KMAX - 1]);
    }
}

// X pieces of one thread: piece q*256 + tid of a slice is row (q*256 + tid)/8,
// 16-byte piece (q*256 + tid) % 8.  They are loaded into registers two
// slices ahead and written to LDS with 16-byte stores.  The resource covers
// the tile's mrows rows, so rows past M read as zero; rows past the tile
// land in the spare rows of the buffer.
template <int MB, int KMAX>
struct LmX {
    static constexpr int XROWS = lm_xrows(MB);
    static constexpr int XP = XROWS * 8 / kWG;
    static_assert(XROWS * 8 % kWG == 0, "whole pieces per thread");
    __device__ static void offsets(int d, uint32_t (&off)[XP]) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            const int pi = q * kWG + tid;
            off[q] = (uint32_t)(((pi >> 3) * d + (pi & 7) * 8) * 2);
        }
    }
    __device__ static void load(__amdgpu_buffer_rsrc_t rx, const uint32_t (&off)[XP], int s,
                                u32x4_t (&xr)[XP]) {
#pragma unroll
        for (int q = 0; q < XP; ++q) xr[q] = lm_load(rx, off[q], (uint32_t)s * (kLmSliceK * 2));
    }
    __device__ static void store(LmLds<MB, KMAX>& sm, int buf, const u32x4_t (&xr)[XP]) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            const int pi = q * kWG + tid;
            const int r = pi >> 3, p = pi & 7;
            sm.xs[buf][r][p ^ ((r >> 1) & 7)] = xr[q];
        }
    }
};

// One chunk's products: acc[i][j] += X rows of m-block i times W rows of the
// wave's block j, over all of d.  The wave multiplies its NBW blocks (the
// chunk's even split gives it that many); every wave meets every barrier.
// rw covers the wave's rows of W_lm (rows past V read as zero).
template <int MB, int KMAX, int NBW>
__device__ __forceinline__ void lm_chunk(__amdgpu_buffer_rsrc_t rx,
                                         const uint32_t (&xoff)[LmX<MB, KMAX>::XP],
                                         __amdgpu_buffer_rsrc_t rw, int d, LmLds<MB, KMAX>& sm,
                                         f32x4_t (&acc)[MB][kLmWaveBlocks]) {
    using XL = LmX<MB, KMAX>;
    constexpr int NB = NBW > 0 ? NBW : 1;
    constexpr int RING = lm_ring(MB);
    const int lane = threadIdx.x & 63;
    const int row = lane & 15, g = lane >> 4;
    const int ns = d / kLmSliceK;
    uint32_t woff[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) woff[j] = (uint32_t)(((16 * j + row) * d + 16 * g) * 2);
    u32x4_t wr[RING][NB][2];
    auto load_w = [&](int s, u32x4_t (&dst)[NB][2]) {
        const uint32_t so = (uint32_t)min(s, ns - 1) * (kLmSliceK * 2);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            dst[j][0] = lm_load(rw, woff[j], so);
            dst[j][1] = lm_load(rw, woff[j] + 16u, so);
        }
    };
    // Step of slice s (ring slot u == s % RING, X buffer s % 2): load X slice
    // s + XA into the registers X slice s left (it reached LDS a step ago),
    // multiply (only for s < ns: past the end the loads repeat the last slice
    // and nothing is added), load W slice s + RING into the slot just used,
    // write X slice s + 1 to the other buffer and meet the other waves.
    // Every X load is issued before the W loads of the same step, so waiting
    // for X slice s + 1 at the end of step s waits for no W slice that is
    // needed later than XA steps after its load.
    constexpr int XA = lm_xahead(MB);
    constexpr int U = lm_unroll(MB);
    static_assert(XA >= 2, "X slice s + 1 is in registers while slice s is read from LDS");
    u32x4_t xr[XA][XL::XP];
    auto step = [&](int s, int u) {
        const int xb = u & 1;
        const int wu = u % RING;
        XL::load(rx, xoff, min(s + XA, ns - 1), xr[u % XA]);
        if constexpr (NBW > 0) {
            if (s < ns) {
                u32x4_t a0 = sm.xs[xb][row][(2 * g) ^ ((row >> 1) & 7)];
                u32x4_t a1 = sm.xs[xb][row][(2 * g + 1) ^ ((row >> 1) & 7)];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    // read block i + 1's operands, then multiply block i; the
                    // fences keep the reads a block ahead of their use
                    u32x4_t n0 = a0, n1 = a1;
                    if (i + 1 < MB) {
                        n0 = sm.xs[xb][16 * (i + 1) + row][(2 * g) ^ ((row >> 1) & 7)];
                        n1 = sm.xs[xb][16 * (i + 1) + row][(2 * g + 1) ^ ((row >> 1) & 7)];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // the two k halves of one block go to different
                    // accumulators first, so no product waits for the last
#pragma unroll
                    for (int j = 0; j < NBW; ++j)
                        acc[i][j] = mfma_bf16(as_bf16x8(a0), as_bf16x8(wr[wu][j][0]), acc[i][j]);
#pragma unroll
                    for (int j = 0; j < NBW; ++j)
                        acc[i][j] = mfma_bf16(as_bf16x8(a1), as_bf16x8(wr[wu][j][1]), acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                    a0 = n0;
                    a1 = n1;
                }
            }
            load_w(s + RING, wr[wu]);
        }
        XL::store(sm, xb ^ 1, xr[(u + 1) % XA]);
        __syncthreads();
    };

    // prologue: X slices 0 .. XA-1 and W slices 0 .. RING-1, interleaved so
    // that waiting for X slice k waits only for the W slices before it; X
    // slice 0 to LDS
#pragma unroll
    for (int u = 0; u < (RING > XA ? RING : XA); ++u) {
        if (u < XA) XL::load(rx, xoff, min(u, ns - 1), xr[u]);
        if (u < RING) load_w(u, wr[u]);
    }
    XL::store(sm, 0, xr[0]);
    __syncthreads();

    for (int s0 = 0; s0 < ns; s0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(s0 + u, u);
    }
}

template <int MB, int KMAX>
__global__ __launch_bounds__(kWG, 1) void k_lmhead(LmArgs a) {
    static_assert(KMAX % 2 == 0, "lists move in 16-byte pairs");
    constexpr int ROWS = 16 * MB;
    using XL = LmX<MB, KMAX>;
    __shared__ LmLds<MB, KMAX> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = lane & 15, g = lane >> 4;

    // Work item: consecutive items (the M tiles of one vocabulary range) go
    // to one XCD, whose L2 then serves their shared W_lm rows.
    const int G = a.n_mt * a.n_vr;
    const int xcd = blockIdx.x & 7, per = G >> 3, extra = G & 7;
    const int item = xcd * per + min(xcd, extra) + (int)(blockIdx.x >> 3);
    const int vr = item / a.n_mt, mt = item - vr * a.n_mt;
    const int64_t m0 = (int64_t)mt * ROWS;
    const int mrows = (int)min<int64_t>(ROWS, a.M - m0);
    // vocabulary range vr: blocks [rb0, rb0 + R), cut into whole chunks of
    // 16 blocks and a last, shorter one (every wave multiplies four blocks
    // in a whole chunk, so no wave waits for another at the barriers)
    const LmSplit ranges(a.nblk, a.n_vr);
    const int rb0 = ranges.start(vr), R = ranges.size(vr);
    const int nch = (R + kLmChunkBlocks - 1) / kLmChunkBlocks;
    const int d = a.d;
    const int col0 = 16 * rb0, col_end = min(16 * (rb0 + R), a.V);

    const __amdgpu_buffer_rsrc_t rx = lm_rsrc(a.X + m0 * d, (uint32_t)(mrows * d * 2));
    uint32_t xoff[XL::XP];
    XL::offsets(d, xoff);

    for (int e = tid; e < (int)(sizeof(sm.lst) / sizeof(double)); e += kWG) (&sm.lst[0][0][0])[e] = 0.0;

    for (int c = 0; c < nch; ++c) {
        const int c0 = rb0 + c * kLmChunkBlocks, nbc = min(kLmChunkBlocks, R - c * kLmChunkBlocks);
        int cb, nbw;
        lm_wave_blocks(c0, nbc, __builtin_amdgcn_readfirstlane(w), cb, nbw);
        // the wave's W_lm rows 16 cb .. 16 (cb + nbw), cut at V
        const int wrows = max(0, min(16 * nbw, a.V - 16 * cb));
        const __amdgpu_buffer_rsrc_t rw =
            lm_rsrc(a.W + (int64_t)min(16 * cb, a.V - 1) * d, (uint32_t)(wrows * d * 2));

        f32x4_t acc[MB][kLmWaveBlocks];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < kLmWaveBlocks; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        switch (nbw) {
            case 0: lm_chunk<MB, KMAX, 0>(rx, xoff, rw, d, sm, acc); break;
            case 1: lm_chunk<MB, KMAX, 1>(rx, xoff, rw, d, sm, acc); break;
            case 2: lm_chunk<MB, KMAX, 2>(rx, xoff, rw, d, sm, acc); break;
            case 3: lm_chunk<MB, KMAX, 3>(rx, xoff, rw, d, sm, acc); break;
            default: lm_chunk<MB, KMAX, 4>(rx, xoff, rw, d, sm, acc); break;
        }

        // ---- epilogue: fold this chunk's columns into the row lists (an
        // entry carries its column, so equal values keep the lower column
        // first whatever the order of folding) ----
        if constexpr (lm_wide(MB, KMAX)) {
            // the wave spills its blocks to its own slab; value v of block
            // (i, j): row 16 i + 4 g + v, column 16 j + row.  Lane (sub, r)
            // then folds its share of row r (columns SUBC sub .. SUBC (sub +
            // 1)) into its own list of that row.
            constexpr int LPR = lm_lpr(MB, KMAX);
            constexpr int SUBC = 16 * kLmWaveBlocks / LPR;
            constexpr int NC = SUBC < kLmSlabCols ? SUBC : kLmSlabCols;
#pragma unroll
            for (int j = 0; j < kLmWaveBlocks; ++j) {
                if (j < nbw) {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            sm.wslab[w][16 * i + 4 * g + v][16 * j + row] = acc[i][j][v];
                }
            }
            wave_sync();
            const int r = lane % ROWS, sub = lane / ROWS;
            if (r < mrows) {
                double lw[KMAX];
#pragma unroll
                for (int j = 0; j < KMAX; ++j) lw[j] = sm.lst[w * LPR + sub][r][j];
                float floor_v = lm_floor(lw[KMAX - 1]);
                const int wcols = min(16 * nbw, col_end - 16 * cb);   // the wave's valid columns
#pragma unroll
                for (int q = 0; q < SUBC / NC; ++q) {
                    const int cq = SUBC * sub + NC * q;
                    const int nc = min(NC, wcols - cq);
                    if (nc > 0)
                        lm_fold<KMAX, NC>(lw, floor_v, &sm.wslab[w][r][cq], nc, 16 * cb - col0 + cq);
                }
#pragma unroll
                for (int j = 0; j < KMAX; ++j) sm.lst[w * LPR + sub][r][j] = lw[j];
            }
        } else {
            const int trow = min(tid, ROWS - 1);
            double lw[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) lw[j] = sm.lst[0][trow][j];
            float floor_v = lm_floor(lw[KMAX - 1]);
            for (int p = 0; p < 2 * kWaves; ++p) {
                const int pw = p >> 1, h = p & 1;
                if (w == pw) {
                    // value v of block (i, j): row 16 i + 4 g + v, column 16 j + row
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                sm.slab[16 * i + 4 * g + v][16 * jj + row] =
                                    h ? acc[i][2 + jj][v] : acc[i][jj][v];
                }
                int pcb, pnb;
                lm_wave_blocks(c0, nbc, pw, pcb, pnb);
                const int v0 = 16 * (pcb + 2 * h);
                const int ncols = max(0, min(min(pnb - 2 * h, 2) * 16, col_end - v0));
                __syncthreads();
                if (tid < mrows && ncols > 0) lm_fold<KMAX, kLmSlabCols>(lw, floor_v, sm.slab[tid], ncols, v0 - col0);
                __syncthreads();
            }
            if (tid < mrows) {
#pragma unroll
                for (int j = 0; j < KMAX; ++j) sm.lst[0][tid][j] = lw[j];
            }
        }
        // the lists and the tile are read before the next chunk's X lands
        __syncthreads();
    }

    // small tiles: merge each row's lists into the first, those of one wave
    // first (in parallel over the waves), then the four waves' results
    if constexpr (lm_wide(MB, KMAX)) {
        constexpr int LPR = lm_lpr(MB, KMAX);
        __syncthreads();
        if constexpr (LPR > 1) {
            if (lane < mrows) {
                double lw[KMAX];
#pragma unroll
                for (int j = 0; j < KMAX; ++j) lw[j] = sm.lst[w * LPR][lane][j];
#pragma unroll
                for (int u = 1; u < LPR; ++u)
                    lm_merge_top<KMAX>(lw, [&](int j) { return sm.lst[w * LPR + u][lane][j]; });
#pragma unroll
                for (int j = 0; j < KMAX; ++j) sm.lst[w * LPR][lane][j] = lw[j];
            }
            __syncthreads();
        }
        if (tid < mrows) {
            double lw[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) lw[j] = sm.lst[0][tid][j];
#pragma unroll
            for (int u = 1; u < kWaves; ++u)
                lm_merge_top<KMAX>(lw, [&](int j) { return sm.lst[u * LPR][tid][j]; });
#pragma unroll
            for (int j = 0; j < KMAX; ++j) sm.lst[0][tid][j] = lw[j];
        }
    }

    // hand the lists to the merge as candidate words (0 = empty)
    if (tid < mrows) {
        uint64_t* plist = a.part + ((m0 + tid) * a.n_vr + vr) * (int64_t)KMAX;
#pragma unroll
        for (int j = 0; j < KMAX; j += 2) {
            uint64_t wd[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const double e = sm.lst[0][tid][j + q];
                const uint32_t key = lm_entry_key(e);
                const int off = kLmMaxRangeCols - 1 - (int)(e - (double)key * kLmOffScale);
                wd[q] = key ? cand_word(key, (uint32_t)(col0 + off)) : 0ull;
            }
            *reinterpret_cast<u32x4_t*>(plist + j) = u32x4_t{
                (uint32_t)wd[0], (uint32_t)(wd[0] >> 32), (uint32_t)wd[1], (uint32_t)(wd[1] >> 32)};
        }
    }
}

// Row merge of the n_vr lists of KMAX words (the first K of each are used).
struct LmMergeLds {
    uint64_t heads[kLmMaxLists];
    uint64_t tk, th;
    uint32_t m;
};

// One workgroup per row; thread l holds list l whole (one round of loads).
template <int KMAX>
__global__ __launch_bounds__(kWG) void k_lmhead_merge(LmArgs a) {
    extern __shared__ uint64_t surv[];      // up to n_vr * K words
    __shared__ LmMergeLds sm;
    const int tid = threadIdx.x;
    const int64_t mrow = blockIdx.x;
    const int nl = a.n_vr, K = a.K;
    const uint64_t* __restrict__ L = a.part + mrow * nl * (int64_t)KMAX;
    if (tid == 0) {
        sm.tk = 0ull;
        sm.th = 0ull;
        sm.m = 0u;
    }
    uint64_t x[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) x[j] = 0ull;
    if (tid < nl) {
#pragma unroll
        for (int j = 0; j < KMAX; j += 2) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(L + (int64_t)tid * KMAX + j);
            x[j] = ((uint64_t)v.y << 32) | v.x;
            x[j + 1] = ((uint64_t)v.w << 32) | v.z;
        }
    }
    uint64_t kth = 0ull;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) kth = (j == K - 1) ? x[j] : kth;
    const uint64_t head = x[0];
    __syncthreads();
    // bound 1: the best K-th word of any list (K words reach it): a maximum
    // within each wave, then one LDS atomic per wave (atomics of all 256
    // threads on one word serialise, about 4 us; lists past nl hold 0)
    uint64_t wk = kth;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t y = __shfl_xor(wk, o);
        wk = y > wk ? y : wk;
    }
    if ((tid & 63) == 0) __hip_atomic_fetch_max(&sm.tk, wk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    sm.heads[tid] = head;
    __syncthreads();
    // bound 2: the K-th best head (K heads reach it)
    if (nl >= K && tid < nl) {
        // all 256 slots (empty lists have head 0, which ranks no head)
        int rank = 0;
#pragma unroll 32
        for (int u = 0; u < kLmMaxLists; ++u) rank += sm.heads[u] > head ? 1 : 0;
        if (rank == K - 1) sm.th = head;
    }
    __syncthreads();
    uint64_t T = sm.tk > sm.th ? sm.tk : sm.th;
    T = T ? T : 1ull;
    // each list hands on its words that reach the bound (a prefix of it)
    int c = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) c += (j < K && x[j] >= T) ? 1 : 0;
    if (c > 0) {
        const uint32_t base = __hip_atomic_fetch_add(&sm.m, (uint32_t)c, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < c) surv[base + j] = x[j];
    }
    __syncthreads();
    const int m = (int)sm.m;
    for (int s0 = 0; s0 < m; s0 += kWG) {
        const int si = s0 + tid;
        const uint64_t y = (si < m) ? surv[si] : 0ull;
        int rank = 0;
        for (int u0 = 0; u0 < m; u0 += 16) {
#pragma unroll
            for (int u = 0; u < 16; ++u) rank += (u0 + u < m && surv[min(u0 + u, m - 1)] > y) ? 1 : 0;
        }
        if (si < m && rank < K) {
            a.out_idx[mrow * K + rank] = (int32_t)cand_index(y);
            a.out_val[mrow * K + rank] = value_of_key_f32((uint32_t)(y >> 32));
        }
    }
}

}  // namespace df2
