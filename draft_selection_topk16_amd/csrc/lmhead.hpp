// The drafter's LM head fused with top-K.
//
// The selector starts from the drafter's own logits ("DFlash 2: Keep Drafting
// Parallel", section "A Lightweight Path Selector": the selector needs no
// extra LM-head pass), read as U_t(v) = <W_lm[v], h_t> over the vocabulary.
// Computing them here, beside the top-K, keeps the [M, V] logits out of HBM:
// the one large read is W_lm itself (V x d bf16), streamed exactly once.
//
// k_lmhead: workgroup (mt, vr) multiplies M tile mt (up to 16 MB rows of X)
// by the W_lm rows of vocabulary range vr on the matrix cores (bf16 operands,
// fp32 sums).  The range's 16-column blocks are split evenly into chunks of
// at most 16 blocks and, inside a chunk, evenly over the four waves, so every
// wave owns at most four blocks (64 columns) of W_lm and streams them from
// HBM straight into registers, five 64-deep k slices ahead (two for the
// largest tile).  X reaches the
// waves through LDS, one 64-deep k slice at a time: buffer loads write it
// there directly, two slices ahead (three buffers).  Within a slice, lane
// group g takes the 16 consecutive k of its 32-byte piece, eight per matrix
// instruction, so that one wave's two loads cover whole 128-byte lines of W_lm.
// After the last slice of a chunk the waves spill their fp32 tiles to LDS
// (where the X slices were), 32 columns at a time, and one thread per row
// folds them, in column order, into that row's running list of its best KMAX
// candidates (value keys and indices), which stays in LDS until the
// workgroup ends.  A value enters only if it beats the list's last entry; an
// insertion is a branch-free update of every entry at once.
//
// k_lmhead_merge: one workgroup per row merges the row's n_vr sorted lists:
// a bound that K words are known to reach (the best K-th word of any list,
// and the K-th best head), compaction of the words that reach it (read only
// from the lists whose head reaches it), and ranks by counting.  Candidate words (key << 32 | ~index) are distinct within a
// row, so results do not depend on timing or on the launch plan.
#pragma once

#include <math.h>

#include "common.hpp"

namespace df2 {

constexpr int kLmWaveBlocks = 4;                          // 16-column blocks per wave
constexpr int kLmChunkBlocks = kWaves * kLmWaveBlocks;    // 256 columns per chunk
constexpr int kLmSliceK = 64;                             // k per X slice
// W slices held in registers per wave (also the unroll of the slice loop,
// whose body is branch-free so that the compiler's memory-counter waits stay
// exact and the loads of later slices stay in flight): six, three for the
// largest tile, whose accumulators leave no room for more
__host__ __device__ constexpr int lm_ring(int mb) { return mb >= 16 ? 3 : 6; }
constexpr int kLmXBufs = 3;                               // X slice buffers in LDS
constexpr int kLmSlabCols = 32;                           // columns per epilogue pass
constexpr int kLmSlabStride = kLmSlabCols + 1;
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
        // X slice: row, 16-byte piece; piece p of row r sits at p ^ (r & 7), so
        // that the eight rows a matrix-operand read touches fall in distinct banks
        u32x4_t xs[kLmXBufs][lm_xrows(MB)][8];
        // a chunk's fp32 tile, 32 columns at a time (between chunks)
        float slab[16 * MB][kLmSlabStride];
    };
    // each row's running list of its best KMAX candidates, best first: value
    // keys (0 = empty) and vocabulary indices; rows padded by 16 bytes so that
    // 16-byte reads of consecutive rows fall in distinct banks
    uint32_t lkey[16 * MB][KMAX + 4];
    uint32_t lidx[16 * MB][KMAX + 4];
};

// s_waitcnt immediate: vmcnt(n) (n <= 63), expcnt and lgkmcnt left alone
__host__ __device__ constexpr int lm_vmcnt(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Blocks [b0, b1) of vocabulary range vr.
__device__ __forceinline__ void lm_range(int nblk, int n_vr, int vr, int& b0, int& b1) {
    b0 = (int)((int64_t)nblk * vr / n_vr);
    b1 = (int)((int64_t)nblk * (vr + 1) / n_vr);
}

// Wave w's blocks [cb, cb + nbw) in chunk c of a range of R blocks from rb0
// split into nch chunks.
__device__ __forceinline__ void lm_wave_blocks(int rb0, int R, int nch, int c, int w, int& cb,
                                               int& nbw) {
    const int c0 = rb0 + (int)((int64_t)R * c / nch);
    const int nb = rb0 + (int)((int64_t)R * (c + 1) / nch) - c0;
    cb = c0 + (nb * w) / kWaves;
    nbw = c0 + (nb * (w + 1)) / kWaves - cb;
}

// Insert (key xk, index xi) into a row's list, sorted by key, best first,
// dropping the last entry.  The new index is larger than every listed one
// (columns arrive in order), so an equal key stays ahead of it.  Every entry
// decides on its own: those that stay ahead keep their place, the first one
// that does not takes the new pair, the rest move down one.
template <int KMAX>
__device__ __forceinline__ void lm_insert(uint32_t (&lk)[KMAX], uint32_t (&li)[KMAX], uint32_t xk,
                                          uint32_t xi) {
    // all-ones where the entry stays ahead; bit selects keep this branch-free
    uint32_t ahead[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ahead[j] = 0u - (uint32_t)(lk[j] >= xk);
#pragma unroll
    for (int j = KMAX - 1; j > 0; --j) {
        const uint32_t nk = (ahead[j - 1] & xk) | (~ahead[j - 1] & lk[j - 1]);
        const uint32_t ni = (ahead[j - 1] & xi) | (~ahead[j - 1] & li[j - 1]);
        lk[j] = (ahead[j] & lk[j]) | (~ahead[j] & nk);
        li[j] = (ahead[j] & li[j]) | (~ahead[j] & ni);
    }
    lk[0] = (ahead[0] & lk[0]) | (~ahead[0] & xk);
    li[0] = (ahead[0] & li[0]) | (~ahead[0] & xi);
}

// the value a candidate must beat to enter a list whose last key is `last`
__device__ __forceinline__ float lm_floor(uint32_t last) {
    return last ? value_of_key_f32(last) : -INFINITY;
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

// X slices go from memory straight into LDS (buffer loads with the lds bit:
// lane l of a wave's load writes the l-th 16 bytes of a 1 KB stretch).
// Load q of wave w fills rows 8 (4 q + w) .. + 7 of a buffer; lane l takes
// row 8 (4 q + w) + l / 8 and physical slot l % 8, which holds piece
// (l % 8) ^ (row % 8) of the row.  The resource covers the tile's mrows rows,
// so rows past M read as zero.
template <int MB, int KMAX>
struct LmX {
    static constexpr int XROWS = lm_xrows(MB);
    static constexpr int NX = XROWS / 32;        // loads per wave per slice
    static_assert(XROWS % 32 == 0, "whole 1 KB stretches per wave");
    __device__ static void offsets(int d, uint32_t (&off)[NX]) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int q = 0; q < NX; ++q) {
            const int r = 8 * (4 * q + w) + (lane >> 3);
            const int p = (lane & 7) ^ ((lane >> 3) & 7);
            off[q] = (uint32_t)((r * d + p * 8) * 2);
        }
    }
    __device__ static void load(__amdgpu_buffer_rsrc_t rx, const uint32_t (&off)[NX], int s,
                                LmLds<MB, KMAX>& sm, int buf) {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int q = 0; q < NX; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)&sm.xs[buf][8 * (4 * q + w)][0], 16,
                (int)off[q], s * (kLmSliceK * 2), 0, 0);
    }
};

// One chunk's products: acc[i][j] += X rows of m-block i times W rows of the
// wave's block j, over all of d.  The wave multiplies its NBW blocks (the
// chunk's even split gives it that many); every wave meets every barrier.
// rw covers the wave's rows of W_lm (rows past V read as zero).
template <int MB, int KMAX, int NBW>
__device__ __forceinline__ void lm_chunk(__amdgpu_buffer_rsrc_t rx,
                                         const uint32_t (&xoff)[LmX<MB, KMAX>::NX],
                                         __amdgpu_buffer_rsrc_t rw, int d, LmLds<MB, KMAX>& sm,
                                         f32x4_t (&acc)[MB][kLmWaveBlocks]) {
    using XL = LmX<MB, KMAX>;
    constexpr int NB = NBW > 0 ? NBW : 1;
    constexpr int RING = lm_ring(MB);
    static_assert(RING % kLmXBufs == 0, "the X buffers cycle inside the unroll");
    // Loads a wave issues after slice s + 1's X: W of slices s - 1 + RING and
    // s + RING, X of slice s + 2.  Waiting until no more are outstanding
    // leaves slice s + 1 in LDS (memory counters complete in order).
    constexpr int kWaitX = XL::NX + 4 * NBW;
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
    // Step of slice s (ring slot u == s % RING, X buffer s % 3): load X slice
    // s + 2, multiply (only for s < ns: past the end the loads repeat the last
    // slice and nothing is added), load W slice s + RING into the slot just
    // used, wait for X slice s + 1 and meet the other waves.
    auto step = [&](int s, int u) {
        const int xb = u % kLmXBufs;
        XL::load(rx, xoff, min(s + 2, ns - 1), sm, (u + 2) % kLmXBufs);
        if constexpr (NBW > 0) {
            if (s < ns) {
                u32x4_t a0 = sm.xs[xb][row][(2 * g) ^ (row & 7)];
                u32x4_t a1 = sm.xs[xb][row][(2 * g + 1) ^ (row & 7)];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    // read block i + 1's operands while block i multiplies
                    u32x4_t n0 = a0, n1 = a1;
                    if (i + 1 < MB) {
                        n0 = sm.xs[xb][16 * (i + 1) + row][(2 * g) ^ (row & 7)];
                        n1 = sm.xs[xb][16 * (i + 1) + row][(2 * g + 1) ^ (row & 7)];
                    }
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        acc[i][j] = mfma_bf16(as_bf16x8(a0), as_bf16x8(wr[u][j][0]), acc[i][j]);
                        acc[i][j] = mfma_bf16(as_bf16x8(a1), as_bf16x8(wr[u][j][1]), acc[i][j]);
                    }
                    if (i + 1 < MB) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // 2 LDS reads
                        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NBW, 0);  // products
                    }
                    a0 = n0;
                    a1 = n1;
                }
            }
            load_w(s + RING, wr[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(lm_vmcnt(kWaitX));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: X slices 0 and 1, then W slices 0 .. RING-1; X slice 0 waited for
    XL::load(rx, xoff, 0, sm, 0);
    XL::load(rx, xoff, min(1, ns - 1), sm, 1);
#pragma unroll
    for (int u = 0; u < RING; ++u) load_w(u, wr[u]);
    constexpr int kWait0 = XL::NX + 2 * NBW * RING < 63 ? XL::NX + 2 * NBW * RING : 63;
    __builtin_amdgcn_s_waitcnt(lm_vmcnt(kWait0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    for (int s0 = 0; s0 < ns; s0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) step(s0 + u, u);
    }
    // the last steps' loads land before the buffers are reused
    __builtin_amdgcn_s_waitcnt(lm_vmcnt(0));
    __syncthreads();
}

template <int MB, int KMAX>
__global__ __launch_bounds__(kWG, 1) void k_lmhead(LmArgs a) {
    static_assert(KMAX % 2 == 0, "lists move in 16-byte pairs");
    constexpr int ROWS = 16 * MB;
    using XL = LmX<MB, KMAX>;
    __shared__ LmLds<MB, KMAX> sm;
    static_assert(sizeof(sm.slab) <= sizeof(sm.xs), "the tile fits where the X slices were");
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
    int rb0, rb1;
    lm_range(a.nblk, a.n_vr, vr, rb0, rb1);
    const int R = rb1 - rb0;
    const int nch = (R + kLmChunkBlocks - 1) / kLmChunkBlocks;
    const int d = a.d;
    const int col_end = min(16 * rb1, a.V);

    const __amdgpu_buffer_rsrc_t rx = lm_rsrc(a.X + m0 * d, (uint32_t)(mrows * d * 2));
    uint32_t xoff[XL::NX];
    XL::offsets(d, xoff);

    for (int e = tid; e < ROWS * (KMAX + 4); e += kWG) (&sm.lkey[0][0])[e] = 0u;

    for (int c = 0; c < nch; ++c) {
        int cb, nbw;
        lm_wave_blocks(rb0, R, nch, c, __builtin_amdgcn_readfirstlane(w), cb, nbw);
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

        // ---- epilogue: fold this chunk's columns into the row lists, in
        // column order (so a value equal to a kept one never displaces it) ----
        const int trow = min(tid, ROWS - 1);
        uint32_t lk[KMAX], li[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; j += 4) {
            const u32x4_t k4 = *reinterpret_cast<const u32x4_t*>(&sm.lkey[trow][j]);
            const u32x4_t i4 = *reinterpret_cast<const u32x4_t*>(&sm.lidx[trow][j]);
            lk[j] = k4.x; lk[j + 1] = k4.y; lk[j + 2] = k4.z; lk[j + 3] = k4.w;
            li[j] = i4.x; li[j + 1] = i4.y; li[j + 2] = i4.z; li[j + 3] = i4.w;
        }
        float floor_v = lm_floor(lk[KMAX - 1]);
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
            lm_wave_blocks(rb0, R, nch, c, pw, pcb, pnb);
            const int v0 = 16 * (pcb + 2 * h);
            const int ncols = max(0, min(min(pnb - 2 * h, 2) * 16, col_end - v0));
            __syncthreads();
            if (tid < mrows && ncols > 0) {
                // all 32 columns at once (columns past ncols are never flagged)
                const float* srow = sm.slab[tid];
                float xv[kLmSlabCols];
#pragma unroll
                for (int cc = 0; cc < kLmSlabCols; ++cc) xv[cc] = srow[cc];
                uint32_t flagged = 0;
#pragma unroll
                for (int cc = 0; cc < kLmSlabCols; ++cc)
                    flagged |= (cc < ncols && xv[cc] > floor_v) ? (1u << cc) : 0u;
                while (flagged) {
                    const int cc = __builtin_ctz(flagged);
                    flagged &= flagged - 1u;
                    const float x = srow[cc];
                    if (x > floor_v) {
                        lm_insert<KMAX>(lk, li, key_f32(__float_as_uint(x)), (uint32_t)(v0 + cc));
                        floor_v = lm_floor(lk[KMAX - 1]);
                    }
                }
            }
            __syncthreads();
        }
        if (tid < mrows) {
#pragma unroll
            for (int j = 0; j < KMAX; j += 4) {
                *reinterpret_cast<u32x4_t*>(&sm.lkey[tid][j]) = u32x4_t{lk[j], lk[j + 1], lk[j + 2], lk[j + 3]};
                *reinterpret_cast<u32x4_t*>(&sm.lidx[tid][j]) = u32x4_t{li[j], li[j + 1], li[j + 2], li[j + 3]};
            }
        }
        // the lists and the tile are read before the next chunk's X lands
        __syncthreads();
    }

    // hand the lists to the merge as candidate words (0 = empty)
    if (tid < mrows) {
        uint64_t* plist = a.part + ((m0 + tid) * a.n_vr + vr) * (int64_t)KMAX;
#pragma unroll
        for (int j = 0; j < KMAX; j += 2) {
            const uint32_t k0 = sm.lkey[tid][j], k1 = sm.lkey[tid][j + 1];
            const uint64_t w0 = k0 ? cand_word(k0, sm.lidx[tid][j]) : 0ull;
            const uint64_t w1 = k1 ? cand_word(k1, sm.lidx[tid][j + 1]) : 0ull;
            *reinterpret_cast<u32x4_t*>(plist + j) =
                u32x4_t{(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
        }
    }
}

// Row merge of the n_vr lists of KMAX words (the first K of each are used).
struct LmMergeLds {
    uint64_t heads[kLmMaxLists];
    uint64_t tk, th;
    uint32_t m;
};

__global__ __launch_bounds__(kWG) void k_lmhead_merge(LmArgs a) {
    extern __shared__ uint64_t surv[];      // up to n_vr * K words
    __shared__ LmMergeLds sm;
    const int tid = threadIdx.x;
    const int64_t mrow = blockIdx.x;
    const int nl = a.n_vr, K = a.K, ks = a.kstride;
    const uint64_t* __restrict__ L = a.part + mrow * nl * (int64_t)ks;
    if (tid == 0) {
        sm.tk = 0ull;
        sm.th = 0ull;
        sm.m = 0u;
    }
    __syncthreads();
    // bound 1: the best K-th word of any list (K words reach it)
    uint64_t head = 0ull;
    if (tid < nl) {
        head = L[(int64_t)tid * ks];
        const uint64_t kth = L[(int64_t)tid * ks + K - 1];
        __hip_atomic_fetch_max(&sm.tk, kth, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    sm.heads[tid] = head;
    __syncthreads();
    // bound 2: the K-th best head (K heads reach it)
    if (nl >= K && tid < nl) {
        int rank = 0;
        for (int u = 0; u < nl; ++u) rank += sm.heads[u] > head ? 1 : 0;
        if (rank == K - 1) sm.th = head;
    }
    __syncthreads();
    uint64_t T = sm.tk > sm.th ? sm.tk : sm.th;
    T = T ? T : 1ull;
    // each list that reaches the bound hands on its words that reach it (a
    // prefix: lists are sorted), eight at a time
    if (tid < nl && head >= T) {
        const uint64_t* lp = L + (int64_t)tid * ks;
        for (int k0 = 0; k0 < K; k0 += 8) {
            uint64_t x[8];
#pragma unroll
            for (int q = 0; q < 8; q += 2) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lp + k0 + q);
                x[q] = ((uint64_t)v.y << 32) | v.x;
                x[q + 1] = ((uint64_t)v.w << 32) | v.z;
            }
            int c = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) c += (k0 + q < K && x[q] >= T) ? 1 : 0;
            const uint32_t base = __hip_atomic_fetch_add(&sm.m, (uint32_t)c, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q < c) surv[base + q] = x[q];
            if (c < 8) break;
        }
    }
    __syncthreads();
    const int m = (int)sm.m;
    for (int s0 = 0; s0 < m; s0 += kWG) {
        const int si = s0 + tid;
        const uint64_t y = (si < m) ? surv[si] : 0ull;
        int rank = 0;
        for (int u = 0; u < m; ++u) rank += surv[u] > y ? 1 : 0;
        if (si < m && rank < K) {
            a.out_idx[mrow * K + rank] = (int32_t)cand_index(y);
            a.out_val[mrow * K + rank] = value_of_key_f32((uint32_t)(y >> 32));
        }
    }
}

}  // namespace df2
