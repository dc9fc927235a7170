// Per-row top-K over the vocabulary ("DFlash 2: Keep Drafting Parallel",
// section "A Lightweight Path Selector": keep the top 16 candidates at each
// draft position).
//
// Stage 1 (segment): a workgroup streams one segment of one row (every
// nseg-th chunk of the row).  Each of its four waves works on its own: it streams every fourth chunk of
// 64 lanes x NV 16-byte vectors, with the next chunk's loads issued before
// the current chunk is processed (two register buffers), and keeps its best
// K candidate words in registers, one word per lane, sorted.  Per chunk each
// lane reduces its values to one statistic, its true maximum, using packed
// 16-bit integer max/min on the raw bf16 bits (non-negative values order like
// their bits; negative values order reversed, so the maximum of a lane is its
// largest bit pattern if it has any non-negative value and its smallest one
// otherwise).  A value can only enter if it reaches a bound that at least K
// values of the row are known to reach: the wave's own K-th kept key, or the
// best K-th kept key of the workgroup's four waves (an LDS word each wave
// raises with an atomic max; any wave's K-th key bounds the row's K-th
// largest value from below).  The first bound of each wave is the K-th
// largest of its 64 lane maxima over its first chunk.  Once a few chunks have been seen, most
// chunks have no lane that reaches the bound and cost a handful of
// instructions.  Vectors that do reach it are keyed exactly from
// registers; words that beat the K-th kept word are compacted (ballot) into
// an LDS buffer, which is merged into the list (all ranks found in parallel)
// once to establish it and then only when it fills.  No step of a chunk
// needs a workgroup barrier.  At the end of the segment each wave's sorted
// list is handed on as it is.
//
// Stage 2 (merge): the last segment of a row to finish merges the row's
// sorted lists (four per segment) with the whole workgroup
// (block_merge_lists): a bound (the best K-th word of any list), compaction
// of the words that reach it, and ranks by counting.
//
// Candidate words (key << 32 | ~index) are distinct within a row, so every
// selection is exact and independent of arrival order: results are
// deterministic.
#pragma once

#include <math.h>

#include "common.hpp"

namespace df2 {

constexpr int kMaxNV = 4;           // 16-byte vectors per lane per chunk
constexpr int kMergeMax = 1024;     // words merged per row (segment lists * K)
static_assert(kMergeMax % kWG == 0, "whole words per thread when a row is loaded");

constexpr int kWCand = 256;         // candidate words buffered per wave
constexpr int kWPend = 64;          // pending vectors per wave before a flush

struct WaveLds {
    u32x4_t pend[kWPend];               // surviving vectors awaiting keying
    uint32_t pend_e0[kWPend];           // row index of each one's first element
    uint64_t cand[kWCand];
    uint64_t L2[64];                    // the merged list
};

struct ChunkLds {
    WaveLds wv[kWaves];
    uint32_t bound;                     // a key at least K values of the segment reach
    uint32_t qkey[kWaves];              // each wave's ceil(K/4)-th kept key
};

struct MergeLds {
    uint64_t surv[kMergeMax];           // words that reach the bound
    uint64_t tk, tc;                    // bound candidates
    uint32_t m;                         // survivors
    uint32_t aux;                       // for the caller's hooks
    uint32_t aux2;                      // head bound
};

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
    static constexpr int kPerVec = 8;
    static constexpr int kKeyBits = 16;
    __device__ static uint32_t key(uint32_t bits) { return key_bf16(bits); }
    __device__ static float value(uint32_t key) { return value_of_key_bf16(key); }
};
template <>
struct Elem<false> {
    static constexpr int kPerVec = 4;
    static constexpr int kKeyBits = 32;
    __device__ static uint32_t key(uint32_t bits) { return key_f32(bits); }
    __device__ static float value(uint32_t key) { return value_of_key_f32(key); }
};

// Raw bits of element p (0 .. kPerVec-1) of a 16-byte vector.
template <bool BF16>
__device__ __forceinline__ uint32_t elem_bits(const u32x4_t& v, int p) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (BF16) {
        uint32_t d = w[p >> 1];
        return (p & 1) ? (d >> 16) : (d & 0xFFFFu);
    } else {
        return w[p];
    }
}

// Element-wise load of the 16-byte vector holding elements [e0, e0 + kPerVec)
// of a row that is not 16-byte aligned (or whose length is not a multiple of
// kPerVec); out-of-row elements read as the all-ones sentinel.
template <bool BF16>
__device__ __forceinline__ u32x4_t load_vec_elems(const void* __restrict__ row, int V, int64_t e0) {
    constexpr int PV = Elem<BF16>::kPerVec;
    uint32_t wv[4] = {~0u, ~0u, ~0u, ~0u};
#pragma unroll
    for (int p = 0; p < PV; ++p) {
        const int64_t e = e0 + p;
        if (e < V) {
            if constexpr (BF16) {
                const uint32_t bits = reinterpret_cast<const uint16_t*>(row)[e];
                const uint32_t sh = (p & 1) * 16;
                wv[p >> 1] = (wv[p >> 1] & ~(0xFFFFu << sh)) | (bits << sh);
            } else {
                wv[p] = reinterpret_cast<const uint32_t*>(row)[e];
            }
        }
    }
    return u32x4_t{wv[0], wv[1], wv[2], wv[3]};
}

// Aligned rows are read through a raw buffer resource that spans exactly the
// row (num_records = its bytes).  A load whose offset lies past the end
// returns zeros without touching memory, so prefetches beyond the segment
// (and the vector slots beyond the row in its last chunk) cost no traffic.
// Loads carry the non-temporal hint: the logits are read once.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, (int)bytes,
                                             0x00020000);
}
constexpr uint32_t kOutOfRow = 0x80000000u;     // beyond any row (rows are < 2^31 bytes)
template <bool BF16>
__device__ __forceinline__ u32x4_t load_vec_rs(__amdgpu_buffer_rsrc_t rs, int V, int64_t e0,
                                               bool live) {
    constexpr int ESZ = BF16 ? 2 : 4;
    const uint32_t off = (live && e0 < V) ? (uint32_t)(e0 * ESZ) : kOutOfRow;
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
}

// At consumption: an aligned vector that lies beyond the row becomes the
// sentinel (its buffer load returned zeros).
template <bool ALIGNED>
__device__ __forceinline__ u32x4_t mask_vec(u32x4_t x, int64_t e0, int V) {
    if constexpr (ALIGNED) {
        const u32x4_t ones = u32x4_t{~0u, ~0u, ~0u, ~0u};
        return (e0 < V) ? x : ones;
    } else {
        return x;
    }
}

// Lane maximum (in value order) of a lane's vectors, as a key.
template <bool BF16, int NV>
__device__ __forceinline__ uint32_t lane_max_key(const u32x4_t (&v)[NV]) {
    uint32_t stat_bits;
    if constexpr (BF16) {
        s16x2_t mx = __builtin_bit_cast(s16x2_t, v[0].x);
        s16x2_t mn = mx;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const s16x2_t s = __builtin_bit_cast(s16x2_t, wd[q]);
                mx = __builtin_elementwise_max(mx, s);
                mn = __builtin_elementwise_min(mn, s);
            }
        }
        const int m = max((int)mx.x, (int)mx.y);
        const int n = min((int)mn.x, (int)mn.y);
        stat_bits = (uint32_t)((m >= 0) ? m : n) & 0xFFFFu;
    } else {
        int mx = (int)v[0].x, mn = mx;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                mx = max(mx, (int)wd[q]);
                mn = min(mn, (int)wd[q]);
            }
        }
        stat_bits = (uint32_t)((mx >= 0) ? mx : mn);
    }
    return Elem<BF16>::key(stat_bits);
}

// Maximum (in value order) of one 16-byte vector, as a key.
template <bool BF16>
__device__ __forceinline__ uint32_t vec_max_key(const u32x4_t& v) {
    const u32x4_t a[1] = {v};
    return lane_max_key<BF16, 1>(a);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Merges m distinct candidate words c[0..m) (LDS, written by this wave) into
// the sorted list held one word per lane (lane k: k-th best; unfilled slots
// and lanes >= K hold 0) and returns the best K.  Candidates are taken 64 at
// a time, one per lane; every rank is counted from registers (readlane over
// the candidates and over the list), then the words whose rank is below K
// are scattered through LDS.
// LDSR: ranks are counted from broadcast LDS reads of the other words
// (independent of each other) instead of readlanes (a dependent chain); it
// needs more registers and is used where the kernel has them to spare.
template <bool LDSR>
__device__ __forceinline__ uint64_t list_merge(uint64_t tk, const uint64_t* c, int m, int K,
                                               WaveLds& sm) {
    const int lane = lane_id();
    if constexpr (LDSR) {
        sm.L2[lane] = (lane < K) ? tk : 0ull;
        wave_sync();
        for (int base = 0; base < m; base += 64) {
            const int mg = min(64, m - base);
            const uint64_t ci = (lane < mg) ? c[base + lane] : 0ull;
            int rc = 0;         // candidates above ci
            int rl = lane;      // new rank of the list word tk
#pragma unroll 8
            for (int i = 0; i < mg; ++i) {
                const uint64_t x = c[base + i];
                rc += (x > ci) ? 1 : 0;
                rl += (x > tk) ? 1 : 0;
            }
            int rk = 0;         // list words above ci
#pragma unroll 8
            for (int k = 0; k < K; ++k) rk += (sm.L2[k] > ci) ? 1 : 0;
            wave_sync();
            sm.L2[lane] = 0ull;
            wave_sync();
            if (lane < K && tk != 0 && rl < K) sm.L2[rl] = tk;
            if (lane < mg && rc + rk < K) sm.L2[rc + rk] = ci;
            wave_sync();
            tk = (lane < K) ? sm.L2[lane] : 0ull;
        }
        wave_sync();
        return tk;
    }
    wave_sync();
    for (int base = 0; base < m; base += 64) {
        const int mg = min(64, m - base);
        const uint64_t ci = (lane < mg) ? c[base + lane] : 0ull;
        int rc = 0;         // candidates above ci
        int rl = lane;      // new rank of the list word tk
        for (int i = 0; i < mg; ++i) {
            const uint64_t x = readlane_u64(ci, i);
            rc += (x > ci) ? 1 : 0;
            rl += (x > tk) ? 1 : 0;
        }
        int rk = 0;         // list words above ci
        for (int k = 0; k < K; ++k) rk += (readlane_u64(tk, k) > ci) ? 1 : 0;
        sm.L2[lane] = 0ull;
        wave_sync();
        if (lane < K && tk != 0 && rl < K) sm.L2[rl] = tk;
        if (lane < mg && rc + rk < K) sm.L2[rc + rk] = ci;
        wave_sync();
        tk = (lane < K) ? sm.L2[lane] : 0ull;
        wave_sync();
    }
    return tk;
}

// Keys the wave's pending vectors and merges every word that beats the K-th
// kept word (and reaches Tm) into the sorted list tk.
template <bool BF16, bool LDSR = false>
__device__ uint64_t flush_pending(int V, int K, uint32_t Tm, uint64_t tk, int np, WaveLds& sm) {
    using E = Elem<BF16>;
    constexpr int PV = E::kPerVec;
    const int lane = lane_id();
    uint64_t kth = readlane_u64(tk, K - 1);
    Tm = max(Tm, (uint32_t)(kth >> 32));
    wave_sync();
    int n = 0;
    const int nel = np * PV;
#pragma unroll 1
    for (int e0 = 0; e0 < nel; e0 += 64) {
        const int e = e0 + lane;
        bool pred = false;
        uint64_t word = 0;
        if (e < nel) {
            const int sl = e / PV, p = e % PV;
            const uint32_t wd = reinterpret_cast<const uint32_t*>(&sm.pend[sl])[BF16 ? (p >> 1) : p];
            const uint32_t bits = BF16 ? ((p & 1) ? (wd >> 16) : (wd & 0xFFFFu)) : wd;
            const int64_t gidx = (int64_t)sm.pend_e0[sl] + p;
            const uint32_t key = E::key(bits);
            word = cand_word(key, (uint32_t)gidx);
            pred = gidx < V && key >= Tm && word > kth;
        }
        const uint64_t b2 = __ballot(pred);
        if (pred) sm.cand[n + __popcll(b2 & ((1ull << lane) - 1ull))] = word;
        n += __popcll(b2);
        if (n > kWCand - 64) {
            tk = list_merge<LDSR>(tk, sm.cand, n, K, sm);
            n = 0;
            kth = readlane_u64(tk, K - 1);
            Tm = max(Tm, (uint32_t)(kth >> 32));
        }
    }
    if (n > 0) tk = list_merge<LDSR>(tk, sm.cand, n, K, sm);
    wave_sync();            // the pending slots are rewritten next
    return tk;
}

// Folds one wave chunk (in registers) into the wave's state: the sorted list
// tk and np pending vectors (vectors that reach the bound, not yet keyed).
//   eb: row index of the chunk's first element; lane l, vector j, element p
//   hold element eb + (j * 64 + l) * kPerVec + p.
//   trow: a key that at least K values of the row are known to reach (the
//   best K-th kept key among the workgroup's waves; 0 if none known).
template <bool BF16, int NV, bool ALIGNED, bool LDSR = false>
__device__ uint64_t wave_chunk(int V, int64_t eb, int K, const u32x4_t (&raw)[NV], uint64_t tk,
                               uint32_t trow, int& np, WaveLds& sm) {
    using E = Elem<BF16>;
    constexpr int PV = E::kPerVec;
    const int lane = lane_id();
    u32x4_t v[NV];
    uint32_t vk[NV];
    uint32_t skey = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        v[j] = mask_vec<ALIGNED>(raw[j], eb + (int64_t)(j * 64 + lane) * PV, V);
        vk[j] = vec_max_key<BF16>(v[j]);
        skey = max(skey, vk[j]);
    }
    const uint64_t kth = readlane_u64(tk, K - 1);     // 0 while the list is filling
    uint32_t Tm = max((uint32_t)(kth >> 32), trow);
    if (Tm == 0) {
        // Nothing known yet: the K-th largest lane maximum of this chunk, by
        // a bitwise search over ballot counts (at least K values reach it).
        uint32_t T = 0;
#pragma unroll 1
        for (int bit = E::kKeyBits - 1; bit >= 0; --bit) {
            const uint32_t c = T | (1u << bit);
            if (ballot_count(skey >= c) >= K) T = c;
        }
        Tm = T;
    }
    Tm = max(Tm, 1u);                           // real values have key >= 1
    if (__ballot(skey >= Tm) == 0) return tk;   // the common case
    // Vectors that reach the bound wait in LDS; they are keyed and merged in
    // batches (flush_pending), so a chunk only pays for copying them.
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const bool vin = vk[j] >= Tm;
        const uint64_t bal = __ballot(vin);
        if (bal == 0) continue;
        if (np + __popcll(bal) > kWPend) {
            tk = flush_pending<BF16, LDSR>(V, K, Tm, tk, np, sm);
            np = 0;
        }
        if (vin) {
            const int slot = np + __popcll(bal & ((1ull << lane) - 1ull));
            sm.pend[slot] = v[j];
            sm.pend_e0[slot] = (uint32_t)(eb + (int64_t)(j * 64 + lane) * PV);
        }
        np += __popcll(bal);
    }
    return tk;
}

// Stage 1: best K candidate words of the chunks of one row that belong to
// this segment: the i-th (i < nc) is (c0 + (i / split) * cs) * split +
// i % split.  A chunk is 4 x 64 x NV vectors; wave w streams its quarter of
// every chunk.  The segments of a row interleave (cs = segments per row), so
// the workgroups of a row read neighbouring chunks at any one time.
//   row: first element of the row; V: row length; K <= 64.
//   ALIGNED: the row start is 16-byte aligned and V is a multiple of kPerVec.
//   out: 4 x K hand-off words, one sorted list per wave (0 for empty slots).
template <bool BF16, int NV, bool ALIGNED, bool LDSR = false>
__device__ void segment_topk_impl(const void* __restrict__ row, int V, int c0, int cs, int nc,
                                  int split, int K, uint64_t* __restrict__ out, ChunkLds& sm) {
    static_assert(NV >= 1 && NV <= kMaxNV, "chunk vectors per lane");
    constexpr int PV = Elem<BF16>::kPerVec;
    constexpr int WE = 64 * PV * NV;           // elements per wave chunk
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t tk = 0;
    int npend = 0;                             // pending vectors of this wave
    const int kq = (K + kWaves - 1) / kWaves;
    auto eb_of = [&](int i) {
        const int c = (c0 + (i / split) * cs) * split + i % split;
        return ((int64_t)c * kWaves + w) * WE;
    };
    // Publishes two bounds that at least K values of the segment reach: the
    // wave's own K-th kept key (raises sm.bound), and its ceil(K/4)-th kept
    // key -- the four waves hold disjoint values, so the smallest of their
    // four such keys is reached by at least K values.  Each word only grows;
    // a reader may see an older value, which is still a valid bound.
    auto publish = [&]() {
        const uint32_t kk = (uint32_t)(readlane_u64(tk, K - 1) >> 32);
        const uint32_t qq = (uint32_t)(readlane_u64(tk, kq - 1) >> 32);
        if (lane == 0) {
            __hip_atomic_fetch_max(&sm.bound, kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(&sm.qkey[w], qq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
    auto wg_bound = [&]() {
        uint32_t q = __hip_atomic_load(&sm.qkey[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int u = 1; u < kWaves; ++u)
            q = min(q, __hip_atomic_load(&sm.qkey[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        return max(q, __hip_atomic_load(&sm.bound, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    };
    // Flushes pending vectors once the buffer is half full (or at the end),
    // filtered by the best bound known now, then republishes the bounds.
    auto settle = [&](bool last) {
        if (npend >= kWPend / 2 || (last && npend > 0)) {
            const uint32_t Tb = max(wg_bound(), 1u);
            tk = flush_pending<BF16, LDSR>(V, K, Tb, tk, npend, sm.wv[w]);
            npend = 0;
            if (!last) publish();
        }
    };
    // Two register buffers, used in turn without copies: while one chunk is
    // processed the next one's loads are in flight.  Aligned rows load
    // through the row's buffer resource, and a prefetch past the segment end
    // reads nothing; otherwise it re-reads the last chunk (in bounds, never
    // consumed).
    u32x4_t b0[NV], b1[NV];
    const int clast = nc - 1;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, (uint32_t)V * (BF16 ? 2u : 4u));
    auto fetch = [&](u32x4_t (&b)[NV], int c) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if constexpr (ALIGNED)
                b[j] = load_vec_rs<BF16>(rs, V, eb_of(min(c, clast)) + (int64_t)(j * 64 + lane) * PV,
                                         c <= clast);
            else
                b[j] = load_vec_elems<BF16>(row, V, eb_of(min(c, clast)) + (int64_t)(j * 64 + lane) * PV);
        }
    };
    // The shared bounds start at zero (one barrier, before any load is in
    // flight).
    if (tid == 0) sm.bound = 0;
    if (tid < kWaves) sm.qkey[tid] = 0;
    __syncthreads();
    fetch(b0, 0);
    {
        // Initial bound, per wave: the K-th largest of its 64 lane maxima
        // over its first chunk (K lane maxima reach it); published with an
        // atomic max, no barrier.
        u32x4_t v[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j)
            v[j] = mask_vec<ALIGNED>(b0[j], eb_of(0) + (int64_t)(j * 64 + lane) * PV, V);
        const uint32_t q0 = lane_max_key<BF16, NV>(v);
        uint32_t T = 0;
#pragma unroll 1
        for (int bit = Elem<BF16>::kKeyBits - 1; bit >= 0; --bit) {
            const uint32_t c = T | (1u << bit);
            if (ballot_count(q0 >= c) >= K) T = c;
        }
        if (lane == 0)
            __hip_atomic_fetch_max(&sm.bound, T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    for (int c = 0; c < nc; c += 2) {
        fetch(b1, c + 1);
        tk = wave_chunk<BF16, NV, ALIGNED, LDSR>(V, eb_of(c), K, b0, tk, wg_bound(), npend, sm.wv[w]);
        settle(false);
        // Keep the next half's uses of its loads below this point: hoisting
        // one would wait on every load in flight, prefetch included.
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 >= nc) break;
        fetch(b0, c + 2);
        tk = wave_chunk<BF16, NV, ALIGNED, LDSR>(V, eb_of(c + 1), K, b1, tk, wg_bound(), npend, sm.wv[w]);
        settle(false);
        __builtin_amdgcn_sched_barrier(0);
    }
    settle(true);
    // Each wave's sorted list leaves as it is; the row merge takes the
    // segments' four lists each.
    if (lane < K) xstore(out + w * K + lane, tk);
}

// Segment seg of nseg of a row of C chunks (chunks seg, seg + nseg, ...).
//   NV >= 1: rows are 16-byte aligned and V is a multiple of kPerVec; chunks
//   of NV vectors per lane.
//   NV == 0: rows that are not aligned load element by element; the C chunks
//   were counted with `split` vectors per lane, and each is taken as `split`
//   one-vector chunks so that this rare path stays small in registers.  It
//   is a kernel instantiation of its own: kept beside the aligned path, the
//   compiler emits it as a called function, and the call stack then gives
//   every workgroup of the launch a private segment.
template <bool BF16, int NV, bool LDSR = false>
__device__ __forceinline__ void segment_topk(const void* __restrict__ row, int V, int C, int seg,
                                             int nseg, int K, int split,
                                             uint64_t* __restrict__ out, ChunkLds& sm) {
    const int nc = (C - seg + nseg - 1) / nseg;
    if constexpr (NV == 0)
        segment_topk_impl<BF16, 1, false, LDSR>(row, V, seg, nseg, nc * split, split, K, out, sm);
    else
        segment_topk_impl<BF16, NV, true, LDSR>(row, V, seg, nseg, nc, 1, K, out, sm);
}

// Stage 2: top K of one row from its nl sorted segment lists (K words each,
// descending, zero padded; written by other workgroups, read with xload);
// nl * K <= kMergeMax.  emit(rank, word) runs once for every rank < K, in
// the thread that holds the word.  Every thread of the workgroup calls.
// The bound, with c = ceil(K / nl): when nl * c <= 64, the K-th largest value
// key among the first ch = max(c, min(K, 64 / nl)) words of every list (at
// least K words reach it; every list's first c words reach its c-th word, so
// this is never below the smallest c-th word), and with fewer lists than K
// also the best K-th word of any list; otherwise the larger of the best K-th
// word of any list and the smallest c-th word over all lists (at least K
// words reach either).
// pre() runs right after the list loads are issued and mid() right after the
// first barrier, so that a caller can overlap loads of its own with the merge.
template <typename Emit, typename Pre, typename Mid>
__device__ void block_merge_lists(const uint64_t* __restrict__ lists, int nl, int K, int keybits,
                                  MergeLds& sm, Emit&& emit, Pre&& pre, Mid&& mid) {
    constexpr int Q = kMergeMax / kWG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = nl * K;
    const int c = (K + nl - 1) / nl;
    uint64_t x[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) x[q] = (q * kWG < n) ? xload(lists + min(q * kWG + tid, n - 1)) : 0ull;
    if (tid == 0) {
        sm.tk = 0ull;
        sm.tc = ~0ull;
        sm.m = 0u;
    }
    pre();
    __syncthreads();
    mid();
    // Up to 64 heads (the first ch words of each list): the K-th largest
    // head key, found by one wave, which is much sharper than the list
    // bounds (at batch 32, 12 lists of 16: 56 words survived the list
    // bounds).  Otherwise the best K-th word of any list and the smallest
    // c-th word (LDS atomics, at most 2 nl of them).
    const bool heads = nl * c <= 64;
    const int ch = heads ? max(c, min(K, 64 / nl)) : c;
    const int nh = nl * ch;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = q * kWG + tid;
        if (e < n) {
            const int k = e % K;
            if (heads) {
                if (k < ch) sm.surv[(e / K) * ch + k] = x[q];
                if (nl < K && k == K - 1)
                    __hip_atomic_fetch_max(&sm.tk, x[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                if (k == K - 1)
                    __hip_atomic_fetch_max(&sm.tk, x[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (k == c - 1)
                    __hip_atomic_fetch_min(&sm.tc, x[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
    uint64_t T = heads ? sm.tk : (sm.tk > sm.tc ? sm.tk : sm.tc);
    if (heads) {
        // The K-th largest value key among the heads (K heads reach it), by
        // a bitwise search over ballot counts.
        if (tid < 64) {
            const uint32_t hk = (lane < nh) ? (uint32_t)(sm.surv[lane] >> 32) : 0u;
            uint32_t th = 0;
            for (int bit = keybits - 1; bit >= 0; --bit) {
                const uint32_t cb = th | (1u << bit);
                if (ballot_count(hk >= cb) >= K) th = cb;
            }
            if (tid == 0) sm.aux2 = th;
        }
        __syncthreads();
        const uint64_t Th = (uint64_t)sm.aux2 << 32;
        T = T > Th ? T : Th;
    }
    T = T ? T : 1ull;
    // compaction: one LDS add per wave reserves the wave's slots
    uint64_t bal[Q];
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        bal[q] = __ballot((q * kWG + tid < n) && x[q] >= T);
        cnt += (uint32_t)__popcll(bal[q]);
    }
    uint32_t base = 0;
    if (lane == 0 && cnt)
        base = __hip_atomic_fetch_add(&sm.m, cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if ((bal[q] >> lane) & 1ull) sm.surv[base + __popcll(bal[q] & ((1ull << lane) - 1ull))] = x[q];
        base += (uint32_t)__popcll(bal[q]);
    }
    __syncthreads();
    const int m = (int)sm.m;
    for (int s0 = 0; s0 < m; s0 += kWG) {
        const int si = s0 + tid;
        const uint64_t y = (si < m) ? sm.surv[si] : 0ull;
        int rank = 0;
        for (int u0 = 0; u0 < m; u0 += 8) {
            uint64_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = sm.surv[min(u0 + j, m - 1)];
#pragma unroll
            for (int j = 0; j < 8; ++j) rank += (u0 + j < m && v[j] > y) ? 1 : 0;
        }
        if (si < m && rank < K) emit(rank, y);
    }
    __syncthreads();
}

// Row merge to (index, value) pairs; a row always has K real values
// (K <= V), so every rank is written.  pre / mid: see block_merge_lists.
template <bool BF16, typename Pre, typename Mid>
__device__ void merge_row(const uint64_t* __restrict__ part, int nseg, int K,
                          int32_t* __restrict__ out_idx, float* __restrict__ out_val,
                          MergeLds& sm, Pre&& pre, Mid&& mid) {
    using E = Elem<BF16>;
    block_merge_lists(
        part, nseg, K, Elem<BF16>::kKeyBits, sm,
        [&](int rank, uint64_t y) {
            xstore(out_idx + rank, (int32_t)cand_index(y));
            xstore(out_val + rank, E::value((uint32_t)(y >> 32)));
        },
        pre, mid);
}

template <bool BF16>
__device__ void merge_row(const uint64_t* __restrict__ part, int nseg, int K,
                          int32_t* __restrict__ out_idx, float* __restrict__ out_val,
                          MergeLds& sm) {
    merge_row<BF16>(part, nseg, K, out_idx, out_val, sm, [] {}, [] {});
}

}  // namespace df2
