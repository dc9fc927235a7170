// Per-row top-K over the vocabulary ("DFlash 2: Keep Drafting Parallel",
// section "A Lightweight Path Selector": keep the top 16 candidates at each
// draft position).
//
// Stage 1 (segment): a workgroup streams a contiguous segment of one row.
// Each of its four waves works on its own: it streams every fourth chunk of
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
// largest value from below).  With nothing known yet, the K-th largest lane
// maximum of the chunk is the bound.  Once a few chunks have been seen, most
// chunks have no lane that reaches the bound and cost a handful of
// instructions.  Vectors that do reach it are keyed exactly from
// registers; words that beat the K-th kept word are compacted (ballot) and
// merged into the list with all ranks found in parallel.  No step of a chunk
// needs a workgroup barrier.
// At the end of the segment the four waves' lists are ranked together.
//
// Stage 2 (merge): the last segment workgroup of a row to finish merges the
// segments' K candidate words with a bound-then-rank scheme (per-wave bounds
// over lane maxima of the words).
//
// Candidate words (key << 32 | ~index) are distinct within a row, so every
// selection is exact and independent of arrival order: results are
// deterministic.
#pragma once

#include "common.hpp"

namespace df2 {

constexpr int kMaxNV = 4;           // 16-byte vectors per lane per chunk
constexpr int kMergeItems = 8;      // candidate words per thread (merge)
constexpr int kMergeCap = 512;      // survivors ranked in LDS (merge)

constexpr int kWCand = 256;         // candidate words buffered per wave before a merge

struct WaveLds {
    u32x4_t slot[64];                   // surviving vectors, one per lane at most
    uint32_t slot_lane[64];
    uint64_t cand[kWCand];
    uint64_t L[64];                     // the list, published for a merge
    uint64_t L2[64];                    // the merged list
};

struct ChunkLds {
    WaveLds wv[kWaves];
    uint64_t fin[kWaves * 64];          // the waves' lists at the end of a segment
    uint32_t bound;                     // best K-th kept key among the four waves
};

struct MergeLds {
    uint64_t thr[kWaves];
    uint32_t red[kWaves];
    uint32_t n;
    uint64_t list[kMergeCap];
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

// Loads of the 16-byte vector holding elements [e0, e0 + kPerVec) of a row.
//   ALIGNED: the row start is 16-byte aligned and V is a multiple of
//   kPerVec, so a vector is all in or all out.  The load is then issued
//   unconditionally from a clamped (in-bounds) address and nothing is done
//   with the value until it is consumed (mask_vec), so consecutive loads stay
//   in flight together.
//   Otherwise elements are loaded one by one; out-of-row ones read as the
//   all-ones sentinel.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ u32x4_t load_vec(const void* __restrict__ row, int V, int64_t e0) {
    constexpr int PV = Elem<BF16>::kPerVec;
    if constexpr (ALIGNED) {
        const int64_t vi = (e0 < V) ? e0 / PV : 0;
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row) + vi);
    } else {
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
}

// At consumption: an aligned vector that lies beyond the row becomes the
// sentinel (its load read an in-bounds stand-in).
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

// Merges m distinct candidate words c[0..m) into the sorted list held one
// word per lane (lane k: k-th best; unfilled slots and lanes >= K hold 0) and
// returns the best K.  Every word finds its new rank in parallel: a list word
// counts the candidates above it; a candidate binary-searches the sorted list
// and counts the candidates above it.  Ranks below K are scattered to LDS.
__device__ __forceinline__ uint64_t list_merge(uint64_t tk, const uint64_t* c, int m, int K,
                                               WaveLds& sm) {
    const int lane = lane_id();
    if (lane < K) sm.L[lane] = tk;
    sm.L2[lane] = 0;
    wave_sync();
    if (lane < K && tk != 0) {
        int r = lane;
        int i = 0;
        for (; i + 4 <= m; i += 4)
            r += (c[i] > tk) + (c[i + 1] > tk) + (c[i + 2] > tk) + (c[i + 3] > tk);
        for (; i < m; ++i) r += (c[i] > tk);
        if (r < K) sm.L2[r] = tk;
    }
    for (int q = lane; q < m; q += 64) {
        const uint64_t x = c[q];
        int lo = 0, hi = K;                     // list words above x: first L[idx] < x
#pragma unroll
        for (int step = 0; step < 7; ++step) {
            if (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (sm.L[mid] > x) lo = mid + 1;
                else hi = mid;
            }
        }
        int r = lo;
        int i = 0;
        for (; i + 4 <= m; i += 4)
            r += (c[i] > x) + (c[i + 1] > x) + (c[i + 2] > x) + (c[i + 3] > x);
        for (; i < m; ++i) r += (c[i] > x);
        if (r < K) sm.L2[r] = x;
    }
    wave_sync();
    return (lane < K) ? sm.L2[lane] : 0ull;
}

// Folds one wave chunk (in registers) into the wave's sorted list tk.
//   eb: row index of the chunk's first element; lane l, vector j, element p
//   hold element eb + (j * 64 + l) * kPerVec + p.
//   trow: a key that at least K values of the row are known to reach (the
//   best K-th kept key among the workgroup's waves; 0 if none known).
template <bool BF16, int NV, bool ALIGNED>
__device__ uint64_t wave_chunk(int V, int64_t eb, int K, const u32x4_t (&raw)[NV], uint64_t tk,
                               uint32_t trow, WaveLds& sm) {
    using E = Elem<BF16>;
    constexpr int PV = E::kPerVec;
    const int lane = lane_id();
    u32x4_t v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = mask_vec<ALIGNED>(raw[j], eb + (int64_t)(j * 64 + lane) * PV, V);
    const uint32_t skey = lane_max_key<BF16, NV>(v);
    uint64_t kth = readlane_u64(tk, K - 1);     // 0 while the list is filling
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
    const bool lane_in = skey >= Tm;
    if (__ballot(lane_in) == 0) return tk;      // the common case
    // Vectors that reach the bound go to LDS slots (one per lane at most per
    // vector index); the wave keys their elements and buffers every word that
    // beats the K-th kept word (ballot compaction), merging when the buffer
    // fills.
    int n = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const bool vin = lane_in && vec_max_key<BF16>(v[j]) >= Tm;
        const uint64_t bal = __ballot(vin);
        if (bal == 0) continue;
        if (vin) {
            const int slot = __popcll(bal & ((1ull << lane) - 1ull));
            sm.slot[slot] = v[j];
            sm.slot_lane[slot] = lane;
        }
        wave_sync();
        const int nel = __popcll(bal) * PV;
#pragma unroll 1
        for (int e0 = 0; e0 < nel; e0 += 64) {
            const int e = e0 + lane;
            bool pred = false;
            uint64_t word = 0;
            if (e < nel) {
                const int sl = e / PV, p = e % PV;
                const uint32_t wd = reinterpret_cast<const uint32_t*>(&sm.slot[sl])[BF16 ? (p >> 1) : p];
                const uint32_t bits = BF16 ? ((p & 1) ? (wd >> 16) : (wd & 0xFFFFu)) : wd;
                const int64_t gidx = eb + (int64_t)(j * 64 + (int)sm.slot_lane[sl]) * PV + p;
                const uint32_t key = E::key(bits);
                word = cand_word(key, (uint32_t)gidx);
                pred = gidx < V && key >= Tm && word > kth;
            }
            const uint64_t b2 = __ballot(pred);
            if (pred) sm.cand[n + __popcll(b2 & ((1ull << lane) - 1ull))] = word;
            n += __popcll(b2);
            if (n > kWCand - 64) {
                tk = list_merge(tk, sm.cand, n, K, sm);
                kth = readlane_u64(tk, K - 1);
                n = 0;
            }
        }
        wave_sync();
    }
    if (n > 0) tk = list_merge(tk, sm.cand, n, K, sm);
    return tk;
}

// Stage 1: best K candidate words of chunks [c0, c1) of one row; chunk c is
// 4 x 64 x NV vectors, wave w streams its quarter of every chunk.
//   row: first element of the row; V: row length; K <= 64.
//   aligned: the row start is 16-byte aligned and V is a multiple of kPerVec.
//   out: K hand-off words (0 for empty slots).
template <bool BF16, int NV, bool ALIGNED>
__device__ void segment_topk_impl(const void* __restrict__ row, int V, int c0, int c1, int K,
                                  uint64_t* __restrict__ out, ChunkLds& sm) {
    static_assert(NV >= 1 && NV <= kMaxNV, "chunk vectors per lane");
    constexpr int PV = Elem<BF16>::kPerVec;
    constexpr int WE = 64 * PV * NV;           // elements per wave chunk
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t tk = 0;
    uint32_t published = 0;
    auto eb_of = [&](int c) { return ((int64_t)c * kWaves + w) * WE; };
    if (tid == 0) sm.bound = 0;
    __syncthreads();
    // Publishes the wave's K-th kept key as a bound for the whole workgroup;
    // a wave may read an older (smaller) bound, which is still valid.
    auto publish = [&]() {
        const uint32_t kk = (uint32_t)(readlane_u64(tk, K - 1) >> 32);
        if (kk > published) {
            if (lane == 0)
                __hip_atomic_fetch_max(&sm.bound, kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            published = kk;
        }
    };
    auto wg_bound = [&]() {
        return __hip_atomic_load(&sm.bound, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // Two register buffers, used in turn without copies: while one chunk is
    // processed the next one's loads are in flight.  Past the segment end a
    // prefetch re-reads the last chunk (in bounds, never consumed).
    u32x4_t b0[NV], b1[NV];
    const int clast = c1 - 1;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        b0[j] = load_vec<BF16, ALIGNED>(row, V, eb_of(c0) + (int64_t)(j * 64 + lane) * PV);
    for (int c = c0; c < c1; c += 2) {
        const int cn = min(c + 1, clast);
#pragma unroll
        for (int j = 0; j < NV; ++j)
            b1[j] = load_vec<BF16, ALIGNED>(row, V, eb_of(cn) + (int64_t)(j * 64 + lane) * PV);
        tk = wave_chunk<BF16, NV, ALIGNED>(V, eb_of(c), K, b0, tk, wg_bound(), sm.wv[w]);
        publish();
        // Keep the next half's uses of its loads below this point: hoisting
        // one would wait on every load in flight, prefetch included.
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 >= c1) break;
        const int cnn = min(c + 2, clast);
#pragma unroll
        for (int j = 0; j < NV; ++j)
            b0[j] = load_vec<BF16, ALIGNED>(row, V, eb_of(cnn) + (int64_t)(j * 64 + lane) * PV);
        tk = wave_chunk<BF16, NV, ALIGNED>(V, eb_of(c + 1), K, b1, tk, wg_bound(), sm.wv[w]);
        publish();
        __builtin_amdgcn_sched_barrier(0);
    }
    // Rank the four waves' lists together; the best K leave in order.
    if (lane < K) sm.fin[w * K + lane] = tk;
    __syncthreads();
    const int n = kWaves * K;
    uint32_t nreal = 0;
    for (int u = 0; u < n; ++u) nreal += (sm.fin[u] != 0) ? 1u : 0u;
    if (tid < n) {
        const uint64_t x = sm.fin[tid];
        if (x != 0) {
            uint32_t rank = 0;
            for (int u = 0; u < n; ++u) rank += (sm.fin[u] > x) ? 1u : 0u;
            if (rank < (uint32_t)K) xstore(out + rank, x);
        }
    }
    // slots beyond the number of real words stay empty
    for (int k = (int)nreal + tid; k < K; k += kWG) xstore(out + k, (uint64_t)0);
}

template <bool BF16, int NV>
__device__ void segment_topk(const void* __restrict__ row, int V, int c0, int c1, int K,
                             bool aligned, uint64_t* __restrict__ out, ChunkLds& sm) {
    // Rows that are not 16-byte aligned load element by element; they use
    // one-vector chunks (the same elements, NV times as many chunks) so that
    // this rare path stays small in registers.
    if (aligned)
        segment_topk_impl<BF16, NV, true>(row, V, c0, c1, K, out, sm);
    else
        segment_topk_impl<BF16, 1, false>(row, V, c0 * NV, c1 * NV, K, out, sm);
}

// Stage 2: merge the K candidate words of each of `nchunks` chunks of a row
// into the row's top-K, written as (index, value).
template <bool BF16>
__device__ void merge_row(const uint64_t* __restrict__ part, int nchunks, int K,
                          int32_t* __restrict__ out_idx, float* __restrict__ out_val,
                          MergeLds& sm) {
    using E = Elem<BF16>;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nitems = nchunks * K;     // host guarantees <= kWG * kMergeItems
    uint64_t it[kMergeItems];
    uint64_t mx = 0;
#pragma unroll
    for (int q = 0; q < kMergeItems; ++q) {
        int i = tid + q * kWG;
        it[q] = (i < nitems) ? xload(part + i) : 0ull;
        mx = it[q] > mx ? it[q] : mx;
    }
    // candidate words of bf16 rows are below 2^48 (16-bit keys)
    const int top = BF16 ? 47 : 63;
    uint64_t T = 0;
#pragma unroll 1
    for (int bit = top; bit >= 0; --bit) {
        uint64_t c = T | (1ull << bit);
        if (ballot_count(mx >= c) >= K) T = c;
    }
    if (lane == 0) sm.thr[w] = T;
    if (tid == 0) sm.n = 0;
    __syncthreads();
    T = sm.thr[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) T = sm.thr[q] > T ? sm.thr[q] : T;
    if (T == 0) T = 1;
#pragma unroll
    for (int q = 0; q < kMergeItems; ++q) {
        if (it[q] >= T) {
            uint32_t pos = atomicAdd(&sm.n, 1u);
            if (pos < (uint32_t)kMergeCap) sm.list[pos] = it[q];
        }
    }
    __syncthreads();
    if (sm.n > (uint32_t)kMergeCap) {
        // Exact fallback: bitwise search for the K-th largest word.
        uint64_t T64 = 0;
#pragma unroll 1
        for (int bit = top; bit >= 0; --bit) {
            uint64_t c = T64 | (1ull << bit);
            uint32_t cnt = 0;
#pragma unroll
            for (int q = 0; q < kMergeItems; ++q) cnt += (it[q] >= c && it[q] != 0) ? 1u : 0u;
            if (block_sum_u32(cnt, sm.red) >= (uint32_t)K) T64 = c;
        }
        if (tid == 0) sm.n = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kMergeItems; ++q) {
            if (it[q] != 0 && it[q] >= T64) {
                uint32_t pos = atomicAdd(&sm.n, 1u);
                sm.list[pos] = it[q];
            }
        }
        __syncthreads();
    }
    const uint32_t n = sm.n;
    for (uint32_t c = tid; c < n; c += kWG) {
        uint64_t x = sm.list[c];
        uint32_t rank = 0;
        for (uint32_t u = 0; u < n; ++u) rank += (sm.list[u] > x) ? 1u : 0u;
        if (rank < (uint32_t)K) {
            xstore(out_idx + rank, (int32_t)cand_index(x));
            xstore(out_val + rank, E::value((uint32_t)(x >> 32)));
        }
    }
}

}  // namespace df2
