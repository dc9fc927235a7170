// Per-row top-K over the vocabulary ("DFlash 2: Keep Drafting Parallel",
// section "A Lightweight Path Selector": keep the top 16 candidates at each
// draft position).
//
// Stage 1 (chunk): a workgroup streams one chunk of a row once from HBM with
// 16-byte loads and keeps it in registers.  Each lane reduces its values to
// one statistic, its true maximum, using packed 16-bit integer max/min on
// the raw bf16 bits (non-negative values order like their bits; negative
// values order reversed, so the maximum of a lane is its largest bit pattern
// if it has any non-negative value and its smallest one otherwise).  The K-th
// largest lane maximum of a wave bounds the chunk's K-th largest value from
// below, so only lanes whose maximum reaches the largest such bound can hold
// a winner.  Those few lanes copy their raw values to LDS; the workgroup then
// keys them exactly and ranks the survivors.  A chunk whose survivors do not
// fit (heavy ties) takes an exact fallback: a bitwise search for the K-th
// largest candidate word over the values still held in registers.
//
// Stage 2 (merge): the last chunk workgroup of a row to finish merges the
// chunks' K candidate words with the same bound-then-rank scheme.
//
// Candidate words (key << 32 | ~index) are distinct within a row, so every
// selection is exact and independent of arrival order: results are
// deterministic.
#pragma once

#include "common.hpp"

namespace df2 {

constexpr int kSlots = 64;          // survivor lanes copied to LDS
constexpr int kMaxNV = 8;           // 16-byte vectors per thread
constexpr int kCandCap = 256;       // survivors ranked in LDS (chunk)
constexpr int kMergeItems = 8;      // candidate words per thread (merge)
constexpr int kMergeCap = 512;      // survivors ranked in LDS (merge)

struct ChunkLds {
    uint32_t thr[kWaves];
    uint32_t red[kWaves];
    uint32_t nslot, ncand;
    uint32_t slot_tid[kSlots];
    uint64_t cand[kCandCap];
    uint32_t slot_data[kSlots][kMaxNV * 4];
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

// The 16-byte vector of elements [e0, e0 + kPerVec) of a row; elements at or
// beyond V read as the all-ones sentinel.  `aligned`: the row start is 16-byte
// aligned and V is a multiple of kPerVec, so a vector is all in or all out.
template <bool BF16>
__device__ __forceinline__ u32x4_t load_vec(const void* __restrict__ row, int V, int64_t e0,
                                            bool aligned) {
    constexpr int PV = Elem<BF16>::kPerVec;
    if (aligned) {
        if (e0 < V) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row) + e0 / PV);
        return u32x4_t{~0u, ~0u, ~0u, ~0u};
    }
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

// Ranks `n` distinct candidate words in LDS and writes the best K, in order,
// to `out`; slots [n, K) get 0.  All threads call it.
__device__ __forceinline__ void rank_and_emit(const uint64_t* list, uint32_t n, int K,
                                              uint64_t* __restrict__ out) {
    for (uint32_t c = threadIdx.x; c < n; c += kWG) {
        uint64_t x = list[c];
        uint32_t rank = 0;
        for (uint32_t u = 0; u < n; ++u) rank += (list[u] > x) ? 1u : 0u;
        if (rank < (uint32_t)K) out[rank] = x;
    }
    for (uint32_t k = n + threadIdx.x; k < (uint32_t)K; k += kWG) out[k] = 0;
}

// Stage 1: best K candidate words of chunk `chunk` of one row.
//   row: first element of the row; V: row length; K <= 64.
//   aligned: the row start is 16-byte aligned and V is a multiple of kPerVec.
template <bool BF16, int NV>
__device__ void chunk_topk(const void* __restrict__ row, int V, int chunk, int K,
                           bool aligned, uint64_t* __restrict__ out, ChunkLds& sm) {
    using E = Elem<BF16>;
    constexpr int PV = E::kPerVec;
    constexpr int CE = kWG * PV * NV;    // elements per chunk
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t cbase = (int64_t)chunk * CE;

    // 1. Stream the chunk into registers; out-of-row elements read as the
    //    all-ones sentinel.
    u32x4_t v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        v[j] = load_vec<BF16>(row, V, cbase + (int64_t)(j * kWG + tid) * PV, aligned);

    // 2. Lane maximum in value order, from signed max/min of the raw bits.
    uint32_t stat_bits;
    if constexpr (BF16) {
        s16x2_t mx = __builtin_bit_cast(s16x2_t, v[0].x);
        s16x2_t mn = mx;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s16x2_t s = __builtin_bit_cast(s16x2_t, wd[q]);
                mx = __builtin_elementwise_max(mx, s);
                mn = __builtin_elementwise_min(mn, s);
            }
        }
        int m = max((int)mx.x, (int)mx.y);
        int n = min((int)mn.x, (int)mn.y);
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
    const uint32_t skey = E::key(stat_bits);

    // 3. K-th largest lane maximum of the wave, by a bitwise search over
    //    ballot counts; the workgroup bound is the largest wave bound.
    uint32_t T = 0;
#pragma unroll 1
    for (int bit = E::kKeyBits - 1; bit >= 0; --bit) {
        uint32_t c = T | (1u << bit);
        if (ballot_count(skey >= c) >= K) T = c;
    }
    if (lane == 0) sm.thr[w] = T;
    if (tid == 0) {
        sm.nslot = 0;
        sm.ncand = 0;
    }
    __syncthreads();
    T = max(max(sm.thr[0], sm.thr[1]), max(sm.thr[2], sm.thr[3]));
    const uint32_t Tm = max(T, 1u);     // real values have key >= 1

    // 4. Lanes that may hold a winner copy their raw vectors to LDS.
    if (skey >= Tm) {
        uint32_t s = atomicAdd(&sm.nslot, 1u);
        if (s < (uint32_t)kSlots) {
            sm.slot_tid[s] = tid;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                sm.slot_data[s][j * 4 + 0] = v[j].x;
                sm.slot_data[s][j * 4 + 1] = v[j].y;
                sm.slot_data[s][j * 4 + 2] = v[j].z;
                sm.slot_data[s][j * 4 + 3] = v[j].w;
            }
        }
    }
    __syncthreads();
    const uint32_t nslot = sm.nslot;
    bool overflow = nslot > (uint32_t)kSlots;

    // 5. Key every copied value exactly; keep those at or above the bound.
    if (!overflow) {
        const uint32_t per = PV * NV;
        const uint32_t nel = nslot * per;
        for (uint32_t e = tid; e < nel; e += kWG) {
            uint32_t s = e / per, k = e % per;
            uint32_t j = k / PV, p = k % PV;
            uint32_t wd = sm.slot_data[s][j * 4 + (BF16 ? (p >> 1) : p)];
            uint32_t bits = BF16 ? ((p & 1) ? (wd >> 16) : (wd & 0xFFFFu)) : wd;
            int64_t gidx = cbase + (int64_t)(j * kWG + sm.slot_tid[s]) * PV + p;
            if (gidx < V) {
                uint32_t key = E::key(bits);
                if (key >= Tm) {
                    uint32_t pos = atomicAdd(&sm.ncand, 1u);
                    if (pos < (uint32_t)kCandCap) sm.cand[pos] = cand_word(key, (uint32_t)gidx);
                }
            }
        }
        __syncthreads();
        overflow = sm.ncand > (uint32_t)kCandCap;
    }

    // 6. Exact fallback: bitwise search for the K-th largest candidate word
    //    (only on heavy ties).  The chunk is read again from memory so that
    //    the register copy is not live across this rarely taken path.
    if (overflow) {
        uint64_t T64 = 0;
        const int top = BF16 ? 47 : 63;
#pragma unroll 1
        for (int bit = top; bit >= 0; --bit) {
            const uint64_t c = T64 | (1ull << bit);
            uint32_t cnt = 0;
#pragma unroll 1
            for (int j = 0; j < NV; ++j) {
                const int64_t e0 = cbase + (int64_t)(j * kWG + tid) * PV;
                const u32x4_t x = load_vec<BF16>(row, V, e0, aligned);
#pragma unroll
                for (int p = 0; p < PV; ++p) {
                    if (e0 + p < V) {
                        const uint64_t wv = cand_word(E::key(elem_bits<BF16>(x, p)), (uint32_t)(e0 + p));
                        cnt += (wv >= c) ? 1u : 0u;
                    }
                }
            }
            if (block_sum_u32(cnt, sm.red) >= (uint32_t)K) T64 = c;
        }
        if (tid == 0) sm.ncand = 0;
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < NV; ++j) {
            const int64_t e0 = cbase + (int64_t)(j * kWG + tid) * PV;
            const u32x4_t x = load_vec<BF16>(row, V, e0, aligned);
#pragma unroll
            for (int p = 0; p < PV; ++p) {
                if (e0 + p < V) {
                    const uint64_t wv = cand_word(E::key(elem_bits<BF16>(x, p)), (uint32_t)(e0 + p));
                    if (wv >= T64) {
                        const uint32_t pos = atomicAdd(&sm.ncand, 1u);
                        sm.cand[pos] = wv;     // at most K <= 64 words qualify
                    }
                }
            }
        }
        __syncthreads();
    }

    // 7. Rank the survivors; the best K leave in order.
    rank_and_emit(sm.cand, sm.ncand, K, out);
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
        it[q] = (i < nitems) ? part[i] : 0ull;
        mx = it[q] > mx ? it[q] : mx;
    }
    uint64_t T = 0;
#pragma unroll 1
    for (int bit = 63; bit >= 0; --bit) {
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
        for (int bit = 63; bit >= 0; --bit) {
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
            out_idx[rank] = (int32_t)cand_index(x);
            out_val[rank] = E::value((uint32_t)(x >> 32));
        }
    }
}

}  // namespace df2
