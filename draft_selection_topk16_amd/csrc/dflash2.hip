// MI355X (gfx950) DFlash 2 path selector: kernels and the C ABI declared in
// include/dflash2.h.
//
// The selector ("DFlash 2: Keep Drafting Parallel", section "A Lightweight
// Path Selector") keeps the top-K candidates per draft position, scores every
// adjacent pair with S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>, and walks
// the scores once from the last verified token.
//
// dflash2_select runs in two launches by default, k_scanm and then
// k_pairs_walk (three stages: scan with the row merges, pairs, walk), and
// in three beyond one resident wave of rows (k_scanm, k_pairs_rows, then
// k_walks); the plan can also run it as k_scan then k_tail, or as the single
// k_select.
// Workgroups are dealt out in index order, and each one's job follows from
// its index:
//   * the first n_gate compute one slice of one gate tile (a partial of H);
//     with M <= 16 rows (outside the fused launch) the tile's last slice sums
//     the partials into H;
//   * every other one streams one segment of one logits row (every nseg-th
//     chunk of it), leaving a sorted list of K candidates per wave, and (in
//     k_scanm and k_select) arrives on the row's counter.
// The work after the segments is handed on by "last arrival": nobody waits
// for a producer except the fused launch's row merges for the gate, below.
//   row:      the last segment of a row merges the row's lists into its
//             top-K (ids and logits).  In k_scanm that is all; k_pairs_walk
//             then scores the transition into every row (one workgroup per
//             row), taking H_t from the tile sums or summing the partials.
//             In k_select and k_tail the row merge also sums H_t and arrives
//             on the counters of the two transitions the row takes part in
//             (t - 1 -> t and t -> t + 1);
//   pairs:    (k_select, k_tail) the second row of a transition to arrive
//             scores it (the first transition of a sequence needs only its
//             own row);
//   walk:     the last transition of a sequence to be scored walks it.
// In k_select and k_tail the row merge sums H_t from the gate partials in
// slice order (or loads the tile sums' row of H) and waits (bounded spin)
// for the gate tile row to be complete; in k_tail it already is.  Gate
// workgroups have the lowest indexes and never wait, so they have all been
// dispatched by the time any row merge runs, and every wait ends.
// Counters live in the scratch buffer and are reset by the workgroup that
// consumes them, so every launch starts from zero without a memset.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "dflash2.h"
#include "common.hpp"
#include "conv.hpp"
#include "gate.hpp"
#include "lmhead.hpp"
#include "pairs.hpp"
#include "topk.hpp"
#include "walk.hpp"

using namespace df2;

namespace {

// ----------------------------------------------------------------------------
// Launch description shared by the kernels (passed by value).
// ----------------------------------------------------------------------------
struct Params {
    const void* logits;
    const void* hidden;
    const void* A;
    const void* Bt;
    const void* W;
    const int32_t* prev;
    int32_t* out_path;
    float* out_score;
    float* H;             // standalone projection output [M, r]
    // scratch
    uint64_t* part;       // [rows, nseg, 4, K] candidate words (a sorted list per wave)
    int32_t* cand;        // [rows, K]
    float* cval;          // [rows, K]
    float* ppart;         // [S, M, r] gate partials
    float* Sb;            // [rows, K, K] pair scores
    float* Hb;            // [rows, r] gate rows (summed by the row merges, or by each
                          // gate tile's last slice with M <= 16 outside k_select)
    uint32_t* err;        // device input-error flags
    uint32_t* row_cnt;    // [rows] segments done
    uint32_t* edge_cnt;   // [rows] rows ready of transition t - 1 -> t
    uint32_t* seq_cnt;    // [B] transitions scored
    uint32_t* gate_cnt;   // [mtiles] gate slices done (M <= 16: tiles summed; unused by k_scanm)
    uint32_t* rd_cnt;     // [mtiles] pair jobs past the gate wait
    // sizes
    int B, P, V, d, r, K;
    int64_t rows;
    int C;                // chunks per row
    int nseg;             // segments per row
    int aligned;          // logits rows are 16-byte aligned and V % per-vector == 0
    int split;            // vectors per lane the chunks were counted with
    int gm_rows;          // rows per gate tile
    int mtiles, ntiles, S, n_gate;
    int64_t n_chunk;      // segment workgroups (rows * nseg)
    int walk;             // kWalkViterbi, kWalkGreedy or kWalkSample
    const float* u;       // [B, P] uniforms of the sampling walk
    float* out_q;         // [B, P] probabilities of the sampled choices
    float inv_tau;        // 1 / temperature of the sampling walk
    // The row merges' gate wait: the arrivals it needs beyond the gate's own
    // (0; 1 only to force a give-up when testing failure handling) and its
    // bound in sleeps.
    uint32_t gate_extra = 0;
    uint32_t gate_spins = 1u << 20;
    uint32_t* tile_cnt;   // [mtiles * ntiles] slices of a gate tile done (tile sums)
};

// Walk modes inside the launch: the two of df2_walk, and the sampling walk.
constexpr int kWalkViterbi = DF2_WALK_VITERBI;
constexpr int kWalkGreedy = DF2_WALK_GREEDY;
constexpr int kWalkSample = 2;

union SharedAll {
    ChunkLds c;
    MergeLds m;
    GateLds g;
    PairLds pr;
    WalkLds wk;
};
// Five workgroups per CU: the LDS a workgroup asks for must stay well under
// a fifth of the CU's 160 KB (32 KB blocks would leave room for four).
static_assert(sizeof(SharedAll) + 64 <= 30720, "LDS budget of five workgroups per CU");

template <int MB>
struct GateShape {
    static constexpr int NB = MB == 1 ? 4 : 2;
};

// One slice of one gate tile.  HSUM (the two-launch kernels with a gate of
// one m-block, M <= 16 rows): the tile's last slice to finish sums the S
// partials in slice order into the gate rows Hb, so that a reader loads one
// row of H instead of S partial rows, and counts the tile on its tile row.
// Otherwise each slice counts itself on the tile row and every reader sums
// its own row's partials (at M = 56 and 224 the tile sums lengthened the
// scan launch by 5-6 us).  Either way the sum runs in slice order, so the
// result never depends on timing.  ARRIVE = false (k_scanm, whose readers
// run in the next launch): no count at all.
template <bool BF16, int MB, bool HSUM, bool ARRIVE = true>
__device__ void gate_role(const Params& p, int gb, GateLds& sm) {
    const int s = gb % p.S, tile = gb / p.S;
    const int mt = tile / p.ntiles, nt = tile % p.ntiles;
    gate_slice<BF16, MB, GateShape<MB>::NB>(p.hidden, p.W, (int)p.rows, p.d, p.r, mt, nt, s, p.S,
                                            p.ppart, sm);
    if constexpr (!HSUM) {
        if constexpr (ARRIVE) {
            drain_stores();
            __syncthreads();
            if (threadIdx.x == 0) arrive(&p.gate_cnt[mt]);
        }
    } else {
        __shared__ uint32_t last;
        if (!block_arrive_last(&p.tile_cnt[tile], (uint32_t)p.S, &last)) return;
        const int tid = threadIdx.x;
        if (tid == 0) reset_counter(&p.tile_cnt[tile]);
        // thread: CG consecutive columns of one tile row (8, or 4 for the
        // 1024-value tiles of one m-block); the partials come in rounds of four
        // slices, all loads of a round in flight at once
        constexpr int TR = 16 * MB, TC = 16 * GateShape<MB>::NB;
        constexpr int CG = TR * TC > 1024 ? 8 : 4;
        static_assert(TR * TC / CG <= kWG, "one group of columns per thread");
        if (tid < TR * TC / CG) {
            const int64_t m = (int64_t)mt * TR + tid / (TC / CG);
            const int c = nt * TC + (tid % (TC / CG)) * CG;
            if (m < p.rows) {
                float h[CG];
    #pragma unroll
                for (int e = 0; e < CG; ++e) h[e] = 0.f;
                for (int s0 = 0; s0 < p.S; s0 += 4) {
                    uint64_t v[4][CG / 2];
    #pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint64_t* q = reinterpret_cast<const uint64_t*>(
                            p.ppart + ((int64_t)min(s0 + u, p.S - 1) * p.rows + m) * p.r + c);
    #pragma unroll
                        for (int i = 0; i < CG / 2; ++i) v[u][i] = xload(q + i);
                    }
    #pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (s0 + u < p.S) {
    #pragma unroll
                            for (int i = 0; i < CG / 2; ++i) {
                                h[2 * i] += __uint_as_float((uint32_t)v[u][i]);
                                h[2 * i + 1] += __uint_as_float((uint32_t)(v[u][i] >> 32));
                            }
                        }
                }
    #pragma unroll
                for (int e = 0; e < CG; ++e) xstore(p.Hb + m * p.r + c + e, h[e]);
            }
        }
        if constexpr (ARRIVE) {
            drain_stores();
            __syncthreads();
            if (tid == 0) arrive(&p.gate_cnt[mt]);
        }
    }
}

template <bool BF16, int NV, bool LDSR = false>
__device__ void segment_of(const Params& p, int64_t row, int seg, ChunkLds& sm) {
    const size_t esz = BF16 ? 2 : 4;
    const char* rowp = reinterpret_cast<const char*>(p.logits) + (size_t)row * p.V * esz;
    segment_topk<BF16, NV, LDSR>(rowp, p.V, p.C, seg, p.nseg, p.K, p.split,
                           p.part + ((size_t)row * p.nseg + seg) * kWaves * p.K, sm);
}

__device__ __forceinline__ int32_t checked_id(int32_t id, int V, uint32_t* err, uint32_t bit) {
    if ((unsigned)id >= (unsigned)V) {
        atomicOr(err, bit);
        return 0;
    }
    return id;
}

// Pair scores of positions e0 .. e0 + ne - 1 of sequence b (fused launch).
// own: the row this workgroup merged; hown: its gate row (floats tid and
// tid + 256 of this thread).  The other position's gate row comes from Hb.
template <bool BF16, bool SUMH = false>
__device__ void pairs_fused(const Params& p, int b, int e0, int ne, int64_t own,
                            const float (&hown)[2], PairLds& sm) {
    const int tid = threadIdx.x, K = p.K, r = p.r;
    const int64_t rb = (int64_t)b * p.P;
    // Every load of a thread is issued before any of them is checked, so the
    // ids, the candidate values and the gate rows cost one round trip
    // (atomic loads are not hoisted past the id check's branch).  Addresses
    // are clamped into their buffers and unused values dropped afterwards.
    const bool prev_row = tid < K;
    const bool cur_row = tid >= 64 && tid < 64 + ne * K;
    const int x = cur_row ? tid - 64 : 0, q = x / K, k = x % K;
    float hv[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    // SUMH (one position, ne == 1): thread t takes the pair of H_t values
    // 2t, 2t + 1 (r <= 512), all S partials of it loaded with the ids
    uint64_t hpv[SUMH ? kMaxFusedSlices : 1];
    const int hk = 2 * min(tid, r / 2 - 1);
    if constexpr (SUMH) {
        const uint64_t* hsrc = reinterpret_cast<const uint64_t*>(p.ppart + (rb + e0) * r + hk);
        const int64_t hstride = p.rows * r / 2;         // one slice, in pairs
#pragma unroll
        for (int s = 0; s < kMaxFusedSlices; ++s) hpv[s] = xload(hsrc + (int64_t)min(s, p.S - 1) * hstride);
    } else {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int64_t grow = min(rb + e0 + qq, (int64_t)p.rows - 1);
            hv[qq][0] = xload(p.Hb + grow * r + min(tid, r - 1));
            if (r > kWG) hv[qq][1] = xload(p.Hb + grow * r + min(tid + kWG, r - 1));
        }
    }
    const int64_t crow = prev_row ? rb + max(e0 - 1, 0) : rb + e0 + q;
    const int ck = prev_row ? tid : k;
    int32_t id = xload(p.cand + crow * K + ck);
    const float uval = xload(p.cval + crow * K + ck);
    const int32_t pid = xload(p.prev + b);
    // Candidate ids come from the row merges and are always in [0, V); they
    // are still checked, so that no gather can leave the tables.
    if (prev_row) {
        if (e0 > 0) {
            id = checked_id(id, p.V, p.err, 2u);
        } else {
            id = pid;
            if ((unsigned)id >= (unsigned)p.V) {
                if (tid == 0) atomicOr(p.err, 1u);
                id = 0;
            }
        }
        sm.ids[0][tid] = id;
    } else if (cur_row) {
        sm.ids[1 + q][k] = checked_id(id, p.V, p.err, 2u);
        sm.u[q][k] = uval;
    }
    if constexpr (SUMH) {
        // summed in slice order, as every other reader of the partials
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int s = 0; s < kMaxFusedSlices; ++s) {
            if (s < p.S) {
                lo += __uint_as_float((uint32_t)hpv[s]);
                hi += __uint_as_float((uint32_t)(hpv[s] >> 32));
            }
        }
        if (tid < r / 2) {
            sm.H[0][hk] = lo;
            sm.H[0][hk + 1] = hi;
        }
    } else {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (qq < ne && tid + u * kWG < r)
                    sm.H[qq][tid + u * kWG] = (rb + e0 + qq == own) ? hown[u] : hv[qq][u];
    }
    __syncthreads();
    pair_tiles<BF16>(p.A, p.Bt, K, r, e0, ne, p.Sb + (rb + e0) * K * K, sm, [] {});
}

// The walk of sequence b over its scored transitions, in the launch's walk
// mode.  Every thread of the workgroup calls.
template <bool SAMPLE, bool PAIR32 = false>
__device__ __forceinline__ void walk_of(const Params& p, int b, SharedAll& sm) {
    const int K = p.K, P = p.P;
    const int64_t rb = (int64_t)b * P;
    const float* Sq = p.Sb + rb * K * K;
    const int32_t* ids = p.cand + rb * K;
    if constexpr (SAMPLE)
        chain_seq<kChainSample>(Sq, ids, p.u + rb, p.inv_tau, P, K, p.out_path + rb, p.out_q + rb,
                                p.out_score + b, sm.wk);
    else if (p.walk == kWalkGreedy)
        chain_seq<kChainGreedy>(Sq, ids, nullptr, 0.f, P, K, p.out_path + rb, nullptr, p.out_score + b, sm.wk);
    else
        walk_seq<PAIR32>(Sq, ids, P, K, p.out_path + rb, p.out_score + b, sm.wk);
}

// Everything after a row's segments: the row merge (with the gate row H_t),
// the pair scores of the transitions the row completes, and the walk of the
// sequence whose last transition it scores.  Every thread of the workgroup
// calls.
template <bool BF16, int MB, bool SAMPLE, bool HSUM>
__device__ __forceinline__ void row_tail(const Params& p, int64_t row, SharedAll& sm,
                                         uint32_t& flag) {
    const int tid = threadIdx.x;
    const int K = p.K, P = p.P, r = p.r;
    // The row's gate H_t: once the gate tile row is complete (its workgroups
    // were dispatched first and never wait; this is almost always so by
    // now), its S partials are loaded while the merge runs and summed in
    // slice order, or (HSUM) its row of Hb, which the gate's tile sums wrote.
    const int mt = (int)(row / p.gm_rows);
    const uint32_t need = (HSUM ? (uint32_t)p.ntiles : (uint32_t)(p.ntiles * p.S)) + p.gate_extra;
    const int S = p.S;
    constexpr int NH = HSUM ? 1 : kMaxFusedSlices;
    uint32_t hp[NH];
    auto issue_h = [&](int k) {
        if constexpr (HSUM) {
            hp[0] = xload(reinterpret_cast<const uint32_t*>(p.Hb) + row * r + min(k, r - 1));
        } else {
#pragma unroll
            for (int s = 0; s < NH; ++s)
                hp[s] = xload(reinterpret_cast<const uint32_t*>(p.ppart) +
                              ((int64_t)min(s, S - 1) * p.rows + row) * r + min(k, r - 1));
        }
    };
    auto sum_h = [&]() {
        if constexpr (HSUM) return __uint_as_float(hp[0]);
        float h = 0.f;
#pragma unroll
        for (int s = 0; s < NH; ++s)
            if (s < S) h += __uint_as_float(hp[s]);
        return h;
    };
    merge_row<BF16>(
        p.part + (size_t)row * p.nseg * kWaves * K, p.nseg * kWaves, K, p.cand + row * K,
        p.cval + row * K, sm.m,
        [&] {
            if (tid == 0) sm.m.aux = xload(&p.gate_cnt[mt]);
        },
        [&] {
            if (sm.m.aux < need) {
                if (tid == 0) {
                    uint32_t it = 0;
                    while (xload(&p.gate_cnt[mt]) < need) {
                        __builtin_amdgcn_s_sleep(2);
                        if (++it > p.gate_spins) {
                            atomicOr(p.err, 4u);
                            break;
                        }
                    }
                }
                __syncthreads();
            }
            issue_h(tid);
        });
    float hown[2];
    hown[0] = sum_h();
    hown[1] = 0.f;
    if (r > kWG) {
        issue_h(tid + kWG);
        hown[1] = sum_h();
    }
    // publish H_t for the pair job of the next position (HSUM: already there)
    if constexpr (!HSUM) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (tid + u * kWG < r) xstore(p.Hb + row * r + tid + u * kWG, hown[u]);
    }
    // arrive on the transitions into and out of this row
    const int b = (int)(row / P), t = (int)(row % P);
    drain_stores();
    __syncthreads();
    if (tid < 64) {
        // one atomic instruction: lane 0 on the transition into this row,
        // lane 1 on the one out of it, lane 2 on the gate tile row's readers
        const int64_t lo = (int64_t)mt * p.gm_rows;
        const uint32_t rows_in = (uint32_t)(std::min<int64_t>(p.rows, lo + p.gm_rows) - lo);
        const bool act = (tid == 0 && t > 0) || (tid == 1 && t + 1 < P) || tid == 2;
        uint32_t* cnt = (tid == 2) ? &p.rd_cnt[mt] : &p.edge_cnt[row + tid];
        const uint32_t old = act ? arrive(cnt) : 0u;
        const bool mine = (tid == 0 && (t == 0 || old == 1u)) || (tid == 1 && act && old == 1u);
        if (tid == 2 && old == rows_in - 1u) {
            // the last row of the gate tile row to be read resets its counters
            reset_counter(&p.gate_cnt[mt]);
            reset_counter(&p.rd_cnt[mt]);
        }
        const uint64_t bal = __ballot(mine);
        if (tid == 0) flag = (uint32_t)bal & 3u;
    }
    __syncthreads();
    const uint32_t em = flag;
    if (!em) return;
    if (tid == 0 && (em & 1u) && t > 0) reset_counter(&p.edge_cnt[row]);
    if (tid == 1 && (em & 2u)) reset_counter(&p.edge_cnt[row + 1]);
    const int e0 = (em & 1u) ? t : t + 1;
    const int ne = (em == 3u) ? 2 : 1;
    pairs_fused<BF16>(p, b, e0, ne, row, hown, sm.pr);
    drain_stores();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&p.seq_cnt[b], (uint32_t)ne, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        flag = (old + (uint32_t)ne == (uint32_t)P) ? 1u : 0u;
    }
    __syncthreads();
    if (!flag) return;
    if (tid == 0) reset_counter(&p.seq_cnt[b]);
    walk_of<SAMPLE>(p, b, sm);
}

// The three-stage plan's scan launch: the last segment of a row merges its
// lists and leaves the row's candidates for the pair launch.  Nothing here
// waits on the gate: the pair launch takes H_t once the whole scan is done.
template <bool BF16>
__device__ __forceinline__ void row_merge_only(const Params& p, int64_t row, SharedAll& sm) {
    merge_row<BF16>(p.part + (size_t)row * p.nseg * kWaves * p.K, p.nseg * kWaves, p.K,
                    p.cand + row * p.K, p.cval + row * p.K, sm.m);
}

// The three-stage plan's second launch, one workgroup per row t of sequence
// b: the pair scores of the transition into t (every input is in memory
// already: no hand-off before it), then the last transition of the sequence
// to be scored walks it.
template <bool BF16, bool SAMPLE, bool HSUM>
__device__ __forceinline__ void pairs_walk(const Params& p, int64_t row, SharedAll& sm,
                                           uint32_t& flag) {
    const int tid = threadIdx.x, P = p.P;
    const int b = (int)(row / P), t = (int)(row % P);
    const float hz[2] = {0.f, 0.f};
    pairs_fused<BF16, !HSUM>(p, b, t, 1, -1, hz, sm.pr);
    drain_stores();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&p.seq_cnt[b], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        flag = (old + 1u == (uint32_t)P) ? 1u : 0u;
    }
    __syncthreads();
    if (!flag) return;
    if (tid == 0) reset_counter(&p.seq_cnt[b]);
    walk_of<SAMPLE>(p, b, sm);
}

// The whole selector in one launch.
template <bool BF16, int NV, int MB, bool SAMPLE>
__global__ __launch_bounds__(kWG, 5) void k_select(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    const int64_t g = blockIdx.x;
    if (g < p.n_gate) {
        // the gate and everything after a segment are on the critical path;
        // the streaming waves that share the SIMDs mostly wait on memory
        __builtin_amdgcn_s_setprio(3);
        gate_role<BF16, MB, false>(p, (int)g, sm.g);
        return;
    }
    const int64_t sb = g - p.n_gate;
    const int64_t row = sb / p.nseg;
    segment_of<BF16, NV>(p, row, (int)(sb % p.nseg), sm.c);
    if (!block_arrive_last(&p.row_cnt[row], (uint32_t)p.nseg, &flag)) return;
    __builtin_amdgcn_s_setprio(3);
    if (threadIdx.x == 0) reset_counter(&p.row_cnt[row]);
    row_tail<BF16, MB, SAMPLE, false>(p, row, sm, flag);
}

// The selector in two launches: k_scan runs the gate slices and the segments
// (each stores its lists and ends), then k_tail runs row_tail for every row,
// one workgroup per row.  Each launch is compiled under its own register
// budget, the scan's without the tail's code.
template <bool BF16, int NV, int MB>
__global__ __launch_bounds__(kWG, 5) void k_scan(Params p) {
    __shared__ SharedAll sm;
    const int64_t g = blockIdx.x;
    if (g < p.n_gate) {
        gate_role<BF16, MB, MB == 1>(p, (int)g, sm.g);
        return;
    }
    const int64_t sb = g - p.n_gate;
    segment_of<BF16, NV, true>(p, sb / p.nseg, (int)(sb % p.nseg), sm.c);
}

template <bool BF16, int MB, bool SAMPLE>
__global__ __launch_bounds__(kWG, 5) void k_tail(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    row_tail<BF16, MB, SAMPLE, MB == 1>(p, (int64_t)blockIdx.x, sm, flag);
}

// The selector in three stages over two launches: k_scanm runs the gate
// slices, the segments and, on a row's last arrival, its merge; k_pairs_walk
// scores every transition (one workgroup per row) and walks each sequence.
template <bool BF16, int NV, int MB>
__global__ __launch_bounds__(kWG, 5) void k_scanm(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    const int64_t g = blockIdx.x;
    if (g < p.n_gate) {
        gate_role<BF16, MB, MB == 1, false>(p, (int)g, sm.g);
        return;
    }
    const int64_t sb = g - p.n_gate;
    const int64_t row = sb / p.nseg;
    // The segments and the merges after them are the launch's critical
    // path; the gate slices that share their CUs are read only by the next
    // launch (batch 32: 28.9 -> 28.6 us per call with the segments above
    // them, whatever the level).
    __builtin_amdgcn_s_setprio(1);
    segment_of<BF16, NV, true>(p, row, (int)(sb % p.nseg), sm.c);
    if (!block_arrive_last(&p.row_cnt[row], (uint32_t)p.nseg, &flag)) return;
    if (threadIdx.x == 0) reset_counter(&p.row_cnt[row]);
    row_merge_only<BF16>(p, row, sm);
}

template <bool BF16, int MB, bool SAMPLE>
__global__ __launch_bounds__(kWG, 5) void k_pairs_walk(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    pairs_walk<BF16, SAMPLE, MB == 1>(p, (int64_t)blockIdx.x, sm, flag);
}

// The three-stage plan with the walks in a launch of their own (rows beyond
// one resident wave of workgroups): the pair scores of the transition into
// every row, then one workgroup per sequence walks.  A walk that fell to the
// last pair job of its sequence landed on the slowest XCD, filled its CUs
// and held back the dispatch of its remaining rows.
template <bool BF16, int MB>
__global__ __launch_bounds__(kWG, 5) void k_pairs_rows(Params p) {
    __shared__ SharedAll sm;
    const int64_t row = blockIdx.x;
    const float hz[2] = {0.f, 0.f};
    pairs_fused<BF16, MB != 1>(p, (int)(row / p.P), (int)(row % p.P), 1, -1, hz, sm.pr);
}

template <bool SAMPLE>
__global__ __launch_bounds__(kWG, 5) void k_walks(Params p) {
    __shared__ SharedAll sm;
    walk_of<SAMPLE, true>(p, (int)blockIdx.x, sm);
}

// Top-K alone: segments, then the row merge on last arrival.
template <bool BF16, int NV>
__global__ __launch_bounds__(kWG, 5) void k_topk(Params p) {
    __shared__ SharedAll sm;
    __shared__ uint32_t flag;
    const int64_t row = blockIdx.x / p.nseg;
    segment_of<BF16, NV>(p, row, (int)(blockIdx.x % p.nseg), sm.c);
    if (!block_arrive_last(&p.row_cnt[row], (uint32_t)p.nseg, &flag)) return;
    if (threadIdx.x == 0) reset_counter(&p.row_cnt[row]);
    merge_row<BF16>(p.part + (size_t)row * p.nseg * kWaves * p.K, p.nseg * kWaves, p.K,
                    p.cand + row * p.K, p.cval + row * p.K, sm.m);
}

// Gate projection alone: slices into H (S == 1) or into partials.
template <bool BF16, int MB>
__global__ __launch_bounds__(kWG) void k_gate(Params p) {
    __shared__ GateLds sm;
    const int s = (int)(blockIdx.x % p.S), tile = (int)(blockIdx.x / p.S);
    gate_slice<BF16, MB, GateShape<MB>::NB>(p.hidden, p.W, (int)p.rows, p.d, p.r,
                                            tile / p.ntiles, tile % p.ntiles, s, p.S,
                                            p.S == 1 ? p.H : p.ppart, sm);
}

// H = sum of the S partials, in slice order; one thread per four floats.
__global__ __launch_bounds__(kWG) void k_gate_sum(const float* __restrict__ part, int S,
                                                  int64_t n4, float* __restrict__ H) {
    const int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x;
    if (i >= n4) return;
    const float4* src = reinterpret_cast<const float4*>(part);
    float4 acc = src[i];
    for (int s = 1; s < S; ++s) {
        const float4 v = src[(int64_t)s * n4 + i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    reinterpret_cast<float4*>(H)[i] = acc;
}

// Pair scores alone: one workgroup per (sequence, position).
struct PairArgs {
    const int32_t* cand;
    const float* cval;
    const float* H;
    const void* A;
    const void* Bt;
    const int32_t* prev;
    float* out_S;
    uint32_t* err;
    int B, P, V, r, K;
};

template <bool BF16>
__global__ __launch_bounds__(kWG) void k_pairs(PairArgs a) {
    __shared__ PairLds sm;
    const int tid = threadIdx.x, K = a.K;
    const int b = (int)(blockIdx.x / a.P), e = (int)(blockIdx.x % a.P);
    const int64_t rb = (int64_t)b * a.P;
    if (tid < K) {
        sm.ids[0][tid] = (e > 0) ? checked_id(a.cand[(rb + e - 1) * K + tid], a.V, a.err, 2u)
                                 : checked_id(a.prev[b], a.V, a.err, 1u);
    } else if (tid >= 64 && tid < 64 + K) {
        const int k = tid - 64;
        sm.ids[1][k] = checked_id(a.cand[(rb + e) * K + k], a.V, a.err, 2u);
        sm.u[0][k] = a.cval[(rb + e) * K + k];
    }
    __syncthreads();
    pair_tiles<BF16>(a.A, a.Bt, K, a.r, e, 1, a.out_S + (rb + e) * K * K, sm, [&]() {
        pair_sum_gate(a.H, 1, (int64_t)a.B * a.P, a.r, rb + e, 1, sm);
    });
}

// The walk alone: one workgroup per sequence.
struct WalkArgs {
    const float* S;
    const int32_t* cand;
    const float* u;       // sampling walk: [B, P] uniforms
    int32_t* out_path;
    float* out_q;         // sampling walk: [B, P] probabilities
    float* out_score;
    int P, K;
    int walk;             // kWalkViterbi, kWalkGreedy or kWalkSample
    float inv_tau;
};

__global__ __launch_bounds__(kWG) void k_walk(WalkArgs a) {
    __shared__ WalkLds sm;
    const int64_t b = blockIdx.x;
    const int64_t rb = b * a.P;
    const float* S = a.S + rb * a.K * a.K;
    const int32_t* ids = a.cand + rb * a.K;
    if (a.walk == kWalkGreedy)
        chain_seq<kChainGreedy>(S, ids, nullptr, 0.f, a.P, a.K, a.out_path + rb, nullptr, a.out_score + b, sm);
    else if (a.walk == kWalkSample)
        chain_seq<kChainSample>(S, ids, a.u + rb, a.inv_tau, a.P, a.K, a.out_path + rb, a.out_q + rb,
                                a.out_score + b, sm);
    else
        walk_seq<true>(S, ids, a.P, a.K, a.out_path + rb, a.out_score + b, sm);
}

// Zeroes n words; clears the arrival counters of the no-allocation entry
// point (a kernel, not a memset, so that callers may capture it in a graph).
__global__ __launch_bounds__(kWG) void k_fill_zero(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Scratch of dflash2_select_noalloc: one copy per device, zero when the
// module loads, kept until the process ends.  Host code uses only the
// address hipGetSymbolAddress returns for the current device, never the
// name.
constexpr size_t kStaticScratchBytes = (size_t)48 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
thread_local std::string g_last_error;

df2_status fail(df2_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

df2_status hip_fail(hipError_t e, const char* what) {
    return fail(DF2_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

struct Scratch {
    void* ptr = nullptr;
    size_t bytes = 0;
    size_t zeroed_counter_bytes = 0;   // prefix known to hold only zeros
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;
std::map<int, void*> g_static_scratch;   // device -> address of `scratch` on it
std::map<int, int> g_capacity;         // device -> resident select workgroups
std::map<int, int> g_cus;              // device -> compute units

// Scratch of at least `bytes`, whose first `counter_bytes` are zero when the
// stream reaches the next launch.
df2_status get_scratch(hipStream_t stream, size_t bytes, size_t counter_bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    Scratch& s = g_scratch[std::make_pair(dev, stream)];
    if (s.bytes < bytes) {
        if (s.ptr) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            (void)hipFree(s.ptr);
            s.ptr = nullptr;
            s.bytes = 0;
        }
        size_t nb = align_up(std::max(bytes, (size_t)1 << 20), (size_t)1 << 20);
        e = hipMalloc(&s.ptr, nb);
        if (e != hipSuccess) {
            s.ptr = nullptr;
            return fail(DF2_ENOMEM, std::string("hipMalloc scratch: ") + hipGetErrorString(e));
        }
        e = hipMemset(s.ptr, 0, nb);
        if (e != hipSuccess) return hip_fail(e, "hipMemset scratch");
        s.bytes = nb;
        s.zeroed_counter_bytes = nb;
    }
    if (s.zeroed_counter_bytes < counter_bytes) {
        e = hipMemsetAsync(s.ptr, 0, counter_bytes, stream);
        if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync counters");
        s.zeroed_counter_bytes = counter_bytes;
    }
    *out = s.ptr;
    return DF2_OK;
}

// The address of the static scratch on the current device (looked up once per
// device).
df2_status static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_static_scratch.find(dev);
    if (it == g_static_scratch.end()) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (no-allocation scratch)");
        it = g_static_scratch.emplace(dev, ptr).first;
    }
    *out = it->second;
    return DF2_OK;
}

// Later layouts may put data where earlier ones kept counters: remember that
// only the counter prefix of the latest layout is known to be zero.
void note_layout(hipStream_t stream, size_t counter_bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_scratch.find(std::make_pair(dev, stream));
    if (it != g_scratch.end()) it->second.zeroed_counter_bytes = counter_bytes;
}

// Plan overrides for measurement (dflash2_plan_override); 0 = automatic.
// Set only through the C ABI: the library never reads the environment.
struct Overrides {
    int wgs = 0;          // target count of top-K segment workgroups
    int nv = 0;           // 16-byte vectors per lane per chunk (1, 2 or 4)
    int mwords = 0;       // most candidate words one row merge takes (<= 1024)
    int gate_s = 0;       // gate slices of d (1..16)
    int conv_s = 0;       // k slices of the convolution's correction GEMM
    int launches = 0;     // dflash2_select: 1 = one fused launch, 2 = scan then tail,
                          // 3 = scan with the row merges, then pairs and walk,
                          // 4 = as 3 with the walks in a third launch
    int lm_ranges = 0;    // vocabulary ranges of the LM head (1..256)
    int gate_giveup = 0;  // 1: the row merges' gate wait gives up (failure-handling tests)
};
Overrides g_over;

Overrides overrides() {
    std::lock_guard<std::mutex> lock(g_mu);
    return g_over;
}

// Workgroups of the select kernel that are resident at once on the current
// device (CUs x workgroups per CU).
int select_capacity() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1024;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_capacity.find(dev);
        if (it != g_capacity.end()) return it->second;
    }
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(&k_select<true, 4, 4, false>), kWG, 0) != hipSuccess)
        per = 4;
    const int cap = std::max(1, cus * std::max(1, per));
    std::lock_guard<std::mutex> lock(g_mu);
    g_capacity[dev] = cap;
    return cap;
}

// Compute units of the current device.
int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_cus.find(dev);
        if (it != g_cus.end()) return it->second;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    std::lock_guard<std::mutex> lock(g_mu);
    g_cus[dev] = cus;
    return cus;
}

struct Plan {
    Params p;
    bool two = false;           // scan and tail as two launches
    bool three = false;         // two launches, the row merges in the first
    bool walks = false;         // three-stage, the walks in a third launch
    int nv = 1;
    int mb = 4;                 // gate tile: 16*mb rows x 16*(mb == 1 ? 4 : 2) columns
    bool bf16 = true;
    int64_t n_chunk_blocks = 0;
    size_t counter_bytes = 0, total_bytes = 0;
    size_t off_part = 0, off_cand = 0, off_cval = 0, off_ppart = 0, off_S = 0, off_Hb = 0;
};

// Chunk size (16-byte vectors per thread) and segmentation of the rows.
// Chunks of 256 x 4 vectors (16 KB of bf16) whenever a row holds at least
// eight of them; for shorter rows, smaller chunks when there are too few
// rows to give every CU a workgroup.  Rows are then cut into segments so
// that about `target` workgroups stream in total; a row's segment lists
// must fit one merge.
void plan_topk(Plan& pl, int64_t rows, int V, int K, bool bf16, const void* logits,
               int64_t target, const Overrides& ov, int mwords_default = kMergeMax) {
    Params& p = pl.p;
    pl.bf16 = bf16;
    const int pv = bf16 ? 8 : 4;
    auto chunks = [&](int nv) { return (int)((V + (int64_t)kWG * pv * nv - 1) / ((int64_t)kWG * pv * nv)); };
    int nv = 1;
    if (chunks(4) >= 8) {
        nv = 4;
    } else {
        for (int cand : {4, 2, 1}) {
            if (rows * chunks(cand) >= 256) { nv = cand; break; }
        }
    }
    if (ov.nv == 1 || ov.nv == 2 || ov.nv == 4) nv = ov.nv;
    pl.nv = nv;
    p.split = nv;
    p.C = chunks(nv);
    if (ov.wgs > 0) target = ov.wgs;
    target = std::max<int64_t>(1, std::min<int64_t>(target, 1 << 30));
    // at most mwords_default (the knob: at most kMergeMax) words per row
    // merge; fewer lists also make the merge bound sharper
    const int mwords = std::min(kMergeMax, ov.mwords > 0 ? ov.mwords : mwords_default);
    const int max_segs = std::max(1, mwords / (kWaves * K));
    int nseg = (int)std::min<int64_t>(p.C, std::max<int64_t>(1, target / rows));
    p.nseg = std::min(nseg, max_segs);
    p.rows = rows;
    p.V = V;
    p.K = K;
    // the aligned path reads a row through a buffer resource: under 2^31 bytes
    p.aligned = (aligned16(logits) && (V % pv) == 0 && (int64_t)V * (bf16 ? 2 : 4) < (1LL << 31))
                    ? 1 : 0;
    pl.n_chunk_blocks = rows * p.nseg;
    p.n_chunk = pl.n_chunk_blocks;
}

// Gate tiles and slices of d.  Tiles are 16 x 64 for a single tile row of
// at most 16 rows, else 64 x 32.  A slice is at least one round of loads
// (4 waves x gate_kb k steps); S is the largest count of such slices that
// stays within kMaxFusedSlices (the pair scores sum the partials) and gives
// about one gate workgroup per CU at most: many short slices finish early,
// beside the streaming segments, but past one per CU the gate's workgroups
// take slots and issue cycles from the streaming.  The standalone
// projection uses the same slices, so both paths round alike.
void plan_gate(Plan& pl, int64_t M, int d, int r, const Overrides& ov) {
    Params& p = pl.p;
    pl.mb = (M <= 16) ? 1 : 4;
    const int nb = (pl.mb == 1) ? 4 : 2;
    p.gm_rows = 16 * pl.mb;
    p.mtiles = (int)((M + p.gm_rows - 1) / p.gm_rows);
    p.ntiles = r / (16 * nb);
    const int KS = d / 32;
    const int per_round = kWaves * gate_kb(pl.bf16);
    int S = std::max(1, std::min(kMaxFusedSlices, (KS + per_round - 1) / per_round));
    // at least four slices; measured at d = 5120: batch 32 runs 37.5 us per
    // cycle with 8 slices against 41.0 with 16, batch 8 keeps 16 (its rows
    // are ready sooner, so its gate must end sooner)
    S = std::min(S, std::max(4, cu_count() / (p.mtiles * p.ntiles)));
    if (ov.gate_s >= 1 && ov.gate_s <= std::min(KS, kMaxFusedSlices)) S = ov.gate_s;
    p.S = S;
    p.n_gate = p.mtiles * p.ntiles * S;
    p.gate_extra = ov.gate_giveup ? 1u : 0u;
    p.gate_spins = ov.gate_giveup ? 64u : (1u << 20);
    p.d = d;
    p.r = r;
}

// Scratch layout: counters first (err, rows, transitions, sequences, gate
// tile rows, gate readers, gate tiles), then data.
void plan_layout(Plan& pl, int64_t rows, int64_t M, int B, bool pairs) {
    Params& p = pl.p;
    const size_t ncnt = 1 + 2 * (size_t)rows + (size_t)B + 2 * (size_t)p.mtiles +
                        (size_t)p.mtiles * p.ntiles;
    pl.counter_bytes = align_up(ncnt * 4, 256);
    size_t off = pl.counter_bytes;
    pl.off_part = off;
    off = align_up(off + (size_t)rows * p.nseg * kWaves * p.K * 8, 256);
    pl.off_cand = off;
    off = align_up(off + (size_t)rows * p.K * 4, 256);
    pl.off_cval = off;
    off = align_up(off + (size_t)rows * p.K * 4, 256);
    pl.off_ppart = off;
    off = align_up(off + (p.S > 1 || pairs ? (size_t)p.S * M * p.r * 4 : 0), 256);
    pl.off_S = off;
    off = align_up(off + (pairs ? (size_t)rows * p.K * p.K * 4 : 0), 256);
    pl.off_Hb = off;
    off = align_up(off + (pairs ? (size_t)rows * p.r * 4 : 0), 256);
    pl.total_bytes = off;
}

void bind_scratch(Plan& pl, void* base, int64_t rows, int B) {
    Params& p = pl.p;
    char* c = reinterpret_cast<char*>(base);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(c);
    p.err = cnt;
    p.row_cnt = cnt + 1;
    p.edge_cnt = p.row_cnt + rows;
    p.seq_cnt = p.edge_cnt + rows;
    p.gate_cnt = p.seq_cnt + B;
    p.rd_cnt = p.gate_cnt + p.mtiles;
    p.tile_cnt = p.rd_cnt + p.mtiles;
    p.part = reinterpret_cast<uint64_t*>(c + pl.off_part);
    p.cand = reinterpret_cast<int32_t*>(c + pl.off_cand);
    p.cval = reinterpret_cast<float*>(c + pl.off_cval);
    p.ppart = reinterpret_cast<float*>(c + pl.off_ppart);
    p.Sb = reinterpret_cast<float*>(c + pl.off_S);
    p.Hb = reinterpret_cast<float*>(c + pl.off_Hb);
}

df2_status check_dims(const df2_dims* dims, bool need_d) {
    if (!dims) return fail(DF2_EINVAL, "dims is NULL");
    if (dims->dtype != DF2_F32 && dims->dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (dims->B < 0) return fail(DF2_EINVAL, "B < 0");
    if (dims->P < 1 || dims->P > kMaxP) return fail(DF2_EINVAL, "P must be in [1, 64]");
    if (dims->V < 1) return fail(DF2_EINVAL, "V < 1");
    if (need_d && (dims->d < 32 || dims->d % 32 != 0))
        return fail(DF2_EUNSUPPORTED, "d must be a positive multiple of 32");
    if (dims->r < 64 || dims->r % 64 != 0 || dims->r > kMaxR)
        return fail(DF2_EUNSUPPORTED, "r must be a multiple of 64 in [64, 512]");
    return DF2_OK;
}

df2_status check_k(int K, int V) {
    if (K < 1 || K > kMaxK || K > V) return fail(DF2_EINVAL, "K must be in [1, min(V, 64)]");
    return DF2_OK;
}

template <typename F>
df2_status launch_checked(F&& f, const char* what) {
    f();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, what);
    return DF2_OK;
}

// One fused launch (k_select), or the scan launch and then the tail launch.
constexpr int kSelectMergeWords = 768;

void launch_select(const Plan& pl, hipStream_t stream) {
    const int64_t n2 = pl.p.n_gate + pl.n_chunk_blocks;
    dim3 block(kWG);
#define DF2_SEL_W(BF, NV_, MB_, SM)                                                            \
    do {                                                                                       \
        if (pl.three) {                                                                        \
            hipLaunchKernelGGL((k_scanm<BF, NV_, MB_>),                                        \
                               dim3((unsigned)(pl.p.n_gate + pl.n_chunk_blocks)), block, 0,    \
                               stream, pl.p);                                                  \
            if (pl.walks) {                                                                    \
                hipLaunchKernelGGL((k_pairs_rows<BF, MB_>), dim3((unsigned)pl.p.rows), block, 0, \
                                   stream, pl.p);                                              \
                hipLaunchKernelGGL((k_walks<SM>), dim3((unsigned)pl.p.B), block, 0, stream,    \
                                   pl.p);                                                      \
                break;                                                                         \
            }                                                                                  \
            hipLaunchKernelGGL((k_pairs_walk<BF, MB_, SM>), dim3((unsigned)pl.p.rows), block, 0,    \
                               stream, pl.p);                                                  \
            break;                                                                             \
        }                                                                                      \
        if (pl.two) {                                                                          \
            hipLaunchKernelGGL((k_scan<BF, NV_, MB_>),                                         \
                               dim3((unsigned)(pl.p.n_gate + pl.n_chunk_blocks)), block, 0,    \
                               stream, pl.p);                                                  \
            hipLaunchKernelGGL((k_tail<BF, MB_, SM>), dim3((unsigned)pl.p.rows), block, 0,     \
                               stream, pl.p);                                                  \
            break;                                                                             \
        }                                                                                      \
        hipLaunchKernelGGL((k_select<BF, NV_, MB_, SM>), dim3((unsigned)n2), block, 0, stream,  \
                           pl.p);                                                              \
    } while (0)
#define DF2_SEL(BF, NV_, MB_)                                     \
    do {                                                          \
        if (pl.p.walk == kWalkSample) DF2_SEL_W(BF, NV_, MB_, true); \
        else DF2_SEL_W(BF, NV_, MB_, false);                      \
    } while (0)
#define DF2_SEL_NV(BF, MB_)                  \
    switch (pl.p.aligned ? pl.nv : 0) {      \
        case 0: DF2_SEL(BF, 0, MB_); break;  \
        case 1: DF2_SEL(BF, 1, MB_); break;  \
        case 2: DF2_SEL(BF, 2, MB_); break;  \
        default: DF2_SEL(BF, 4, MB_); break; \
    }
    if (pl.bf16) {
        if (pl.mb == 1) { DF2_SEL_NV(true, 1) } else { DF2_SEL_NV(true, 4) }
    } else {
        if (pl.mb == 1) { DF2_SEL_NV(false, 1) } else { DF2_SEL_NV(false, 4) }
    }
#undef DF2_SEL_NV
#undef DF2_SEL
#undef DF2_SEL_W
}

void launch_topk(const Plan& pl, hipStream_t stream) {
    dim3 grid((unsigned)pl.n_chunk_blocks), block(kWG);
#define DF2_TOPK(BF)                                                                          \
    switch (pl.p.aligned ? pl.nv : 0) {                                                       \
        case 0: hipLaunchKernelGGL((k_topk<BF, 0>), grid, block, 0, stream, pl.p); break;   \
        case 1: hipLaunchKernelGGL((k_topk<BF, 1>), grid, block, 0, stream, pl.p); break;   \
        case 2: hipLaunchKernelGGL((k_topk<BF, 2>), grid, block, 0, stream, pl.p); break;   \
        default: hipLaunchKernelGGL((k_topk<BF, 4>), grid, block, 0, stream, pl.p); break;  \
    }
    if (pl.bf16) { DF2_TOPK(true) } else { DF2_TOPK(false) }
#undef DF2_TOPK
}

void launch_gate(const Plan& pl, hipStream_t stream) {
    dim3 grid((unsigned)pl.p.n_gate), block(kWG);
    if (pl.bf16) {
        if (pl.mb == 1) hipLaunchKernelGGL((k_gate<true, 1>), grid, block, 0, stream, pl.p);
        else hipLaunchKernelGGL((k_gate<true, 4>), grid, block, 0, stream, pl.p);
    } else {
        if (pl.mb == 1) hipLaunchKernelGGL((k_gate<false, 1>), grid, block, 0, stream, pl.p);
        else hipLaunchKernelGGL((k_gate<false, 4>), grid, block, 0, stream, pl.p);
    }
    if (pl.p.S > 1) {
        const int64_t n4 = pl.p.rows * pl.p.r / 4;
        dim3 g2((unsigned)((n4 + kWG - 1) / kWG));
        hipLaunchKernelGGL(k_gate_sum, g2, block, 0, stream, pl.p.ppart, pl.p.S, n4, pl.p.H);
    }
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------
extern "C" {

const char* dflash2_version(void) { return "0.1.0"; }

const char* dflash2_status_string(df2_status s) {
    switch (s) {
        case DF2_OK: return "ok";
        case DF2_EINVAL: return "invalid argument";
        case DF2_EUNSUPPORTED: return "unsupported argument";
        case DF2_EHIP: return "HIP error";
        case DF2_ENOMEM: return "out of device memory";
    }
    return "unknown status";
}

const char* dflash2_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// The fused selector with any walk; the sampling walk also takes u, 1 / tau
// and out_q (checked by the caller).
df2_status select_common(const df2_dims* dims, const void* logits, const void* hidden,
                         const void* A_tab, const void* B_tab, const void* W_H,
                         const int32_t* prev_tok, int32_t K, int walk, const float* u, float inv_tau,
                         int32_t* out_path, float* out_q, float* out_score, hipStream_t stream,
                         bool noalloc = false) {
    df2_status st = check_dims(dims, true);
    if (st != DF2_OK) return st;
    if ((st = check_k(K, dims->V)) != DF2_OK) return st;
    if (dims->B == 0) return DF2_OK;
    if (!logits || !hidden || !A_tab || !B_tab || !W_H || !prev_tok || !out_path || !out_score)
        return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(hidden) || !aligned16(A_tab) || !aligned16(B_tab) || !aligned16(W_H))
        return fail(DF2_EINVAL, "hidden, A_tab, B_tab and W_H must be 16-byte aligned");
    if (((uintptr_t)prev_tok & 3u) || ((uintptr_t)out_path & 3u) || ((uintptr_t)out_score & 3u))
        return fail(DF2_EINVAL, "prev_tok, out_path and out_score must be 4-byte aligned");
    const bool bf16 = dims->dtype == DF2_BF16;
    if (!bf16 && ((uintptr_t)logits & 3u)) return fail(DF2_EINVAL, "fp32 logits must be 4-byte aligned");
    if (bf16 && ((uintptr_t)logits & 1u)) return fail(DF2_EINVAL, "bf16 logits must be 2-byte aligned");
    const int64_t rows = (int64_t)dims->B * dims->P;
    const Overrides ov = overrides();
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    pl.bf16 = bf16;
    plan_gate(pl, rows, dims->d, dims->r, ov);
    // Row merges of the selector take at most 768 words (12 segments per row
    // at K = 16): at batch 8 (V = 151936, d = 5120) 21.1 us per call against
    // 21.6 with 13 segments per row (832 words), batch 1 and 32 unchanged.
    // Three stages in two launches by default: k_scanm (gate slices,
    // segments, and each row's merge on its last segment's arrival), then
    // k_pairs_walk.  Nothing in k_scanm waits: a row merge that waited there
    // for its gate tile row slowed the gate slices on its CU (at batch 32 the
    // slowest slices went from 16 to 27 us).  Measured at V = 151936 (bf16,
    // us per call, three stages / scan then tail / fused): batch 1 (d = 2560)
    // 18.2 / 19.6 / 20.8, batch 8 (d = 5120) 22.3 / 23.4 / 26.4, batch 32
    // 31.9 / 33.8 / 37.0; B = 256, P = 15, V = 262144: 481 / 527 / 488 (as
    // first measured).  Beyond one resident wave of rows the walks move to a
    // third launch: left to the last pair job of each sequence they gathered
    // on the slowest XCD and held back its dispatch (B = 256, P = 15: 484 ->
    // 421 us).  The launches plan knob forces any plan.  Segment workgroups: about
    // three per CU for the two-launch plans, two and a half for the fused one,
    // within what the gate leaves of one resident wave (batch 32, three
    // stages: 31.8 us with 3 segments per row, 33.0 with 2, 34.2 with 4).
    const int64_t cap = select_capacity();
    const int mode = ov.launches ? ov.launches : (rows > cap ? 4 : 3);
    pl.two = mode >= 2;
    pl.three = mode >= 3;
    pl.walks = mode == 4;
    const int64_t cus = cu_count();
    const int64_t target = std::min<int64_t>(cap - pl.p.n_gate, pl.two ? 3 * cus : (5 * cus) / 2);
    plan_topk(pl, rows, dims->V, K, bf16, logits, std::max<int64_t>(rows, target), ov, kSelectMergeWords);
    if (pl.p.n_gate + pl.n_chunk_blocks > 0x7FFFFFFF) return fail(DF2_EUNSUPPORTED, "problem too large");
    plan_layout(pl, rows, rows, dims->B, true);
    Params& p = pl.p;
    p.logits = logits;
    p.hidden = hidden;
    p.A = A_tab;
    p.Bt = B_tab;
    p.W = W_H;
    p.prev = prev_tok;
    p.out_path = out_path;
    p.out_score = out_score;
    p.B = dims->B;
    p.P = dims->P;
    p.walk = walk;
    p.u = u;
    p.out_q = out_q;
    p.inv_tau = inv_tau;
    void* base = nullptr;
    if (noalloc) {
        if (pl.total_bytes > kStaticScratchBytes)
            return fail(DF2_EUNSUPPORTED, "problem needs " + std::to_string(pl.total_bytes) +
                                              " bytes of scratch; the no-allocation entry point holds " +
                                              std::to_string(kStaticScratchBytes));
        if ((st = static_scratch(&base)) != DF2_OK) return st;
    } else {
        if ((st = get_scratch(stream, pl.total_bytes, pl.counter_bytes, &base)) != DF2_OK) return st;
        note_layout(stream, pl.counter_bytes);
    }
    bind_scratch(pl, base, rows, dims->B);
    return launch_checked([&] {
        if (noalloc) {
            // the counters (all words after the device flag word) start at
            // zero; the previous call may have left data there
            const int64_t n = (int64_t)(pl.counter_bytes / 4) - 1;
            hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + kWG - 1) / kWG)), dim3(kWG), 0, stream,
                               pl.p.err + 1, n);
        }
        launch_select(pl, stream);
    }, "dflash2_select launch");
}

// 1 / tau for the sampling walk, or an error for a temperature that is not
// positive and finite, or whose reciprocal overflows fp32.
df2_status sample_inv_tau(float temperature, float* inv_tau) {
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(DF2_EINVAL, "temperature must be positive and finite");
    const double it = 1.0 / (double)temperature;
    if (it > 3.0e38) return fail(DF2_EINVAL, "temperature too small (1 / temperature overflows fp32)");
    *inv_tau = (float)it;
    return DF2_OK;
}

}  // namespace

extern "C" {

df2_status dflash2_select_walk(const df2_dims* dims, const void* logits, const void* hidden,
                               const void* A_tab, const void* B_tab, const void* W_H,
                               const int32_t* prev_tok, int32_t K, df2_walk walk,
                               int32_t* out_path, float* out_score, hipStream_t stream) {
    g_last_error.clear();
    if (walk != DF2_WALK_VITERBI && walk != DF2_WALK_GREEDY)
        return fail(DF2_EINVAL, "unknown walk mode");
    return select_common(dims, logits, hidden, A_tab, B_tab, W_H, prev_tok, K, (int)walk, nullptr,
                         0.f, out_path, nullptr, out_score, stream);
}

df2_status dflash2_select_sample(const df2_dims* dims, const void* logits, const void* hidden,
                                 const void* A_tab, const void* B_tab, const void* W_H,
                                 const int32_t* prev_tok, int32_t K, float temperature,
                                 const float* u, int32_t* out_path, float* out_q,
                                 float* out_score, hipStream_t stream) {
    g_last_error.clear();
    float inv_tau = 0.f;
    df2_status st = sample_inv_tau(temperature, &inv_tau);
    if (st != DF2_OK) return st;
    if (dims && dims->B > 0) {
        if (!u || !out_q) return fail(DF2_EINVAL, "NULL pointer argument");
        if (((uintptr_t)u & 3u) || ((uintptr_t)out_q & 3u))
            return fail(DF2_EINVAL, "u and out_q must be 4-byte aligned");
    }
    return select_common(dims, logits, hidden, A_tab, B_tab, W_H, prev_tok, K, kWalkSample, u,
                         inv_tau, out_path, out_q, out_score, stream);
}

df2_status dflash2_select(const df2_dims* dims, const void* logits, const void* hidden,
                          const void* A_tab, const void* B_tab, const void* W_H,
                          const int32_t* prev_tok, int32_t K, int32_t* out_path,
                          float* out_score, hipStream_t stream) {
    return dflash2_select_walk(dims, logits, hidden, A_tab, B_tab, W_H, prev_tok, K,
                               DF2_WALK_VITERBI, out_path, out_score, stream);
}

df2_status dflash2_select_noalloc(const df2_dims* dims, const void* logits, const void* hidden,
                                  const void* A_tab, const void* B_tab, const void* W_H,
                                  const int32_t* prev_tok, int32_t K, int32_t* out_path,
                                  float* out_score, hipStream_t stream) {
    g_last_error.clear();
    return select_common(dims, logits, hidden, A_tab, B_tab, W_H, prev_tok, K, kWalkViterbi, nullptr, 0.f,
                         out_path, nullptr, out_score, stream, true);
}

df2_status dflash2_topk(const void* logits, int64_t rows, int32_t V, df2_dtype dtype, int32_t K,
                        int32_t* out_idx, float* out_val, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != DF2_F32 && dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (rows < 0) return fail(DF2_EINVAL, "rows < 0");
    if (V < 1) return fail(DF2_EINVAL, "V < 1");
    df2_status st = check_k(K, V);
    if (st != DF2_OK) return st;
    if (rows == 0) return DF2_OK;
    if (!logits || !out_idx || !out_val) return fail(DF2_EINVAL, "NULL pointer argument");
    const bool bf16 = dtype == DF2_BF16;
    if (((uintptr_t)out_idx & 3u) || ((uintptr_t)out_val & 3u))
        return fail(DF2_EINVAL, "outputs must be 4-byte aligned");
    if ((bf16 && ((uintptr_t)logits & 1u)) || (!bf16 && ((uintptr_t)logits & 3u)))
        return fail(DF2_EINVAL, "logits misaligned for its dtype");
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    plan_topk(pl, rows, V, K, bf16, logits, select_capacity(), overrides());
    if (pl.n_chunk_blocks > 0x7FFFFFFF) return fail(DF2_EUNSUPPORTED, "too many rows");
    pl.p.S = 1;
    plan_layout(pl, rows, 0, 0, false);
    Params& p = pl.p;
    p.logits = logits;
    p.P = 1;
    void* base = nullptr;
    if ((st = get_scratch(stream, pl.total_bytes, pl.counter_bytes, &base)) != DF2_OK) return st;
    note_layout(stream, pl.counter_bytes);
    bind_scratch(pl, base, rows, 0);
    // results go straight to the caller's buffers
    p.cand = out_idx;
    p.cval = out_val;
    return launch_checked([&] { launch_topk(pl, stream); }, "dflash2_topk launch");
}

df2_status dflash2_project(const void* hidden, const void* W_H, int64_t M, int32_t d, int32_t r,
                           df2_dtype dtype, float* out_H, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != DF2_F32 && dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (M < 0) return fail(DF2_EINVAL, "M < 0");
    if (d < 32 || d % 32 != 0) return fail(DF2_EUNSUPPORTED, "d must be a positive multiple of 32");
    if (r < 64 || r % 64 != 0 || r > 1024)
        return fail(DF2_EUNSUPPORTED, "r must be a multiple of 64 in [64, 1024]");
    if (M == 0) return DF2_OK;
    if (M > (1 << 24)) return fail(DF2_EUNSUPPORTED, "M too large");
    if (!hidden || !W_H || !out_H) return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(hidden) || !aligned16(W_H) || ((uintptr_t)out_H & 15u))
        return fail(DF2_EINVAL, "hidden, W_H and out_H must be 16-byte aligned");
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    pl.bf16 = dtype == DF2_BF16;
    plan_gate(pl, M, d, r, overrides());
    pl.p.C = 0;
    pl.p.K = 0;
    plan_layout(pl, 0, M, 0, false);
    Params& p = pl.p;
    p.rows = M;
    p.hidden = hidden;
    p.W = W_H;
    void* base = nullptr;
    df2_status st;
    if ((st = get_scratch(stream, pl.total_bytes, pl.counter_bytes, &base)) != DF2_OK) return st;
    note_layout(stream, pl.counter_bytes);
    bind_scratch(pl, base, 0, 0);
    p.H = out_H;
    return launch_checked([&] { launch_gate(pl, stream); }, "dflash2_project launch");
}

df2_status dflash2_pair_scores(const df2_dims* dims, const int32_t* cand_idx,
                               const float* cand_val, const float* H, const void* A_tab,
                               const void* B_tab, const int32_t* prev_tok, int32_t K,
                               float* out_S, hipStream_t stream) {
    g_last_error.clear();
    df2_status st = check_dims(dims, false);
    if (st != DF2_OK) return st;
    if ((st = check_k(K, dims->V)) != DF2_OK) return st;
    if (dims->B == 0) return DF2_OK;
    if (!cand_idx || !cand_val || !H || !A_tab || !B_tab || !prev_tok || !out_S)
        return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(H) || !aligned16(A_tab) || !aligned16(B_tab))
        return fail(DF2_EINVAL, "H, A_tab and B_tab must be 16-byte aligned");
    if ((int64_t)dims->B * dims->P > 0x7FFFFFFF) return fail(DF2_EUNSUPPORTED, "too many rows");
    void* base = nullptr;
    if ((st = get_scratch(stream, 256, 4, &base)) != DF2_OK) return st;
    PairArgs a;
    std::memset(&a, 0, sizeof(a));
    a.cand = cand_idx;
    a.cval = cand_val;
    a.H = H;
    a.A = A_tab;
    a.Bt = B_tab;
    a.prev = prev_tok;
    a.out_S = out_S;
    a.err = reinterpret_cast<uint32_t*>(base);
    a.B = dims->B;
    a.P = dims->P;
    a.V = dims->V;
    a.r = dims->r;
    a.K = K;
    dim3 grid((unsigned)((int64_t)dims->B * dims->P)), block(kWG);
    return launch_checked([&] {
        if (dims->dtype == DF2_BF16)
            hipLaunchKernelGGL((k_pairs<true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_pairs<false>), grid, block, 0, stream, a);
    }, "dflash2_pair_scores launch");
}

}  // extern "C"

namespace {

df2_status walk_common(const float* S, const int32_t* cand_idx, int32_t B, int32_t P, int32_t K,
                       int walk, const float* u, float inv_tau, int32_t* out_path, float* out_q,
                       float* out_score, hipStream_t stream) {
    if (B < 0) return fail(DF2_EINVAL, "B < 0");
    if (P < 1 || P > kMaxP) return fail(DF2_EINVAL, "P must be in [1, 64]");
    if (K < 1 || K > kMaxK) return fail(DF2_EINVAL, "K must be in [1, 64]");
    if (B == 0) return DF2_OK;
    if (!S || !cand_idx || !out_path || !out_score) return fail(DF2_EINVAL, "NULL pointer argument");
    if (((uintptr_t)S & 3u) || ((uintptr_t)cand_idx & 3u) || ((uintptr_t)out_path & 3u) ||
        ((uintptr_t)out_score & 3u))
        return fail(DF2_EINVAL, "arguments must be 4-byte aligned");
    WalkArgs a;
    a.S = S;
    a.cand = cand_idx;
    a.out_path = out_path;
    a.out_score = out_score;
    a.P = P;
    a.K = K;
    a.walk = walk;
    a.u = u;
    a.out_q = out_q;
    a.inv_tau = inv_tau;
    dim3 grid((unsigned)B), block(kWG);
    return launch_checked([&] { hipLaunchKernelGGL(k_walk, grid, block, 0, stream, a); },
                          "dflash2_walk launch");
}

}  // namespace

// The sampling walk's uniforms: a kernel family of its own (philox.hpp),
// launched only by dflash2_philox_uniforms below.
#include "philox.hpp"

extern "C" {

df2_status dflash2_walk(const float* S, const int32_t* cand_idx, int32_t B, int32_t P, int32_t K,
                        df2_walk walk, int32_t* out_path, float* out_score, hipStream_t stream) {
    g_last_error.clear();
    if (walk != DF2_WALK_VITERBI && walk != DF2_WALK_GREEDY)
        return fail(DF2_EINVAL, "unknown walk mode");
    return walk_common(S, cand_idx, B, P, K, (int)walk, nullptr, 0.f, out_path, nullptr, out_score,
                       stream);
}

df2_status dflash2_sample_walk(const float* S, const int32_t* cand_idx, const float* u, int32_t B,
                               int32_t P, int32_t K, float temperature, int32_t* out_path,
                               float* out_q, float* out_score, hipStream_t stream) {
    g_last_error.clear();
    float inv_tau = 0.f;
    df2_status st = sample_inv_tau(temperature, &inv_tau);
    if (st != DF2_OK) return st;
    if (B > 0) {
        if (!u || !out_q) return fail(DF2_EINVAL, "NULL pointer argument");
        if (((uintptr_t)u & 3u) || ((uintptr_t)out_q & 3u))
            return fail(DF2_EINVAL, "u and out_q must be 4-byte aligned");
    }
    return walk_common(S, cand_idx, B, P, K, kWalkSample, u, inv_tau, out_path, out_q, out_score,
                       stream);
}

namespace {

// Checks shared by both uniforms entry points; *grid receives the launch width.
df2_status philox_args(int64_t n, const float* out, unsigned* grid) {
    if (n < 0) return fail(DF2_EINVAL, "n < 0");
    if (n > ((int64_t)1 << 31)) return fail(DF2_EUNSUPPORTED, "n above 2^31");
    if (n == 0) return DF2_OK;
    if (!out) return fail(DF2_EINVAL, "NULL pointer argument");
    if ((uintptr_t)out & 3u) return fail(DF2_EINVAL, "out must be 4-byte aligned");
    // one thread per Philox block of four uniforms: at most 2^29 threads
    const int64_t blocks = (n + 3) / 4;
    *grid = (unsigned)((blocks + kPhiloxWG - 1) / kPhiloxWG);
    return DF2_OK;
}

}  // namespace

df2_status dflash2_philox_uniforms(uint64_t seed, uint64_t offset, int64_t n, float* out,
                                   hipStream_t stream) {
    g_last_error.clear();
    unsigned grid = 0;
    const df2_status st = philox_args(n, out, &grid);
    if (st != DF2_OK || n == 0) return st;
    const int vec = aligned16(out) ? 1 : 0;
    return launch_checked(
        [&] {
            hipLaunchKernelGGL(k_philox_uniforms, dim3(grid), dim3(kPhiloxWG), 0, stream, seed,
                               offset, (uint64_t*)nullptr, n, out, vec, 0);
        },
        "philox uniforms launch");
}

df2_status dflash2_philox_uniforms_next(uint64_t seed, uint64_t* offset, int64_t n, float* out,
                                        hipStream_t stream) {
    g_last_error.clear();
    unsigned grid = 0;
    const df2_status st = philox_args(n, out, &grid);
    if (st != DF2_OK || n == 0) return st;
    if (!offset) return fail(DF2_EINVAL, "NULL pointer argument");
    if ((uintptr_t)offset & 7u) return fail(DF2_EINVAL, "offset must be 8-byte aligned");
    const int vec = aligned16(out) ? 1 : 0;
    // one workgroup (n <= 1024) advances the offset itself after a barrier;
    // a wider grid leaves it to a one-thread launch behind it
    const int bump = grid == 1 ? 1 : 0;
    const df2_status s1 = launch_checked(
        [&] {
            hipLaunchKernelGGL(k_philox_uniforms, dim3(grid), dim3(kPhiloxWG), 0, stream, seed,
                               (uint64_t)0, offset, n, out, vec, bump);
        },
        "philox uniforms launch");
    if (s1 != DF2_OK || bump) return s1;
    return launch_checked(
        [&] { hipLaunchKernelGGL(k_philox_bump, dim3(1), dim3(64), 0, stream, offset); },
        "philox offset launch");
}

df2_status dflash2_viterbi(const float* S, const int32_t* cand_idx, int32_t B, int32_t P,
                           int32_t K, int32_t* out_path, float* out_score, hipStream_t stream) {
    return dflash2_walk(S, cand_idx, B, P, K, DF2_WALK_VITERBI, out_path, out_score, stream);
}

df2_status dflash2_conv2(const void* x, const void* x_prev, const void* base, const void* W_c,
                         int32_t B, int32_t P, int32_t d, df2_dtype dtype, void* out,
                         hipStream_t stream) {
    g_last_error.clear();
    if (dtype != DF2_F32 && dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (B < 0) return fail(DF2_EINVAL, "B < 0");
    if (P < 1) return fail(DF2_EINVAL, "P < 1");
    if (d < 512 || d % 512 != 0 || d > 8192)
        return fail(DF2_EUNSUPPORTED, "d must be a multiple of 512 in [512, 8192]");
    if (B == 0) return DF2_OK;
    const int64_t M = (int64_t)B * P;
    if (M > (1 << 24)) return fail(DF2_EUNSUPPORTED, "B * P too large");
    if (!x || !x_prev || !base || !W_c || !out) return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(x) || !aligned16(x_prev) || !aligned16(base) || !aligned16(W_c) || !aligned16(out))
        return fail(DF2_EINVAL, "x, x_prev, base, W_c and out must be 16-byte aligned");
    // the corrections [M, d/8] = x [M, d] times W_c^T on the gate's slices,
    // then the combine by the last slice of each tile, in one launch
    const int N = d / 8;
    Plan pl;
    std::memset(&pl.p, 0, sizeof(pl.p));
    pl.bf16 = dtype == DF2_BF16;
    const Overrides ov = overrides();
    plan_gate(pl, M, d, N, ov);
    {
        // fewer, longer slices than the selector's: the last slice of a tile
        // sums them all (measured best: 4 with 64-row tiles, B = 32,
        // d = 5120; with one 16-row tile as many as one round of loads per
        // slice allows, 10 at B = 1, d = 2560: 11.0 us against 13.0 with 4)
        const int KS = d / 32;
        const int s_def = pl.mb == 1 ? 16 : 4;
        int S = std::max(1, std::min(ov.conv_s > 0 ? ov.conv_s : s_def, KS / (kWaves * gate_kb(pl.bf16))));
        pl.p.S = S;
    }
    const int ntiles_total = pl.p.mtiles * pl.p.ntiles;
    const size_t counter_bytes = align_up(4 * (1 + (size_t)ntiles_total), 256);
    const size_t off_ppart = counter_bytes;
    const size_t total = align_up(off_ppart + (size_t)pl.p.S * M * N * 4, 256);
    void* sbase = nullptr;
    df2_status st;
    if ((st = get_scratch(stream, total, counter_bytes, &sbase)) != DF2_OK) return st;
    note_layout(stream, counter_bytes);
    char* c = reinterpret_cast<char*>(sbase);
    ConvArgs a;
    a.x = x;
    a.x_prev = x_prev;
    a.base = base;
    a.Wc = W_c;
    a.out = out;
    a.ppart = reinterpret_cast<float*>(c + off_ppart);
    a.tile_cnt = reinterpret_cast<uint32_t*>(c) + 1;    // word 0 is the error flag
    a.M = M;
    a.P = P;
    a.d = d;
    a.S = pl.p.S;
    a.ntiles = pl.p.ntiles;
    dim3 grid((unsigned)(ntiles_total * pl.p.S)), block(kWG);
    return launch_checked([&] {
        if (pl.bf16) {
            if (pl.mb == 1) hipLaunchKernelGGL((k_conv2<true, 1>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((k_conv2<true, 4>), grid, block, 0, stream, a);
        } else {
            if (pl.mb == 1) hipLaunchKernelGGL((k_conv2<false, 1>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((k_conv2<false, 4>), grid, block, 0, stream, a);
        }
    }, "dflash2_conv2 launch");
}

df2_status dflash2_device_error(hipStream_t stream, uint32_t* flags) {
    g_last_error.clear();
    if (!flags) return fail(DF2_EINVAL, "flags is NULL");
    *flags = 0;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    void* ptr = nullptr;
    void* sptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto is = g_static_scratch.find(dev);
        if (is != g_static_scratch.end()) sptr = is->second;
        auto it = g_scratch.find(std::make_pair(dev, stream));
        if (it != g_scratch.end()) ptr = it->second.ptr;
    }
    uint32_t sv = 0;
    if (sptr) {
        // flags of no-allocation calls on this device
        if ((e = hipMemcpy(&sv, sptr, 4, hipMemcpyDeviceToHost)) != hipSuccess)
            return hip_fail(e, "hipMemcpy flags");
        if (sv) {
            const uint32_t zero = 0;
            if ((e = hipMemcpy(sptr, &zero, 4, hipMemcpyHostToDevice)) != hipSuccess)
                return hip_fail(e, "hipMemcpy flags");
        }
    }
    if (!ptr) {
        *flags = sv;
        return DF2_OK;
    }
    uint32_t v = 0;
    if ((e = hipMemcpy(&v, ptr, 4, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy flags");
    if (v) {
        const uint32_t zero = 0;
        if ((e = hipMemcpy(ptr, &zero, 4, hipMemcpyHostToDevice)) != hipSuccess)
            return hip_fail(e, "hipMemcpy flags");
        // A raised flag may come from a launch that left arrival counters
        // behind (a gate wait that gave up): the next call on this stream
        // clears its whole counter prefix before it launches.
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_scratch.find(std::make_pair(dev, stream));
        if (it != g_scratch.end()) it->second.zeroed_counter_bytes = 0;
    }
    *flags = v | sv;
    return DF2_OK;
}

df2_status dflash2_plan_override(df2_plan_knob knob, int32_t value) {
    g_last_error.clear();
    if (value < 0) return fail(DF2_EINVAL, "override values are >= 0 (0 restores the automatic plan)");
    std::lock_guard<std::mutex> lock(g_mu);
    switch (knob) {
        case DF2_PLAN_SEGMENT_WGS: g_over.wgs = value; break;
        case DF2_PLAN_CHUNK_VECTORS:
            if (value != 0 && value != 1 && value != 2 && value != 4)
                return fail(DF2_EINVAL, "chunk vectors must be 0, 1, 2 or 4");
            g_over.nv = value;
            break;
        case DF2_PLAN_MERGE_WORDS: g_over.mwords = value; break;
        case DF2_PLAN_GATE_SLICES: g_over.gate_s = value; break;
        case DF2_PLAN_CONV_SLICES: g_over.conv_s = value; break;
        case DF2_PLAN_LAUNCHES:
            if (value > 4) return fail(DF2_EINVAL, "launches must be 0 to 4");
            g_over.launches = value;
            break;
        case DF2_PLAN_LM_RANGES:
            if (value > kLmMaxLists) return fail(DF2_EINVAL, "LM-head ranges must be in [0, 256]");
            g_over.lm_ranges = value;
            break;
        case DF2_PLAN_GATE_GIVEUP:
            if (value > 1) return fail(DF2_EINVAL, "gate give-up must be 0 or 1");
            g_over.gate_giveup = value;
            break;
        default: return fail(DF2_EINVAL, "unknown plan knob");
    }
    return DF2_OK;
}

df2_status dflash2_release(void) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lock(g_mu);
    df2_status st = DF2_OK;
    for (auto& kv : g_scratch) {
        if (!kv.second.ptr) continue;
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(kv.first.first);
        hipError_t e = hipFree(kv.second.ptr);
        (void)hipSetDevice(cur);
        if (e != hipSuccess) st = hip_fail(e, "hipFree");
    }
    g_scratch.clear();
    return st;
}

}  // extern "C"

// ----------------------------------------------------------------------------
// The drafter's LM head fused with top-K (k_lmhead, then k_lmhead_merge).
// ----------------------------------------------------------------------------
namespace {

constexpr int kLmTiles[] = {1, 2, 4, 8, 12, 14};   // m-blocks per tile with a kernel

struct LmPlan {
    int mb = 1, kmax = 16;
    int n_mt = 1, n_vr = 1, nblk = 1;
    size_t part_bytes = 0, merge_lds = 0;
};

// Tiles of up to 14 m-blocks (16 would spill registers; 8 for K > 32,
// whose lists take more LDS and registers), the smallest tile kernel that
// covers an even split of the rows; then enough vocabulary ranges to give
// every CU one workgroup.
LmPlan plan_lmhead(int64_t M, int V, int K, int cus, const Overrides& ov) {
    LmPlan pl;
    pl.kmax = K <= 16 ? 16 : (K <= 32 ? 32 : 64);
    const int maxmb = pl.kmax == 64 ? 8 : 14;
    const int64_t nbm = (M + 15) / 16;
    const int64_t nmt = (nbm + maxmb - 1) / maxmb;
    const int64_t want = (nbm + nmt - 1) / nmt;
    for (int t : kLmTiles)
        if (t <= maxmb && t >= want) {
            pl.mb = t;
            break;
        }
    pl.n_mt = (int)((nbm + pl.mb - 1) / pl.mb);
    pl.nblk = (V + 15) / 16;
    int nvr = ov.lm_ranges > 0 ? ov.lm_ranges : (int)std::max<int64_t>(1, cus / pl.n_mt);
    // a range spans fewer than 2^21 columns (its candidates encode the offset)
    const int min_vr = (int)(((int64_t)pl.nblk * 16 + kLmMaxRangeCols - 1) / kLmMaxRangeCols);
    nvr = std::max(nvr, min_vr);
    pl.n_vr = std::max(1, std::min(std::min(nvr, kLmMaxLists), pl.nblk));
    pl.part_bytes = (size_t)M * pl.n_vr * pl.kmax * sizeof(uint64_t);
    pl.merge_lds = (size_t)pl.n_vr * K * sizeof(uint64_t);
    return pl;
}

df2_status launch_lmhead(const LmPlan& pl, const LmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)pl.n_mt * pl.n_vr)), block(kWG);
#define DF2_LM(MB_, KM_)                                                                   \
    if (pl.mb == MB_ && pl.kmax == KM_) {                                                  \
        hipLaunchKernelGGL((k_lmhead<MB_, KM_>), grid, block, 0, stream, a);               \
        launched = true;                                                                   \
    }
    bool launched = false;
    DF2_LM(1, 16) DF2_LM(2, 16) DF2_LM(4, 16) DF2_LM(8, 16) DF2_LM(12, 16) DF2_LM(14, 16)
    DF2_LM(1, 32) DF2_LM(2, 32) DF2_LM(4, 32) DF2_LM(8, 32) DF2_LM(12, 32) DF2_LM(14, 32)
    DF2_LM(1, 64) DF2_LM(2, 64) DF2_LM(4, 64) DF2_LM(8, 64)
#undef DF2_LM
    if (!launched) return fail(DF2_EUNSUPPORTED, "no LM-head kernel for this tile");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "dflash2_lmhead_topk launch");
    const void* merge_fn = pl.kmax == 16 ? reinterpret_cast<const void*>(&k_lmhead_merge<16>)
                           : pl.kmax == 32 ? reinterpret_cast<const void*>(&k_lmhead_merge<32>)
                                           : reinterpret_cast<const void*>(&k_lmhead_merge<64>);
    if (pl.merge_lds > 65536) {
        static std::mutex mu;
        static std::map<const void*, hipError_t> done;
        std::lock_guard<std::mutex> lock(mu);
        auto it = done.find(merge_fn);
        if (it == done.end())
            it = done.emplace(merge_fn, hipFuncSetAttribute(merge_fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                            (int)(kLmMaxLists * 64 * sizeof(uint64_t))))
                     .first;
        if (it->second != hipSuccess) return hip_fail(it->second, "hipFuncSetAttribute (LM-head merge)");
    }
    if (pl.kmax == 16)
        hipLaunchKernelGGL(k_lmhead_merge<16>, dim3((unsigned)a.M), block, pl.merge_lds, stream, a);
    else if (pl.kmax == 32)
        hipLaunchKernelGGL(k_lmhead_merge<32>, dim3((unsigned)a.M), block, pl.merge_lds, stream, a);
    else
        hipLaunchKernelGGL(k_lmhead_merge<64>, dim3((unsigned)a.M), block, pl.merge_lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "dflash2_lmhead_topk merge launch");
    return DF2_OK;
}

}  // namespace

extern "C" {

df2_status dflash2_lmhead_topk(const void* hidden, const void* W_lm, int64_t M, int32_t V,
                               int32_t d, df2_dtype dtype, int32_t K, int32_t* out_idx,
                               float* out_val, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != DF2_F32 && dtype != DF2_BF16) return fail(DF2_EINVAL, "unknown dtype");
    if (dtype != DF2_BF16)
        return fail(DF2_EUNSUPPORTED, "the LM head takes bf16 hidden states and weights");
    if (M < 0) return fail(DF2_EINVAL, "M < 0");
    if (V < 1) return fail(DF2_EINVAL, "V < 1");
    df2_status st = check_k(K, V);
    if (st != DF2_OK) return st;
    if (d < 64 || d % 64 != 0 || d > 32768)
        return fail(DF2_EUNSUPPORTED, "d must be a multiple of 64 in [64, 32768]");
    if (M == 0) return DF2_OK;
    if (M > (1 << 24)) return fail(DF2_EUNSUPPORTED, "M too large (at most 2^24 rows)");
    if (V > (1 << 29)) return fail(DF2_EUNSUPPORTED, "V too large for the LM head (at most 2^29)");
    if (!hidden || !W_lm || !out_idx || !out_val) return fail(DF2_EINVAL, "NULL pointer argument");
    if (!aligned16(hidden) || !aligned16(W_lm))
        return fail(DF2_EINVAL, "hidden and W_lm must be 16-byte aligned");
    if (((uintptr_t)out_idx & 3u) || ((uintptr_t)out_val & 3u))
        return fail(DF2_EINVAL, "outputs must be 4-byte aligned");
    const LmPlan pl = plan_lmhead(M, V, K, cu_count(), overrides());
    // the first 256 bytes keep the device flag word; the lists follow
    void* base = nullptr;
    if ((st = get_scratch(stream, 256 + pl.part_bytes, 4, &base)) != DF2_OK) return st;
    note_layout(stream, 4);
    LmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.X = reinterpret_cast<const uint16_t*>(hidden);
    a.W = reinterpret_cast<const uint16_t*>(W_lm);
    a.part = reinterpret_cast<uint64_t*>(reinterpret_cast<unsigned char*>(base) + 256);
    a.out_idx = out_idx;
    a.out_val = out_val;
    a.M = M;
    a.V = V;
    a.d = d;
    a.K = K;
    a.kstride = pl.kmax;
    a.n_mt = pl.n_mt;
    a.n_vr = pl.n_vr;
    a.nblk = pl.nblk;
    return launch_lmhead(pl, a, stream);
}

}  // extern "C"
