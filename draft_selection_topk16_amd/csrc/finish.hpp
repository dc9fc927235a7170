// Per-sequence finish: row merges, pair scores and the walk, run by one
// workgroup.
//
// "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path Selector":
// the top-K candidates of every draft position are kept, every adjacent
// candidate pair is scored at once with
//     S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >,
// and the only sequential work is one walk over the precomputed scores,
// starting from the last verified token.  The walk is read as a max-sum
// (Viterbi) pass with backtrack.
//
// Positions are handled in groups of G, sized so that a group's candidate
// words, gate rows and scores fit the workgroup's LDS.  Per group:
//   1. the group's inputs land in LDS in one batch of loads (candidate
//      words of the segment lists, or a caller's candidates; gate rows);
//   2. each wave merges whole rows (wave_merge_lists);
//   3. each wave scores whole 16 x 16 tiles on the matrix cores, gathering
//      the embedding rows straight into operand registers, several k steps
//      in flight together;
//   4. wave 0 advances the walk by the group's positions.
// Scores: for position t the K x K block is G_t B_t^T + U, where
// G_t[i] = A(pred_i) (.) H_t (fp32) and B_t[j] = B(cand_j).  With bf16
// tables G is split into bf16 high and low parts (two products), which keeps
// about 16 significant bits of G; B is exact in bf16.  fp32 tables use the
// fp32 matrix instruction.  All sums accumulate in fp32.
// Walk: lane (g, j) of wave 0 holds delta[j] and scans predecessors
// i = g, g + NG, ...; the NG lane groups are combined with a butterfly.
// Ties keep the smaller predecessor rank and the smaller final rank.
#pragma once

#include <math.h>

#include "common.hpp"
#include "topk.hpp"

namespace df2 {

constexpr int kMaxP = 64;
constexpr int kMaxK = 64;
constexpr int kMaxR = 512;
constexpr int kFinS = 4096;           // floats of scores per group (G*K*K)
constexpr int kFinWords = kFinS / 2;  // candidate words per group (share the scores' space)
constexpr int kFinH = 1920;           // floats of gate rows per group (G*r)
constexpr int kFinCand = 512;         // candidate ids kept, a ring over positions
constexpr int kFinVal = 512;          // candidate values per group (G*K)

// 32 KB in all, so that five workgroups fit a CU's LDS.
struct FinLds {
    union {
        float S[kFinS];
        uint64_t words[kFinWords];
    };
    float H[kFinH];
    int32_t cand[kFinCand];
    union {
        float cval[kFinVal];
        int32_t rank[kMaxP];        // after the last group's walk
    };
    uint8_t psi[kMaxP * kMaxK];
};

// Everything one sequence's finish needs.
struct FinArgs {
    // candidate source: segment lists (fused) or a caller's candidates
    const uint64_t* part;   // [rows, nseg, K] words (fused)
    const int32_t* cand;    // [B, P, K] (scores stage)
    const float* cval;      // [B, P, K] (scores stage)
    const float* H;         // [B, P, r] gate rows
    const void* A;          // [V, r]
    const void* Bt;         // [V, r]
    const int32_t* prev;    // [B]
    const float* in_S;      // [B, P, K, K] (walk stage)
    const int32_t* in_cand; // [B, P, K] (walk stage: ids for the path)
    float* out_S;           // [B, P, K, K] (scores stage)
    int32_t* cand_out;      // [B, P, K] merged ids (fused; read back for long paths)
    float* cval_out;        // [B, P, K] merged values (fused)
    int32_t* out_path;      // [B, P]
    float* out_score;       // [B]
    uint32_t* err;          // device input-error flags
    int P, V, r, K, nseg;
};

enum { kFinFused = 0, kFinScores = 1, kFinWalk = 2 };

// Positions per group for the LDS budget.
template <int mode>
__device__ __forceinline__ int fin_group(const FinArgs& a) {
    const int K = a.K;
    int G = kFinS / (K * K);
    if constexpr (mode != kFinWalk) {
        G = min(G, kFinH / a.r);
        G = min(G, kFinVal / K);
        G = min(G, kFinCand / K - 1);
    }
    if constexpr (mode == kFinFused) G = min(G, kFinWords / (a.nseg * K));
    return max(1, min(G, a.P));
}

// Ring slot of position t's candidate ids.
__device__ __forceinline__ int fin_slot(int t, int K) { return t % (kFinCand / K); }

// Step 1 (fused): candidate words and gate rows of positions [t0, t1); all
// loads of a round are issued before any is used.
__device__ void fin_load_fused(const FinArgs& a, int b, int t0, int t1, FinLds& sm) {
    constexpr int U = 4;
    const int tid = threadIdx.x;
    const int K = a.K, r = a.r;
    const int nw = (t1 - t0) * a.nseg * K;
    const uint64_t* wsrc = a.part + ((int64_t)b * a.P + t0) * a.nseg * K;
    const int np = (t1 - t0) * r / 2;               // gate float pairs
    const uint64_t* hsrc = reinterpret_cast<const uint64_t*>(a.H + ((int64_t)b * a.P + t0) * r);
    for (int base = 0; base < max(nw, np); base += U * kWG) {
        uint64_t wv[U], hv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + u * kWG + tid;
            wv[u] = xload(wsrc + min(e, nw - 1));
            hv[u] = xload(hsrc + min(e, np - 1));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + u * kWG + tid;
            if (e < nw) sm.words[e] = wv[u];
            if (e < np) {
                sm.H[2 * e] = __uint_as_float((uint32_t)hv[u]);
                sm.H[2 * e + 1] = __uint_as_float((uint32_t)(hv[u] >> 32));
            }
        }
    }
}

// Step 2 (fused): each wave merges whole rows of the group.
template <bool BF16>
__device__ void fin_merge_rows(const FinArgs& a, int b, int t0, int t1, FinLds& sm) {
    const int lane = lane_id(), w = wave_id();
    const int K = a.K, nl = a.nseg;
    for (int tt = t0 + w; tt < t1; tt += kWaves) {
        uint64_t* lists = sm.words + (tt - t0) * nl * K;
        int32_t* cid = sm.cand + fin_slot(tt, K) * K;
        float* cv = sm.cval + (tt - t0) * K;
        const int64_t o = ((int64_t)b * a.P + tt) * K;
        // a row always has K real values (K <= V); the fill is a safe default
        if (lane < K) {
            cid[lane] = 0;
            cv[lane] = -INFINITY;
        }
        wave_sync();
        wave_merge_lists_emit(lists, nl, K, [&](int rank, uint64_t x) {
            const uint32_t key = (uint32_t)(x >> 32);
            const int32_t id = (int32_t)cand_index(x);
            const float v = BF16 ? value_of_key_bf16(key) : value_of_key_f32(key);
            cid[rank] = id;
            cv[rank] = v;
            xstore(a.cand_out + o + rank, id);
            xstore(a.cval_out + o + rank, v);
        });
    }
}

// Step 1 (scores stage): a caller's candidates and gate rows.  Ids outside
// [0, V) are replaced by token 0 and flagged (bit 1), so gathers stay in
// bounds.
__device__ void fin_load_given(const FinArgs& a, int b, int t0, int t1, FinLds& sm) {
    const int tid = threadIdx.x;
    const int K = a.K, r = a.r;
    const int nc = (t1 - t0) * K;
    for (int e = tid; e < nc; e += kWG) {
        const int tt = t0 + e / K, k = e % K;
        const int64_t o = ((int64_t)b * a.P + tt) * K + k;
        int32_t id = a.cand[o];
        if ((unsigned)id >= (unsigned)a.V) {
            atomicOr(a.err, 2u);
            id = 0;
        }
        sm.cand[fin_slot(tt, K) * K + k] = id;
        sm.cval[e] = a.cval[o];
    }
    // the predecessor row of the group's first position (needed by its tile)
    if (t0 > 0) {
        for (int k = tid; k < K; k += kWG) {
            int32_t id = a.cand[((int64_t)b * a.P + t0 - 1) * K + k];
            if ((unsigned)id >= (unsigned)a.V) {
                atomicOr(a.err, 2u);
                id = 0;
            }
            sm.cand[fin_slot(t0 - 1, K) * K + k] = id;
        }
    }
    const int nh = (t1 - t0) * r;
    const float* src = a.H + ((int64_t)b * a.P + t0) * r;
    for (int e = tid; e < nh; e += kWG) sm.H[e] = src[e];
}

// One 16 x 16 tile (rows ti, columns tj) of S_t into sm.S (group-relative).
template <bool BF16>
__device__ void fin_tile(const FinArgs& a, int t, int t0, int ti, int tj, int prev,
                         FinLds& sm) {
    const int lane = lane_id(), row = lane & 15, g = lane >> 4;
    const int K = a.K, r = a.r, nks = r / 32;
    const int i = ti * 16 + row, j = tj * 16 + row;
    const int ic = min(i, K - 1), jc = min(j, K - 1);
    const int atok = (t == 0) ? prev : sm.cand[fin_slot(t - 1, K) * K + ic];
    const int btok = sm.cand[fin_slot(t, K) * K + jc];
    const float* Hs = sm.H + (t - t0) * r;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
        constexpr int KB = 4;       // k steps per batch: 8 loads of 16 bytes in flight
        const uint16_t* Ar = reinterpret_cast<const uint16_t*>(a.A) + (int64_t)atok * r;
        const uint16_t* Br = reinterpret_cast<const uint16_t*>(a.Bt) + (int64_t)btok * r;
        for (int ks0 = 0; ks0 < nks; ks0 += KB) {
            u32x4_t av[KB], bv[KB];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int k0 = min(ks0 + q, nks - 1) * 32 + g * 8;
                av[q] = *reinterpret_cast<const u32x4_t*>(Ar + k0);
                bv[q] = *reinterpret_cast<const u32x4_t*>(Br + k0);
            }
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                // one k step at a time: keeps the gate reads from being
                // hoisted next to the gathers (registers)
                __builtin_amdgcn_sched_barrier(0);
                if (ks0 + q < nks) {
                    const int k0 = (ks0 + q) * 32 + g * 8;
                    const float4 h0 = *reinterpret_cast<const float4*>(Hs + k0);
                    const float4 h1 = *reinterpret_cast<const float4*>(Hs + k0 + 4);
                    const float gv[8] = {bf16_lo(av[q].x) * h0.x, bf16_hi(av[q].x) * h0.y,
                                         bf16_lo(av[q].y) * h0.z, bf16_hi(av[q].y) * h0.w,
                                         bf16_lo(av[q].z) * h1.x, bf16_hi(av[q].z) * h1.y,
                                         bf16_lo(av[q].w) * h1.z, bf16_hi(av[q].w) * h1.w};
                    bf16x8_t hi, lo;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const __bf16 hb = (__bf16)gv[e];
                        hi[e] = hb;
                        lo[e] = (__bf16)(gv[e] - (float)hb);
                    }
                    acc = mfma_bf16(hi, as_bf16x8(bv[q]), acc);
                    acc = mfma_bf16(lo, as_bf16x8(bv[q]), acc);
                }
            }
        }
    } else {
        constexpr int KB = 2;
        const float* Ar = reinterpret_cast<const float*>(a.A) + (int64_t)atok * r;
        const float* Br = reinterpret_cast<const float*>(a.Bt) + (int64_t)btok * r;
        for (int ks0 = 0; ks0 < nks; ks0 += KB) {
            float4 av[KB][2], bv[KB][2];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int k0 = min(ks0 + q, nks - 1) * 32 + g * 8;
                av[q][0] = *reinterpret_cast<const float4*>(Ar + k0);
                av[q][1] = *reinterpret_cast<const float4*>(Ar + k0 + 4);
                bv[q][0] = *reinterpret_cast<const float4*>(Br + k0);
                bv[q][1] = *reinterpret_cast<const float4*>(Br + k0 + 4);
            }
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                __builtin_amdgcn_sched_barrier(0);
                if (ks0 + q < nks) {
                    const int k0 = (ks0 + q) * 32 + g * 8;
                    const float4 h0 = *reinterpret_cast<const float4*>(Hs + k0);
                    const float4 h1 = *reinterpret_cast<const float4*>(Hs + k0 + 4);
                    const float gv[8] = {av[q][0].x * h0.x, av[q][0].y * h0.y, av[q][0].z * h0.z,
                                         av[q][0].w * h0.w, av[q][1].x * h1.x, av[q][1].y * h1.y,
                                         av[q][1].z * h1.z, av[q][1].w * h1.w};
                    const float bw[8] = {bv[q][0].x, bv[q][0].y, bv[q][0].z, bv[q][0].w,
                                         bv[q][1].x, bv[q][1].y, bv[q][1].z, bv[q][1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = mfma_f32(gv[e], bw[e], acc);
                }
            }
        }
    }
    const int KK = K * K;
    float* dst = sm.S + (t - t0) * KK;
    if (j < K) {
        const float u = sm.cval[(t - t0) * K + j];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int ii = ti * 16 + g * 4 + v;
            if (ii < K) dst[ii * K + j] = acc[v] + u;
        }
    }
}

// Step 3: every tile of positions [t0, t1), spread over the waves.  At
// t = 0 every row is the last verified token, so only tile row 0 is formed.
template <bool BF16>
__device__ void fin_scores(const FinArgs& a, int t0, int t1, int prev, FinLds& sm) {
    const int w = wave_id();
    const int nT = (a.K + 15) / 16;
    const int per = nT * nT;
    const int items = (t1 - t0) * per;
    for (int it = w; it < items; it += kWaves) {
        const int tt = t0 + it / per, rem = it % per;
        const int ti = rem / nT, tj = rem % nT;
        if (tt == 0 && ti > 0) continue;
        fin_tile<BF16>(a, tt, t0, ti, tj, prev, sm);
    }
}

// Step 4 (wave 0): delta over positions [t0, t1).  Lane (g, j): j = lane %
// (64 / NG) is the candidate, g the predecessor phase; predecessors are read
// four at a time (indexes clamped into range) before any is compared.
template <int NG>
__device__ float fin_walk_ng(const FinArgs& a, int t0, int t1, float delta, FinLds& sm) {
    constexpr int W = 64 / NG;
    const int lane = lane_id();
    const int K = a.K, KK = K * K;
    const int j = lane % W, g = lane / W;
    const bool jv = j < K;
    const int jc = min(j, K - 1);
    for (int t = t0; t < t1; ++t) {
        const float* St = sm.S + (t - t0) * KK;
        if (t == 0) {
            delta = jv ? St[jc] : -INFINITY;
            continue;
        }
        // predecessors i = g, g + NG, ...: the first one seeds the max
        float best = -INFINITY;
        int arg = g;
        for (int q0 = 0; q0 * NG < K; q0 += 4) {
            float dv[4], sv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ic = min(g + NG * (q0 + u), K - 1);
                if constexpr (NG == 1)
                    dv[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(delta), ic));
                else
                    dv[u] = __shfl(delta, ic);
                sv[u] = St[ic * K + jc];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = g + NG * (q0 + u);
                const float v = dv[u] + sv[u];
                if (i < K && (i == g || v > best)) {
                    best = v;
                    arg = i;
                }
            }
        }
        // combine the NG phases: larger value, then smaller predecessor
#pragma unroll
        for (int o = W; o < 64; o <<= 1) {
            const float ob = __shfl_xor(best, o);
            const int oa = __shfl_xor(arg, o);
            if (ob > best || (ob == best && oa < arg)) {
                best = ob;
                arg = oa;
            }
        }
        delta = jv ? best : -INFINITY;
        if (g == 0 && jv) sm.psi[t * K + j] = (uint8_t)arg;
    }
    return delta;
}

__device__ float fin_walk(const FinArgs& a, int t0, int t1, float delta, FinLds& sm) {
    if (a.K <= 16) return fin_walk_ng<4>(a, t0, t1, delta, sm);
    if (a.K <= 32) return fin_walk_ng<2>(a, t0, t1, delta, sm);
    return fin_walk_ng<1>(a, t0, t1, delta, sm);
}

// Final pick, backtrack and outputs (wave 0).  ids: position t's candidate
// ids come from the LDS ring while every position is still held there,
// else from ids_global ([B, P, K], drained before the call).
__device__ void fin_backtrack(const FinArgs& a, int b, float delta, const int32_t* ids_global,
                              FinLds& sm) {
    const int lane = lane_id();
    const int K = a.K, P = a.P;
    const int W = 64 / ((K <= 16) ? 4 : (K <= 32 ? 2 : 1));
    const bool mine = lane < W && lane < K;     // phase-0 lanes hold delta[j]
    const float m = wave_max_f32(mine ? delta : -INFINITY);
    const uint64_t mask = __ballot(mine && delta == m);
    const int jb = mask ? (__ffsll((unsigned long long)mask) - 1) : 0;
    if (lane == 0) {
        int jj = jb;
        for (int t = P - 1; t >= 0; --t) {
            sm.rank[t] = jj;
            if (t > 0) jj = sm.psi[t * K + jj];
        }
        a.out_score[b] = m;
    }
    wave_sync();
    for (int t = lane; t < P; t += 64) {
        const int rk = sm.rank[t];
        int32_t id;
        if (ids_global)
            id = xload(ids_global + ((int64_t)b * P + t) * K + rk);
        else
            id = sm.cand[fin_slot(t, K) * K + rk];
        a.out_path[(int64_t)b * P + t] = id;
    }
}

// The whole finish of sequence b.  Every thread of the workgroup calls it.
template <bool BF16, int mode>
__device__ void finish_seq(const FinArgs& a, int b, FinLds& sm) {
    const int tid = threadIdx.x, w = wave_id();
    const int K = a.K, P = a.P, KK = K * K;
    const int G = fin_group<mode>(a);
    // The finish is on the critical path; streaming waves that share the
    // SIMDs are mostly waiting on memory.
    __builtin_amdgcn_s_setprio(3);
    int prev = 0;
    if constexpr (mode != kFinWalk) {
        prev = a.prev[b];
        if (prev < 0 || prev >= a.V) {
            if (tid == 0) atomicOr(a.err, 1u);
            prev = 0;
        }
    }
    float delta = -INFINITY;
    for (int t0 = 0; t0 < P; t0 += G) {
        const int t1 = min(P, t0 + G);
        if constexpr (mode == kFinWalk) {
            for (int x = tid; x < (t1 - t0) * KK; x += kWG) {
                const int tt = t0 + x / KK;
                sm.S[x] = a.in_S[((int64_t)b * P + tt) * KK + x % KK];
            }
        } else if constexpr (mode == kFinFused) {
            fin_load_fused(a, b, t0, t1, sm);
            __syncthreads();
            fin_merge_rows<BF16>(a, b, t0, t1, sm);
        } else {
            fin_load_given(a, b, t0, t1, sm);
        }
        __syncthreads();
        if constexpr (mode != kFinWalk) {
            fin_scores<BF16>(a, t0, t1, prev, sm);
            __syncthreads();
        }
        if constexpr (mode == kFinScores) {
            for (int x = tid; x < (t1 - t0) * KK; x += kWG) {
                const int tt = t0 + x / KK, rem = x % KK;
                const int src = (tt == 0) ? (rem % K) : rem;   // t = 0: row 0 for every i
                a.out_S[((int64_t)b * P + tt) * KK + rem] = sm.S[(tt - t0) * KK + src];
            }
        } else if (w == 0) {
            delta = fin_walk(a, t0, t1, delta, sm);
        }
        __syncthreads();
    }
    if constexpr (mode == kFinScores) return;
    const int32_t* ids = nullptr;
    if constexpr (mode == kFinWalk) {
        ids = a.in_cand;
    } else if (P > kFinCand / K) {
        // the early positions' ids have left the ring: read them back from
        // the copy every wave stored
        drain_stores();
        __syncthreads();
        ids = a.cand_out;
    }
    if (w == 0) fin_backtrack(a, b, delta, ids, sm);
}

}  // namespace df2
