// The walk over precomputed pair scores.
//
// "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path Selector":
// the only sequential work of the selector is one walk over the scores,
// starting from the last verified token.  The walk is read as a max-sum
// (Viterbi) pass with backtrack:
//     delta_0(j) = S_0(prev, j)
//     delta_t(j) = max_i delta_{t-1}(i) + S_t(i, j),  psi_t(j) = its argmax
// then the best final state and psi backwards.  Ties keep the smaller
// predecessor rank and the smaller final rank.  Sums are fp32.
//
// One wave walks; lane j owns candidate j and reads the whole previous delta
// from scalar registers (no LDS round trip per step).  Scores enter LDS
// transposed (column j contiguous, padded to Kp = K rounded up to 16, 32 or
// 64), a group of positions at a time.
//
// The same section also describes the walk literally as greedy (from the
// last verified token, each position takes the best successor of the token
// chosen one step earlier) and as sampling from the same scores.  chain_seq
// does both: every thread of the workgroup decides the successor of one
// (position, predecessor) row at once, and the chain through those choices
// is then a few register reads.
#pragma once

#include <math.h>

#include "common.hpp"
#include "pairs.hpp"

namespace df2 {

constexpr int kWalkS = 4096;        // floats of scores per group of positions
constexpr int kWalkIds = 1024;      // candidate ids kept in LDS (P * K at most)

struct WalkLds {
    float ST[kWalkS];               // [t][j][i] over Kp x Kp, zero padded
    uint8_t psi[kMaxP * kMaxK];     // Viterbi: [j][t], row j of kMaxP positions
    int32_t ids[kWalkIds];
    int32_t rank[kMaxP];
    union {
        float qpick[kMaxP];         // sampling walk: probability of each choice
        float dq[kMaxK];            // Viterbi, 16 < K <= 32: delta of the last step
    };
};

// The larger of two floats, as the plain instruction (fmaxf quiets each
// operand first; a NaN never decides a choice here).
__device__ __forceinline__ float walk_max(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Best of one lane's values v[0..16) (predecessors i0 .. i0 + 15): the
// largest value by a max tree, then its smallest index.
__device__ __forceinline__ void best_of16(const float (&v)[16], int i0, float& best, int& arg) {
    float m8[8], m4[4], m2[2];
#pragma unroll
    for (int u = 0; u < 8; ++u) m8[u] = walk_max(v[2 * u], v[2 * u + 1]);
#pragma unroll
    for (int u = 0; u < 4; ++u) m4[u] = walk_max(m8[2 * u], m8[2 * u + 1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) m2[u] = walk_max(m4[2 * u], m4[2 * u + 1]);
    best = walk_max(m2[0], m2[1]);
    arg = i0 + 15;
#pragma unroll
    for (int u = 14; u >= 0; --u) arg = (v[u] == best) ? i0 + u : arg;
}

// Wave 0: delta over positions [t0, t1) of a group held in sm.ST.  Lane j
// owns candidate j; delta_{t-1} reaches every lane through readlane (scalar
// registers), 16 predecessors at a time, and the column S_t(., j) comes from
// LDS with 16-byte reads.  Lanes j >= K carry -inf.
template <int KP>
__device__ float walk_steps(int t0, int t1, int K, float delta, WalkLds& sm) {
    const int lane = lane_id();
    const int j = lane % KP;
    const bool jv = lane < K;
    const uint32_t keep = jv ? ~0u : 0u;
    const uint32_t ninf = (uint32_t)__float_as_int(-INFINITY);
#pragma unroll 1
    for (int t = t0; t < t1; ++t) {
        const float* col = sm.ST + (t - t0) * KP * KP + j * KP;
        if (t == 0) {
            delta = jv ? col[0] : -INFINITY;
            continue;
        }
        float sv[KP];
#pragma unroll
        for (int q = 0; q < KP / 4; ++q) {
            const float4 x = *reinterpret_cast<const float4*>(col + 4 * q);
            sv[4 * q] = x.x;
            sv[4 * q + 1] = x.y;
            sv[4 * q + 2] = x.z;
            sv[4 * q + 3] = x.w;
        }
        float best = -INFINITY;
        int arg = 0;
#pragma unroll
        for (int c = 0; c < KP; c += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = sv[c + u] + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(delta), c + u));
            float cb;
            int ca;
            best_of16(v, c, cb, ca);
            if (c == 0 || cb > best) {
                best = cb;
                arg = ca;
            }
        }
        delta = __int_as_float((int)((__float_as_int(best) & keep) | (ninf & ~keep)));
        // arg < K for finite scores; the clamp keeps NaN inputs in bounds
        if (jv) sm.psi[j * kMaxP + t] = (uint8_t)min(arg, K - 1);
    }
    return delta;
}

// One quad_perm DPP move: lane l of each group of four takes lane sel[l].
template <int CTRL>
__device__ __forceinline__ uint32_t quad_mov(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;    // lanes 1, 0, 3, 2
constexpr int kQuadSwap2 = 0x4E;    // lanes 2, 3, 0, 1

// Wave 0, K <= 16: delta over positions [t0, t1) of a group held in sm.ST
// (Kp = 16), four lanes per candidate.  Lane 4 j + q takes predecessors
// 4 q .. 4 q + 3 of candidate j: delta_{t-1} of those four comes from the
// lanes that hold it (ds_bpermute from lanes 16 q + 4 k), the column piece
// S_t(4q .. 4q + 3, j) with one 16-byte LDS read one step ahead, and the
// quad combines its four partial results by DPP: the largest value, then
// the smallest predecessor that reaches it.  Lane 4 j writes psi_t(j).
// dl: delta(j) of the position before t0 in every lane of quad j (any value
// when t0 = 0); returns it for the group's last position.  Candidates j >= K
// hold -inf.
__device__ float walk_steps_quad(int t0, int t1, int K, float dl, WalkLds& sm) {
    const int lane = lane_id();
    const int j = lane >> 2, q = lane & 3;
    const bool jv = j < K;
    const float* col = sm.ST + j * 16 + 4 * q;
    const int src = 64 * q;                     // byte address of lane 16 q
    float4 s = *reinterpret_cast<const float4*>(col);
#pragma unroll 1
    for (int t = t0; t < t1; ++t) {
        if (t == 0) {
            // delta_0(j) = S_0(prev, j): row 0 of the first block
            dl = jv ? s.x : -INFINITY;
            s = *reinterpret_cast<const float4*>(col + min(1, t1 - 1 - t0) * 256);
            continue;
        }
        const int di = __float_as_int(dl);
        const float dx = __int_as_float(__builtin_amdgcn_ds_bpermute(src, di));
        const float dy = __int_as_float(__builtin_amdgcn_ds_bpermute(src + 16, di));
        const float dz = __int_as_float(__builtin_amdgcn_ds_bpermute(src + 32, di));
        const float dw = __int_as_float(__builtin_amdgcn_ds_bpermute(src + 48, di));
        const float4 sn = *reinterpret_cast<const float4*>(col + min(t + 1 - t0, t1 - 1 - t0) * 256);
        const float v0 = s.x + dx, v1 = s.y + dy, v2 = s.z + dz, v3 = s.w + dw;
        const float m = walk_max(walk_max(v0, v1), walk_max(v2, v3));
        int a = 3;
        a = (v2 == m) ? 2 : a;
        a = (v1 == m) ? 1 : a;
        a = (v0 == m) ? 0 : a;
        float mq = walk_max(m, __uint_as_float(quad_mov<kQuadSwap1>(__float_as_uint(m))));
        mq = walk_max(mq, __uint_as_float(quad_mov<kQuadSwap2>(__float_as_uint(mq))));
        uint32_t c = (m == mq) ? (uint32_t)(4 * q + a) : 255u;
        c = min(c, quad_mov<kQuadSwap1>(c));
        c = min(c, quad_mov<kQuadSwap2>(c));
        dl = jv ? mq : -INFINITY;
        // c < K for finite scores; the clamp keeps NaN inputs in bounds
        if (q == 0 && jv) sm.psi[j * kMaxP + t] = (uint8_t)min((int)c, K - 1);
        s = sn;
    }
    return dl;
}

// Wave 0, 16 < K <= 32: the same over a group with Kp = 32, two lanes per
// candidate.  Lane 2 j + h takes predecessors 16 h .. 16 h + 15 of candidate
// j: delta_{t-1} of those sixteen from sm.dq and the column piece S_t(16h ..
// 16h + 15, j), four 16-byte LDS reads each, issued together (lane 2 j
// writes delta_t(j) once the wave's reads of the step are issued, and LDS
// keeps one wave's accesses in order); the pair combines its two partial
// maxima by DPP.  Returns delta(j) in lane 2 j.
__device__ float walk_steps_pair(int t0, int t1, int K, float dl, WalkLds& sm) {
    const int lane = lane_id();
    const int j = lane >> 1, h = lane & 1;
    const bool jv = j < K;
    const float* col = sm.ST + j * 32 + 16 * h;
#pragma unroll 1
    for (int t = t0; t < t1; ++t) {
        const float* cp = col + (t - t0) * 1024;
        if (t == 0) {
            // delta_0(j) = S_0(prev, j): row 0 of the first block
            dl = jv ? cp[0] : -INFINITY;
            if (h == 0) sm.dq[j] = dl;
            continue;
        }
        float v[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 sv = *reinterpret_cast<const float4*>(cp + 4 * g);
            const float4 dv = *reinterpret_cast<const float4*>(sm.dq + 16 * h + 4 * g);
            v[4 * g] = sv.x + dv.x;
            v[4 * g + 1] = sv.y + dv.y;
            v[4 * g + 2] = sv.z + dv.z;
            v[4 * g + 3] = sv.w + dv.w;
        }
        float m;
        int a;
        best_of16(v, 16 * h, m, a);
        const float mq = walk_max(m, __uint_as_float(quad_mov<kQuadSwap1>(__float_as_uint(m))));
        uint32_t c = (m == mq) ? (uint32_t)a : 255u;
        c = min(c, quad_mov<kQuadSwap1>(c));
        dl = jv ? mq : -INFINITY;
        if (h == 0) {
            sm.dq[j] = dl;
            // c < K for finite scores; the clamp keeps NaN inputs in bounds
            if (jv) sm.psi[j * kMaxP + t] = (uint8_t)min((int)c, K - 1);
        }
    }
    return dl;
}

// Wave 0, after the steps: the final pick (smaller rank on ties) over the
// deltas -- candidate j in lane ls * j (ls = 4 or 2: candidates j >= K hold
// -inf already), or ls = 0: in lane j, candidates j >= K skipped -- then
// the backtrack through psi and the outputs.  ids_lds: the candidate ids
// are in sm.ids, else they are read from ids.
__device__ __forceinline__ void walk_finish(float delta, int ls, int P, int K, bool ids_lds,
                                            const int32_t* __restrict__ ids,
                                            int32_t* __restrict__ out_path,
                                            float* __restrict__ out_score, WalkLds& sm) {
    const int lane = lane_id();
    float m = -INFINITY;
    int jb = 0;
    if (ls > 0) {
        for (int c = 0; c < 64 / ls; c += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(delta), (c + u) * ls));
            float cb;
            int ca;
            best_of16(v, c, cb, ca);
            if (c == 0 || cb > m) {
                m = cb;
                jb = ca;
            }
        }
    } else {
        for (int c = 0; c < K; c += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = (c + u < K) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(delta), min(c + u, 63)))
                                   : -INFINITY;
            float cb;
            int ca;
            best_of16(v, c, cb, ca);
            if (c == 0 || cb > m) {
                m = cb;
                jb = ca;
            }
        }
    }
    // backtrack (jj is uniform): lane j holds psi_t(j) of sixteen positions
    // (one 16-byte read of its row), each step is one readlane, and lane t
    // keeps the rank chosen at position t (P <= 64)
    int jj = __builtin_amdgcn_readfirstlane(min(jb, K - 1));
    int rk = 0;
    for (int g = (P - 1) & ~15; g >= 0; g -= 16) {
        const uint4 pw = *reinterpret_cast<const uint4*>(sm.psi + lane * kMaxP + g);
#pragma unroll
        for (int u = 15; u >= 0; --u) {
            const int t = g + u;
            if (t > P - 1 || t < 1) continue;
            rk = (lane == t) ? jj : rk;
            const uint32_t wd = u < 4 ? pw.x : (u < 8 ? pw.y : (u < 12 ? pw.z : pw.w));
            jj = (int)((__builtin_amdgcn_readlane(wd, jj) >> (8 * (u & 3))) & 0xffu);
        }
    }
    rk = (lane == 0) ? jj : rk;
    if (lane == 0) *out_score = m;
    if (lane < P) out_path[lane] = ids_lds ? sm.ids[lane * K + rk] : xload(ids + (int64_t)lane * K + rk);
}

// The walk of one sequence.  S: [P, K, K] scores (row i = predecessor rank,
// column j = candidate rank; row 0 is used at t = 0), ids: [P, K] candidate
// ids; both read with xload.  Writes out_path[0 .. P) and *out_score.
// Every thread of the workgroup calls.  PAIR32: 16 < K <= 32 takes two lanes
// per candidate (a kernel of its own can afford the registers; inlined
// beside the pair job it spilled), else one.
template <bool PAIR32 = false>
__device__ __forceinline__ void walk_seq(const float* __restrict__ S, const int32_t* __restrict__ ids, int P,
                         int K, int32_t* __restrict__ out_path, float* __restrict__ out_score,
                         WalkLds& sm) {
    constexpr int U = 8;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int KP = K <= 16 ? 16 : (K <= 32 ? 32 : 64);
    const int KK = K * K, KP2 = KP * KP;
    const int G = kWalkS / KP2;
    const bool ids_lds = P * K <= kWalkIds;
    float delta = -INFINITY;
    for (int t0 = 0; t0 < P; t0 += G) {
        const int t1 = min(P, t0 + G);
        if (KP != K) {
            for (int x = tid; x < (t1 - t0) * KP2; x += kWG) sm.ST[x] = 0.f;
            __syncthreads();
        }
        // the group's scores, all loads of a thread issued before any is
        // stored
        const int nt = t1 - t0;
        for (int e = tid; e < KK; e += kWG) {
            const int i = e / K, j = e % K;
            const float* src = S + (int64_t)t0 * KK + e;
            float* dst = sm.ST + j * KP + i;
            for (int tb = 0; tb < nt; tb += U) {
                float v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = xload(src + (int64_t)min(tb + u, nt - 1) * KK);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (tb + u < nt) dst[(tb + u) * KP2] = v[u];
            }
        }
        __syncthreads();
        if (w == 0) {
            if (KP == 16) delta = walk_steps_quad(t0, t1, K, delta, sm);
            else if (KP == 32) delta = PAIR32 ? walk_steps_pair(t0, t1, K, delta, sm)
                                              : walk_steps<32>(t0, t1, K, delta, sm);
            else delta = walk_steps<64>(t0, t1, K, delta, sm);
        } else if (t0 == 0 && ids_lds) {
            // the other waves bring the candidate ids into LDS meanwhile, so
            // their round trip is off the walk's path
            constexpr int NW = kWG - 64;
            constexpr int QI = (kWalkIds + NW - 1) / NW;
            int32_t idv[QI];
#pragma unroll
            for (int q = 0; q < QI; ++q)
                idv[q] = q * NW + tid - 64 < P * K ? xload(ids + q * NW + tid - 64) : 0;
#pragma unroll
            for (int q = 0; q < QI; ++q)
                if (q * NW + tid - 64 < P * K) sm.ids[q * NW + tid - 64] = idv[q];
        }
        __syncthreads();
    }
    if (w != 0) return;
    walk_finish(delta, KP == 16 ? 4 : ((PAIR32 && KP == 32) ? 2 : 0), P, K, ids_lds, ids, out_path,
                out_score, sm);
}

// Walks whose choice at t depends only on the row of the token chosen at
// t - 1 ("chain" walks: greedy and sampling).  Each row (t, i) has its own
// successor nx(t, i), so all rows are decided at once and the walk is the
// chain j_t = nx(t, j_{t-1}) from row 0 at t = 0.
enum ChainRule { kChainGreedy = 0, kChainSample = 1 };

constexpr int kChainRows = kWalkS / 2;  // rows (t, i) decided per group of positions

// Greedy rule: the first maximiser of the row and its score.
__device__ __forceinline__ void row_best(const float* __restrict__ row, int K, int& arg, float& best) {
    best = -INFINITY;
    arg = 0;
    for (int c = 0; c < K; c += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = xload(row + min(c + u, K - 1));
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            // strictly greater: the lower rank keeps a tie
            if (c + u < K && (c + u == 0 || v[u] > best)) {
                best = v[u];
                arg = c + u;
            }
        }
    }
}

// Sampling rule (section "A Lightweight Path Selector": sampling draws from
// the same scores): e_j = exp((s_j - max s) / tau), z = e_0 + ... + e_{K-1}
// summed in rank order, and the draw is the first j whose running sum
// exceeds uu * z (the running sum ends exactly at z: the same additions of
// the same values in the same order); if rounding leaves none, the last j
// with e_j > 0.
// Outputs the rank, its score and its probability e_j / z.
__device__ __forceinline__ void row_draw(const float* __restrict__ row, int K, float uu, float inv_tau,
                                         int& arg, float& val, float& q) {
    int pick = -1, last = 0;
    float vp = 0.f, ep = 0.f, vl = 0.f, el = 0.f, z = 0.f;
    if (K <= 16) {
        float v[16], e[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = xload(row + min(u, K - 1));
        float m = v[0];
#pragma unroll
        for (int u = 1; u < 16; ++u) m = (u < K) ? fmaxf(m, v[u]) : m;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            e[u] = (u < K) ? expf((v[u] - m) * inv_tau) : 0.f;
            z += e[u];
        }
        const float target = uu * z;
        float c = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            c += e[u];
            if (e[u] > 0.f) {
                last = u;
                vl = v[u];
                el = e[u];
            }
            if (pick < 0 && target < c) {
                pick = u;
                vp = v[u];
                ep = e[u];
            }
        }
    } else {
        // three passes over the row, reloading 16 values at a time
        float m = -INFINITY;
        for (int c0 = 0; c0 < K; c0 += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = xload(row + min(c0 + u, K - 1));
#pragma unroll
            for (int u = 0; u < 16; ++u) m = (c0 + u < K) ? fmaxf(m, v[u]) : m;
        }
        for (int c0 = 0; c0 < K; c0 += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = xload(row + min(c0 + u, K - 1));
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (c0 + u < K) z += expf((v[u] - m) * inv_tau);
        }
        const float target = uu * z;
        float c = 0.f;
        for (int c0 = 0; c0 < K; c0 += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = xload(row + min(c0 + u, K - 1));
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (c0 + u < K) {
                    const float e = expf((v[u] - m) * inv_tau);
                    c += e;
                    if (e > 0.f) {
                        last = c0 + u;
                        vl = v[u];
                        el = e;
                    }
                    if (pick < 0 && target < c) {
                        pick = c0 + u;
                        vp = v[u];
                        ep = e;
                    }
                }
            }
        }
    }
    if (pick < 0) {
        pick = last;
        vp = vl;
        ep = el;
    }
    arg = pick;
    val = vp;
    q = ep / z;
}

// A chain walk of one sequence.  S: [P, K, K] scores (row 0 used at t = 0),
// ids: [P, K] candidate ids, both read with xload; u: [P] uniforms (sampling
// only; values outside [0, 1) are clamped into it, NaN to 0).  Writes
// out_path[0 .. P), *out_score (the chosen scores summed in order of t, fp32)
// and, when sampling, out_q[0 .. P) (each choice's probability).
// Step 1, every thread: for each row (t, i) it owns, nx(t, i), its score and
// (sampling) its probability go to LDS.  Step 2, wave 0: lane i holds them
// for eight positions at a time and the chain runs through readlane.
// Positions are taken in groups of kChainRows / K.  Every thread calls.
template <int RULE>
__device__ __forceinline__ void chain_seq(const float* __restrict__ S, const int32_t* __restrict__ ids,
                                          const float* __restrict__ u, float inv_tau, int P, int K,
                                          int32_t* __restrict__ out_path, float* __restrict__ out_q,
                                          float* __restrict__ out_score, WalkLds& sm) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int PK = P * K;
    const bool ids_lds = PK <= kWalkIds;
    constexpr int QI = kWalkIds / kWG;
    float* val = sm.ST;
    float* prob = sm.ST + kChainRows;
    const int GT = kChainRows / K;      // K <= 64, so at least 32 positions a group
    int j = 0;
    float score = 0.f;
    for (int t0 = 0; t0 < P; t0 += GT) {
        const int t1 = min(P, t0 + GT);
        const int n = (t1 - t0) * K;
        const bool load_ids = t0 == 0 && ids_lds;
        int32_t idv[QI];
#pragma unroll
        for (int q = 0; q < QI; ++q) idv[q] = load_ids ? xload(ids + min(q * kWG + tid, PK - 1)) : 0;
        for (int e = tid; e < n; e += kWG) {
            // row (t, i) = (t0 + e / K, e % K) starts at S + (t0 * K + e) * K
            const float* row = S + ((int64_t)t0 * K + e) * K;
            int arg;
            float best;
            if constexpr (RULE == kChainSample) {
                float uu = u[t0 + e / K];
                uu = (uu >= 0.f) ? fminf(uu, 0x1.fffffep-1f) : 0.f;
                float q;
                row_draw(row, K, uu, inv_tau, arg, best, q);
                prob[e] = q;
            } else {
                row_best(row, K, arg, best);
            }
            sm.psi[e] = (uint8_t)arg;
            val[e] = best;
        }
        if (load_ids) {
#pragma unroll
            for (int q = 0; q < QI; ++q)
                if (q * kWG + tid < PK) sm.ids[q * kWG + tid] = idv[q];
        }
        __syncthreads();
        if (w == 0) {
            // eight positions at a time: their LDS reads go out together, then
            // the chain runs through readlane (more at once costs registers)
            constexpr int G = 8;
            const int li = min(lane, K - 1);
#pragma unroll 1
            for (int ta = t0; ta < t1; ta += G) {
                int nx[G];
                float sv[G], qv[G];
#pragma unroll
                for (int x = 0; x < G; ++x) {
                    const int e = (min(ta + x, t1 - 1) - t0) * K + li;
                    nx[x] = sm.psi[e];
                    sv[x] = val[e];
                    qv[x] = (RULE == kChainSample) ? prob[e] : 0.f;
                }
#pragma unroll
                for (int x = 0; x < G; ++x) {
                    if (ta + x < t1) {
                        score += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv[x]), j));
                        if constexpr (RULE == kChainSample) {
                            const float qs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv[x]), j));
                            if (lane == 0) sm.qpick[ta + x] = qs;
                        }
                        j = __builtin_amdgcn_readlane(nx[x], j);
                        if (lane == 0) sm.rank[ta + x] = j;
                    }
                }
            }
        }
        __syncthreads();
    }
    if (w != 0) return;
    if (lane == 0) *out_score = score;
    for (int t = lane; t < P; t += 64) {
        const int rk = sm.rank[t];
        out_path[t] = ids_lds ? sm.ids[t * K + rk] : xload(ids + (int64_t)t * K + rk);
        if constexpr (RULE == kChainSample) out_q[t] = sm.qpick[t];
    }
}

}  // namespace df2
