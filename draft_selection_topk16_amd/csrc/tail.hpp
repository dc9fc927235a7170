// Pair scores and the walk, one workgroup per sequence.
//
// "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path Selector":
// every adjacent candidate pair is scored at once with
//     S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >,
// and the only sequential work is one walk over the precomputed scores,
// starting from the last verified token.  The walk is read as a max-sum
// (Viterbi) pass with backtrack.
//
// Scores: for position t the K x K block is the product G_t B_t^T plus U,
// where G_t[i] = A(pred_i) (.) H_t (fp32) and B_t[j] = B(cand_j).  One wave
// forms a 16 x 16 tile on the matrix cores, gathering the 512-byte embedding
// rows straight into operand registers.  With bf16 tables G is split into
// bf16 high and low parts (two products), which keeps about 16 significant
// bits of G; B is exact in bf16.  fp32 tables use the fp32 matrix
// instruction.  All sums accumulate in fp32.
//
// Walk: wave 0, lane j holds delta_t[j]; backpointers go to LDS as bytes.
// Ties keep the smaller predecessor rank and the smaller final rank.
#pragma once

#include <math.h>

#include "common.hpp"

namespace df2 {

constexpr int kTailFloats = 4096;   // scores of a group of positions in LDS
constexpr int kMaxP = 64;
constexpr int kMaxK = 64;
constexpr int kMaxR = 512;

struct TailLds {
    float S[kTailFloats];
    float Hw[kWaves][kMaxR];        // each wave's copy of the gate row it scores
    uint8_t psi[kMaxP * kMaxK];
    int32_t rank[kMaxP];
};

struct TailArgs {
    const int32_t* cand;    // [B, P, K]
    const float* cval;      // [B, P, K]
    const float* H;         // [B, P, r]
    const void* A;          // [V, r]
    const void* Bt;         // [V, r]
    const int32_t* prev;    // [B]
    const float* in_S;      // [B, P, K, K] (walk-only mode)
    float* out_S;           // [B, P, K, K] (scores-only mode)
    int32_t* out_path;      // [B, P]
    float* out_score;       // [B]
    uint32_t* err;          // device input-error flags
    int P, V, r, K;
};

enum { kTailFull = 0, kTailScoresOnly = 1, kTailWalkOnly = 2 };

// One 16 x 16 tile (rows ti, columns tj) of S_t, computed by the calling wave
// and stored to dst[i * K + j] (i, j < K).  Hs: this wave's LDS copy of H_t.
template <bool BF16>
__device__ void pair_tile(const TailArgs& a, int b, int t, int ti, int tj, int prev,
                          const float* __restrict__ Hs, float* __restrict__ dst) {
    const int lane = lane_id(), row = lane & 15, g = lane >> 4;
    const int K = a.K, r = a.r, nks = r / 32;
    const int i = ti * 16 + row, j = tj * 16 + row;
    const int ic = min(i, K - 1), jc = min(j, K - 1);
    const int64_t rt = (int64_t)b * a.P + t;
    int atok = (t == 0) ? prev : xload(a.cand + (rt - 1) * K + ic);
    int ctok = xload(a.cand + rt * K + jc);
    const float u = xload(a.cval + rt * K + jc);
    // Ids outside [0, V) (possible only from a caller's own candidate list)
    // are replaced by token 0 and flagged, so the gathers stay in bounds.
    if ((unsigned)atok >= (unsigned)a.V || (unsigned)ctok >= (unsigned)a.V) {
        atomicOr(a.err, 2u);
        atok = ((unsigned)atok >= (unsigned)a.V) ? 0 : atok;
        ctok = ((unsigned)ctok >= (unsigned)a.V) ? 0 : ctok;
    }
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // k steps in batches of four: all row loads of a batch are in flight
    // together.
    if constexpr (BF16) {
        const uint16_t* Ar = reinterpret_cast<const uint16_t*>(a.A) + (int64_t)atok * r;
        const uint16_t* Br = reinterpret_cast<const uint16_t*>(a.Bt) + (int64_t)ctok * r;
        for (int ks0 = 0; ks0 < nks; ks0 += 4) {
            u32x4_t av[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k0 = (ks0 + q) * 32 + g * 8;
                if (ks0 + q < nks) {
                    av[q] = *reinterpret_cast<const u32x4_t*>(Ar + k0);
                    bv[q] = *reinterpret_cast<const u32x4_t*>(Br + k0);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (ks0 + q >= nks) break;
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
    } else {
        const float* Ar = reinterpret_cast<const float*>(a.A) + (int64_t)atok * r;
        const float* Br = reinterpret_cast<const float*>(a.Bt) + (int64_t)ctok * r;
        for (int ks0 = 0; ks0 < nks; ks0 += 2) {
            float4 av[2][2], bv[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int k0 = (ks0 + q) * 32 + g * 8;
                if (ks0 + q < nks) {
                    av[q][0] = *reinterpret_cast<const float4*>(Ar + k0);
                    av[q][1] = *reinterpret_cast<const float4*>(Ar + k0 + 4);
                    bv[q][0] = *reinterpret_cast<const float4*>(Br + k0);
                    bv[q][1] = *reinterpret_cast<const float4*>(Br + k0 + 4);
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (ks0 + q >= nks) break;
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
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int ii = ti * 16 + g * 4 + v;
        if (ii < K && j < K) dst[ii * K + j] = acc[v] + u;
    }
}

// Scores and/or walk for sequence b.  Every thread of the workgroup calls it.
template <bool BF16>
__device__ void tail_seq(const TailArgs& a, int b, int mode, TailLds& sm) {
    const int K = a.K, P = a.P, r = a.r;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nT = (K + 15) / 16;
    const int KK = K * K;
    const int G = max(1, min(P, kTailFloats / KK));
    int prev = 0;
    if (mode != kTailWalkOnly) {
        prev = a.prev[b];
        if (prev < 0 || prev >= a.V) {
            if (tid == 0) atomicOr(a.err, 1u);
            prev = 0;
        }
    }
    float delta = -INFINITY;
    int hw_t = -1;                       // position whose H row this wave holds
    for (int t0 = 0; t0 < P; t0 += G) {
        const int t1 = min(P, t0 + G);
        if (mode == kTailWalkOnly) {
            for (int x = tid; x < (t1 - t0) * KK; x += kWG) {
                const int tt = t0 + x / KK, rem = x % KK;
                const int i = (tt == 0) ? 0 : rem / K, j = rem % K;
                sm.S[x] = xload(a.in_S + (((int64_t)b * P + tt) * K + i) * K + j);
            }
        } else {
            const int items = (t1 - t0) * nT * nT;
            for (int it = w; it < items; it += kWaves) {
                const int tt = t0 + it / (nT * nT), rem = it % (nT * nT);
                const int ti = rem / nT, tj = rem % nT;
                if (tt == 0 && ti > 0) continue;   // at t = 0 every row is row 0
                if (hw_t != tt) {                  // stage H_t in this wave's LDS row
                    const uint64_t* Hr =
                        reinterpret_cast<const uint64_t*>(a.H + ((int64_t)b * P + tt) * r);
                    for (int q = lane; q < r / 2; q += 64) {
                        const uint64_t v = xload(Hr + q);
                        sm.Hw[w][2 * q] = __uint_as_float((uint32_t)v);
                        sm.Hw[w][2 * q + 1] = __uint_as_float((uint32_t)(v >> 32));
                    }
                    wave_sync();
                    hw_t = tt;
                }
                pair_tile<BF16>(a, b, tt, ti, tj, prev, sm.Hw[w], sm.S + (tt - t0) * KK);
            }
        }
        __syncthreads();
        if (mode == kTailScoresOnly) {
            for (int x = tid; x < (t1 - t0) * KK; x += kWG) {
                const int tt = t0 + x / KK, rem = x % KK;
                const int src = (tt == 0) ? (rem % K) : rem;
                a.out_S[((int64_t)b * P + tt) * KK + rem] = sm.S[(tt - t0) * KK + src];
            }
        } else if (w == 0) {
            for (int t = t0; t < t1; ++t) {
                const float* St = sm.S + (t - t0) * KK;
                if (t == 0) {
                    delta = (lane < K) ? St[lane] : -INFINITY;
                    continue;
                }
                // delta_{t-1}[i] is broadcast from lane i with readlane; the
                // column S_t[., lane] is read from LDS 16 rows at a time.
                float best = -INFINITY;
                int arg = 0;
                for (int i0 = 0; i0 < K; i0 += 16) {
                    float sv[16];
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        sv[q] = (i0 + q < K && lane < K) ? St[(i0 + q) * K + lane] : 0.f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        if (i0 + q < K) {
                            const float di = __int_as_float(
                                __builtin_amdgcn_readlane(__float_as_int(delta), i0 + q));
                            const float v = di + sv[q];
                            if (v > best) {
                                best = v;
                                arg = i0 + q;
                            }
                        }
                    }
                }
                delta = (lane < K) ? best : -INFINITY;
                if (lane < K) sm.psi[t * K + lane] = (uint8_t)arg;
            }
        }
        __syncthreads();
    }
    if (mode != kTailScoresOnly && w == 0) {
        const float m = wave_max_f32(delta);
        const uint64_t mask = __ballot(lane < K && delta == m);
        const int jb = mask ? (__ffsll((unsigned long long)mask) - 1) : 0;
        if (lane == 0) {
            int j = jb;
            for (int t = P - 1; t >= 0; --t) {
                sm.rank[t] = j;
                if (t > 0) j = sm.psi[t * K + j];
            }
            a.out_score[b] = m;
        }
        wave_sync();
        if (lane < P) {
            const int64_t rt = (int64_t)b * P + lane;
            a.out_path[rt] = xload(a.cand + rt * K + sm.rank[lane]);
        }
    }
}

}  // namespace df2
