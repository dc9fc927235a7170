// Pair scores of adjacent draft positions.
//
// "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path Selector":
// every adjacent candidate pair is scored at once with
//     S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >.
// For position t the K x K block is G_t B_t^T + U_t, where
// G_t[i] = A(pred_i) (.) H_t (fp32), pred_i is the i-th candidate of position
// t - 1 (the last verified token at t = 0, for every i) and B_t[j] = B(cand_j).
// With bf16 tables G is split into bf16 high and low parts (two products),
// which keeps about 16 significant bits of G; B is exact in bf16.  fp32
// tables use the fp32 matrix instruction.  All sums accumulate in fp32.
//
// One workgroup scores one or two consecutive positions.  The 16 x 16 tiles
// are taken a batch at a time; inside a batch the four waves split the k
// steps (wave w takes adjacent steps 2w, 2w + 1, then 2w + 8, ...: adjacent
// steps of an embedding row share cache lines), each wave gathers its embedding
// slices straight into operand registers with all loads of the batch in
// flight, and the four partial tiles are summed in LDS in wave order.
#pragma once

#include <math.h>

#include "common.hpp"
#include "gate.hpp"

namespace df2 {

constexpr int kMaxP = 64;
constexpr int kMaxK = 64;
constexpr int kMaxR = 512;

struct PairLds {
    float H[2][kMaxR];              // gate rows of the positions
    int32_t ids[3][kMaxK];          // predecessors of the first position, then each position's candidates
    float u[2][kMaxK];              // the positions' candidate logits
    float part[kWaves][2][256];     // per-wave partial tiles of a batch
};

// Tiles of one position: 16 x 16 blocks (ti, tj); at t = 0 every predecessor
// row is the same token, so only ti = 0 is formed.
__device__ __forceinline__ int pair_ntiles(int e, int nT) { return (e == 0 ? 1 : nT) * nT; }

// Scores of positions e0 .. e0 + ne - 1 (ne <= 2) from sm.ids, sm.u and sm.H
// (which load_h fills; it is called once, by every thread, after the first
// batch's gathers are issued, and is followed by a barrier).  S_e goes to
// dst + (e - e0) * K * K, row i = predecessor rank, column j = candidate
// rank; at e == 0 every row holds the same values.  Every thread calls.
template <bool BF16, typename LoadH>
__device__ void pair_tiles(const void* __restrict__ A, const void* __restrict__ Bt, int K, int r,
                           int e0, int ne, float* __restrict__ dst, PairLds& sm,
                           LoadH&& load_h) {
    constexpr int TB = BF16 ? 2 : 1;        // tiles per batch
    constexpr int KSW = 2;                  // k steps per wave per round
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = lane & 15, g = lane >> 4;
    const int nT = (K + 15) / 16, nks = r / 32;
    const int n0 = pair_ntiles(e0, nT);
    const int ntot = n0 + (ne > 1 ? pair_ntiles(e0 + 1, nT) : 0);
    bool h_loaded = false;
    for (int t0 = 0; t0 < ntot; t0 += TB) {
        int tq[TB], tti[TB], ttj[TB], atok[TB], btok[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            int ix = min(t0 + tb, ntot - 1);
            const int q = ix < n0 ? 0 : 1;
            ix -= q ? n0 : 0;
            tq[tb] = q;
            tti[tb] = ix / nT;
            ttj[tb] = ix % nT;
            atok[tb] = sm.ids[q][min(tti[tb] * 16 + row, K - 1)];
            btok[tb] = sm.ids[q + 1][min(ttj[tb] * 16 + row, K - 1)];
        }
        f32x4_t acc[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int kr = KSW * w; kr < nks || !h_loaded; kr += kWaves * KSW) {
            if constexpr (BF16) {
                const uint16_t* A16 = reinterpret_cast<const uint16_t*>(A);
                const uint16_t* B16 = reinterpret_cast<const uint16_t*>(Bt);
                u32x4_t av[TB][KSW], bv[TB][KSW];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int q = 0; q < KSW; ++q) {
                        const int ks = min(kr + q, nks - 1);
                        const int k0 = ks * 32 + g * 8;
                        av[tb][q] = *reinterpret_cast<const u32x4_t*>(A16 + (int64_t)atok[tb] * r + k0);
                        bv[tb][q] = *reinterpret_cast<const u32x4_t*>(B16 + (int64_t)btok[tb] * r + k0);
                    }
                if (!h_loaded) {
                    load_h();
                    __syncthreads();
                    h_loaded = true;
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    if (t0 + tb >= ntot) continue;
                    const float* Hs = sm.H[tq[tb]];
#pragma unroll
                    for (int q = 0; q < KSW; ++q) {
                        const int ks = kr + q;
                        if (ks >= nks) continue;
                        const int k0 = ks * 32 + g * 8;
                        const float4 h0 = *reinterpret_cast<const float4*>(Hs + k0);
                        const float4 h1 = *reinterpret_cast<const float4*>(Hs + k0 + 4);
                        const u32x4_t a = av[tb][q];
                        const float gv[8] = {bf16_lo(a.x) * h0.x, bf16_hi(a.x) * h0.y,
                                             bf16_lo(a.y) * h0.z, bf16_hi(a.y) * h0.w,
                                             bf16_lo(a.z) * h1.x, bf16_hi(a.z) * h1.y,
                                             bf16_lo(a.w) * h1.z, bf16_hi(a.w) * h1.w};
                        bf16x8_t hi, lo;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const __bf16 hb = (__bf16)gv[e];
                            hi[e] = hb;
                            lo[e] = (__bf16)(gv[e] - (float)hb);
                        }
                        acc[tb] = mfma_bf16(hi, as_bf16x8(bv[tb][q]), acc[tb]);
                        acc[tb] = mfma_bf16(lo, as_bf16x8(bv[tb][q]), acc[tb]);
                    }
                }
            } else {
                const float* A32 = reinterpret_cast<const float*>(A);
                const float* B32 = reinterpret_cast<const float*>(Bt);
                float4 av[KSW][2], bv[KSW][2];
#pragma unroll
                for (int q = 0; q < KSW; ++q) {
                    const int ks = min(kr + q, nks - 1);
                    const int k0 = ks * 32 + g * 8;
                    const float* ap = A32 + (int64_t)atok[0] * r + k0;
                    const float* bp = B32 + (int64_t)btok[0] * r + k0;
                    av[q][0] = *reinterpret_cast<const float4*>(ap);
                    av[q][1] = *reinterpret_cast<const float4*>(ap + 4);
                    bv[q][0] = *reinterpret_cast<const float4*>(bp);
                    bv[q][1] = *reinterpret_cast<const float4*>(bp + 4);
                }
                if (!h_loaded) {
                    load_h();
                    __syncthreads();
                    h_loaded = true;
                }
                const float* Hs = sm.H[tq[0]];
#pragma unroll
                for (int q = 0; q < KSW; ++q) {
                    const int ks = kr + q;
                    if (ks >= nks) continue;
                    const int k0 = ks * 32 + g * 8;
                    const float4 h0 = *reinterpret_cast<const float4*>(Hs + k0);
                    const float4 h1 = *reinterpret_cast<const float4*>(Hs + k0 + 4);
                    const float gv[8] = {av[q][0].x * h0.x, av[q][0].y * h0.y, av[q][0].z * h0.z,
                                         av[q][0].w * h0.w, av[q][1].x * h1.x, av[q][1].y * h1.y,
                                         av[q][1].z * h1.z, av[q][1].w * h1.w};
                    const float bw[8] = {bv[q][0].x, bv[q][0].y, bv[q][0].z, bv[q][0].w,
                                         bv[q][1].x, bv[q][1].y, bv[q][1].z, bv[q][1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[0] = mfma_f32(gv[e], bw[e], acc[0]);
                }
            }
            if (kr >= nks) break;           // a wave with no k steps only joined the H load
        }
        // Sum the four waves' partial tiles in wave order, add U, store.
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.part[w][tb][v * 64 + lane] = acc[tb][v];
        __syncthreads();
        for (int x = tid; x < TB * 256; x += kWG) {
            const int tb = x >> 8, v = (x >> 6) & 3, l = x & 63;
            if (t0 + tb < ntot) {
                const float sum = sm.part[0][tb][x & 255] + sm.part[1][tb][x & 255] +
                                  sm.part[2][tb][x & 255] + sm.part[3][tb][x & 255];
                const int q = tb == 0 ? tq[0] : tq[TB - 1];
                const int ti = tb == 0 ? tti[0] : tti[TB - 1];
                const int tj = tb == 0 ? ttj[0] : ttj[TB - 1];
                const int rr = 4 * (l >> 4) + v, j = tj * 16 + (l & 15);
                if (j < K) {
                    const float val = sum + sm.u[q][j];
                    float* out = dst + (int64_t)q * K * K;
                    if (e0 + q == 0) {
                        for (int i = rr; i < K; i += 16) xstore(out + (int64_t)i * K + j, val);
                    } else {
                        const int i = ti * 16 + rr;
                        if (i < K) xstore(out + (int64_t)i * K + j, val);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Fills sm.H[q] (q < ne) with the gate rows grow0 + q, each the sum of the
// S partials hpart[s][row][:] in slice order (S == 1: hpart is H).  The
// partials are read with xload.  Every thread calls; no barrier inside.
__device__ __forceinline__ void pair_sum_gate(const float* __restrict__ hpart, int S, int64_t M,
                                              int r, int64_t grow0, int ne, PairLds& sm) {
    const int tid = threadIdx.x;
    const int hp = r / 2;                       // float pairs per row
    for (int pi = tid; pi < ne * hp; pi += kWG) {
        const int q = pi / hp, k = 2 * (pi % hp);
        const uint64_t* src = reinterpret_cast<const uint64_t*>(hpart + (grow0 + q) * r + k);
        const int64_t stride = M * r / 2;       // one slice, in pairs
        uint64_t v[kMaxFusedSlices];
#pragma unroll
        for (int s = 0; s < kMaxFusedSlices; ++s) v[s] = xload(src + (int64_t)min(s, S - 1) * stride);
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int s = 0; s < kMaxFusedSlices; ++s) {
            if (s < S) {
                lo += __uint_as_float((uint32_t)v[s]);
                hi += __uint_as_float((uint32_t)(v[s] >> 32));
            }
        }
        sm.H[q][k] = lo;
        sm.H[q][k + 1] = hi;
    }
}

}  // namespace df2
