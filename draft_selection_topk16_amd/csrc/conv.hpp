// Two-tap dynamic depthwise convolution of the block drafter.
//
// "DFlash 2: Keep Drafting Parallel", section "A Lightweight Local
// Convolution": before and after each attention and feed-forward sublayer,
//     y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1},
// the first draft position reading the last verified token's representation.
// Each coefficient is a learned base plus a correction computed from the
// current hidden state, one correction per 16 channels.  The correction's
// formula is not printed; this library reads it as a bias-free linear map
//     corr_t[tap][g] = sum_m W_c[tap][g][m] x_t[m],  k_{t,tap}[c] = base[tap][c] + corr_t[tap][c / 16].
//
// One launch.  The corrections are a small GEMM ([B*P, d] x [d, d/8]) on
// the gate projection's matrix-core slices, with the output columns ordered
// (group, tap) so that a tile of 16*NB columns holds both taps of 8*NB
// channel groups.  Every slice stores its partial tile and arrives on the
// tile's counter; the last to arrive sums the S partials in slice order and
// applies the combine to its rows and 128*NB channels: one thread per 8
// channels of one position (16-byte loads of x_t, x_{t-1} and both base
// rows), fp32 arithmetic, output in the input type (bf16 rounded to nearest
// even).  HBM-bound: W_c, x_prev, base and y move once, x twice (GEMM and
// combine, the second mostly from L2).
#pragma once

#include "common.hpp"
#include "gate.hpp"

namespace df2 {

template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ p, int64_t off, float (&v)[8]) {
    if constexpr (BF16) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p) + off);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(w[q] << 16);
            v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
    } else {
        const float* f = reinterpret_cast<const float*>(p) + off;
        const float4 a = *reinterpret_cast<const float4*>(f);
        const float4 b = *reinterpret_cast<const float4*>(f + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <bool BF16>
__device__ __forceinline__ void store8(void* __restrict__ p, int64_t off, const float (&v)[8]) {
    if constexpr (BF16) {
        u32x4_t w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = bf16_rne(v[2 * q]) | (bf16_rne(v[2 * q + 1]) << 16);
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(p) + off) = w;
    } else {
        float* f = reinterpret_cast<float*>(p) + off;
        *reinterpret_cast<float4*>(f) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(f + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

struct ConvArgs {
    const void* x;         // [M, d]
    const void* x_prev;    // [B, d]
    const void* base;      // [2, d]
    const void* Wc;        // [2, d/16, d]
    void* out;             // [M, d]
    float* ppart;          // [S, M, d/8] partial corrections, columns (group, tap)
    uint32_t* tile_cnt;    // [mtiles * ntiles] slices done, reset by the last
    int64_t M;
    int P, d, S, ntiles;
};

struct ConvLds {
    union {
        GateLds g;
        float corr[64 * 64];       // the tile's summed corrections [row][column]
    };
    uint32_t flag;
};

template <bool BF16, int MB>
__global__ __launch_bounds__(kWG) void k_conv2(ConvArgs a) {
    constexpr int NB = MB == 1 ? 4 : 2;
    constexpr int TR = 16 * MB, TC = 16 * NB;      // tile rows, tile columns
    __shared__ ConvLds sm;
    const int tid = threadIdx.x;
    const int N = a.d / 8, G = a.d / 16;
    const int s = (int)(blockIdx.x % a.S), tile = (int)(blockIdx.x / a.S);
    const int mt = tile / a.ntiles, nt = tile % a.ntiles;
    gate_slice<BF16, MB, NB>(a.x, a.Wc, (int)a.M, a.d, N, mt, nt, s, a.S, a.ppart, sm.g, G);
    if (!block_arrive_last(&a.tile_cnt[tile], (uint32_t)a.S, &sm.flag)) return;
    if (tid == 0) reset_counter(&a.tile_cnt[tile]);
    // sum the S partials of the tile in slice order; a thread's loads all
    // go out before the first add
    const int64_t m0 = (int64_t)mt * TR;
    constexpr int PER = TR * TC / kWG;              // entries per thread (4 or 8)
    const int64_t plane = a.M * N;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int q0 = 0; q0 < a.S; q0 += 4) {
        float v[4][PER];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int x = e * kWG + tid, row = x / TC, col = x % TC;
                const int64_t mm = min(m0 + row, a.M - 1);
                const int q = min(q0 + qq, a.S - 1);
                v[qq][e] = xload(a.ppart + q * plane + mm * N + nt * TC + col);
            }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < PER; ++e)
                if (q0 + qq < a.S) acc[e] = (q0 + qq == 0) ? v[qq][e] : acc[e] + v[qq][e];
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) sm.corr[e * kWG + tid] = acc[e];
    __syncthreads();
    // combine: rows m0 .., channels of groups g0 .. g0 + TC / 2.  Vector v
    // (8 channels of one row) goes to thread v % kWG; since kWG is a
    // multiple of the vectors per row, all of a thread's vectors cover the
    // same 8 channels, so the two base rows are loaded once, and the x loads
    // of a batch of vectors all go out before the first is used.
    const int g0 = nt * (TC / 2);
    constexpr int VPR = TC / 2 * 2;                 // 8-channel vectors per row (2 per group)
    static_assert(kWG % VPR == 0, "a thread's vectors share their channels");
    constexpr int NVEC = TR * VPR / kWG;            // vectors per thread
    constexpr int BATCH = BF16 ? NVEC : (NVEC > 2 ? NVEC / 2 : NVEC);
    const int vc = tid % VPR, gl = vc >> 1;
    const int c0 = (g0 + gl) * 16 + (vc & 1) * 8;
    float b0[8], b1[8];
    load8<BF16>(a.base, c0, b0);
    load8<BF16>(a.base, (int64_t)a.d + c0, b1);
#pragma unroll
    for (int k0 = 0; k0 < NVEC; k0 += BATCH) {
        float xt[BATCH][8], xp[BATCH][8];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int row = (tid + (k0 + u) * kWG) / VPR;
            const int64_t m = min(m0 + row, a.M - 1);   // rows past M load row M - 1, unused
            const int t = (int)(m % a.P);
            load8<BF16>(a.x, m * a.d + c0, xt[u]);
            if (t == 0)
                load8<BF16>(a.x_prev, (m / a.P) * a.d + c0, xp[u]);
            else
                load8<BF16>(a.x, (m - 1) * a.d + c0, xp[u]);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int row = (tid + (k0 + u) * kWG) / VPR;
            const int64_t m = m0 + row;
            if (m >= a.M) continue;
            const float k0c = sm.corr[row * TC + 2 * gl];
            const float k1c = sm.corr[row * TC + 2 * gl + 1];
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (b0[e] + k0c) * xt[u][e] + (b1[e] + k1c) * xp[u][e];
            store8<BF16>(a.out, m * a.d + c0, y);
        }
    }
}

}  // namespace df2
