// Gate projection H_t = W_H h_t.
//
// The selector equation ("DFlash 2: Keep Drafting Parallel", section "A
// Lightweight Path Selector") matches two token embeddings under a context
// gate H(h_t) computed from the drafter hidden state; the formula of H is not
// printed, and this library reads it as a bias-free linear map d -> r.
//
// The map is a GEMM of M = B*P rows: hidden [M, d] times W_H^T [d, r], fp32
// accumulation on the matrix cores (bf16 x bf16 products are exact in fp32;
// fp32 inputs use the fp32 matrix instruction).
//
// A workgroup computes one slice s of d for one output tile of MB x NB
// 16 x 16 blocks.  Its four waves take turns at groups of KB adjacent
// 32-wide k steps (adjacent steps of a row share cache lines) and issue the
// loads of a group before its first product, so a slice of 4 * KB steps
// costs one memory round trip.  The four waves' tiles are summed
// in LDS in wave order and the slice is written as a partial [S, M, r]
// (or straight into H when S == 1).  The S partials are summed in slice order
// by whoever needs H_t (a row merge, or in the selector's two launches with a
// one-m-block gate the tile's last slice to finish), so results never depend
// on timing.
#pragma once

#include "common.hpp"

namespace df2 {

constexpr int kMaxFusedSlices = 16; // d slices of a tile (whoever needs H sums them)

// k steps each wave loads before its first product
__host__ __device__ constexpr int gate_kb(bool bf16) { return bf16 ? 2 : 1; }

struct GateLds {
    float red[kWaves][4][256];      // four 16 x 16 blocks per wave at a time
};

// Slice s (of S) of tile (mt, nt); tile rows mt*16*MB.., columns nt*16*NB..
// dst: [S, M, r] partials (slice s at dst + s*M*r); with S == 1 this is H.
// Rows m >= M load row M - 1 and are not written.  With pair_half > 0,
// output column q takes row (q % 2) * pair_half + q / 2 of W (two
// half-matrices interleaved column by column).  Every thread calls.
template <bool BF16, int MB, int NB>
__device__ void gate_slice(const void* __restrict__ hidden, const void* __restrict__ W, int M,
                           int d, int r, int mt, int nt, int s, int S, float* __restrict__ dst,
                           GateLds& sm, int pair_half = 0) {
    static_assert((MB * NB) % 4 == 0, "blocks are summed four at a time");
    constexpr int KB = gate_kb(BF16);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = lane & 15, g = lane >> 4;
    // slices start on even k steps, so that the two adjacent steps a wave
    // loads together share their 128-byte lines
    const int KS = d / 32, KP = (KS + 1) / 2;
    const int ks0 = 2 * (int)((int64_t)KP * s / S);
    const int ks1 = min(KS, 2 * (int)((int64_t)KP * (s + 1) / S));

    f32x4_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    int64_t arow[MB], brow[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        arow[i] = (int64_t)min(mt * 16 * MB + 16 * i + row, M - 1) * d;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int q = nt * 16 * NB + 16 * j + row;
        brow[j] = (int64_t)(pair_half > 0 ? (q & 1) * pair_half + (q >> 1) : q) * d;
    }

    // wave w takes steps kb .. kb + KB - 1, kb = ks0 + KB * (w + 4 i)
    for (int kb = ks0 + KB * w; kb < ks1; kb += kWaves * KB) {
        if constexpr (BF16) {
            const uint16_t* h16 = reinterpret_cast<const uint16_t*>(hidden);
            const uint16_t* w16 = reinterpret_cast<const uint16_t*>(W);
            u32x4_t a[KB][MB], b[KB][NB];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int kq = kb + q;
                const int k0 = ((kq < ks1) ? kq : kb) * 32 + g * 8;
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    a[q][i] = *reinterpret_cast<const u32x4_t*>(h16 + arow[i] + k0);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    b[q][j] = *reinterpret_cast<const u32x4_t*>(w16 + brow[j] + k0);
            }
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                if (kb + q < ks1) {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            acc[i][j] = mfma_bf16(as_bf16x8(a[q][i]), as_bf16x8(b[q][j]), acc[i][j]);
                }
            }
        } else {
            const float* h32 = reinterpret_cast<const float*>(hidden);
            const float* w32 = reinterpret_cast<const float*>(W);
            float4 a[MB][2], b[NB][2];
            const int k0 = kb * 32 + g * 8;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                a[i][0] = *reinterpret_cast<const float4*>(h32 + arow[i] + k0);
                a[i][1] = *reinterpret_cast<const float4*>(h32 + arow[i] + k0 + 4);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                b[j][0] = *reinterpret_cast<const float4*>(w32 + brow[j] + k0);
                b[j][1] = *reinterpret_cast<const float4*>(w32 + brow[j] + k0 + 4);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const float av[8] = {a[i][0].x, a[i][0].y, a[i][0].z, a[i][0].w,
                                     a[i][1].x, a[i][1].y, a[i][1].z, a[i][1].w};
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const float bv[8] = {b[j][0].x, b[j][0].y, b[j][0].z, b[j][0].w,
                                         b[j][1].x, b[j][1].y, b[j][1].z, b[j][1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[i][j] = mfma_f32(av[e], bv[e], acc[i][j]);
                }
            }
        }
    }

    // Sum the four waves' tiles in wave order, four blocks at a time.  Block
    // (i, j), value v of lane l is row 16 i + 4 (l / 16) + v, column
    // 16 j + l % 16 of the tile.
    float* out = dst + (int64_t)s * M * r;
#pragma unroll
    for (int part = 0; part < MB * NB / 4; ++part) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ij = part * 4 + u;
#pragma unroll
            for (int v = 0; v < 4; ++v) sm.red[w][u][v * 64 + lane] = acc[ij / NB][ij % NB][v];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int x = q * kWG + tid;            // [u][v][lane]
            const int u = x >> 8, v = (x >> 6) & 3, l = x & 63;
            const float sum = sm.red[0][u][x & 255] + sm.red[1][u][x & 255] +
                              sm.red[2][u][x & 255] + sm.red[3][u][x & 255];
            const int ij = part * 4 + u;
            const int mm = mt * 16 * MB + 16 * (ij / NB) + 4 * (l >> 4) + v;
            const int col = nt * 16 * NB + 16 * (ij % NB) + (l & 15);
            if (mm < M) xstore(out + (int64_t)mm * r + col, sum);
        }
        __syncthreads();
    }
}

}  // namespace df2
