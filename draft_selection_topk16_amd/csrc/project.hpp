// Gate projection H_t = W_H h_t.
//
// The selector equation ("DFlash 2: Keep Drafting Parallel", section "A
// Lightweight Path Selector") matches two token embeddings under a context
// gate H(h_t) computed from the drafter hidden state; the formula of H is not
// printed, and this library reads it as a bias-free linear map d -> r.
//
// The map is a GEMM of M = B*P rows: hidden [M, d] times W_H^T [d, r], fp32
// accumulation on the matrix cores (bf16 x bf16 products are exact in fp32;
// fp32 inputs use the fp32 matrix instruction).  A workgroup owns a 16-row by
// 16*NQ-column output tile over one slice of d; its four waves take
// interleaved 32-wide k steps and are summed in LDS in a fixed order.  With
// S > 1 slices (at most 8) the slices write partial tiles that are summed in
// slice order (by the last slice to arrive, or by the reader of H), so the
// result does not depend on timing.  Slice
// s of every tile runs on XCD s when S is 8 (workgroups are dealt to the
// eight XCDs round-robin), so the re-reads of one d-slice stay in one L2.
#pragma once

#include "common.hpp"

namespace df2 {

constexpr int kMaxSlices = 8;      // d slices of one H tile

// k steps whose loads a wave issues together: about sixty registers of
// operands (bf16: 1 + NQ 16-byte loads per step; fp32: 2 + 2 NQ).
__host__ __device__ constexpr int proj_kb(bool bf16, int nq) {
    return bf16 ? (nq >= 4 ? 3 : (nq == 2 ? 5 : 8)) : (nq >= 4 ? 1 : (nq == 2 ? 2 : 4));
}

struct ProjLds {
    float red[kWaves][4][4][64];   // [wave][q tile][row group][lane]
    uint32_t flag;
};

// One slice of one output tile.  dst is H [M, r] or the partial buffer
// [S, M, r] (slice s at dst + s * M * r).  Rows m >= M of the last tile load
// row M - 1 and are not written.  A wave issues the loads of KB of its k
// steps before the first product that uses them.
template <bool BF16, int NQ>
__device__ void proj_block(const void* __restrict__ hidden, const void* __restrict__ W,
                           int M, int d, int r, int mt, int qt, int s, int S,
                           float* __restrict__ dst, ProjLds& sm) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = lane & 15, g = lane >> 4;
    const int KS = d / 32;
    const int ks0 = (int)((int64_t)KS * s / S), ks1 = (int)((int64_t)KS * (s + 1) / S);
    const int m = min(mt * 16 + row, M - 1);
    const int qbase = qt * 16 * NQ;

    f32x4_t acc[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if constexpr (BF16) {
        constexpr int KB = proj_kb(true, NQ);
        const uint16_t* h16 = reinterpret_cast<const uint16_t*>(hidden) + (int64_t)m * d + g * 8;
        const uint16_t* w16 = reinterpret_cast<const uint16_t*>(W) + (int64_t)(qbase + row) * d + g * 8;
        for (int ks = ks0 + w; ks < ks1; ks += kWaves * KB) {
            u32x4_t a[KB], b[KB][NQ];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int kq = ks + q * kWaves;
                const int k0 = ((kq < ks1) ? kq : ks) * 32;
                a[q] = *reinterpret_cast<const u32x4_t*>(h16 + k0);
#pragma unroll
                for (int n = 0; n < NQ; ++n)
                    b[q][n] = *reinterpret_cast<const u32x4_t*>(w16 + (int64_t)n * 16 * d + k0);
            }
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                if (ks + q * kWaves < ks1) {
#pragma unroll
                    for (int n = 0; n < NQ; ++n)
                        acc[n] = mfma_bf16(as_bf16x8(a[q]), as_bf16x8(b[q][n]), acc[n]);
                }
            }
        }
    } else {
        constexpr int KB = proj_kb(false, NQ);
        const float* h32 = reinterpret_cast<const float*>(hidden) + (int64_t)m * d + g * 8;
        const float* w32 = reinterpret_cast<const float*>(W) + (int64_t)(qbase + row) * d + g * 8;
        for (int ks = ks0 + w; ks < ks1; ks += kWaves * KB) {
            float4 a[KB][2], b[KB][NQ][2];
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                const int kq = ks + q * kWaves;
                const int k0 = ((kq < ks1) ? kq : ks) * 32;
                a[q][0] = *reinterpret_cast<const float4*>(h32 + k0);
                a[q][1] = *reinterpret_cast<const float4*>(h32 + k0 + 4);
#pragma unroll
                for (int n = 0; n < NQ; ++n) {
                    const float* wr = w32 + (int64_t)n * 16 * d + k0;
                    b[q][n][0] = *reinterpret_cast<const float4*>(wr);
                    b[q][n][1] = *reinterpret_cast<const float4*>(wr + 4);
                }
            }
#pragma unroll
            for (int q = 0; q < KB; ++q) {
                if (ks + q * kWaves < ks1) {
                    const float av[8] = {a[q][0].x, a[q][0].y, a[q][0].z, a[q][0].w,
                                         a[q][1].x, a[q][1].y, a[q][1].z, a[q][1].w};
#pragma unroll
                    for (int n = 0; n < NQ; ++n) {
                        const float bv[8] = {b[q][n][0].x, b[q][n][0].y, b[q][n][0].z, b[q][n][0].w,
                                             b[q][n][1].x, b[q][n][1].y, b[q][n][1].z, b[q][n][1].w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[n] = mfma_f32(av[e], bv[e], acc[n]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.red[w][n][v][lane] = acc[n][v];
    __syncthreads();
    float* out = dst + (int64_t)s * M * r;
    for (int x = tid; x < NQ * 4 * 64; x += kWG) {
        const int n = x >> 8, v = (x >> 6) & 3, l = x & 63;
        const float sum = sm.red[0][n][v][l] + sm.red[1][n][v][l] + sm.red[2][n][v][l] +
                          sm.red[3][n][v][l];
        const int mm = mt * 16 + (l >> 4) * 4 + v;
        const int q = qbase + n * 16 + (l & 15);
        if (mm < M) xstore(out + (int64_t)mm * r + q, sum);
    }
}

// Sum the S partial slices of one tile into H, in slice order.  Every
// slice load of an element is issued before the sum.
template <int NQ>
__device__ void proj_reduce_tile(const float* __restrict__ part, int M, int r, int mt, int qt,
                                 int S, float* __restrict__ H) {
    const int cols = 16 * NQ;
    for (int x = threadIdx.x; x < 16 * cols; x += kWG) {
        const int mm = mt * 16 + x / cols;
        const int q = qt * cols + x % cols;
        const int mc = min(mm, M - 1);
        float v[kMaxSlices];
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s)
            v[s] = xload(part + ((int64_t)min(s, S - 1) * M + mc) * r + q);
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s)
            if (s < S) acc += v[s];
        if (mm < M) xstore(H + (int64_t)mm * r + q, acc);
    }
}

}  // namespace df2
