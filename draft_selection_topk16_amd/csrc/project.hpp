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
// S > 1 slices the slices write partial tiles and the last slice to arrive
// sums them in slice order, so the result does not depend on timing.  Slice
// s of every tile runs on XCD s when S is 8 (workgroups are dealt to the
// eight XCDs round-robin), so the re-reads of one d-slice stay in one L2.
#pragma once

#include "common.hpp"

namespace df2 {

struct ProjLds {
    float red[kWaves][4][4][64];   // [wave][q tile][row group][lane]
    uint32_t flag;
};

// One slice of one output tile.  dst is H [M, r] when S == 1, else the
// partial buffer [S, M, r].  Rows m >= M of the last tile are not written.
template <bool BF16, int NQ>
__device__ void proj_block(const void* __restrict__ hidden, const void* __restrict__ W,
                           int M, int d, int r, int mt, int qt, int s, int S,
                           float* __restrict__ dst, ProjLds& sm) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int row = lane & 15, g = lane >> 4;
    const int KS = d / 32;
    const int ks0 = (int)((int64_t)KS * s / S), ks1 = (int)((int64_t)KS * (s + 1) / S);
    const int m = mt * 16 + row;
    const bool mvalid = m < M;
    const int qbase = qt * 16 * NQ;

    f32x4_t acc[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if constexpr (BF16) {
        const uint16_t* h16 = reinterpret_cast<const uint16_t*>(hidden);
        const uint16_t* w16 = reinterpret_cast<const uint16_t*>(W);
        for (int ks = ks0 + w; ks < ks1; ks += kWaves) {
            const int k0 = ks * 32 + g * 8;
            u32x4_t a = u32x4_t{0u, 0u, 0u, 0u};
            if (mvalid) a = *reinterpret_cast<const u32x4_t*>(h16 + (int64_t)m * d + k0);
            u32x4_t b[NQ];
#pragma unroll
            for (int n = 0; n < NQ; ++n)
                b[n] = *reinterpret_cast<const u32x4_t*>(w16 + (int64_t)(qbase + n * 16 + row) * d + k0);
#pragma unroll
            for (int n = 0; n < NQ; ++n) acc[n] = mfma_bf16(as_bf16x8(a), as_bf16x8(b[n]), acc[n]);
        }
    } else {
        const float* h32 = reinterpret_cast<const float*>(hidden);
        const float* w32 = reinterpret_cast<const float*>(W);
        for (int ks = ks0 + w; ks < ks1; ks += kWaves) {
            const int k0 = ks * 32 + g * 8;
            float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
            if (mvalid) {
                a0 = *reinterpret_cast<const float4*>(h32 + (int64_t)m * d + k0);
                a1 = *reinterpret_cast<const float4*>(h32 + (int64_t)m * d + k0 + 4);
            }
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const float* wr = w32 + (int64_t)(qbase + n * 16 + row) * d + k0;
                float4 b0 = *reinterpret_cast<const float4*>(wr);
                float4 b1 = *reinterpret_cast<const float4*>(wr + 4);
                const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[n] = mfma_f32(av[e], bv[e], acc[n]);
            }
        }
    }

#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.red[w][n][v][lane] = acc[n][v];
    __syncthreads();
    float* out = (S == 1) ? dst : dst + (int64_t)s * M * r;
    for (int x = tid; x < NQ * 4 * 64; x += kWG) {
        const int n = x >> 8, v = (x >> 6) & 3, l = x & 63;
        const float sum = sm.red[0][n][v][l] + sm.red[1][n][v][l] + sm.red[2][n][v][l] +
                          sm.red[3][n][v][l];
        const int mm = mt * 16 + (l >> 4) * 4 + v;
        const int q = qbase + n * 16 + (l & 15);
        if (mm < M) xstore(out + (int64_t)mm * r + q, sum);
    }
}

// Sum the S partial slices of one tile into H, in slice order.
template <int NQ>
__device__ void proj_reduce_tile(const float* __restrict__ part, int M, int r, int mt, int qt,
                                 int S, float* __restrict__ H) {
    const int cols = 16 * NQ;
    for (int x = threadIdx.x; x < 16 * cols; x += kWG) {
        const int mm = mt * 16 + x / cols;
        const int q = qt * cols + x % cols;
        if (mm >= M) continue;
        float acc = 0.f;
        for (int s = 0; s < S; ++s) acc += xload(part + ((int64_t)s * M + mm) * r + q);
        xstore(H + (int64_t)mm * r + q, acc);
    }
}

}  // namespace df2
