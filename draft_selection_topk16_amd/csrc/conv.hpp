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
// The corrections are a small GEMM ([B*P, d] x [d, d/8]) done by the gate
// projection's matrix-core slices; this file holds the combine: one thread
// per 8 channels of one position (16-byte loads of x_t, x_{t-1} and both
// base rows, two correction values), fp32 arithmetic, output in the input
// type (bf16 rounded to nearest even).  HBM-bound: every byte is read once
// apart from x, which the GEMM also reads.
#pragma once

#include "common.hpp"

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

// x [M = B*P, d], x_prev [B, d], base [2, d], corr [M, d/8] (tap 0 groups,
// then tap 1 groups), out [M, d].  One thread per 8 channels.
template <bool BF16>
__global__ __launch_bounds__(kWG) void k_conv2(const void* __restrict__ x, const void* __restrict__ x_prev,
                                               const void* __restrict__ base,
                                               const float* __restrict__ corr, void* __restrict__ out,
                                               int64_t M, int P, int d) {
    const int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x;
    const int dv = d / 8, N = d / 8, G = d / 16;
    if (i >= M * dv) return;
    const int64_t m = i / dv;
    const int c0 = (int)(i % dv) * 8;
    const int t = (int)(m % P);
    const float k0c = corr[m * N + (c0 >> 4)];
    const float k1c = corr[m * N + G + (c0 >> 4)];
    float xt[8], xp[8], b0[8], b1[8], y[8];
    load8<BF16>(x, m * d + c0, xt);
    if (t == 0)
        load8<BF16>(x_prev, (m / P) * d + c0, xp);
    else
        load8<BF16>(x, (m - 1) * d + c0, xp);
    load8<BF16>(base, c0, b0);
    load8<BF16>(base, (int64_t)d + c0, b1);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (b0[e] + k0c) * xt[e] + (b1[e] + k1c) * xp[e];
    store8<BF16>(out, m * d + c0, y);
}

}  // namespace df2
