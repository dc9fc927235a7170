// Counter-based uniforms for the sampling walk ("DFlash 2: Keep Drafting
// Parallel", section "A Lightweight Path Selector": sampling draws from the
// same scores, one uniform per draft position).
//
// The generator is Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds over a 4-word
// counter under a 2-word key; in each round words 0 and 2 are multiplied by
// the two round multipliers, the high halves are crossed with words 1 and 3
// and the key, and the key then advances by the two Weyl increments.
//
// Uniform i of a call (seed, offset) is word i mod 4 of the block at counter
// (i / 4, offset, 0, 0) under key (seed, 0); a word x becomes the fp32 value
// (x >> 40) * 2^-24, exact and in [0, 1).  One thread makes one block, so a
// draw depends only on (seed, offset, i): the stream is the same for any
// launch shape, and a caller advances `offset` once per draft-verify cycle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace df2 {

constexpr uint64_t kPhiloxMul0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxMul1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxWeyl0 = 0x9E3779B97F4A7C15ull;  // 2^64 / golden ratio
constexpr uint64_t kPhiloxWeyl1 = 0xBB67AE8584CAA73Bull;  // 2^64 * (sqrt(3) - 1)
constexpr int kPhiloxWG = 256;                            // threads per workgroup

struct PhiloxBlock {
    uint64_t w[4];
};

__device__ __forceinline__ PhiloxBlock philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                     uint64_t c3, uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t hi0 = __umul64hi(kPhiloxMul0, c0), lo0 = kPhiloxMul0 * c0;
        const uint64_t hi1 = __umul64hi(kPhiloxMul1, c2), lo1 = kPhiloxMul1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0;
        const uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kPhiloxWeyl0;
        k1 += kPhiloxWeyl1;
    }
    return PhiloxBlock{{c0, c1, c2, c3}};
}

__device__ __forceinline__ float philox_unit(uint64_t x) {
    return (float)(uint32_t)(x >> 40) * 0x1.0p-24f;   // 24 bits: exact in fp32
}

// Thread t of the grid writes uniforms 4t .. 4t+3 (those below n).  The grid
// covers ceil(n / 4) threads; `vec` (out 16-byte aligned) lets whole blocks
// go out as one 16-byte store.  With offset_ptr set, the offset is read from
// device memory, so a captured graph draws fresh uniforms on every replay;
// it then moves on by one: inside this kernel when the grid is one
// workgroup (`bump`: every thread holds the value in a register before the
// barrier, and only then does thread 0 write), else by k_philox_bump
// afterwards in stream order.
__global__ void __launch_bounds__(kPhiloxWG)
k_philox_uniforms(uint64_t seed, uint64_t offset, uint64_t* __restrict__ offset_ptr,
                  int64_t n, float* __restrict__ out, int vec, int bump) {
    const int64_t blk = (int64_t)blockIdx.x * kPhiloxWG + threadIdx.x;
    const int64_t i0 = blk * 4;
    if (offset_ptr) {
        const uint64_t v = *offset_ptr;
        // wave-uniform value moved to scalar registers: the load has
        // returned before the barrier below
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
        offset = ((uint64_t)hi << 32) | lo;
        if (bump) {
            __syncthreads();
            if (threadIdx.x == 0) *offset_ptr = offset + 1;
        }
    }
    if (i0 >= n) return;
    const PhiloxBlock b = philox4x64_10((uint64_t)blk, offset, 0, 0, seed, 0);
    float u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = philox_unit(b.w[q]);
    if (vec && i0 + 4 <= n) {
        *reinterpret_cast<float4*>(out + i0) = make_float4(u[0], u[1], u[2], u[3]);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (i0 + q < n) out[i0 + q] = u[q];
    }
}

// One thread: the device-resident offset moves to the next cycle.
__global__ void k_philox_bump(uint64_t* __restrict__ offset_ptr) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *offset_ptr += 1;
}

}  // namespace df2
