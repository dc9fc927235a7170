// Device helpers shared by the selector kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace df2 {

constexpr int kWG = 256;     // threads per workgroup
constexpr int kWaves = 4;    // wave64 waves per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__ballot(p)); }

// ---------------------------------------------------------------------------
// Order-preserving keys.  A larger key means a larger value; -0 and +0 share
// one key (IEEE equality).  The all-ones bit pattern (a NaN) is the padding
// sentinel and maps to key 0, below every number (-inf included).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t key_bf16(uint32_t x) {
    x = (x == 0x8000u) ? 0u : x;
    return (x & 0x8000u) ? (~x & 0xFFFFu) : (x | 0x8000u);
}
__device__ __forceinline__ uint32_t key_f32(uint32_t x) {
    x = (x == 0x80000000u) ? 0u : x;
    return (x & 0x80000000u) ? ~x : (x | 0x80000000u);
}
__device__ __forceinline__ float value_of_key_bf16(uint32_t k) {
    uint32_t bits = (k & 0x8000u) ? (k ^ 0x8000u) : (~k & 0xFFFFu);
    return __uint_as_float(bits << 16);
}
__device__ __forceinline__ float value_of_key_f32(uint32_t k) {
    uint32_t bits = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
    return __uint_as_float(bits);
}

// Candidate word: key in the high half, complemented vocabulary index in the
// low half, so that comparing words orders by (value desc, index asc) and all
// words of one row are distinct.  0 marks an empty slot.
__device__ __forceinline__ uint64_t cand_word(uint32_t key, uint32_t gidx) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - gidx);
}
__device__ __forceinline__ uint32_t cand_index(uint64_t w) {
    return 0xFFFFFFFFu - (uint32_t)w;
}

// ---------------------------------------------------------------------------
// Wave and workgroup reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over the workgroup; `red` holds kWaves words of LDS.  Every thread of
// the workgroup must call it.
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t x, uint32_t* red) {
    x = wave_sum_u32(x);
    if (lane_id() == 0) red[wave_id()] = x;
    __syncthreads();
    uint32_t t = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return t;
}

// ---------------------------------------------------------------------------
// Matrix cores (CDNA4).  For the 16x16 output tile, lane l holds rows
// 4*(l/16) + v (v = 0..3) of column l % 16.  Operand A row / operand B column
// is l % 16; both operands assign the same k values to a lane, so any k order
// inside one instruction gives the same sum.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Reinterpret four dwords (eight bf16) as an MFMA operand.
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// ---------------------------------------------------------------------------
// Workgroup-to-workgroup hand-off inside one launch.
//
// Each XCD has its own L2.  A device-scope fence on gfx950 writes back and
// invalidates the whole L2 (buffer_wbl2 / buffer_inv), which is far too
// costly to pay once per workgroup.  Instead, every value that one
// workgroup writes for another goes through an agent-scope atomic store and
// is read back with an agent-scope atomic load: both carry the sc1 bit and
// are coherent across XCDs by themselves.  A producer drains its own stores
// (s_waitcnt vmcnt(0)), meets the workgroup barrier, and one thread then
// bumps a counter with a device-scope atomic add.  The workgroup that sees
// the last count reads the data after that add has returned.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void xstore(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T xload(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Eight consecutive floats (32-byte aligned) through four 8-byte loads.
__device__ __forceinline__ void xload_f8(const float* p, float out[8]) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint64_t w = xload(q + i);
        out[2 * i] = __uint_as_float((uint32_t)w);
        out[2 * i + 1] = __uint_as_float((uint32_t)(w >> 32));
    }
}

// Wait until this wave's outstanding vector-memory operations (in particular
// its stores) have completed.  simm16 0x0F70 = vmcnt(0), expcnt and lgkmcnt
// left at their maxima.
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint32_t arrive(uint32_t* cnt) {
    return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* cnt) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave publishes its hand-off stores, then one thread arrives.  Returns
// true (uniformly) in the workgroup that arrives last; that workgroup then
// reads the other arrivals' data with xload.
__device__ __forceinline__ bool block_arrive_last(uint32_t* cnt, uint32_t expected,
                                                  uint32_t* lds_flag) {
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) *lds_flag = (arrive(cnt) == expected - 1u) ? 1u : 0u;
    __syncthreads();
    return *lds_flag != 0u;
}

}  // namespace df2
