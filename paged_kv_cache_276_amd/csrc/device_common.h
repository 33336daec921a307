// device_common.h -- small device helpers shared by the HIP kernels of libpagedkv.
// gfx950 (CDNA4): wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 is the upper half of a binary32: widening is a 16-bit shift.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Value of lane `lane` (wave-uniform index) broadcast to the whole wave.
__device__ __forceinline__ float read_lane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Element storage types: fp32 as float, bf16 as its raw 16 bits.
struct F32 {
    using storage = float;
    static constexpr int kBytes = 4;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int kBytes = 2;
};

// Widen the 16 bytes at p (8 bf16 or 4 fp32 elements) to fp32.
template <typename E>
struct Chunk16;

template <>
struct Chunk16<BF16> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void load(const void* p, float (&f)[8]) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
        f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
        f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
        f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
    }
};

template <>
struct Chunk16<F32> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void load(const void* p, float (&f)[4]) {
        const float4 u = *reinterpret_cast<const float4*>(p);
        f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
    }
};

// Widen N consecutive elements at p (N in 1, 2, 4) to fp32.
template <typename E, int N>
__device__ __forceinline__ void load_small(const void* p, float (&f)[N]);

template <>
__device__ __forceinline__ void load_small<BF16, 1>(const void* p, float (&f)[1]) {
    f[0] = __uint_as_float(((uint32_t)*reinterpret_cast<const uint16_t*>(p)) << 16);
}
template <>
__device__ __forceinline__ void load_small<BF16, 2>(const void* p, float (&f)[2]) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    f[0] = bf16_lo(u); f[1] = bf16_hi(u);
}
template <>
__device__ __forceinline__ void load_small<BF16, 4>(const void* p, float (&f)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
}
template <>
__device__ __forceinline__ void load_small<F32, 1>(const void* p, float (&f)[1]) {
    f[0] = *reinterpret_cast<const float*>(p);
}
template <>
__device__ __forceinline__ void load_small<F32, 2>(const void* p, float (&f)[2]) {
    const float2 u = *reinterpret_cast<const float2*>(p);
    f[0] = u.x; f[1] = u.y;
}
template <>
__device__ __forceinline__ void load_small<F32, 4>(const void* p, float (&f)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
}

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// Sequence bookkeeping shared by the partition and combine kernels.
struct SeqSpan {
    int ctx;     // valid tokens (0 when the stored length is out of range)
    int nparts;  // partitions holding tokens (1 for an empty sequence)
    bool bad;    // the stored length is negative or exceeds the block table
};

__device__ __forceinline__ SeqSpan seq_span(int ctx_raw, int table_tokens, int part_tokens) {
    SeqSpan s;
    s.bad = ctx_raw < 0 || ctx_raw > table_tokens;
    s.ctx = s.bad ? 0 : ctx_raw;
    s.nparts = s.ctx == 0 ? 1 : (s.ctx + part_tokens - 1) / part_tokens;
    return s;
}

}  // namespace pkv
