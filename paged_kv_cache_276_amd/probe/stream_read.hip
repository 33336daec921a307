// stream_read.hip -- libpkvprobe.so: plain streaming reads of one device
// buffer, the achievable HBM read rate that the decode kernels are compared
// with.  Not part of the decode library; the benchmark loads it by itself and
// keeps the fastest variant.
//
// Variants (all read each 16-byte chunk of the buffer exactly once and fold
// it into one register by XOR; a store taken only when the fold equals a
// constant keeps the loads alive):
//   0  grid stride: load k of a thread is chunk i + k * (grid threads)
//   1  contiguous: workgroup b reads its own 1/grid of the buffer, 256 threads
//      x 16 B = 4 KiB per step
//   2  as 1 with non-temporal loads (streamed, not kept in the caches)
// Every thread has kInFlight loads issued before the first is used.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int VARIANT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
    if constexpr (VARIANT == 2) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <int VARIANT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    if constexpr (VARIANT == 0) {
        const int64_t stride = (int64_t)gridDim.x * kThreads;
        int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
            uint4 v[kInFlight];
#pragma unroll
            for (int k = 0; k < kInFlight; ++k) v[k] = load16<VARIANT>(buf + i + k * stride);
#pragma unroll
            for (int k = 0; k < kInFlight; ++k) acc ^= fold(v[k]);
        }
        for (; i < n16; i += stride) acc ^= fold(load16<VARIANT>(buf + i));
    } else {
        const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
        const int64_t lo = (int64_t)blockIdx.x * per;
        const int64_t hi = lo + per < n16 ? lo + per : n16;
        int64_t i = lo + threadIdx.x;
        for (; i + (kInFlight - 1) * kThreads < hi; i += kInFlight * kThreads) {
            uint4 v[kInFlight];
#pragma unroll
            for (int k = 0; k < kInFlight; ++k) v[k] = load16<VARIANT>(buf + i + k * kThreads);
#pragma unroll
            for (int k = 0; k < kInFlight; ++k) acc ^= fold(v[k]);
        }
        for (; i < hi; i += kThreads) acc ^= fold(load16<VARIANT>(buf + i));
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) at `buf` (16-byte aligned) with `blocks`
// workgroups of 256 threads on `stream`, in access pattern `variant` (0, 1 or
// 2 above).  `sink` (device, at least `blocks` uint32) receives a value only
// in the rare case that a workgroup's fold equals a fixed constant.  Returns
// the hipError_t of the launch.
extern "C" __attribute__((visibility("default"))) int pkv_probe_stream_read(const void* buf, uint64_t bytes,
                                                                            int32_t blocks, int32_t variant,
                                                                            uint32_t* sink, void* stream) {
    if (!buf || !sink || blocks <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
        return (int)hipErrorInvalidValue;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* b = static_cast<const uint4*>(buf);
    const int64_t n16 = (int64_t)(bytes / 16);
    switch (variant) {
        case 0: hipLaunchKernelGGL(stream_read_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, s, b, n16, sink); break;
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, b, n16, sink); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, s, b, n16, sink); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}
