// kv_write.hip -- append step of the paged KV cache: each new token's K and V
// rows go to their slot (physical block slot / block_size, offset
// slot % block_size) for every KV head.  Raw 16-byte copies, so every bit
// pattern arrives unchanged.
//
// One thread moves one 16-byte chunk of one row of K and the same chunk of V.
// Consecutive threads cover consecutive chunks of a row, then the next KV head,
// then the next token, so both the reads of k_new/v_new and the writes of one
// destination row are contiguous.  Slots outside [0, num_blocks * block_size)
// are skipped, which keeps every store inside the pools whatever the slot
// mapping holds.
#include "launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ slot_mapping, int64_t total_chunks, int32_t chunks_per_row,
    int32_t num_kv_heads, int32_t block_size, int64_t num_slots, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total_chunks) return;
    const int32_t c = (int32_t)(idx % chunks_per_row);
    const int64_t row = idx / chunks_per_row;  // token * num_kv_heads + head
    const int32_t h = (int32_t)(row % num_kv_heads);
    const int64_t t = row / num_kv_heads;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + c;
    const uint4 kv = k_new[idx];
    const uint4 vv = v_new[idx];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
}

hipError_t launch_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                           int32_t num_tokens, void* k_cache, void* v_cache, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t row_bytes,
                           hipStream_t stream) {
    const int32_t chunks_per_row = row_bytes / 16;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                       slot_mapping, total, chunks_per_row, num_kv_heads, block_size,
                       (int64_t)num_blocks * block_size, static_cast<uint4*>(k_cache),
                       static_cast<uint4*>(v_cache));
    return hipGetLastError();
}

// Whole-block copy inside both pools (copy-on-write of a shared block): one
// workgroup row per pair, consecutive threads on consecutive 16-byte chunks of
// the block (all KV heads, all slots), so reads and writes are contiguous.
__global__ __launch_bounds__(256) void block_copy_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                         const int32_t* __restrict__ pairs, int64_t chunks_per_block,
                                                         int32_t num_blocks) {
    const int64_t p = blockIdx.x;
    const int32_t src = pairs[2 * p];
    const int32_t dst = pairs[2 * p + 1];
    if ((uint32_t)src >= (uint32_t)num_blocks || (uint32_t)dst >= (uint32_t)num_blocks) return;
    const int64_t so = (int64_t)src * chunks_per_block;
    const int64_t d0 = (int64_t)dst * chunks_per_block;
    for (int64_t j = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; j < chunks_per_block;
         j += (int64_t)gridDim.y * blockDim.x) {
        const uint4 kv = k_cache[so + j];
        const uint4 vv = v_cache[so + j];
        k_cache[d0 + j] = kv;
        v_cache[d0 + j] = vv;
    }
}

hipError_t launch_block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                             int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
    if (num_pairs == 0) return hipSuccess;
    const int64_t chunks = block_bytes / 16;
    const int threads = 256;
    int64_t ys = (chunks + threads - 1) / threads;
    if (ys > 16) ys = 16;
    hipLaunchKernelGGL(block_copy_kernel, dim3((unsigned)num_pairs, (unsigned)ys), dim3(threads), 0, stream,
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs, chunks, num_blocks);
    return hipGetLastError();
}

}  // namespace pkv
