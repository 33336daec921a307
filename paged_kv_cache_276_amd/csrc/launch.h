// launch.h -- host-side launchers of the libpagedkv kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Arguments of one decode call after host validation.  Workspace: ws_ml holds
// (running max in log2 units, softmax denominator) per [seq][q_head][partition];
// ws_acc the unnormalised output per [seq][q_head][partition][head_dim].
struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t block_size;
    int32_t head_dim;
    int32_t dtype;  // pkv_dtype
    float scale;
    float* out;
    float* ws_acc;
    float2* ws_ml;
    int2* ws_rec;  // fast kernel: per (seq, kv head) first partial slot and partial count
    uint32_t* ws_cnt;  // multi-query chunk kernel: arrival counter per (seq, kv head, row block), zero between calls
    int32_t part_tokens;
    int32_t max_parts;
    int32_t grid_waves;  // fast kernel: requested waves (0 = resident capacity)
    int32_t xcd_balance; // fast kernel: share of a wave on an odd XCD, in 64ths (64 = equal); 0 = library choice
    // Shared-prefix path (paged_attn_decode_prefix); zero/null otherwise.
    const int32_t* seq_start;    // [S] tokens of each sequence covered by its group's shared prefix
    const int32_t* groups;       // [num_groups][2] first sequence, member count
    int32_t num_groups;
    int32_t prefix_chunk_tiles;  // 16-token tiles per prefix chunk
    int32_t prefix_max_chunks;   // chunk partials kept per (sequence, KV head)
    float2* ws_pml;              // prefix partials (m, l): [S][Hkv][max_chunks][G]
    float* ws_pacc;              // prefix partials acc: [S][Hkv][max_chunks][G][head_dim]
    // Several new tokens per sequence (paged_attn_decode_multi); chunk partials
    // go to ws_pml / ws_pacc as [total_q][Hq][max_chunks] (m, l) and acc.
    const int32_t* cu_q;         // [S + 1] offsets of each sequence's query rows
    int32_t total_q;
    int32_t max_q_len;
    int32_t multi_row_blocks;    // row blocks (16 * multi_waves rows each) per KV head
    int32_t multi_waves;         // 16-row groups per workgroup of the multi-query kernel: 1, 4 or 16 (1, 4, 8 waves)
    int32_t multi_split_runs;    // 1: equal runs of tiles over the resident waves (multi_waves 1),
                                 // partials in ws_rec / ws_ml / ws_acc with 16 rows per slot
};

constexpr int32_t kMaxGridWaves = 8192;  // PKV_MAX_GRID_WAVES

// Every workspace starts with this many uint32 arrival counters
// (PKV_WORKSPACE_COUNTER_BYTES), used by the multi-query chunk kernel to merge
// its chunks in-kernel when the batch has at most that many units.
constexpr int64_t kCounterUnits = 65536;

hipError_t launch_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                           int32_t num_tokens, void* k_cache, void* v_cache, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t row_bytes,
                           hipStream_t stream);

hipError_t launch_block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                             int32_t num_blocks, int64_t block_bytes, hipStream_t stream);

// Returns hipErrorInvalidValue when no instantiation matches the shape.
// The calling thread's last decode launch (kernel family, grid, XCD share,
// partition tokens), set by the launchers and read by pkv_last_launch_info.
struct LaunchInfo {
    int32_t kernel, grid, xcd_balance, partition_tokens, k_stream;
};
LaunchInfo& last_launch();

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t stream);
// Shared-prefix decode: prefix kernel, suffix tiles (fast kernel), merge.
hipError_t launch_decode_prefix(const DecodeArgs& a, hipStream_t stream);
// Several new tokens per sequence (causal): chunk kernel, merge.
hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t stream);
constexpr int32_t kPrefixGroupMax = 8;  // sequences per prefix group (one wave each)
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream);

bool generic_supports(int32_t dtype, int32_t head_dim, int32_t group);
bool fast_supports(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group);

}  // namespace pkv
