// api.hip -- the extern "C" device entry points of libpagedkv.so (declared in
// include/pagedkv.h and include/pagedkv_blocks.h).  Host code only: argument validation, the launch plan,
// and dispatch to the kernels.  Every check runs before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <cstring>
#include <mutex>

#include "launch.h"
#include "pagedkv.h"
#include "pagedkv_blocks.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int32_t kDefaultPartitionTokens = 512;

bool is_pow2_in(int32_t v, int32_t lo, int32_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pkv_status check_desc(const pkv_cache_desc* c) {
    if (!c) return PKV_ERR_NULL;
    if (c->dtype != PKV_F32 && c->dtype != PKV_BF16) return PKV_ERR_DTYPE;
    if (c->num_blocks <= 0 || c->block_size <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
        return PKV_ERR_SHAPE;
    if (!is_pow2_in(c->block_size, 8, 64)) return PKV_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return PKV_ERR_UNSUPPORTED;
    if ((int64_t)c->num_blocks * c->block_size > INT32_MAX) return PKV_ERR_SHAPE;
    return PKV_OK;
}

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Every workspace starts with the same fixed counter region
// (PKV_WORKSPACE_COUNTER_BYTES: pkv::kCounterUnits uint32 arrival counters).
// Only the multi-query chunk kernel uses it; it needs the counters at zero when a
// call starts and leaves them at zero.  No layout puts other data there,
// whatever the shape, so one zero-filled workspace can serve calls of any shape
// and entry point in turn.
constexpr uint64_t kCounterBytes = PKV_WORKSPACE_COUNTER_BYTES;
static_assert(kCounterBytes == pkv::kCounterUnits * sizeof(uint32_t), "counter region");

struct WorkspaceLayout {
    uint64_t rec_bytes;  // fast: int2 (first partial slot, partial count) [S][Hkv]
    uint64_t ml_bytes;   // generic: float2 [S][Hq][P]; fast: float2 [slots][G]
    uint64_t acc_bytes;  // generic: float [S][Hq][P][D]; fast: float [slots][G][D]
    uint64_t total;      // counter region included
};

// Generic kernel: one partial per (sequence, query head, partition).
WorkspaceLayout generic_layout(int32_t num_seqs, int32_t num_q_heads, int32_t max_parts,
                               int32_t head_dim) {
    WorkspaceLayout w{0, 0, 0, 0};
    if (max_parts <= 1) return w;
    const uint64_t rows = (uint64_t)num_seqs * (uint64_t)num_q_heads * (uint64_t)max_parts;
    w.ml_bytes = align_up(rows * sizeof(float2), 256);
    w.acc_bytes = rows * (uint64_t)head_dim * sizeof(float);
    w.total = kCounterBytes + w.ml_bytes + w.acc_bytes;
    return w;
}

// Fast kernel: per-unit records first, then partial slot u + w for unit
// u = seq * Hkv + kv_head met by wave w; at most (units + waves) slots, each
// holding the unit's G query heads.
WorkspaceLayout fast_layout(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t head_dim) {
    WorkspaceLayout w{0, 0, 0, 0};
    const uint64_t units = (uint64_t)num_seqs * (uint64_t)num_kv_heads;
    const uint64_t slots = units + (uint64_t)pkv::kMaxGridWaves;
    // rows of a partial slot: the group, or 16 on the split-run kernel (group
    // size 16, head dims 64 and 256)
    const uint64_t rows = (head_dim == 128 && group <= 8) ? (uint64_t)group : 16;
    w.rec_bytes = align_up(units * sizeof(int2), 256);
    w.ml_bytes = align_up(slots * rows * sizeof(float2), 256);
    w.acc_bytes = slots * rows * (uint64_t)head_dim * sizeof(float);
    w.total = kCounterBytes + w.rec_bytes + w.ml_bytes + w.acc_bytes;
    return w;
}

pkv_status make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                     const pkv_cache_desc* cache, const pkv_decode_opts* opts,
                     pkv_decode_plan* plan) {
    pkv_status st = check_desc(cache);
    if (st != PKV_OK) return st;
    if (!plan) return PKV_ERR_NULL;
    if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
    if (num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
    if ((int64_t)max_blocks_per_seq * cache->block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
    const int32_t group = num_q_heads / cache->num_kv_heads;

    const int64_t table_tokens = (int64_t)max_blocks_per_seq * cache->block_size;
    // the fast kernel indexes 16-token tiles of all (sequence, KV head) pairs with int32
    const int64_t fast_tiles = (int64_t)num_seqs * ((table_tokens + 15) / 16) * cache->num_kv_heads;
    int32_t kernel = opts ? opts->kernel : PKV_KERNEL_AUTO;
    const bool fast_ok = pkv::fast_supports(cache->dtype, cache->head_dim, cache->block_size, group) &&
                         fast_tiles < INT32_MAX;
    const bool generic_ok = pkv::generic_supports(cache->dtype, cache->head_dim, group);
    if (kernel == PKV_KERNEL_AUTO) {
        kernel = fast_ok ? PKV_KERNEL_FAST : PKV_KERNEL_GENERIC;
    }
    if (kernel == PKV_KERNEL_FAST && !fast_ok) return PKV_ERR_UNSUPPORTED;
    if (kernel == PKV_KERNEL_GENERIC && !generic_ok) return PKV_ERR_UNSUPPORTED;
    if (kernel != PKV_KERNEL_FAST && kernel != PKV_KERNEL_GENERIC) return PKV_ERR_UNSUPPORTED;
    if ((int64_t)num_seqs * num_q_heads > INT32_MAX) return PKV_ERR_SHAPE;

    const int32_t waves = opts ? opts->grid_waves : 0;
    if (waves < 0 || waves > pkv::kMaxGridWaves) return PKV_ERR_SHAPE;
    if (opts && (opts->xcd_balance < 0 || opts->xcd_balance > 127)) return PKV_ERR_SHAPE;

    if (kernel == PKV_KERNEL_FAST) {
        const bool split = group == 16 || cache->head_dim != 128;  // the split-run kernel
        if (split && cache->num_kv_heads > 65535) return PKV_ERR_SHAPE;  // its merge grid's third dimension
        plan->kernel = kernel;
        plan->partition_tokens = 16;
        plan->max_partitions = pkv::kMaxGridWaves;
        plan->threads_per_block = 64;
        plan->grid_blocks = waves;
        plan->workspace_bytes = fast_layout(num_seqs, cache->num_kv_heads, group, cache->head_dim).total;
        return PKV_OK;
    }

    int32_t part = opts && opts->partition_tokens ? opts->partition_tokens : kDefaultPartitionTokens;
    if (part <= 0 || part % 64 != 0) return PKV_ERR_SHAPE;
    const int64_t max_parts = (table_tokens + part - 1) / part;
    const int64_t grid = max_parts * cache->num_kv_heads * (int64_t)num_seqs;
    if (grid > INT32_MAX) return PKV_ERR_SHAPE;

    plan->kernel = kernel;
    plan->partition_tokens = part;
    plan->max_partitions = (int32_t)max_parts;
    plan->threads_per_block = 64;
    plan->grid_blocks = grid;
    plan->workspace_bytes = generic_layout(num_seqs, num_q_heads, (int32_t)max_parts, cache->head_dim).total;
    return PKV_OK;
}

}  // namespace

PKV_API pkv_status paged_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                  int32_t num_tokens, void* k_cache, void* v_cache,
                                  const pkv_cache_desc* cache, void* stream) {
    pkv_status st = check_desc(cache);
    if (st != PKV_OK) return st;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (!k_cache || !v_cache) return PKV_ERR_NULL;
    if (num_tokens > 0 && (!k_new || !v_new || !slot_mapping)) return PKV_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return PKV_ERR_ALIGN;
    if (num_tokens == 0) return PKV_OK;
    const int32_t elem = cache->dtype == PKV_F32 ? 4 : 2;
    const hipError_t e = pkv::launch_kv_write(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache,
                                              cache->num_blocks, cache->block_size, cache->num_kv_heads,
                                              cache->head_dim * elem, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_API pkv_status paged_block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                                    const pkv_cache_desc* cache, void* stream) {
    pkv_status st = check_desc(cache);
    if (st != PKV_OK) return st;
    if (num_pairs < 0 || num_pairs > INT32_MAX / 2) return PKV_ERR_SHAPE;
    if (!k_cache || !v_cache) return PKV_ERR_NULL;
    if (num_pairs == 0) return PKV_OK;
    if (!pairs) return PKV_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_ALIGN;
    const int64_t elem = cache->dtype == PKV_BF16 ? 2 : 4;
    const int64_t block_bytes = (int64_t)cache->num_kv_heads * cache->block_size * cache->head_dim * elem;
    const hipError_t e = pkv::launch_block_copy(k_cache, v_cache, pairs, num_pairs, cache->num_blocks, block_bytes,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_API pkv_status paged_attn_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                   const pkv_cache_desc* cache, const pkv_decode_opts* opts,
                                   pkv_decode_plan* plan) {
    return make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, opts, plan);
}

PKV_API pkv_status paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                              const pkv_decode_opts* opts, uint64_t* bytes) {
    if (!bytes) return PKV_ERR_NULL;
    pkv_decode_plan plan;
    const pkv_status st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, opts, &plan);
    if (st != PKV_OK) return st;
    *bytes = plan.workspace_bytes;
    return PKV_OK;
}

namespace {

// Checks of paged_attn_decode that come before the workspace's (same order in both entry points).
pkv_status check_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        const int32_t* context_lens, const float* out) {
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PKV_ERR_ALIGN;
    return PKV_OK;
}

// paged_attn_decode after validation, with a workspace of at least plan.workspace_bytes.
pkv_status decode_with_workspace(const pkv_decode_plan& plan, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                 float* out, void* workspace, const pkv_cache_desc* cache,
                                 const pkv_decode_opts* opts, void* stream) {

    const int32_t group = num_q_heads / cache->num_kv_heads;
    const WorkspaceLayout wl =
        plan.kernel == PKV_KERNEL_FAST ? fast_layout(num_seqs, cache->num_kv_heads, group, cache->head_dim)
                                       : generic_layout(num_seqs, num_q_heads, plan.max_partitions, cache->head_dim);
    char* ws = static_cast<char*>(workspace) + (wl.total ? kCounterBytes : 0);  // past the counter region
    pkv::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.num_blocks = cache->num_blocks;
    a.block_size = cache->block_size;
    a.head_dim = cache->head_dim;
    a.dtype = cache->dtype;
    a.scale = scale;
    a.out = out;
    a.ws_rec = wl.total ? reinterpret_cast<int2*>(ws) : nullptr;
    a.ws_ml = wl.total ? reinterpret_cast<float2*>(ws + wl.rec_bytes) : nullptr;
    a.ws_acc = wl.total ? reinterpret_cast<float*>(ws + wl.rec_bytes + wl.ml_bytes) : nullptr;
    a.part_tokens = plan.partition_tokens;
    a.max_parts = plan.max_partitions;
    a.grid_waves = opts ? opts->grid_waves : 0;
    a.xcd_balance = opts ? opts->xcd_balance : 0;  // 0: the launch decides

    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (plan.kernel == PKV_KERNEL_FAST) {
        e = pkv::launch_decode_fast(a, s);  // tile kernel + merge kernel
    } else {
        e = pkv::launch_decode_generic(a, s);
        if (e == hipSuccess && plan.max_partitions > 1) e = pkv::launch_combine(a, s);
        if (e == hipSuccess)
            pkv::last_launch() = pkv::LaunchInfo{PKV_KERNEL_GENERIC, (int32_t)plan.grid_blocks, 0,
                                                 plan.partition_tokens, 0};
    }
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

PKV_API pkv_status paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     float scale, float* out, void* workspace, uint64_t workspace_bytes,
                                     const pkv_cache_desc* cache, const pkv_decode_opts* opts,
                                     void* stream) {
    pkv_decode_plan plan;
    pkv_status st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, opts, &plan);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return PKV_OK;
    st = check_decode(q, k_cache, v_cache, block_tables, context_lens, out);
    if (st != PKV_OK) return st;
    if (plan.workspace_bytes > 0) {
        if (!workspace) return PKV_ERR_WORKSPACE;
        if (workspace_bytes < plan.workspace_bytes) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    }
    return decode_with_workspace(plan, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                 num_seqs, num_q_heads, scale, out, workspace, cache, opts, stream);
}

// ---- The allocation-free variant: its workspace is this file-scope device
// array.  In host code the name `scratch` is only a stand-in for the symbol:
// its device address, which differs per GPU, comes from hipGetSymbolAddress,
// taken once per device (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call per device).
pkv_status scratch_address(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

PKV_API pkv_status paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                             float scale, float* out, const pkv_cache_desc* cache,
                                             const pkv_decode_opts* opts, void* stream) {
    pkv_decode_plan plan;
    pkv_status st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, opts, &plan);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return PKV_OK;
    st = check_decode(q, k_cache, v_cache, block_tables, context_lens, out);
    if (st != PKV_OK) return st;
    pkv_decode_opts generic = opts ? *opts : pkv_decode_opts{0, PKV_KERNEL_AUTO, 0, 0};
    if (plan.workspace_bytes > PKV_NOALLOC_SCRATCH_BYTES) {
        // The library's choice does not fit the array: the generic kernel, if it does.
        if (generic.kernel != PKV_KERNEL_AUTO || plan.kernel != PKV_KERNEL_FAST) return PKV_ERR_TOO_LARGE;
        generic.kernel = PKV_KERNEL_GENERIC;
        if (make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, &generic, &plan) != PKV_OK ||
            plan.workspace_bytes > PKV_NOALLOC_SCRATCH_BYTES)
            return PKV_ERR_TOO_LARGE;
        opts = &generic;
    }
    void* ws = nullptr;
    if (plan.workspace_bytes > 0) {
        st = scratch_address(&ws);
        if (st != PKV_OK) return st;
    }
    return decode_with_workspace(plan, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                 num_seqs, num_q_heads, scale, out, ws, cache, opts, stream);
}

namespace pkv {
LaunchInfo& last_launch() {
    thread_local LaunchInfo info{0, 0, 0, 0, 0};
    return info;
}
}  // namespace pkv

PKV_API pkv_status pkv_last_launch_info(pkv_launch_info* info) {
    if (!info) return PKV_ERR_NULL;
    const pkv::LaunchInfo& l = pkv::last_launch();
    info->kernel = l.kernel;
    info->grid = l.grid;
    info->xcd_balance = l.xcd_balance;
    info->partition_tokens = l.partition_tokens;
    info->k_stream = l.k_stream;
    return PKV_OK;
}

namespace {

// Shared-prefix path: the fast plan plus the chunking of the prefixes and the
// chunk partials after the fast workspace.
struct PrefixPlan {
    pkv_decode_plan base;      // fast plan of the suffix pass
    int32_t chunk_tiles;       // 16-token tiles per prefix chunk
    int32_t max_chunks;        // chunks of the longest prefix
    WorkspaceLayout fast;      // suffix pass workspace
    uint64_t pml_bytes, pacc_bytes;
    uint64_t total;
};

constexpr int32_t kPrefixChunkTilesMax = 64;
constexpr int64_t kPrefixTargetWorkgroups = 512;  // about two per CU of the largest parts
constexpr int32_t kMultiChunkTilesMax = 128;
// Multi-query workgroups of 16 row groups (8 waves of 254 registers) fit one
// per CU: aim for one round of them on the largest parts, so that fewer
// chunks leave fewer partials to write and merge.
constexpr int64_t kMultiWideTargetWorkgroups = 256;

pkv_status make_prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                            int32_t num_groups, int32_t max_prefix_tokens, const pkv_cache_desc* cache,
                            const pkv_decode_opts* opts, PrefixPlan* pp) {
    pkv_decode_opts o = opts ? *opts : pkv_decode_opts{0, PKV_KERNEL_AUTO, 0};
    const int32_t chunk_tokens = o.partition_tokens;
    o.partition_tokens = 0;
    o.kernel = PKV_KERNEL_FAST;
    pkv_status st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, &o, &pp->base);
    if (st != PKV_OK) return st;
    if (cache->block_size < 16) return PKV_ERR_UNSUPPORTED;  // the prefix pass reads whole 16-token tiles of one block
    if (num_q_heads / cache->num_kv_heads > pkv::kPrefixGroupMax || cache->head_dim != 128)
        return PKV_ERR_UNSUPPORTED;  // up to 8 heads per KV head, head dim 128
    if (opts && opts->kernel != PKV_KERNEL_AUTO && opts->kernel != PKV_KERNEL_FAST) return PKV_ERR_UNSUPPORTED;
    if (num_groups < 0 || max_prefix_tokens < 0) return PKV_ERR_SHAPE;
    if ((int64_t)max_prefix_tokens > (int64_t)max_blocks_per_seq * cache->block_size) return PKV_ERR_SHAPE;
    if (cache->num_kv_heads > 65535) return PKV_ERR_SHAPE;
    const int64_t prefix_tiles = (max_prefix_tokens + 15) / 16;
    int64_t ct;
    if (chunk_tokens) {
        if (chunk_tokens < 0 || chunk_tokens % 16 != 0 || chunk_tokens / 16 > kPrefixChunkTilesMax) return PKV_ERR_SHAPE;
        ct = chunk_tokens / 16;
    } else {
        // about kPrefixTargetWorkgroups workgroups for the whole prefix pass
        ct = (prefix_tiles * num_groups * cache->num_kv_heads + kPrefixTargetWorkgroups - 1) / kPrefixTargetWorkgroups;
        ct = ct < 8 ? 8 : (ct > kPrefixChunkTilesMax ? kPrefixChunkTilesMax : ct);
    }
    const int64_t mc = (prefix_tiles + ct - 1) / ct;
    if (mc > 65535) return PKV_ERR_SHAPE;
    const int32_t group = num_q_heads / cache->num_kv_heads;
    pp->chunk_tiles = (int32_t)ct;
    pp->max_chunks = num_groups ? (int32_t)mc : 0;
    pp->fast = fast_layout(num_seqs, cache->num_kv_heads, group, cache->head_dim);
    const uint64_t rows = (uint64_t)num_seqs * cache->num_kv_heads * (uint64_t)pp->max_chunks * group;
    pp->pml_bytes = align_up(rows * sizeof(float2), 256);
    pp->pacc_bytes = rows * (uint64_t)cache->head_dim * sizeof(float);
    pp->total = align_up(pp->fast.total, 256) + pp->pml_bytes + pp->pacc_bytes;
    pp->base.partition_tokens = (int32_t)ct * 16;
    pp->base.max_partitions = pp->max_chunks;
    pp->base.workspace_bytes = pp->total;
    return PKV_OK;
}

}  // namespace

PKV_API pkv_status paged_attn_prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                          int32_t num_groups, int32_t max_prefix_tokens,
                                          const pkv_cache_desc* cache, const pkv_decode_opts* opts,
                                          pkv_decode_plan* plan) {
    if (!plan) return PKV_ERR_NULL;
    PrefixPlan pp;
    const pkv_status st = make_prefix_plan(num_seqs, num_q_heads, max_blocks_per_seq, num_groups,
                                           max_prefix_tokens, cache, opts, &pp);
    if (st == PKV_OK) *plan = pp.base;
    return st;
}

PKV_API pkv_status paged_attn_decode_prefix(const void* q, const void* k_cache, const void* v_cache,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                            const int32_t* seq_prefix_tokens, const int32_t* groups,
                                            int32_t num_groups, int32_t max_prefix_tokens, float scale,
                                            float* out, void* workspace, uint64_t workspace_bytes,
                                            const pkv_cache_desc* cache, const pkv_decode_opts* opts,
                                            void* stream) {
    PrefixPlan pp;
    pkv_status st = make_prefix_plan(num_seqs, num_q_heads, max_blocks_per_seq, num_groups, max_prefix_tokens,
                                     cache, opts, &pp);
    if (st != PKV_OK) return st;
    if (num_seqs == 0) return PKV_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !seq_prefix_tokens) return PKV_ERR_NULL;
    if (num_groups > 0 && !groups) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PKV_ERR_ALIGN;
    if (!workspace || workspace_bytes < pp.total) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;

    char* ws = static_cast<char*>(workspace) + kCounterBytes;  // past the counter region
    const WorkspaceLayout& wl = pp.fast;
    pkv::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.num_blocks = cache->num_blocks;
    a.block_size = cache->block_size;
    a.head_dim = cache->head_dim;
    a.dtype = cache->dtype;
    a.scale = scale;
    a.out = out;
    a.ws_rec = reinterpret_cast<int2*>(ws);
    a.ws_ml = reinterpret_cast<float2*>(ws + wl.rec_bytes);
    a.ws_acc = reinterpret_cast<float*>(ws + wl.rec_bytes + wl.ml_bytes);
    a.part_tokens = 16;
    a.max_parts = pkv::kMaxGridWaves;
    a.grid_waves = opts ? opts->grid_waves : 0;
    a.xcd_balance = opts ? opts->xcd_balance : 0;  // 0: the launch decides
    a.seq_start = seq_prefix_tokens;
    a.groups = groups;
    a.num_groups = num_groups;
    a.prefix_chunk_tiles = pp.chunk_tiles;
    a.prefix_max_chunks = pp.max_chunks;
    const uint64_t poff = align_up(wl.total - kCounterBytes, 256);
    a.ws_pml = reinterpret_cast<float2*>(ws + poff);
    a.ws_pacc = reinterpret_cast<float*>(ws + poff + pp.pml_bytes);
    const hipError_t e = pkv::launch_decode_prefix(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

namespace {

// Several new tokens per sequence: chunks of the context per (sequence, KV
// head, row block of 16 * waves rows) and the chunk partials.
// With one wave per row block and no chunk asked for, the tiles are split in
// equal runs over the resident waves instead (partials per slot unit + wave,
// 16 rows each, after one record per unit, as in fast_layout).
struct MultiPlan {
    pkv_decode_plan base;
    int32_t chunk_tiles, max_chunks, row_blocks, waves;
    bool split_runs;
    uint64_t pml_bytes, pacc_bytes, total;
    WorkspaceLayout runs;
};

pkv_status make_multi_plan(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                           int32_t max_blocks_per_seq, const pkv_cache_desc* cache, const pkv_decode_opts* opts,
                           MultiPlan* mp) {
    pkv_decode_opts o = opts ? *opts : pkv_decode_opts{0, PKV_KERNEL_AUTO, 0};
    const int32_t chunk_tokens = o.partition_tokens;
    o.partition_tokens = 0;
    o.kernel = PKV_KERNEL_FAST;
    pkv_status st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, &o, &mp->base);
    if (st != PKV_OK) return st;
    if (cache->block_size < 16) return PKV_ERR_UNSUPPORTED;  // the chunk kernel reads whole 16-token tiles of one block
    if (num_q_heads / cache->num_kv_heads > 8 || cache->head_dim != 128)
        return PKV_ERR_UNSUPPORTED;  // up to 8 heads per KV head, head dim 128
    if (opts && opts->kernel != PKV_KERNEL_AUTO && opts->kernel != PKV_KERNEL_FAST) return PKV_ERR_UNSUPPORTED;
    if (total_q < 0 || max_q_len < 1) return PKV_ERR_SHAPE;
    const int32_t group = num_q_heads / cache->num_kv_heads;
    // Groups of 16 query rows per workgroup: one when a sequence's rows fit a
    // group (speculative decoding: every wave then loads its own tiles and
    // all workgroups fit on the chip at once), 4 (one wave each), or 16 (two
    // per wave, 8 waves) so that up to 256 rows share each tile read.
    const int64_t rows_max = (int64_t)max_q_len * group;
    const int32_t waves = rows_max <= 16 ? 1 : rows_max <= 64 ? 4 : 16;
    const int64_t rb = (rows_max + 16 * waves - 1) / (16 * waves);
    if (rb * cache->num_kv_heads > 65535 || (int64_t)max_q_len > 65535 || num_seqs > INT32_MAX - 1) return PKV_ERR_SHAPE;
    mp->waves = waves;
    mp->row_blocks = (int32_t)rb;
    mp->split_runs = waves == 1 && chunk_tokens == 0;
    if (mp->split_runs) {
        const uint64_t units = (uint64_t)num_seqs * (uint64_t)cache->num_kv_heads;
        const uint64_t slots = units + (uint64_t)pkv::kMaxGridWaves;
        WorkspaceLayout& w = mp->runs;
        w.rec_bytes = align_up(units * sizeof(int2), 256);
        w.ml_bytes = align_up(slots * 16 * sizeof(float2), 256);
        w.acc_bytes = slots * 16 * (uint64_t)cache->head_dim * sizeof(float);
        w.total = kCounterBytes + w.rec_bytes + w.ml_bytes + w.acc_bytes;
        mp->chunk_tiles = 0;
        mp->max_chunks = 0;
        mp->pml_bytes = mp->pacc_bytes = 0;
        mp->total = w.total;
        mp->base.partition_tokens = 16;
        mp->base.max_partitions = pkv::kMaxGridWaves;
        mp->base.grid_blocks = opts ? opts->grid_waves : 0;
        mp->base.threads_per_block = 64;
        mp->base.workspace_bytes = mp->total;
        return PKV_OK;
    }
    const int64_t tiles = ((int64_t)max_blocks_per_seq * cache->block_size + 15) / 16;
    int64_t ct;
    if (chunk_tokens) {
        if (chunk_tokens < 0 || chunk_tokens % 16 != 0 || chunk_tokens / 16 > kMultiChunkTilesMax) return PKV_ERR_SHAPE;
        ct = chunk_tokens / 16;
    } else {
        const int64_t target = waves == 16 ? kMultiWideTargetWorkgroups : kPrefixTargetWorkgroups;
        ct = (tiles * num_seqs * cache->num_kv_heads * rb + target - 1) / target;
        ct = ct < 8 ? 8 : (ct > kMultiChunkTilesMax ? kMultiChunkTilesMax : ct);
    }
    const int64_t mc = (tiles + ct - 1) / ct;
    if (mc > 65535) return PKV_ERR_SHAPE;
    mp->chunk_tiles = (int32_t)ct;
    mp->max_chunks = (int32_t)mc;
    const uint64_t rows = (uint64_t)total_q * num_q_heads * (uint64_t)mc;
    mp->pml_bytes = align_up(rows * sizeof(float2), 256);
    mp->pacc_bytes = rows * (uint64_t)cache->head_dim * sizeof(float);
    mp->total = kCounterBytes + mp->pml_bytes + mp->pacc_bytes;
    mp->base.partition_tokens = (int32_t)ct * 16;
    mp->base.max_partitions = mp->max_chunks;
    mp->base.grid_blocks = (int64_t)num_seqs * cache->num_kv_heads * rb * mc;
    mp->base.threads_per_block = 64 * (waves == 16 ? 8 : waves);
    mp->base.workspace_bytes = mp->total;
    return PKV_OK;
}

}  // namespace

PKV_API pkv_status paged_attn_multi_plan(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                                         int32_t max_blocks_per_seq, const pkv_cache_desc* cache,
                                         const pkv_decode_opts* opts, pkv_decode_plan* plan) {
    if (!plan) return PKV_ERR_NULL;
    MultiPlan mp;
    const pkv_status st = make_multi_plan(num_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq, cache, opts, &mp);
    if (st == PKV_OK) *plan = mp.base;
    return st;
}

PKV_API pkv_status paged_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, const int32_t* cu_q_lens, int32_t num_seqs,
                                           int32_t total_q, int32_t max_q_len, int32_t num_q_heads, float scale,
                                           float* out, void* workspace, uint64_t workspace_bytes,
                                           const pkv_cache_desc* cache, const pkv_decode_opts* opts, void* stream) {
    MultiPlan mp;
    pkv_status st = make_multi_plan(num_seqs, total_q, max_q_len, num_q_heads, max_blocks_per_seq, cache, opts, &mp);
    if (st != PKV_OK) return st;
    if (num_seqs == 0 || total_q == 0) return PKV_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !cu_q_lens || !out) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PKV_ERR_ALIGN;
    if (!workspace || workspace_bytes < mp.total) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    char* ws = static_cast<char*>(workspace);
    pkv::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.num_blocks = cache->num_blocks;
    a.block_size = cache->block_size;
    a.head_dim = cache->head_dim;
    a.dtype = cache->dtype;
    a.scale = scale;
    a.out = out;
    a.cu_q = cu_q_lens;
    a.total_q = total_q;
    a.max_q_len = max_q_len;
    a.multi_row_blocks = mp.row_blocks;
    a.multi_waves = mp.waves;
    a.prefix_chunk_tiles = mp.chunk_tiles;
    a.prefix_max_chunks = mp.max_chunks;
    a.multi_split_runs = mp.split_runs ? 1 : 0;
    a.ws_cnt = reinterpret_cast<uint32_t*>(ws);  // the counter region
    ws += kCounterBytes;
    if (mp.split_runs) {
        a.ws_rec = reinterpret_cast<int2*>(ws);
        a.ws_ml = reinterpret_cast<float2*>(ws + mp.runs.rec_bytes);
        a.ws_acc = reinterpret_cast<float*>(ws + mp.runs.rec_bytes + mp.runs.ml_bytes);
        a.grid_waves = opts ? opts->grid_waves : 0;
    } else {
        a.ws_pml = reinterpret_cast<float2*>(ws);
        a.ws_pacc = reinterpret_cast<float*>(ws + mp.pml_bytes);
    }
    const hipError_t e = pkv::launch_decode_multi(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_API const char* pkv_status_string(pkv_status status) {
    // A caller may pass any int: read its bits as one (loading an out-of-range
    // value as the enum type is undefined behaviour in C++).
    int code = 0;
    static_assert(sizeof(code) == sizeof(status), "pkv_status is int-sized");
    std::memcpy(&code, &status, sizeof(code));
    switch (code) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_SHAPE: return "invalid or inconsistent size";
        case PKV_ERR_DTYPE: return "unknown element type";
        case PKV_ERR_UNSUPPORTED: return "no kernel for this shape";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PKV_ERR_HIP: return "HIP runtime error while enqueueing";
        case PKV_ERR_ALIGN: return "pointer not 16-byte aligned";
        case PKV_ERR_NO_BLOCKS: return "not enough free blocks in the pool";
        case PKV_ERR_SEQ: return "unknown, repeated or existing sequence id";
        case PKV_ERR_TOO_LARGE: return "needs more scratch than the allocation-free entry point holds";
    }
    return "unknown status";
}

PKV_API const char* pkv_version(void) { return "pagedkv 0.1.0 gfx950"; }
