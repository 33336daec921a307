/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged KV-cache append and single-token
 * decode attention on AMD Instinct MI355X (gfx950).
 *
 * The method (pages this library follows):
 *  - Attention(Q,K,V) = softmax(Q K^T / sqrt(d_head)) V; at decode time each
 *    sequence contributes one query row per head and attends over every cached
 *    key/value of that sequence.  Page "x321.org/?p=939", section "First
 *    understand what the KV cache is storing".
 *  - The KV cache grows by one token per step and old K/V are reused as is:
 *    same page and section.
 *  - The cache of a sequence is cut into fixed-size blocks; a block table maps
 *    each logical block to a physical block anywhere in a shared pool, and the
 *    attention kernel follows that mapping in logical order.  Page
 *    "x321.org/?p=939", section "PagedAttention borrows an operating-system
 *    trick"; page "chenhuiyu.github.io/blog/llm-infra-vllm-en", sections "Why
 *    naive KV allocation wastes memory" and "Logical continuity, physical
 *    flexibility".
 *  - Blocks holding an identical prefix may be named by several block tables;
 *    page "praveentn.live/architecture/quiz/pagedattention-kv-cache-constraint",
 *    section "What the change bought".  Reads through shared blocks are
 *    supported; copying a shared block before writing into it is the caller's
 *    job.
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are HIP device pointers, (host) are host
 *    pointers.  Every array is dense and row-major as documented.  The caller
 *    owns all memory; the library allocates nothing and keeps no pointer after
 *    a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; the caller keeps the buffers alive until the stream
 *    has passed the enqueued work.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error nothing is enqueued (all-or-nothing).  No C++ exception crosses the
 *    ABI.
 *  - Device-side contents are not validated on the host, but the kernels stay
 *    inside the buffers whatever those contents are: an out-of-range slot is
 *    not written; an out-of-range block-table entry or context length turns
 *    the affected output rows into NaN.
 *  - Layouts.  Cache pools K and V: [num_blocks][num_kv_heads][block_size]
 *    [head_dim] of `dtype`.  A slot number is physical_block * block_size +
 *    offset.  Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is NULL */
    PKV_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
    PKV_ERR_DTYPE = 3,       /* unknown element type */
    PKV_ERR_UNSUPPORTED = 4, /* valid, but no kernel for this head_dim / block_size / group size */
    PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than paged_attn_workspace_bytes */
    PKV_ERR_HIP = 6,         /* the HIP runtime reported an error while enqueueing */
    PKV_ERR_ALIGN = 7,       /* a pointer is not 16-byte aligned */
    PKV_ERR_NO_BLOCKS = 8,   /* block manager: the pool has too few free blocks */
    PKV_ERR_SEQ = 9,         /* block manager: unknown, repeated or already existing sequence id */
    PKV_ERR_TOO_LARGE = 10   /* paged_attn_decode_noalloc: the call needs more than PKV_NOALLOC_SCRATCH_BYTES */
} pkv_status;

typedef enum pkv_dtype {
    PKV_F32 = 0, /* IEEE binary32 */
    PKV_BF16 = 1 /* bfloat16 (upper half of a binary32) */
} pkv_dtype;

/* Shape of the K and V pools (host struct).  Supported: head_dim 64, 128 or
 * 256; block_size 8, 16, 32 or 64; dtype PKV_F32 or PKV_BF16;
 * num_blocks * block_size < 2^31. */
typedef struct pkv_cache_desc {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype; /* a pkv_dtype */
} pkv_cache_desc;

/* Kernel families of paged_attn_decode. */
#define PKV_KERNEL_AUTO 0    /* library choice */
#define PKV_KERNEL_GENERIC 1 /* any supported shape and dtype */
#define PKV_KERNEL_FAST 2    /* bf16, head_dim 128, block_size 8, 16, 32 or 64, group size 1, 2, 4 or 8
                                (block size 8: a 16-token tile reads two blocks); or, with
                                block_size 16, 32 or 64, group size 16 at head_dim 128 and group
                                size 1 .. 16 at head_dim 64 or 256 (the split-run kernel of
                                paged_attn_decode_multi with one query row per sequence: its rows
                                are the group's heads) */

/* Optional decode settings (host struct; NULL = all defaults). */
typedef struct pkv_decode_opts {
    int32_t partition_tokens; /* generic kernel: tokens per split-K partition, a multiple of 64;
                                 0 = library choice */
    int32_t kernel;           /* a PKV_KERNEL_* value */
    int32_t grid_waves;       /* fast kernel: number of waves that share the work, 1 ..
                                 PKV_MAX_GRID_WAVES; 0 = library choice: as many as the device
                                 keeps resident, or half of them when num_seqs * num_kv_heads
                                 is at most a quarter of that (fewer, longer units) */
    int32_t xcd_balance;      /* fast kernel: work share of each wave on an odd-numbered XCD, in
                                 64ths of an equal share (waves on even XCDs get 128 minus it),
                                 1 .. 127; 64 = equal shares; 0 = library choice
                                 (PKV_XCD_BALANCE_DEFAULT with two waves per SIMD, equal shares
                                 when the library launches one per SIMD and in the suffix pass
                                 of paged_attn_decode_prefix).  Applies when the
                                 wave count is a multiple of 8 and there are enough tiles for
                                 every wave to hold one.  With it, when every XCD has an even
                                 number of waves, the first half of each XCD's waves (in
                                 dispatch order) take 84/64 of their share and the second half
                                 44/64.  Results do not depend on it. */
} pkv_decode_opts;

/* On the MI355X boxes measured, waves on odd-numbered XCDs drained the same reads 4-9% more
 * slowly than waves on even ones, so an equal split left the odd XCDs finishing last; their
 * waves get this share (in 64ths) by default. */
#define PKV_XCD_BALANCE_DEFAULT 62

/* Upper bound of the fast kernel's wave count (sizes its workspace). */
#define PKV_MAX_GRID_WAVES 8192

/* Every decode workspace (paged_attn_decode, _prefix, _multi) starts with a
 * counter region of this many bytes: 65536 uint32 arrival counters that
 * paged_attn_decode_multi uses to merge a unit's context chunks in the chunk
 * kernel itself.  They must be zero before a workspace's first use with
 * paged_attn_decode_multi (zero-fill a workspace when allocating it); every
 * call leaves them zero once its kernels have completed, and no entry point
 * writes anything else there, so one workspace can serve all of them in turn. */
#define PKV_WORKSPACE_COUNTER_BYTES (65536u * 4u)

/* What paged_attn_decode will launch for a given shape (host struct). */
typedef struct pkv_decode_plan {
    int32_t kernel;           /* PKV_KERNEL_GENERIC or PKV_KERNEL_FAST */
    int32_t partition_tokens; /* generic: tokens per partition; fast: 16 (tokens per work tile) */
    int32_t max_partitions;   /* generic: ceil(max_blocks_per_seq * block_size / partition_tokens);
                                 fast: most partial results one (sequence, KV head) can leave */
    int32_t threads_per_block;
    int64_t grid_blocks;      /* generic: workgroups of the partition kernel; fast: the requested
                                 wave count, or 0 for the library's choice (see grid_waves) */
    uint64_t workspace_bytes; /* required workspace (0 when nothing needs merging) */
} pkv_decode_plan;

/*
 * paged_kv_write -- append step: store each new token's key and value rows in
 * its slot (page "x321.org/?p=939", section "First understand what the KV
 * cache is storing": the cache grows as tokens are produced).
 *
 *   k_new, v_new  (device) [num_tokens][num_kv_heads][head_dim] of cache->dtype
 *   slot_mapping  (device) int32 [num_tokens]; slot s goes to block s / block_size,
 *                 offset s % block_size; s < 0 = skip this token; s >= num_blocks *
 *                 block_size is not written
 *   k_cache, v_cache (device) pools as described above, updated in place
 *   cache         (host) pool shape
 *
 * The copy is bit-exact (NaN payloads, -0.0 and subnormals arrive unchanged).
 * Two tokens with the same slot race; the result is then unspecified.
 * num_tokens == 0 enqueues nothing and returns PKV_OK.
 */
pkv_status paged_kv_write(const void *k_new, const void *v_new, const int32_t *slot_mapping,
                          int32_t num_tokens, void *k_cache, void *v_cache,
                          const pkv_cache_desc *cache, void *stream);

/*
 * paged_attn_plan -- host-only: which kernel, partition size, grid and
 * workspace size paged_attn_decode uses for these sizes.  Touches no device.
 */
pkv_status paged_attn_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                           const pkv_cache_desc *cache, const pkv_decode_opts *opts,
                           pkv_decode_plan *plan);

/* paged_attn_workspace_bytes -- host-only: plan->workspace_bytes of paged_attn_plan. */
pkv_status paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_blocks_per_seq, const pkv_cache_desc *cache,
                                      const pkv_decode_opts *opts, uint64_t *bytes);

/*
 * paged_attn_decode -- single-token decode attention over paged K/V:
 * out[i][h] = softmax(scale * q[i][h] . K_i^T) V_i, where K_i, V_i are the
 * context_lens[i] tokens of sequence i, token j read from physical block
 * block_tables[i][j / block_size] at offset j % block_size, KV head
 * h / (num_q_heads / num_kv_heads)  (page "x321.org/?p=939", sections "First
 * understand what the KV cache is storing" and "PagedAttention borrows an
 * operating-system trick").
 *
 *   q             (device) [num_seqs][num_q_heads][head_dim] of cache->dtype
 *   k_cache, v_cache (device) pools
 *   block_tables  (device) int32 [num_seqs][max_blocks_per_seq]; only the first
 *                 ceil(context_lens[i] / block_size) entries of row i are read;
 *                 rows may name the same physical blocks (shared prefixes)
 *   context_lens  (device) int32 [num_seqs]; tokens of each sequence, including
 *                 the one appended this step; 0 gives an all-zero output row
 *   scale         softmax scale (normally 1/sqrt(head_dim))
 *   out           (device) fp32 [num_seqs][num_q_heads][head_dim]
 *   workspace     (device) scratch of at least paged_attn_workspace_bytes bytes,
 *                 16-byte aligned; may be NULL when that size is 0.  Its first
 *                 PKV_WORKSPACE_COUNTER_BYTES bytes are a counter region that
 *                 only paged_attn_decode_multi uses; the rest needs no
 *                 initialisation and is garbage afterwards.
 *   opts          (host) NULL or settings
 *
 * Work splitting.  The generic kernel cuts every sequence into partitions of
 * plan.partition_tokens tokens and merges them in a second kernel.  The fast
 * kernel lays all (sequence, KV head, 16-token tile) triples end to end and
 * gives each wave of its grid a contiguous run of tiles (equal runs, or runs
 * weighted by the wave's XCD and its half of the XCD's waves: opts->xcd_balance), so a long sequence spreads
 * over several waves and many short ones share a wave; a second kernel merges
 * the pieces of each (sequence, KV head); at group size 16 and head dims 64
 * and 256 the runs are equal and the pieces go through the multi-query path's
 * tile pipeline and merge.
 * Either way every piece yields a
 * running max, a softmax denominator and an unnormalised output, merged by a
 * log-sum-exp combine.  Results do not depend on the physical placement of
 * blocks (the summation order is fixed by logical token positions, the wave
 * count and the XCD shares).
 * Calls that share a workspace must be serialised on one stream.
 */
pkv_status paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                             float scale, float *out, void *workspace, uint64_t workspace_bytes,
                             const pkv_cache_desc *cache, const pkv_decode_opts *opts,
                             void *stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results, with the workspace
 * taken from a device array that the library holds on every GPU it runs on
 * (PKV_NOALLOC_SCRATCH_BYTES, kept until the process ends).  The call
 * allocates nothing; the first call on a device looks the array's address up
 * (hipGetSymbolAddress) with that device current.
 *
 * Arguments as paged_attn_decode without workspace and workspace_bytes.  A
 * call whose plan (paged_attn_plan) needs a workspace larger than
 * PKV_NOALLOC_SCRATCH_BYTES runs the generic kernel instead when opts leaves
 * the kernel to the library (PKV_KERNEL_AUTO) and that plan fits (the
 * split-run shapes of PKV_KERNEL_FAST size 16 rows for every one of up to
 * PKV_MAX_GRID_WAVES partial slots); otherwise it returns PKV_ERR_TOO_LARGE
 * and enqueues nothing.
 * Nothing in the array needs clearing: every byte a call reads was written
 * earlier in that call.  All calls on one GPU share its array, so calls that
 * may overlap on one GPU (two streams, two threads) race: serialise them.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
pkv_status paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     float scale, float *out, const pkv_cache_desc *cache,
                                     const pkv_decode_opts *opts, void *stream);

/*
 * paged_attn_prefix_plan -- host-only plan of paged_attn_decode_prefix: the
 * fast kernel's plan with partition_tokens = tokens per prefix chunk,
 * max_partitions = chunks of the longest prefix, workspace_bytes = the
 * workspace paged_attn_decode_prefix needs.  Shapes as PKV_KERNEL_FAST with
 * block_size 16, 32 or 64 and group size at most 8 (PKV_ERR_UNSUPPORTED
 * otherwise).
 * opts->partition_tokens, if nonzero, sets the prefix chunk: a multiple of 16,
 * at most 1024.
 */
pkv_status paged_attn_prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                  int32_t num_groups, int32_t max_prefix_tokens,
                                  const pkv_cache_desc *cache, const pkv_decode_opts *opts,
                                  pkv_decode_plan *plan);

/*
 * paged_attn_decode_prefix -- the result of paged_attn_decode for a batch in
 * which groups of sequences share the first blocks of their block tables
 * (parallel samples of one prompt: page
 * "praveentn.live/architecture/quiz/pagedattention-kv-cache-constraint",
 * section "What the change bought").  Each shared block is read from HBM once
 * per group and KV head rather than once per sequence: a prefix pass runs one
 * wave per member over the group's prefix tiles held in LDS, the fast kernel
 * covers each sequence's own tokens after its prefix, and a merge combines
 * the pieces by log-sum-exp in token order.
 *
 *   seq_prefix_tokens (device) int32 [num_seqs]: tokens at the start of
 *                 sequence i that its group shares, a whole number of blocks
 *                 and at most context_lens[i]; 0 for a sequence in no group
 *   groups       (device) int32 [num_groups][2]: first sequence and member
 *                 count (1 .. 8) of each group.  Members are consecutive, have
 *                 equal seq_prefix_tokens and the same first
 *                 seq_prefix_tokens / block_size table entries (the first
 *                 member's entries are read).
 *   num_groups   (host) rows of `groups`; 0 is allowed (then every
 *                 seq_prefix_tokens entry must be 0)
 *   max_prefix_tokens (host) at least every seq_prefix_tokens entry, at most
 *                 max_blocks_per_seq * block_size; sizes the prefix grid
 * Everything else as paged_attn_decode; the workspace is
 * paged_attn_prefix_plan's workspace_bytes (no initialisation needed).
 *
 * Device contents are not validated on the host.  A prefix that is not a
 * whole number of blocks, longer than its sequence or than max_prefix_tokens,
 * or that differs from its group's, gives NaN rows.  A sequence with a
 * nonzero prefix that no group lists gives unspecified rows.  The kernels
 * stay inside their buffers in every case.
 */
pkv_status paged_attn_decode_prefix(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                    const int32_t *seq_prefix_tokens, const int32_t *groups,
                                    int32_t num_groups, int32_t max_prefix_tokens, float scale,
                                    float *out, void *workspace, uint64_t workspace_bytes,
                                    const pkv_cache_desc *cache, const pkv_decode_opts *opts,
                                    void *stream);

/*
 * paged_attn_multi_plan -- host-only plan of paged_attn_decode_multi:
 * partition_tokens = tokens per context chunk, max_partitions = chunks of the
 * longest table, grid_blocks = workgroups of the chunk kernel,
 * workspace_bytes.  Shapes as PKV_KERNEL_FAST with block_size 16, 32 or 64
 * and group size at most 8 (PKV_ERR_UNSUPPORTED otherwise).  The rows of a KV head, max_q_len *
 * (num_q_heads / num_kv_heads), go to workgroups of 1, 4 or 16 groups of 16
 * rows (the fewest that hold them, at most 16; 16 groups are 8 waves of two
 * groups each, so grid threads = 64, 256 or 512), in row blocks; at most 65535
 * row blocks in all.  opts->partition_tokens, if nonzero, sets the chunk (a
 * multiple of 16, at most 2048).
 * With one wave per row block (max_q_len * G <= 16) and no chunk asked for,
 * the 16-token tiles of all (sequence, KV head) pairs are instead split in
 * equal runs over opts->grid_waves waves (0: the waves the device keeps
 * resident): partition_tokens = 16, max_partitions = PKV_MAX_GRID_WAVES,
 * grid_blocks = opts->grid_waves, and the workspace holds one record per
 * (sequence, KV head) and partial slots of 16 rows.
 */
pkv_status paged_attn_multi_plan(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq, const pkv_cache_desc *cache,
                                 const pkv_decode_opts *opts, pkv_decode_plan *plan);

/*
 * paged_attn_decode_multi -- attention from several new tokens per sequence
 * over the paged cache, each token seeing the tokens up to its own position:
 * the step of a prefill split into chunks, or the verification of several
 * drafted tokens (page "x321.org/?p=939", section "Continuous batching is the
 * other half of the story"; attention over the existing context, section
 * "First understand what the KV cache is storing").  Sequence i's new tokens
 * are the last q_len = cu_q_lens[i + 1] - cu_q_lens[i] of its
 * context_lens[i] tokens (already written with paged_kv_write); new token j
 * is at position context_lens[i] - q_len + j and
 *   out[cu_q_lens[i] + j][h] = softmax over tokens 0 .. that position of
 *                              scale * q[cu_q_lens[i] + j][h] . K  times V.
 * Each context tile is read once per (sequence, KV head) for all of its new
 * tokens; the q . K and P . V products run on the matrix cores.
 *
 *   q            (device) [total_q][num_q_heads][head_dim] bf16
 *   cu_q_lens    (device) int32 [num_seqs + 1], cu_q_lens[0] = 0, nondecreasing,
 *                cu_q_lens[num_seqs] = total_q
 *   max_q_len    (host) at least every q_len; sizes the grid
 *   out          (device) fp32 [total_q][num_q_heads][head_dim]
 * Everything else as paged_attn_decode; the workspace is
 * paged_attn_multi_plan's, with its counter region (PKV_WORKSPACE_COUNTER_BYTES)
 * zero before its first use; the rest needs no initialisation.  When the
 * counters of all (sequence, KV head, row block) units fit that region, the
 * last chunk workgroup of a unit to finish merges the unit's chunks (one
 * kernel); larger batches merge them in a second kernel.
 *
 * Device contents are not validated on the host.  A sequence with
 * q_len > max_q_len or > context_lens[i], or a length past the table, gets NaN
 * rows (for its first max_q_len tokens); q_len < 1 or offsets outside
 * [0, total_q] leave that sequence's rows unwritten.  A block-table entry
 * outside the pool among the blocks a (sequence, KV head) reads gives NaN
 * rows: all of its rows on the split runs, the rows that see the entry's
 * chunk with chunks.  The kernels stay inside their buffers.
 */
pkv_status paged_attn_decode_multi(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *cu_q_lens, int32_t num_seqs,
                                   int32_t total_q, int32_t max_q_len, int32_t num_q_heads, float scale,
                                   float *out, void *workspace, uint64_t workspace_bytes,
                                   const pkv_cache_desc *cache, const pkv_decode_opts *opts, void *stream);

/*
 * What the calling thread's last successful paged_attn_decode or
 * paged_attn_decode_prefix call launched (host struct), so that a caller can
 * see which kernel ran and the launch choices the library made:
 *   kernel            PKV_KERNEL_FAST or PKV_KERNEL_GENERIC (0 before any call)
 *   grid              fast: waves sharing the tiles; generic: workgroups of the
 *                     partition kernel
 *   xcd_balance       fast: the odd-XCD share used, in 64ths (64 = equal); 0 generic
 *   partition_tokens  fast: 16 (tokens per tile); generic: tokens per partition
 *   k_stream          fast: 1 when K rows were read with non-temporal loads
 *                     (the units were few and long, at most 1/16 of the
 *                     resident waves, the prefix path's suffix pass, or head
 *                     dim 256), 0 when with ordinary loads; V rows are always
 *                     streamed; 0 generic
 * Per thread and per process; NULL info gives PKV_ERR_NULL.  For callers that
 * check or report the path taken (for example a benchmark).
 */
typedef struct pkv_launch_info {
    int32_t kernel;
    int32_t grid;
    int32_t xcd_balance;
    int32_t partition_tokens;
    int32_t k_stream;
} pkv_launch_info;
pkv_status pkv_last_launch_info(pkv_launch_info *info);

/* Human-readable name of a status code (static string). */
const char *pkv_status_string(pkv_status status);

/* Library version string (static). */
const char *pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
