/*
 * pagedkv_blocks.h -- host-side block manager of a paged KV cache, and the
 * device block copy it asks for.  Part of libpagedkv.so (same status codes as
 * pagedkv.h).
 *
 * What the manager does (pages it follows):
 *  - A sequence's cache is a list of fixed-size blocks taken from a shared pool
 *    as the sequence grows; only the last block can be partly filled, so the
 *    waste per sequence is under one block.  Page "x321.org/?p=939", section
 *    "PagedAttention borrows an operating-system trick" (a request grows by
 *    taking more free blocks when it needs them); page
 *    "chenhuiyu.github.io/blog/llm-infra-vllm-en", sections "Why naive KV
 *    allocation wastes memory" and "Logical continuity, physical flexibility"
 *    (block counts, slack, one table per sequence).
 *  - Sequences forked from a common prefix name the same physical blocks
 *    (reference counted); a shared block that is only partly filled is copied
 *    before a sequence writes into it (copy-on-write).  Page
 *    "praveentn.live/architecture/quiz/pagedattention-kv-cache-constraint",
 *    section "What the change bought".
 *
 * Policy choices the pages leave open (stated here once):
 *  - A new block is always the lowest-numbered free block, so every result is
 *    a function of the call sequence alone.
 *  - When several sharers of one partly filled block append in the same call,
 *    they are served in the order given; the last remaining sharer keeps the
 *    original block and the others get copies.
 *  - Every call is all-or-nothing: on any error the manager is unchanged.
 *
 * The manager is plain host memory; it is not thread-safe (callers serialise
 * calls on one manager).  Sequence ids are caller-chosen 64-bit integers.
 */
#ifndef PAGEDKV_BLOCKS_H
#define PAGEDKV_BLOCKS_H

#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* New manager over a pool of num_blocks blocks of block_size tokens (both > 0,
 * num_blocks * block_size < 2^31).  *out receives the handle; free it with
 * pkv_bm_destroy.  PKV_ERR_SHAPE on bad sizes, PKV_ERR_NULL if out is NULL. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager **out);

/* Release a manager (NULL is ignored). */
void pkv_bm_destroy(pkv_block_manager *bm);

/* Free blocks in the pool (-1 if bm is NULL). */
int32_t pkv_bm_num_free(const pkv_block_manager *bm);

/* Number of sequences holding block `block` (0 for a free block, -1 if the id
 * is outside the pool or bm is NULL). */
int32_t pkv_bm_refcount(const pkv_block_manager *bm, int32_t block);

/* Tokens of sequence seq_id (-1 if unknown or bm is NULL). */
int32_t pkv_bm_seq_len(const pkv_block_manager *bm, int64_t seq_id);

/* Register a new sequence holding num_tokens >= 0 tokens (a prompt) and give
 * it ceil(num_tokens / block_size) blocks.  PKV_ERR_SEQ if the id exists,
 * PKV_ERR_NO_BLOCKS if the pool has too few free blocks. */
pkv_status pkv_bm_add(pkv_block_manager *bm, int64_t seq_id, int32_t num_tokens);

/* New sequence `child` sharing every block of `parent` (same length).
 * PKV_ERR_SEQ if the parent is unknown or the child exists. */
pkv_status pkv_bm_fork(pkv_block_manager *bm, int64_t parent, int64_t child);

/* Drop a sequence; blocks no other sequence holds return to the pool.
 * PKV_ERR_SEQ if unknown. */
pkv_status pkv_bm_free(pkv_block_manager *bm, int64_t seq_id);

/*
 * One decode step: append one token to each of the n listed sequences (ids
 * distinct).  For sequence k:
 *   - its length is a multiple of block_size: a new block is added and the
 *     token goes to its offset 0;
 *   - its last block is partly filled and held by no other sequence: the
 *     token goes to the next offset of that block;
 *   - its last block is partly filled and shared: a new block replaces it in
 *     this sequence's table, the pair (old, new) is appended to `copies`
 *     (host, int32 [max_copies][2]: source block, destination block), and
 *     the token goes to the next offset of the new block.  The caller copies
 *     the blocks (paged_block_copy) before writing the step's tokens.
 * slot_mapping (host, int32 [n]) receives each token's slot, block *
 * block_size + offset, for paged_kv_write.  *num_copies receives the number
 * of pairs written.  PKV_ERR_SEQ for an unknown or repeated id,
 * PKV_ERR_NO_BLOCKS if the pool cannot supply the new blocks, PKV_ERR_SHAPE if
 * more than max_copies copies would be needed.
 */
pkv_status pkv_bm_append(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                         int32_t *slot_mapping, int32_t *copies, int32_t max_copies,
                         int32_t *num_copies);

/* Slots of tokens [first, first + count) of sequence seq_id (host, int32
 * [count]), e.g. to write a prompt with paged_kv_write.  PKV_ERR_SHAPE if the
 * range is outside [0, length). */
pkv_status pkv_bm_slots(const pkv_block_manager *bm, int64_t seq_id, int32_t first, int32_t count,
                        int32_t *slots);

/* Block tables and lengths of n sequences, as paged_attn_decode takes them:
 * tables (host, int32 [n][max_blocks_per_seq], unused entries -1), context_lens
 * (host, int32 [n]).  PKV_ERR_SHAPE if a sequence has more than
 * max_blocks_per_seq blocks. */
pkv_status pkv_bm_block_tables(const pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                               int32_t max_blocks_per_seq, int32_t *tables, int32_t *context_lens);

/*
 * paged_block_copy -- copy whole blocks inside the K and V pools (every KV
 * head, every slot), bit for bit: for each pair p, block pairs[2p + 1] becomes
 * a copy of block pairs[2p].  This is the device half of copy-on-write (page
 * "praveentn.live/architecture/quiz/pagedattention-kv-cache-constraint",
 * section "What the change bought").
 *
 *   k_cache, v_cache (device) pools [num_blocks][num_kv_heads][block_size][head_dim]
 *   pairs       (device) int32 [num_pairs][2] (source, destination)
 *   cache       (host) pool shape
 *
 * Pairs with an id outside the pool are skipped.  A destination that is also
 * a source, or two pairs with one destination, give unspecified contents.
 * num_pairs == 0 enqueues nothing.
 */
pkv_status paged_block_copy(void *k_cache, void *v_cache, const int32_t *pairs, int32_t num_pairs,
                            const pkv_cache_desc *cache, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_BLOCKS_H */
