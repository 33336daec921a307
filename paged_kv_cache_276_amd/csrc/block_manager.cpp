// block_manager.cpp -- host-side block manager of the paged KV cache (C ABI in
// include/pagedkv_blocks.h).
//
// A sequence is a list of physical block ids plus its token count; block b
// holds refcount[b] sequences.  Free blocks sit in an ordered set and the
// lowest id is always taken first.  Every entry point checks everything it
// needs (including a dry run of the allocation) before it changes anything, so
// an error leaves the manager as it was.
#include <new>
#include <set>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedkv_blocks.h"

#define PKV_API extern "C" __attribute__((visibility("default")))

struct pkv_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;
        int32_t len = 0;
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> refcount;
    std::set<int32_t> free_blocks;
    std::unordered_map<int64_t, Seq> seqs;

    int32_t take() {  // caller has checked that a block is free
        const int32_t b = *free_blocks.begin();
        free_blocks.erase(free_blocks.begin());
        refcount[b] = 1;
        return b;
    }
    void release(int32_t b) {
        if (--refcount[b] == 0) free_blocks.insert(b);
    }
    int32_t blocks_for(int64_t tokens) const {
        return (int32_t)((tokens + block_size - 1) / block_size);
    }
};

namespace {

template <typename F>
pkv_status guarded(F&& f) {
    try {
        return f();
    } catch (const std::bad_alloc&) {
        return PKV_ERR_SHAPE;  // host memory exhausted: treated as an impossible size
    } catch (...) {
        return PKV_ERR_SHAPE;
    }
}

}  // namespace

PKV_API pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager** out) {
    if (!out) return PKV_ERR_NULL;
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0 || (int64_t)num_blocks * block_size > INT32_MAX)
        return PKV_ERR_SHAPE;
    return guarded([&] {
        auto* bm = new pkv_block_manager();
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->refcount.assign((size_t)num_blocks, 0);
        for (int32_t b = 0; b < num_blocks; ++b) bm->free_blocks.insert(bm->free_blocks.end(), b);
        *out = bm;
        return PKV_OK;
    });
}

PKV_API void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

PKV_API int32_t pkv_bm_num_free(const pkv_block_manager* bm) {
    return bm ? (int32_t)bm->free_blocks.size() : -1;
}

PKV_API int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->refcount[block];
}

PKV_API int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

PKV_API pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens) {
    if (!bm) return PKV_ERR_NULL;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (bm->seqs.count(seq_id)) return PKV_ERR_SEQ;
    const int32_t need = bm->blocks_for(num_tokens);
    if ((size_t)need > bm->free_blocks.size()) return PKV_ERR_NO_BLOCKS;
    return guarded([&] {
        pkv_block_manager::Seq s;
        s.blocks.reserve((size_t)need);
        s.len = num_tokens;
        auto& slot = bm->seqs[seq_id];  // may throw before any block is taken
        for (int32_t k = 0; k < need; ++k) s.blocks.push_back(bm->take());
        slot = std::move(s);
        return PKV_OK;
    });
}

PKV_API pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PKV_ERR_SEQ;
    return guarded([&] {
        pkv_block_manager::Seq copy = it->second;
        bm->seqs.emplace(child, std::move(copy));
        for (int32_t b : bm->seqs[child].blocks) ++bm->refcount[b];
        return PKV_OK;
    });
}

PKV_API pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_SEQ;
    for (int32_t b : it->second.blocks) bm->release(b);
    bm->seqs.erase(it);
    return PKV_OK;
}

PKV_API pkv_status pkv_bm_append(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                 int32_t* slot_mapping, int32_t* copies, int32_t max_copies,
                                 int32_t* num_copies) {
    if (!bm || !num_copies) return PKV_ERR_NULL;
    if (n < 0 || max_copies < 0) return PKV_ERR_SHAPE;
    if (n > 0 && (!seq_ids || !slot_mapping)) return PKV_ERR_NULL;
    if (max_copies > 0 && !copies) return PKV_ERR_NULL;
    return guarded([&] {
        // Dry run: ids known and distinct, new blocks and copies needed, with
        // the refcount drops of earlier copies in this call taken into account.
        std::unordered_set<int64_t> seen;
        std::unordered_map<int32_t, int32_t> dropped;  // block -> sharers that copied away
        int64_t need = 0, ncopy = 0;
        for (int32_t k = 0; k < n; ++k) {
            auto it = bm->seqs.find(seq_ids[k]);
            if (it == bm->seqs.end() || !seen.insert(seq_ids[k]).second) return PKV_ERR_SEQ;
            const auto& s = it->second;
            if ((int64_t)s.len + 1 > (int64_t)INT32_MAX / 2) return PKV_ERR_SHAPE;
            if (s.len % bm->block_size == 0) {
                ++need;
            } else {
                const int32_t last = s.blocks.back();
                if (bm->refcount[last] - dropped[last] > 1) {
                    ++need;
                    ++ncopy;
                    ++dropped[last];
                }
            }
        }
        if (need > (int64_t)bm->free_blocks.size()) return PKV_ERR_NO_BLOCKS;
        if (ncopy > max_copies) return PKV_ERR_SHAPE;
        // Apply.
        int32_t c = 0;
        for (int32_t k = 0; k < n; ++k) {
            auto& s = bm->seqs[seq_ids[k]];
            const int32_t off = s.len % bm->block_size;
            int32_t blk;
            if (off == 0) {
                blk = bm->take();
                s.blocks.push_back(blk);
            } else {
                blk = s.blocks.back();
                if (bm->refcount[blk] > 1) {
                    const int32_t fresh = bm->take();
                    copies[2 * c] = blk;
                    copies[2 * c + 1] = fresh;
                    ++c;
                    bm->release(blk);
                    s.blocks.back() = fresh;
                    blk = fresh;
                }
            }
            slot_mapping[k] = blk * bm->block_size + off;
            ++s.len;
        }
        *num_copies = c;
        return PKV_OK;
    });
}

PKV_API pkv_status pkv_bm_slots(const pkv_block_manager* bm, int64_t seq_id, int32_t first, int32_t count,
                                int32_t* slots) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PKV_ERR_SEQ;
    const auto& s = it->second;
    if (first < 0 || count < 0 || (int64_t)first + count > s.len) return PKV_ERR_SHAPE;
    if (count > 0 && !slots) return PKV_ERR_NULL;
    for (int32_t j = 0; j < count; ++j) {
        const int32_t t = first + j;
        slots[j] = s.blocks[(size_t)(t / bm->block_size)] * bm->block_size + t % bm->block_size;
    }
    return PKV_OK;
}

PKV_API pkv_status pkv_bm_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                       int32_t max_blocks_per_seq, int32_t* tables, int32_t* context_lens) {
    if (!bm) return PKV_ERR_NULL;
    if (n < 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
    if (n > 0 && (!seq_ids || !tables || !context_lens)) return PKV_ERR_NULL;
    for (int32_t k = 0; k < n; ++k) {
        auto it = bm->seqs.find(seq_ids[k]);
        if (it == bm->seqs.end()) return PKV_ERR_SEQ;
        if (it->second.blocks.size() > (size_t)max_blocks_per_seq) return PKV_ERR_SHAPE;
    }
    for (int32_t k = 0; k < n; ++k) {
        const auto& s = bm->seqs.find(seq_ids[k])->second;
        int32_t* row = tables + (int64_t)k * max_blocks_per_seq;
        for (int32_t b = 0; b < max_blocks_per_seq; ++b)
            row[b] = (size_t)b < s.blocks.size() ? s.blocks[(size_t)b] : -1;
        context_lens[k] = s.len;
    }
    return PKV_OK;
}
