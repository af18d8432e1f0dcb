// pa_blocks.cpp -- host-side block manager for the paged KV cache (C ABI in
// include/pa.h, functions pa_bm_*).
//
// What it does: the cache is a pool of fixed-size blocks; a sequence gets a
// new block only when its last one is full, and gives all of them back when it
// ends (page "轻量级的vLLM", section 核心机制一：分页 KV Cache).  Sequences
// join and leave the running batch at every step (same page, section
// 核心机制二：连续批处理).  Requests may share the blocks of a common prompt
// prefix (page "vllm-v0 版本介绍", section 为什么需要推理框架？, PagedAttention
// item): here a sequence can be forked, sharing every block with reference
// counts, and a shared last block is copied before the first write into it
// (copy on write; the copy itself is pa_copy_blocks on the GPU).
//
// Policy (fixed, so that results are reproducible):
//  * free blocks form a stack; initially block 0 is on top, then 1, 2, ...;
//    allocation pops, release pushes (most recently freed block reused first);
//  * a sequence's blocks are released from its last block to its first;
//  * an operation that cannot get all the blocks it needs fails with
//    PA_ENOMEM and changes nothing.  So does one that runs out of host memory:
//    every allocation is made before the first change, and no C++ exception
//    crosses the C ABI.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

constexpr int kBlockTokens = 16;

struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
};

}  // namespace

struct pa_block_manager {
    int64_t num_blocks = 0;
    std::vector<int32_t> free_stack;  // back() is the next block handed out
    std::vector<int32_t> refcount;
    std::unordered_map<int64_t, Seq> seqs;

    int32_t pop() {
        const int32_t b = free_stack.back();
        free_stack.pop_back();
        refcount[b] = 1;
        return b;
    }
    void release(int32_t b) {
        if (--refcount[b] == 0) free_stack.push_back(b);
    }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size) {
    if (num_blocks <= 0 || num_blocks > INT32_MAX / kBlockTokens || block_size != kBlockTokens) return nullptr;
    pa_block_manager* m = new (std::nothrow) pa_block_manager;
    if (!m) return nullptr;
    try {
        m->num_blocks = num_blocks;
        m->refcount.assign((size_t)num_blocks, 0);
        m->free_stack.reserve((size_t)num_blocks);  // release never reallocates
        for (int64_t b = num_blocks - 1; b >= 0; --b) m->free_stack.push_back((int32_t)b);
    } catch (...) {
        delete m;
        return nullptr;
    }
    return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int64_t pa_bm_num_free(const pa_block_manager* m) { return m ? (int64_t)m->free_stack.size() : -1; }

int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, int64_t num_tokens) {
    if (!m || num_tokens < 0) return PA_EINVAL;
    if (m->seqs.count(seq_id)) return PA_EINVAL;
    const int64_t need = (num_tokens + kBlockTokens - 1) / kBlockTokens;
    if (need > (int64_t)m->free_stack.size()) return PA_ENOMEM;
    try {
        Seq s;
        s.tokens = num_tokens;
        s.blocks.reserve((size_t)need);
        Seq& dst = m->seqs.emplace(seq_id, std::move(s)).first->second;  // allocations done
        for (int64_t i = 0; i < need; ++i) dst.blocks.push_back(m->pop());
    } catch (...) {
        return PA_ENOMEM;
    }
    return PA_OK;
}

int pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id) {
    if (!m || parent_id == child_id) return PA_EINVAL;
    auto it = m->seqs.find(parent_id);
    if (it == m->seqs.end() || m->seqs.count(child_id)) return PA_EINVAL;
    try {
        Seq child = it->second;  // same blocks, same tokens
        const Seq& c = m->seqs.emplace(child_id, std::move(child)).first->second;  // allocations done
        for (int32_t b : c.blocks) ++m->refcount[b];
    } catch (...) {
        return PA_ENOMEM;
    }
    return PA_OK;
}

int pa_bm_free(pa_block_manager* m, int64_t seq_id) {
    if (!m) return PA_EINVAL;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PA_EINVAL;
    const std::vector<int32_t>& bl = it->second.blocks;
    for (size_t i = bl.size(); i-- > 0;) m->release(bl[i]);
    m->seqs.erase(it);
    return PA_OK;
}

int64_t pa_bm_num_tokens(const pa_block_manager* m, int64_t seq_id) {
    if (!m) return -1;
    auto it = m->seqs.find(seq_id);
    return it == m->seqs.end() ? -1 : it->second.tokens;
}

namespace {

int append_batch(pa_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t* slot_mapping, int32_t* copies,
                 int32_t max_copies, int32_t* num_copies) {
    // Check first, replaying the batch on the reference counts alone: every id
    // known and distinct, enough free blocks and copy room.  (A shared block
    // copied away by one sequence may be left to a single owner, who then
    // writes it in place.)
    int64_t need_blocks = 0, need_copies = 0;
    std::unordered_map<int64_t, int> seen;
    std::unordered_map<int32_t, int32_t> dropped;  // references given up earlier in this batch
    for (int32_t i = 0; i < n; ++i) {
        auto it = m->seqs.find(seq_ids[i]);
        if (it == m->seqs.end() || seen.count(seq_ids[i])) return PA_EINVAL;
        seen[seq_ids[i]] = 1;
        const Seq& s = it->second;
        if (s.tokens % kBlockTokens == 0) {
            ++need_blocks;  // the last block is full (or there is none)
        } else {
            const int32_t last = s.blocks.back();
            auto d = dropped.find(last);
            const int32_t refs = m->refcount[last] - (d == dropped.end() ? 0 : d->second);
            if (refs > 1) {  // shared partial block: copy before writing
                ++need_blocks;
                ++need_copies;
                ++dropped[last];
            }
        }
    }
    if (need_blocks > (int64_t)m->free_stack.size()) return PA_ENOMEM;
    if (need_copies > max_copies) return PA_EINVAL;
    // room for the new last blocks, so that nothing below allocates
    for (int32_t i = 0; i < n; ++i) {
        Seq& s = m->seqs.find(seq_ids[i])->second;
        if (s.tokens % kBlockTokens == 0) s.blocks.reserve(s.blocks.size() + 1);
    }
    int32_t nc = 0;
    for (int32_t i = 0; i < n; ++i) {
        Seq& s = m->seqs.find(seq_ids[i])->second;
        if (s.tokens % kBlockTokens == 0) {
            s.blocks.push_back(m->pop());
        } else if (m->refcount[s.blocks.back()] > 1) {
            const int32_t old = s.blocks.back();
            const int32_t fresh = m->pop();
            copies[2 * nc] = old;
            copies[2 * nc + 1] = fresh;
            ++nc;
            m->release(old);  // drops one reference; still held by the others
            s.blocks.back() = fresh;
        }
        slot_mapping[i] = s.blocks.back() * kBlockTokens + (int32_t)(s.tokens % kBlockTokens);
        ++s.tokens;
    }
    *num_copies = nc;
    return PA_OK;
}

}  // namespace

int pa_bm_append_batch(pa_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t* slot_mapping,
                       int32_t* copies, int32_t max_copies, int32_t* num_copies) {
    if (!m || n < 0 || (n > 0 && (!seq_ids || !slot_mapping)) || max_copies < 0 || !num_copies) return PA_EINVAL;
    if (max_copies > 0 && !copies) return PA_EINVAL;
    try {
        return append_batch(m, seq_ids, n, slot_mapping, copies, max_copies, num_copies);
    } catch (...) {  // only the checks allocate (their maps): nothing has changed
        return PA_ENOMEM;
    }
}

int pa_bm_batch_tables(const pa_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t* block_tables,
                       int32_t max_blocks_per_seq, int32_t* context_lens) {
    if (!m || n < 0 || max_blocks_per_seq <= 0) return PA_EINVAL;
    if (n > 0 && (!seq_ids || !block_tables || !context_lens)) return PA_EINVAL;
    for (int32_t i = 0; i < n; ++i) {
        auto it = m->seqs.find(seq_ids[i]);
        if (it == m->seqs.end()) return PA_EINVAL;
        if ((int64_t)it->second.blocks.size() > max_blocks_per_seq) return PA_EINVAL;
        if (it->second.tokens > INT32_MAX) return PA_EINVAL;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq& s = m->seqs.find(seq_ids[i])->second;
        int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
        size_t j = 0;
        for (; j < s.blocks.size(); ++j) row[j] = s.blocks[j];
        for (; j < (size_t)max_blocks_per_seq; ++j) row[j] = -1;
        context_lens[i] = (int32_t)s.tokens;
    }
    return PA_OK;
}

int32_t pa_bm_refcount(const pa_block_manager* m, int32_t block) {
    if (!m || block < 0 || block >= m->num_blocks) return -1;
    return m->refcount[block];
}

}  // extern "C"
