// Host-side block pool of the paged KV cache: free list, reference counts,
// block tables and copy-on-write.
//
// Follows the block allocator of the "vLLM 核心工程深度剖析" page (section
// 2.2: a free list used as a stack, one reference count per block, one table
// per request; a new block only when the last one is full; blocks return to
// the free list when their count reaches zero; running out is an error),
// its fork (section 4.1: the child copies the parent's table and adds a
// reference to each block), and the copy-on-write rule of the
// "PagedAttention 笔记" page (a block referenced by more than one sequence
// is never written: the writer takes a new block, the shared one is copied
// into it, the writer's table points at the copy and the shared block loses
// one reference).
//
// The pool only does the bookkeeping; the block copies it asks for are done
// on the device by pkv_copy_blocks, before the token is written.
#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_block_pool {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> free_list;  // stack: back() is handed out next
    std::vector<int32_t> ref_count;
    struct Seq {
        std::vector<int32_t> table;
        int64_t len = 0;
    };
    std::unordered_map<int64_t, Seq> seqs;

    int32_t take()
    {
        const int32_t b = free_list.back();
        free_list.pop_back();
        ++ref_count[b];
        return b;
    }
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t B) { return (tokens + B - 1) / B; }

// Reserves position L = len for the next token of s (the caller has checked
// that a free block exists when one is needed).
int64_t append_one(pkv_block_pool* p, pkv_block_pool::Seq& s, int32_t* copy_src, int32_t* copy_dst)
{
    const int32_t B = p->block_size;
    const int64_t L = s.len;
    *copy_src = -1;
    *copy_dst = -1;
    if (L % B == 0) {
        s.table.push_back(p->take());
    } else {
        int32_t& last = s.table[L / B];
        if (p->ref_count[last] > 1) {
            const int32_t fresh = p->take();
            *copy_src = last;
            *copy_dst = fresh;
            --p->ref_count[last];
            last = fresh;
        }
    }
    s.len = L + 1;
    return (int64_t)s.table[L / B] * B + L % B;
}

}  // namespace

extern "C" {

pkv_block_pool* pkv_pool_create(int32_t num_blocks, int32_t block_size)
{
    if (num_blocks <= 0 || block_size <= 0)
        return nullptr;
    pkv_block_pool* p = new (std::nothrow) pkv_block_pool;
    if (!p)
        return nullptr;
    try {
        p->num_blocks = num_blocks;
        p->block_size = block_size;
        p->free_list.resize(num_blocks);
        for (int32_t b = 0; b < num_blocks; ++b)
            p->free_list[b] = b;
        p->ref_count.assign(num_blocks, 0);
    } catch (...) {
        delete p;
        return nullptr;
    }
    return p;
}

pkv_block_pool* pkv_pool_create_with_free_list(int32_t num_blocks, int32_t block_size, const int32_t* free_list,
                                               int32_t count)
{
    if (!free_list || count < 0 || count > num_blocks)
        return nullptr;
    std::vector<char> seen(num_blocks > 0 ? num_blocks : 0, 0);
    for (int32_t i = 0; i < count; ++i) {
        const int32_t b = free_list[i];
        if (b < 0 || b >= num_blocks || seen[b])
            return nullptr;
        seen[b] = 1;
    }
    pkv_block_pool* p = pkv_pool_create(num_blocks, block_size);
    if (!p)
        return nullptr;
    p->free_list.assign(free_list, free_list + count);
    return p;
}

void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

pkv_status pkv_pool_add_sequence(pkv_block_pool* p, int64_t seq, int64_t num_tokens)
{
    if (!p || num_tokens < 0 || p->seqs.count(seq))
        return PKV_ERR_INVALID_ARG;
    const int64_t need = blocks_for(num_tokens, p->block_size);
    if (need > (int64_t)p->free_list.size())
        return PKV_ERR_OUT_OF_BLOCKS;
    try {
        pkv_block_pool::Seq s;
        s.len = num_tokens;
        s.table.reserve(need);
        for (int64_t i = 0; i < need; ++i)
            s.table.push_back(p->take());
        p->seqs.emplace(seq, std::move(s));
    } catch (...) {
        return PKV_ERR_INVALID_ARG;
    }
    return PKV_OK;
}

pkv_status pkv_pool_append_slots(pkv_block_pool* p, const int64_t* seqs, int32_t num_seqs, int64_t* slots,
                                 int32_t* copies, int32_t* num_copies)
{
    if (!p || num_seqs < 0 || (num_seqs > 0 && (!seqs || !slots || !copies || !num_copies)))
        return PKV_ERR_INVALID_ARG;
    if (num_copies)
        *num_copies = 0;
    // check everything first, so that a failed call changes nothing: count
    // the blocks the appends will take, in order (a copy-on-write by one
    // sequence can leave a shared block to a later one in the same call)
    int64_t need = 0;
    std::vector<pkv_block_pool::Seq*> ss(num_seqs);
    std::unordered_map<int32_t, int32_t> dropped;  // references given up by earlier copies
    const int32_t B = p->block_size;
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = p->seqs.find(seqs[i]);
        if (it == p->seqs.end())
            return PKV_ERR_INVALID_ARG;
        for (int32_t j = 0; j < i; ++j)
            if (seqs[j] == seqs[i])
                return PKV_ERR_INVALID_ARG;  // one token per sequence per call
        ss[i] = &it->second;
        const pkv_block_pool::Seq& sq = it->second;
        if (sq.len % B == 0) {
            ++need;
        } else {
            const int32_t last = sq.table[sq.len / B];
            if (p->ref_count[last] - dropped[last] > 1) {
                ++need;
                ++dropped[last];
            }
        }
    }
    if (need > (int64_t)p->free_list.size())
        return PKV_ERR_OUT_OF_BLOCKS;
    int32_t nc = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        int32_t src, dst;
        slots[i] = append_one(p, *ss[i], &src, &dst);
        if (src >= 0) {
            copies[2 * nc] = src;
            copies[2 * nc + 1] = dst;
            ++nc;
        }
    }
    *num_copies = nc;
    return PKV_OK;
}

pkv_status pkv_pool_fork(pkv_block_pool* p, int64_t parent, int64_t child)
{
    if (!p || p->seqs.count(child))
        return PKV_ERR_INVALID_ARG;
    auto it = p->seqs.find(parent);
    if (it == p->seqs.end())
        return PKV_ERR_INVALID_ARG;
    try {
        pkv_block_pool::Seq s = it->second;
        for (int32_t b : s.table)
            ++p->ref_count[b];
        p->seqs.emplace(child, std::move(s));
    } catch (...) {
        return PKV_ERR_INVALID_ARG;
    }
    return PKV_OK;
}

pkv_status pkv_pool_free(pkv_block_pool* p, int64_t seq)
{
    if (!p)
        return PKV_ERR_INVALID_ARG;
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end())
        return PKV_ERR_INVALID_ARG;
    for (int32_t b : it->second.table)
        if (--p->ref_count[b] == 0)
            p->free_list.push_back(b);
    p->seqs.erase(it);
    return PKV_OK;
}

int32_t pkv_pool_num_free(const pkv_block_pool* p) { return p ? (int32_t)p->free_list.size() : -1; }

int32_t pkv_pool_ref_count(const pkv_block_pool* p, int32_t block)
{
    if (!p || block < 0 || block >= p->num_blocks)
        return -1;
    return p->ref_count[block];
}

int64_t pkv_pool_seq_len(const pkv_block_pool* p, int64_t seq)
{
    if (!p)
        return -1;
    auto it = p->seqs.find(seq);
    return it == p->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_pool_block_table(const pkv_block_pool* p, int64_t seq, int32_t* out, int32_t capacity)
{
    if (!p || capacity < 0 || (capacity > 0 && !out))
        return -1;
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end())
        return -1;
    const auto& t = it->second.table;
    const int32_t n = (int32_t)t.size();
    std::copy(t.begin(), t.begin() + std::min(n, capacity), out);
    return n;
}

pkv_status pkv_pool_export(const pkv_block_pool* p, const int64_t* seqs, int32_t num_seqs,
                           int32_t max_blocks_per_seq, int32_t pad_block, int32_t* block_tables, int32_t* seq_lens)
{
    if (!p || num_seqs < 0 || max_blocks_per_seq <= 0 ||
        (num_seqs > 0 && (!seqs || !block_tables || !seq_lens)))
        return PKV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = p->seqs.find(seqs[i]);
        if (it == p->seqs.end() || (int64_t)it->second.table.size() > max_blocks_per_seq ||
            it->second.len > INT32_MAX)
            return PKV_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const auto& s = p->seqs.find(seqs[i])->second;
        int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
        const int32_t n = (int32_t)s.table.size();
        std::copy(s.table.begin(), s.table.end(), row);
        std::fill(row + n, row + max_blocks_per_seq, pad_block);
        seq_lens[i] = (int32_t)s.len;
    }
    return PKV_OK;
}

}  // extern "C"
