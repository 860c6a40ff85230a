// kvp_manager.cpp -- host block manager: block pool, per-sequence block tables, fork and
// copy-on-write.
//
// Semantics (chatgpz.de "Aufmerksamkeit", paged-attention article, SECTION 2 "Paged
// Attention: Pages + Block Table" and SECTION 3 "Copy-on-Write: Shared System Prompts";
// neuralialabs chapter, PagedAttention passage):
//   - a flat pool of equal blocks; the free list starts as 0..N-1, allocation takes the
//     front and a released block goes to the back, so block ids are deterministic;
//   - every allocated block has a reference count; sharing adds one, releasing subtracts
//     one, and the block is free again when the count reaches zero;
//   - a sequence owns a block table (logical block -> block id) and a token count; a new
//     block is taken whenever the token count sits on a block boundary;
//   - copy-on-write takes a new block and releases the old one; it is only done when the
//     block is shared (count > 1), i.e. private only when needed.
// Every call checks everything it needs before changing anything, so an error (OOM,
// unknown id, double free) leaves the pool exactly as it was, free-list order included.
#include <algorithm>
#include <cstring>
#include <deque>
#include <unordered_map>
#include <vector>

#include "kvp_internal.h"

namespace kvp {

static thread_local std::string g_err;

void set_error(const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
}

void clear_error() { g_err.clear(); }

} // namespace kvp

using kvp::fail;

struct Seq {
    std::vector<int32_t> table;
    int32_t tokens = 0;
};

struct kvp_pool {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::deque<int32_t> free_list;
    std::vector<int32_t> ref; // 0 = free
    std::unordered_map<int32_t, Seq> seqs;
    int32_t next_seq = 0;

    int32_t take()
    { // caller has checked free_list is not empty
        int32_t b = free_list.front();
        free_list.pop_front();
        ref[b] = 1;
        return b;
    }
    void release(int32_t b)
    { // caller has checked ref[b] > 0
        if (--ref[b] == 0)
            free_list.push_back(b);
    }
    Seq *find(int32_t id)
    {
        auto it = seqs.find(id);
        return it == seqs.end() ? nullptr : &it->second;
    }
    const Seq *find(int32_t id) const
    {
        auto it = seqs.find(id);
        return it == seqs.end() ? nullptr : &it->second;
    }
};

extern "C" {

const char *kvp_last_error(void) { return kvp::g_err.c_str(); }

const char *kvp_version(void) { return "kvpaged-mi355x 0.1.0 (gfx950)"; }

kvp_status block_pool_create(int32_t num_blocks, int32_t block_size, kvp_pool **out)
{
    if (!out)
        return fail(KVP_ERR_INVALID, "block_pool_create: out is NULL");
    if (num_blocks <= 0 || block_size <= 0)
        return fail(KVP_ERR_INVALID, "block_pool_create: num_blocks=%d block_size=%d must be > 0",
                    num_blocks, block_size);
    kvp_pool *p = new (std::nothrow) kvp_pool;
    if (!p)
        return fail(KVP_ERR_OOM, "block_pool_create: host allocation failed");
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->ref.assign(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i)
        p->free_list.push_back(i);
    *out = p;
    return KVP_OK;
}

void block_pool_destroy(kvp_pool *pool) { delete pool; }

kvp_status block_pool_set_free_order(kvp_pool *pool, const int32_t *perm, int32_t n)
{
    if (!pool || !perm)
        return fail(KVP_ERR_INVALID, "block_pool_set_free_order: NULL argument");
    if ((int32_t)pool->free_list.size() != pool->num_blocks)
        return fail(KVP_ERR_INVALID, "block_pool_set_free_order: blocks are in use");
    if (n != pool->num_blocks)
        return fail(KVP_ERR_INVALID, "block_pool_set_free_order: n=%d != num_blocks=%d", n,
                    pool->num_blocks);
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
        if (perm[i] < 0 || perm[i] >= n || seen[perm[i]])
            return fail(KVP_ERR_INVALID, "block_pool_set_free_order: not a permutation");
        seen[perm[i]] = 1;
    }
    pool->free_list.assign(perm, perm + n);
    return KVP_OK;
}

kvp_status block_table_alloc(kvp_pool *pool, int32_t n_tokens, int32_t *seq_id)
{
    if (!pool || !seq_id)
        return fail(KVP_ERR_INVALID, "block_table_alloc: NULL argument");
    if (n_tokens < 0)
        return fail(KVP_ERR_INVALID, "block_table_alloc: n_tokens=%d < 0", n_tokens);
    int64_t need = ((int64_t)n_tokens + pool->block_size - 1) / pool->block_size;
    if (need > (int64_t)pool->free_list.size())
        return fail(KVP_ERR_OOM, "block_table_alloc: need %lld blocks, %zu free", (long long)need,
                    pool->free_list.size());
    Seq s;
    s.tokens = n_tokens;
    s.table.reserve(need);
    for (int64_t i = 0; i < need; ++i)
        s.table.push_back(pool->take());
    int32_t id = pool->next_seq++;
    pool->seqs.emplace(id, std::move(s));
    *seq_id = id;
    return KVP_OK;
}

kvp_status block_table_append_slot(kvp_pool *pool, int32_t seq, int64_t *slot, kvp_copy *cow)
{
    if (!pool || !slot || !cow)
        return fail(KVP_ERR_INVALID, "block_table_append_slot: NULL argument");
    Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_append_slot: unknown sequence %d", seq);
    if (s->tokens == INT32_MAX)
        return fail(KVP_ERR_INVALID, "block_table_append_slot: sequence %d is full", seq);
    const int32_t bs = pool->block_size;
    const int32_t lb = s->tokens / bs, off = s->tokens % bs;
    kvp_copy c = {-1, -1};
    if (off == 0) {
        if (pool->free_list.empty())
            return fail(KVP_ERR_OOM, "block_table_append_slot: no free block");
        s->table.push_back(pool->take());
    } else {
        int32_t old = s->table[lb];
        if (pool->ref[old] > 1) {
            if (pool->free_list.empty())
                return fail(KVP_ERR_OOM, "block_table_append_slot: no free block for copy-on-write");
            int32_t nb = pool->take();
            pool->release(old);
            s->table[lb] = nb;
            c.src = old;
            c.dst = nb;
        }
    }
    *slot = (int64_t)s->table[lb] * bs + off;
    *cow = c;
    s->tokens += 1;
    return KVP_OK;
}

kvp_status block_table_append_slots(kvp_pool *pool, const int32_t *seqs, int32_t n,
                                    int64_t *slots, kvp_copy *cows)
{
    if (!pool || n < 0 || (n > 0 && (!seqs || !slots || !cows)))
        return fail(KVP_ERR_INVALID, "block_table_append_slots: bad arguments");
    // validate ids and count the blocks the batch will take, simulating the reference
    // counts of shared partial blocks (the last of several sharers writes in place)
    std::unordered_map<int32_t, int32_t> seen, ref_sim;
    int64_t need = 0;
    const int32_t bs = pool->block_size;
    for (int32_t i = 0; i < n; ++i) {
        const Seq *s = pool->find(seqs[i]);
        if (!s)
            return fail(KVP_ERR_NOT_FOUND, "block_table_append_slots: unknown sequence %d", seqs[i]);
        if (seen.count(seqs[i]))
            return fail(KVP_ERR_INVALID, "block_table_append_slots: sequence %d repeated", seqs[i]);
        seen[seqs[i]] = 1;
        if (s->tokens == INT32_MAX)
            return fail(KVP_ERR_INVALID, "block_table_append_slots: sequence %d is full", seqs[i]);
        if (s->tokens % bs == 0) {
            need += 1;
        } else {
            const int32_t b = s->table[s->tokens / bs];
            auto it = ref_sim.find(b);
            int32_t &r = it == ref_sim.end() ? (ref_sim[b] = pool->ref[b]) : it->second;
            if (r > 1) {
                need += 1;
                r -= 1;
            }
        }
    }
    if (need > (int64_t)pool->free_list.size())
        return fail(KVP_ERR_OOM, "block_table_append_slots: need %lld blocks, %zu free",
                    (long long)need, pool->free_list.size());
    for (int32_t i = 0; i < n; ++i) {
        kvp_status st = block_table_append_slot(pool, seqs[i], &slots[i], &cows[i]);
        if (st != KVP_OK) // cannot happen after the checks above
            return st;
    }
    return KVP_OK;
}

kvp_status block_table_reserve(kvp_pool *pool, int32_t seq, int32_t n, int64_t *slots,
                               kvp_copy *cow)
{
    if (!pool || !cow || n < 0 || (n > 0 && !slots))
        return fail(KVP_ERR_INVALID, "block_table_reserve: bad arguments");
    Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_reserve: unknown sequence %d", seq);
    if ((int64_t)s->tokens + n > INT32_MAX)
        return fail(KVP_ERR_INVALID, "block_table_reserve: sequence %d would overflow", seq);
    const int32_t bs = pool->block_size;
    const int64_t have = (int64_t)s->table.size();
    const int64_t need_total = ((int64_t)s->tokens + n + bs - 1) / bs;
    int64_t need = need_total - have;
    const bool partial = n > 0 && s->tokens % bs != 0;
    const bool copy = partial && pool->ref[s->table[s->tokens / bs]] > 1;
    if (need + (copy ? 1 : 0) > (int64_t)pool->free_list.size())
        return fail(KVP_ERR_OOM, "block_table_reserve: need %lld blocks, %zu free",
                    (long long)(need + copy), pool->free_list.size());
    kvp_copy c = {-1, -1};
    if (copy) {
        const int32_t lb = s->tokens / bs;
        const int32_t old = s->table[lb];
        const int32_t nb = pool->take();
        pool->release(old);
        s->table[lb] = nb;
        c.src = old;
        c.dst = nb;
    }
    for (int64_t i = 0; i < need; ++i)
        s->table.push_back(pool->take());
    for (int32_t i = 0; i < n; ++i) {
        const int32_t j = s->tokens + i;
        slots[i] = (int64_t)s->table[j / bs] * bs + j % bs;
    }
    s->tokens += n;
    *cow = c;
    return KVP_OK;
}

kvp_status block_table_fork(kvp_pool *pool, int32_t parent, int32_t *child)
{
    if (!pool || !child)
        return fail(KVP_ERR_INVALID, "block_table_fork: NULL argument");
    const Seq *p = pool->find(parent);
    if (!p)
        return fail(KVP_ERR_NOT_FOUND, "block_table_fork: unknown sequence %d", parent);
    Seq s = *p;
    for (int32_t b : s.table)
        pool->ref[b] += 1;
    int32_t id = pool->next_seq++;
    pool->seqs.emplace(id, std::move(s));
    *child = id;
    return KVP_OK;
}

kvp_status block_table_cow(kvp_pool *pool, int32_t seq, int32_t logical_block, int32_t *src,
                           int32_t *dst)
{
    if (!pool || !src || !dst)
        return fail(KVP_ERR_INVALID, "block_table_cow: NULL argument");
    Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_cow: unknown sequence %d", seq);
    if (logical_block < 0 || logical_block >= (int32_t)s->table.size())
        return fail(KVP_ERR_INVALID, "block_table_cow: logical block %d out of range [0,%zu)",
                    logical_block, s->table.size());
    int32_t old = s->table[logical_block];
    if (pool->ref[old] == 1) {
        *src = *dst = old;
        return KVP_OK;
    }
    if (pool->free_list.empty())
        return fail(KVP_ERR_OOM, "block_table_cow: no free block");
    int32_t nb = pool->take();
    pool->release(old);
    s->table[logical_block] = nb;
    *src = old;
    *dst = nb;
    return KVP_OK;
}

kvp_status block_table_truncate(kvp_pool *pool, int32_t seq, int32_t n_tokens)
{
    if (!pool)
        return fail(KVP_ERR_INVALID, "block_table_truncate: NULL pool");
    Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_truncate: unknown sequence %d", seq);
    if (n_tokens < 0 || n_tokens > s->tokens)
        return fail(KVP_ERR_INVALID, "block_table_truncate: n_tokens=%d outside [0,%d]", n_tokens,
                    s->tokens);
    const size_t keep = ((size_t)n_tokens + pool->block_size - 1) / pool->block_size;
    for (size_t i = keep; i < s->table.size(); ++i)
        pool->release(s->table[i]);
    s->table.resize(keep);
    s->tokens = n_tokens;
    return KVP_OK;
}

kvp_status block_table_free(kvp_pool *pool, int32_t seq)
{
    if (!pool)
        return fail(KVP_ERR_INVALID, "block_table_free: NULL pool");
    Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_free: unknown sequence %d", seq);
    for (int32_t b : s->table) {
        if (pool->ref[b] <= 0) // would be a double free: the pool is corrupted
            return fail(KVP_ERR_INVALID, "block_table_free: block %d already free", b);
    }
    for (int32_t b : s->table)
        pool->release(b);
    pool->seqs.erase(seq);
    return KVP_OK;
}

kvp_status block_table_export(const kvp_pool *pool, const int32_t *seqs, int32_t n,
                              int32_t max_blocks, int32_t *host_table, int32_t *context_lens)
{
    if (!pool || (n > 0 && (!seqs || !host_table || !context_lens)) || n < 0 || max_blocks < 0)
        return fail(KVP_ERR_INVALID, "block_table_export: bad arguments");
    for (int32_t i = 0; i < n; ++i) {
        const Seq *s = pool->find(seqs[i]);
        if (!s)
            return fail(KVP_ERR_NOT_FOUND, "block_table_export: unknown sequence %d", seqs[i]);
        if ((int32_t)s->table.size() > max_blocks)
            return fail(KVP_ERR_INVALID, "block_table_export: sequence %d has %zu blocks > max_blocks %d",
                        seqs[i], s->table.size(), max_blocks);
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq *s = pool->find(seqs[i]);
        int32_t *row = host_table + (size_t)i * max_blocks;
        size_t nb = s->table.size();
        if (nb)
            std::memcpy(row, s->table.data(), nb * sizeof(int32_t));
        for (size_t j = nb; j < (size_t)max_blocks; ++j)
            row[j] = -1;
        context_lens[i] = s->tokens;
    }
    return KVP_OK;
}

kvp_status block_table_slots(const kvp_pool *pool, int32_t seq, int32_t start, int32_t n,
                             int64_t *slots)
{
    if (!pool || (n > 0 && !slots))
        return fail(KVP_ERR_INVALID, "block_table_slots: NULL argument");
    const Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_slots: unknown sequence %d", seq);
    if (start < 0 || n < 0 || (int64_t)start + n > s->tokens)
        return fail(KVP_ERR_INVALID, "block_table_slots: range [%d,%lld) outside [0,%d)", start,
                    (long long)start + n, s->tokens);
    const int32_t bs = pool->block_size;
    for (int32_t i = 0; i < n; ++i) {
        int32_t j = start + i;
        slots[i] = (int64_t)s->table[j / bs] * bs + j % bs;
    }
    return KVP_OK;
}

kvp_status block_table_get(const kvp_pool *pool, int32_t seq, int32_t *n_tokens,
                           int32_t *n_blocks, int32_t *blocks, int32_t cap)
{
    if (!pool || !n_tokens || !n_blocks || (cap > 0 && !blocks) || cap < 0)
        return fail(KVP_ERR_INVALID, "block_table_get: bad arguments");
    const Seq *s = pool->find(seq);
    if (!s)
        return fail(KVP_ERR_NOT_FOUND, "block_table_get: unknown sequence %d", seq);
    *n_tokens = s->tokens;
    *n_blocks = (int32_t)s->table.size();
    int32_t m = std::min<int32_t>(cap, (int32_t)s->table.size());
    for (int32_t i = 0; i < m; ++i)
        blocks[i] = s->table[i];
    return KVP_OK;
}

kvp_status block_pool_stats(const kvp_pool *pool, kvp_pool_stats *st)
{
    if (!pool || !st)
        return fail(KVP_ERR_INVALID, "block_pool_stats: NULL argument");
    st->total_blocks = pool->num_blocks;
    st->free_blocks = (int32_t)pool->free_list.size();
    st->used_blocks = pool->num_blocks - st->free_blocks;
    int32_t shared = 0;
    for (int32_t r : pool->ref)
        shared += r > 1;
    st->shared_blocks = shared;
    st->num_seqs = (int32_t)pool->seqs.size();
    st->utilisation_pct = 100.0 * st->used_blocks / pool->num_blocks;
    return KVP_OK;
}

kvp_status block_pool_refcount(const kvp_pool *pool, int32_t block, int32_t *refcount)
{
    if (!pool || !refcount)
        return fail(KVP_ERR_INVALID, "block_pool_refcount: NULL argument");
    if (block < 0 || block >= pool->num_blocks)
        return fail(KVP_ERR_INVALID, "block_pool_refcount: block %d out of range", block);
    *refcount = pool->ref[block];
    return KVP_OK;
}

int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                           int32_t elem_bytes)
{
    if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0 || elem_bytes < 0)
        return -1;
    return (int64_t)2 * num_layers * num_kv_heads * head_dim * elem_bytes;
}

} // extern "C"
