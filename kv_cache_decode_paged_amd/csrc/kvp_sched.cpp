// kvp_sched.cpp -- static vs continuous batching over the block pool (host C++).
//
//   neuralialabs "Tornar a inferencia barata", batching passage: a fixed batch runs until
//   its longest member finishes, finished members keeping their places as padding;
//   continuous batching admits the next queued request into a freed place at the next step.
//   chatgpz.de "Aufmerksamkeit", paged-attention article, SECTION 1 (the naive cache
//   reserves max_seq_len tokens per request), SECTION 2 (pages taken on demand from a free
//   list, returned on release), SECTION 4 (utilisation = tokens written / tokens reserved).
//
// The schedule drives a real kvp_pool: admission allocates the prompt's pages (paged) or
// max_seq_len tokens' pages (naive), every produced token goes through
// block_table_append_slot, returns free the sequence.  Step rules are documented at
// sched_simulate in kvp.h.
#include <cstdint>
#include <vector>

#include "kvp_internal.h"

namespace {

struct Active {
    int req;
    int32_t seq;        // sequence id in the pool
    int64_t tokens;     // resident tokens
    int64_t blocks;     // pages held
    int64_t generated;  // tokens produced so far
    bool done;
};

} // namespace

using namespace kvp;

extern "C" kvp_status sched_simulate(const kvp_sched_config *cfg, const int32_t *prompt_lens,
                                     const int32_t *output_lens, int32_t n, int32_t *latency,
                                     int32_t *service, kvp_sched_result *res)
{
    const char *who = "sched_simulate";
    if (!cfg || !res || n < 0 || (n > 0 && (!prompt_lens || !output_lens)))
        return fail(KVP_ERR_INVALID, "%s: NULL argument or n=%d", who, n);
    if (cfg->slots <= 0 || cfg->block_size <= 0 || cfg->num_blocks <= 0 ||
        (cfg->policy != KVP_SCHED_STATIC && cfg->policy != KVP_SCHED_CONTINUOUS) ||
        (cfg->alloc != KVP_ALLOC_PAGED && cfg->alloc != KVP_ALLOC_NAIVE) || cfg->max_seq_len < 0)
        return fail(KVP_ERR_INVALID, "%s: slots=%d policy=%d alloc=%d max_seq_len=%d block_size=%d num_blocks=%d",
                    who, cfg->slots, cfg->policy, cfg->alloc, cfg->max_seq_len, cfg->block_size, cfg->num_blocks);
    for (int i = 0; i < n; ++i) {
        if (prompt_lens[i] < 0 || output_lens[i] < 1)
            return fail(KVP_ERR_INVALID, "%s: request %d has prompt %d, output %d", who, i, prompt_lens[i],
                        output_lens[i]);
        if (cfg->alloc == KVP_ALLOC_NAIVE && (int64_t)prompt_lens[i] + output_lens[i] > cfg->max_seq_len)
            return fail(KVP_ERR_INVALID, "%s: request %d needs more than max_seq_len=%d tokens", who, i,
                        cfg->max_seq_len);
    }
    *res = kvp_sched_result{};
    if (n == 0)
        return KVP_OK;
    kvp_pool *pool = nullptr;
    kvp_status st = block_pool_create(cfg->num_blocks, cfg->block_size, &pool);
    if (st != KVP_OK)
        return st;
    const int64_t bs = cfg->block_size;
    auto pages = [bs](int64_t t) { return (t + bs - 1) / bs; };
    const bool paged = cfg->alloc == KVP_ALLOC_PAGED;
    const bool continuous = cfg->policy == KVP_SCHED_CONTINUOUS;

    std::vector<Active> active;
    active.reserve(cfg->slots);
    std::vector<int64_t> lat(n, 0), adm(n, 0);
    int queue = 0, returned = 0;
    int64_t step = 0, busy = 0, padding = 0, peak = 0, deferrals = 0, stalls = 0, held = 0;
    double util_sum = 0.0;
    while (returned < n) {
        int64_t progress = 0;
        // admission: free places take queued requests in order (static: only an empty batch)
        if (continuous || active.empty()) {
            while ((int)active.size() < cfg->slots && queue < n) {
                const int r = queue;
                const int32_t alloc_tokens = paged ? prompt_lens[r] : cfg->max_seq_len;
                int32_t seq = -1;
                st = block_table_alloc(pool, alloc_tokens, &seq);
                if (st == KVP_ERR_OOM) {
                    ++deferrals;
                    break;
                }
                if (st != KVP_OK) {
                    block_pool_destroy(pool);
                    return st;
                }
                const int64_t nb = pages(alloc_tokens);
                held += nb;
                active.push_back(Active{r, seq, prompt_lens[r], nb, 0, false});
                adm[r] = step;
                ++queue;
                ++progress;
            }
        }
        // one token for every unfinished admitted request
        for (Active &a : active) {
            if (a.done) { // finished earlier, holding its place (static policy)
                ++padding;
                continue;
            }
            if (paged) {
                int64_t slot;
                kvp_copy cow;
                st = block_table_append_slot(pool, a.seq, &slot, &cow);
                if (st == KVP_ERR_OOM) {
                    ++stalls;
                    continue;
                }
                if (st != KVP_OK) {
                    block_pool_destroy(pool);
                    return st;
                }
                if (pages(a.tokens + 1) > a.blocks) {
                    ++a.blocks;
                    ++held;
                }
            }
            ++a.tokens;
            ++a.generated;
            ++busy;
            ++progress;
            if (a.generated == output_lens[a.req])
                a.done = true;
        }
        ++step;
        // statistics after the step, before returns
        if (held > peak)
            peak = held;
        int64_t resident = 0;
        for (const Active &a : active)
            resident += a.tokens;
        util_sum += held ? (double)resident / (double)(held * bs) : 0.0;
        // returns
        bool all_done = !active.empty();
        for (const Active &a : active)
            all_done = all_done && a.done;
        if (continuous || all_done) {
            size_t k = 0;
            for (size_t i = 0; i < active.size(); ++i) {
                Active &a = active[i];
                if (a.done) {
                    lat[a.req] = step;
                    held -= a.blocks;
                    block_table_free(pool, a.seq);
                    ++returned;
                } else {
                    active[k++] = a;
                }
            }
            active.resize(k);
        }
        if (progress == 0 && !active.empty() && !all_done) {
            block_pool_destroy(pool);
            return fail(KVP_ERR_OOM, "%s: at step %lld every admitted request waits for a page and none can "
                        "be admitted (the pool of %d blocks is too small; there is no preemption)", who,
                        (long long)step, cfg->num_blocks);
        }
    }
    block_pool_destroy(pool);
    int64_t lsum = 0, ssum = 0, lmax = 0, tokens = 0;
    for (int i = 0; i < n; ++i) {
        lsum += lat[i];
        ssum += lat[i] - adm[i];
        lmax = lat[i] > lmax ? lat[i] : lmax;
        tokens += output_lens[i];
        if (latency)
            latency[i] = (int32_t)lat[i];
        if (service)
            service[i] = (int32_t)(lat[i] - adm[i]);
    }
    res->steps = step;
    res->tokens = tokens;
    res->busy_slot_steps = busy;
    res->padding_slot_steps = padding;
    res->peak_blocks = peak;
    res->deferrals = deferrals;
    res->stalls = stalls;
    res->max_latency = lmax;
    res->mean_latency = (double)lsum / n;
    res->mean_service = (double)ssum / n;
    res->mean_utilisation = util_sum / (double)step;
    return KVP_OK;
}
