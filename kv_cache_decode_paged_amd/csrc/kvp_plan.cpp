// kvp_plan.cpp -- host planner for the fp16 decode kernel: work items (one wave each), the
// partial-slot layout of split pairs, and shared-prefix items for requests whose block
// tables start with the same physical blocks.
//
// Pages: [PAGED] (paged-attention article, SECTION 3): forked requests share the physical
// blocks of a common prefix until copy-on-write makes a block private; [CHAP] (PagedAttention
// passage): sharing prefix blocks among requests.  Reading a shared block once for all of
// its readers is this library's choice; the attention each request receives is unchanged
// (same keys and values, only the order of the fp32 sums differs).
#include <algorithm>
#include <cstring>
#include <vector>

#include "kvp_internal.h"
#include "kvp_plan_format.h"

using namespace kvp;
using namespace kvp::plan;

namespace {

constexpr int BS = 16;

size_t align16(size_t x) { return (x + 15) / 16 * 16; }

kvp_status check_plan_dims(const kvp_dims *d, const char *who)
{
    if (!d)
        return fail(KVP_ERR_INVALID, "%s: dims is NULL", who);
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
        return fail(KVP_ERR_INVALID, "%s: num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                    who, d->num_q_heads, d->num_kv_heads);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(KVP_ERR_UNSUPPORTED, "%s: head_dim=%d (64 or 128)", who, d->head_dim);
    if (d->dtype != KVP_F16 && d->dtype != KVP_I8)
        return fail(d->dtype == KVP_F32 ? KVP_ERR_UNSUPPORTED : KVP_ERR_INVALID,
                    "%s: planned decode is implemented for fp16 and int8 (dtype=%d)", who, d->dtype);
    if (!group_supported(d->num_q_heads / d->num_kv_heads, d->head_dim))
        return fail(KVP_ERR_UNSUPPORTED, "%s: %d query heads per KV head (1..16, or a multiple of 16 up to %d at head "
                    "dim %d)", who, d->num_q_heads / d->num_kv_heads, 16 * max_col_blocks(d->head_dim), d->head_dim);
    return KVP_OK;
}

constexpr int MAX_BUNDLE = 8; // shared items kept together on one XCD


long long max_items(long long B, long long hkv, long long max_blocks, bool i8, int hd)
{
    const long long ipp = std::max<long long>(1, (max_blocks + split_blocks(i8, hd) - 1) / split_blocks(i8, hd));
    // private items: at most ipp per pair; shared items: a sub-run of n >= 2 members has at
    // most 4 ipp parts when it takes 4 column blocks (then n >= 3), 2 ipp with 2 blocks and
    // ipp with one, so fewer than 2 ipp per request; plus the padding that evens out the XCD
    // queues and rounds them to whole CU rounds
    // (KVP_PLAN_FILL: private items shorter than split_blocks only while they fit the
    // resident waves)
    const long long waves = i8 ? LONG_TARGET_WAVES_I8 : LONG_TARGET_WAVES_F16;
    const long long work = std::max(B * hkv * ipp, waves) + 2 * B * hkv * ipp;
    return XCDS * ((work + XCDS - 1) / XCDS + MAX_BUNDLE + CU_SLOTS - 1);
}

// records, the pair and request arrays, and the id area of long items (at most every block
// of every pair)
size_t image_bytes_for(long long items, long long B, long long hkv, long long max_blocks)
{
    return align16((size_t)items * REC * 4) + 2 * align16((size_t)B * hkv * 4) + align16((size_t)B * 4) +
           align16((size_t)B * hkv * max_blocks * 4);
}

// parts of a range of nb blocks: one item up to unsplit_blocks blocks unless `forced` (the
// pair has other parts anyway), else ceil(nb / split_blocks) parts of equal tile counts
int split_parts(int nb, bool forced, bool i8, int hd)
{
    if (nb <= 0 || (!forced && nb <= unsplit_blocks(i8, hd)))
        return 1;
    return (nb + split_blocks(i8, hd) - 1) / split_blocks(i8, hd);
}
// first block of part k of n over nb blocks (part k holds tiles [k T / n, (k+1) T / n))
int split_start(int nb, int n, int k, int slack = 0)
{
    return std::min(nb, 4 * part_tile_begin((nb + 3) / 4, n, k, slack));
}

// v in stable order of cost, highest first (cost: an item's tiles plus 2, at most
// LONG_BPI + 2, so a counting sort; equal costs keep their order, as a stable sort would)
void sort_by_cost_desc(std::vector<long long> &v, const std::vector<long long> &cost, std::vector<long long> &tmp)
{
    long long maxc = 0;
    for (long long i : v)
        maxc = std::max(maxc, cost[i]);
    if (maxc > 4 * LONG_BPI) {
        std::stable_sort(v.begin(), v.end(), [&](long long x, long long y) { return cost[x] > cost[y]; });
        return;
    }
    std::vector<size_t> start((size_t)maxc + 2, 0);
    for (long long i : v)
        ++start[(size_t)(maxc - cost[i]) + 1];
    for (size_t k = 1; k < start.size(); ++k)
        start[k] += start[k - 1];
    tmp.resize(v.size());
    for (long long i : v)
        tmp[start[(size_t)(maxc - cost[i])]++] = i;
    v.swap(tmp);
}

struct SubRun {
    int a, n, shared_tokens, run;
};

// Parts of a shared range of nsb blocks read for n members at group size G: an item scores
// each tile against ncb blocks of 16 query columns (ncb = 1, 2 or 4), so its work per tile
// grows with ncb; its length is cut to split_blocks / ncb blocks (the private parts' length
// over ncb) to keep items of equal work.
int shared_split(int nsb, int n, int G, int hd, bool i8)
{
    const int mpb = G <= 16 ? 16 / G : 1;
    int ncb = (n + mpb - 1) / mpb;
    ncb = ncb <= 1 ? 1 : (ncb <= 2 ? 2 : 4);
    ncb = std::min(ncb, max_col_blocks(hd));
    const int len = split_blocks(i8, hd) / ncb;
    return nsb <= 0 ? 1 : (nsb + len - 1) / len;
}

} // namespace

extern "C" {

size_t decode_plan_bytes(const kvp_dims *dims, int32_t B, int32_t max_blocks, int32_t pad_items)
{
    if (check_plan_dims(dims, "decode_plan_bytes") != KVP_OK || B < 0 || max_blocks <= 0 || pad_items < 0)
        return 0;
    const long long pad = ((long long)pad_items + XCDS - 1) / XCDS * XCDS;
    return image_bytes_for(std::max(pad, max_items(B, dims->num_kv_heads, max_blocks, dims->dtype == KVP_I8,
                                                     dims->head_dim)), B,
                           dims->num_kv_heads,
                           max_blocks);
}

kvp_status decode_plan_build(const kvp_dims *dims, const int32_t *table, int32_t max_blocks,
                             const int32_t *ctx_lens, int32_t B, int32_t num_blocks, uint32_t flags,
                             int32_t pad_items, void *h_image, size_t image_bytes, kvp_decode_plan *plan)
{
    const char *who = "decode_plan_build";
    kvp_status st = check_plan_dims(dims, who);
    if (st != KVP_OK)
        return st;
    if (B < 0 || max_blocks <= 0 || num_blocks <= 0)
        return fail(KVP_ERR_INVALID, "%s: B=%d max_blocks=%d num_blocks=%d", who, B, max_blocks, num_blocks);
    if (!plan || !h_image || (B > 0 && (!table || !ctx_lens)))
        return fail(KVP_ERR_INVALID, "%s: NULL pointer argument", who);
    if (flags & ~(KVP_PLAN_SHARE_PREFIX | KVP_PLAN_LONG_ITEMS | KVP_PLAN_SHARE_WIDE2 | KVP_PLAN_SHARE_WIDE4 |
                  KVP_PLAN_FILL))
        return fail(KVP_ERR_INVALID, "%s: unknown flags 0x%x", who, flags);
    if ((flags & KVP_PLAN_SHARE_WIDE2) && (flags & KVP_PLAN_SHARE_WIDE4))
        return fail(KVP_ERR_INVALID, "%s: KVP_PLAN_SHARE_WIDE2 and KVP_PLAN_SHARE_WIDE4 together", who);
    const int width = (flags & KVP_PLAN_SHARE_WIDE4) ? 4 : (flags & KVP_PLAN_SHARE_WIDE2) ? 2 : 1;
    if (pad_items < 0)
        return fail(KVP_ERR_INVALID, "%s: pad_items=%d", who, pad_items);
    if ((long long)max_blocks * BS > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "%s: max_blocks too large", who);
    const int hkv = dims->num_kv_heads;
    const bool i8 = dims->dtype == KVP_I8; // the int8 kernel's split sizes
    const int hd = dims->head_dim;
    const int G = dims->num_q_heads / hkv;
    const int maxm = shared_members(G, hd, width); // members of a shared item (1: no sharing)
    const long long npairs = (long long)B * hkv;

    std::vector<int> c(B), nbt(B), E(B, 0);
    auto ent = [&](int b, int j) -> int {
        const int e = table[(size_t)b * max_blocks + j];
        return (e >= 0 && e < num_blocks) ? e : -1;
    };
    for (int b = 0; b < B; ++b) {
        c[b] = std::min(std::max(ctx_lens[b], 0), max_blocks * BS);
        nbt[b] = (c[b] + BS - 1) / BS;
    }

    // ---- shared prefixes: runs of consecutive requests with the same first block, cut
    // into sub-runs of at most maxm members; member m shares E[m] tokens (whole blocks
    // equal to the sub-run leader's, never the block holding its last token) ----
    std::vector<SubRun> subs;
    if (flags & KVP_PLAN_SHARE_PREFIX) {
        int b = 0, run = 0;
        while (b < B) {
            if (nbt[b] == 0 || ent(b, 0) < 0) {
                ++b;
                continue;
            }
            int r = b + 1;
            while (r < B && nbt[r] > 0 && ent(r, 0) == ent(b, 0))
                ++r;
            for (int a = b; a < r; a += maxm) {
                const int n = std::min(maxm, r - a);
                if (n < 2)
                    continue;
                int S = 0;
                for (int m = a + 1; m < a + n; ++m) {
                    const int lim = std::min(nbt[a], nbt[m]);
                    int k = 0;
                    while (k < lim && ent(m, k) >= 0 && ent(m, k) == ent(a, k))
                        ++k;
                    E[m] = std::min(BS * k, BS * ((c[m] - 1) / BS));
                    S = std::max(S, E[m]);
                }
                E[a] = std::min(S, BS * ((c[a] - 1) / BS));
                if (S > 0)
                    subs.push_back({a, n, S, run});
                else
                    for (int m = a; m < a + n; ++m)
                        E[m] = 0;
            }
            b = r;
            ++run;
        }
    }

    // ---- parts per pair and slot ranges ----
    // shared items a member takes part in: those starting below its shared extent
    std::vector<int> shared_parts(B, 0);
    for (const SubRun &sr : subs) {
        const int nsb = sr.shared_tokens / BS;
        const int ns = shared_split(nsb, sr.n, G, hd, i8);
        for (int m = sr.a; m < sr.a + sr.n; ++m)
            for (int k = 0; k < ns; ++k)
                if (BS * split_start(nsb, ns, k) < E[m])
                    ++shared_parts[m];
    }
    long long n_shared = 0;
    for (const SubRun &s : subs)
        n_shared += (long long)hkv * shared_split(s.shared_tokens / BS, s.n, G, hd, i8);
    // long items: parts of up to S blocks, S sized so the private blocks fill about one
    // generation of waves (whole tiles, between SPLIT_BLOCKS and LONG_BPI); S = SPLIT_BLOCKS
    // leaves the plan as without the flag
    const long long waves = i8 ? LONG_TARGET_WAVES_I8 : LONG_TARGET_WAVES_F16;
    const int S0 = split_blocks(i8, hd);
    int S = S0;
    if (flags & KVP_PLAN_LONG_ITEMS) {
        long long priv_blocks = 0;
        for (int b = 0; b < B; ++b)
            priv_blocks += (long long)hkv * std::max(0, nbt[b] - E[b] / BS);
        const long long per_wave = (priv_blocks + waves - 1) / waves;
        S = (int)std::min<long long>(LONG_BPI, std::max<long long>(S0, (per_wave + 3) / 4 * 4));
    }
    // fill: the shortest parts (whole tiles, from FILL_MIN_BLOCKS) whose private items all
    // fit the waves the shared items leave
    if ((flags & KVP_PLAN_FILL) && S == S0) {
        const long long avail = waves - n_shared;
        for (int s = FILL_MIN_BLOCKS; s < S0; s += 4) {
            long long items = 0;
            for (int b = 0; b < B; ++b) {
                const int nb = nbt[b] - E[b] / BS;
                items += (long long)hkv * (nb <= 0 ? 1 : (nb + s - 1) / s);
            }
            if (items <= avail) {
                S = s;
                break;
            }
        }
    }
    auto private_items = [&](int b) -> int {
        const int nb = nbt[b] - E[b] / BS;
        if (S < S0) // fill
            return nb <= 0 ? 1 : (nb + S - 1) / S;
        if (S == S0 || nb <= unsplit_blocks(i8, hd))
            return split_parts(nb, E[b] > 0, i8, hd);
        return (nb + S - 1) / S;
    };
    std::vector<int> pair_base(npairs, -1), pair_nparts(npairs, 1);
    long long slots = 0, n_items = 0;
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < hkv; ++g) {
            const long long p = (long long)b * hkv + g;
            pair_nparts[p] = shared_parts[b] + private_items(b);
            if (pair_nparts[p] > 1) {
                pair_base[p] = (int)slots;
                slots += pair_nparts[p];
            }
            n_items += private_items(b);
        }
    n_items += n_shared;
    if (slots > 0x7fffffffLL || n_items > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "%s: plan too large", who);

    // ---- records (built in plan order, placed into XCD queues below) ----
    std::vector<int32_t> recs((size_t)n_items * REC); // every field of a record is written
    std::vector<int32_t> long_ids; // id area
    std::vector<long long> cost(n_items);
    long long idx = 0, blocks_read = 0;
    auto record = [&](int fl, int b, int g, int nmem, int blk0, int nblk, int end, int slot, int nparts,
                      int pbase, int src_req) {
        int32_t *r = recs.data() + (size_t)idx * REC;
        r[R_FLAGS] = fl;
        r[R_B] = b;
        r[R_G] = g;
        r[R_NMEM] = nmem;
        r[R_BLK0] = blk0;
        r[R_NBLK] = nblk;
        r[R_END] = end;
        r[R_SLOT] = slot;
        r[R_NPARTS] = nparts;
        r[R_PBASE] = pbase;
        for (int j = R_PBASE + 1; j < R_ENT; ++j)
            r[j] = 0;
        if (nblk > BPI) { // long item (private only): ids in the id area
            r[R_FLAGS] |= F_LONG;
            for (int j = 0; j < BPI; ++j)
                r[R_ENT + j] = -1;
            r[R_IDS] = (int32_t)long_ids.size();
            for (int j = 0; j < nblk; ++j)
                long_ids.push_back(ent(src_req, blk0 + j));
        } else {
            const int32_t *row = table + (size_t)src_req * max_blocks + blk0;
            for (int j = 0; j < nblk; ++j)
                r[R_ENT + j] = (uint32_t)row[j] < (uint32_t)num_blocks ? row[j] : -1;
            for (int j = std::max(nblk, 0); j < BPI; ++j)
                r[R_ENT + j] = -1;
        }
        blocks_read += nblk;
        cost[idx] = nblk + 2; // a tile stream plus the fixed start / finish of a wave
        ++idx;
    };
    // bundles: the shared items of one run and KV head (at most MAX_BUNDLE per bundle)
    std::vector<std::vector<long long>> bundles;
    {
        std::vector<std::pair<long long, long long>> keyed; // (run * hkv + g, item)
        for (const SubRun &sr : subs) {
            const int nsb = sr.shared_tokens / BS;
            const int ns = shared_split(nsb, sr.n, G, hd, i8);
            for (int g = 0; g < hkv; ++g)
                for (int k = 0; k < ns; ++k) {
                    const int b0 = split_start(nsb, ns, k), b1 = split_start(nsb, ns, k + 1);
                    keyed.push_back({(long long)sr.run * hkv + g, idx});
                    record(F_SHARED, sr.a, g, sr.n, b0, b1 - b0, 0, k, 0, -1, sr.a);
                }
        }
        std::stable_sort(keyed.begin(), keyed.end(),
                         [](const std::pair<long long, long long> &x, const std::pair<long long, long long> &y) {
                             return x.first < y.first;
                         });
        for (size_t i = 0; i < keyed.size(); ++i) {
            if (i == 0 || keyed[i].first != keyed[i - 1].first || bundles.back().size() >= (size_t)MAX_BUNDLE)
                bundles.push_back({});
            bundles.back().push_back(keyed[i].second);
        }
    }
    const long long first_private = idx;
    for (int b = 0; b < B; ++b) {
        const int first = E[b] / BS;
        const int npriv = private_items(b);
        for (int g = 0; g < hkv; ++g) {
            const long long p = (long long)b * hkv + g;
            for (int k = 0; k < npriv; ++k) {
                const int nb = nbt[b] - first;
                const int blk0 = first + split_start(nb, npriv, k, SPLIT_SLACK);
                const int nblk = nb <= 0 ? 0 : first + split_start(nb, npriv, k + 1, SPLIT_SLACK) - blk0;
                const int slot = pair_nparts[p] > 1 ? pair_base[p] + shared_parts[b] + k : -1;
                record(0, b, g, 1, blk0, nblk, c[b], slot, pair_nparts[p], pair_base[p], b);
            }
        }
    }

    if (idx != n_items)
        return fail(KVP_ERR_INVALID, "%s: internal error (%lld records for %lld items)", who, idx, n_items);

    // ---- XCD queues: item p of the image runs on XCD p % XCDS.  Bundles first, then private
    // items longest first, each to the least-loaded queue that stays within the length cap;
    // shorter queues are padded with empty items ----
    const long long cap = (n_items + XCDS - 1) / XCDS + MAX_BUNDLE;
    std::vector<std::vector<long long>> q(XCDS);
    for (auto &v : q)
        v.reserve((size_t)cap);
    long long load[XCDS] = {};
    // bundles: the least-loaded XCD (lowest index among equals) with room for the bundle
    for (const auto &bd : bundles) {
        long long c = 0;
        for (long long i : bd)
            c += cost[i];
        int best = -1;
        for (int x = 0; x < XCDS; ++x)
            if ((long long)(q[x].size() + bd.size()) <= cap && (best < 0 || load[x] < load[best]))
                best = x;
        for (long long i : bd)
            q[best].push_back(i);
        load[best] += c;
    }
    // single items, longest first, the same rule: a min-heap of (load, XCD) over the XCDs
    // with room (popping the least load, the lowest index among equal loads)
    std::vector<long long> priv(n_items - first_private);
    for (size_t i = 0; i < priv.size(); ++i)
        priv[i] = first_private + (long long)i;
    std::vector<long long> tmp;
    sort_by_cost_desc(priv, cost, tmp);
    typedef std::pair<long long, int> LoadIdx;
    const auto after = [](const LoadIdx &a, const LoadIdx &b) { return a > b; }; // min-heap order
    LoadIdx heap[XCDS > CU_SLOTS ? XCDS : CU_SLOTS];
    int nh = 0;
    for (int x = 0; x < XCDS; ++x)
        if ((long long)q[x].size() < cap)
            heap[nh++] = {load[x], x};
    std::make_heap(heap, heap + nh, after);
    for (long long i : priv) {
        if (nh == 0) // cannot happen: the queues hold n_items + XCDS MAX_BUNDLE items
            return fail(KVP_ERR_INVALID, "%s: internal error (XCD queues full)", who);
        std::pop_heap(heap, heap + nh, after);
        const int x = heap[nh - 1].second;
        q[x].push_back(i);
        load[x] += cost[i];
        if ((long long)q[x].size() < cap) {
            heap[nh - 1] = {load[x], x};
            std::push_heap(heap, heap + nh, after);
        } else {
            --nh;
        }
    }
    // within each XCD: items to CU slots, longest first to the least-loaded slot that has
    // fewer than K items (K = the XCD's items over its slots, rounded up; lowest slot among
    // equal loads); the k-th item of slot s takes queue position CU_SLOTS k + s
    std::vector<std::vector<long long>> qpos(XCDS);
    size_t qlen = 0;
    for (int x = 0; x < XCDS; ++x) {
        std::vector<long long> &its = q[x];
        sort_by_cost_desc(its, cost, tmp);
        const size_t K = (its.size() + CU_SLOTS - 1) / CU_SLOTS;
        qpos[x].assign(K * CU_SLOTS, -1);
        int cnt[CU_SLOTS] = {};
        nh = 0;
        for (int c = 0; c < CU_SLOTS; ++c)
            heap[nh++] = {0, c};
        // all loads are 0: already a heap in (load, slot) order
        for (long long i : its) {
            std::pop_heap(heap, heap + nh, after);
            const int c = heap[nh - 1].second;
            qpos[x][(size_t)cnt[c] * CU_SLOTS + c] = i;
            if ((size_t)++cnt[c] < K) {
                heap[nh - 1] = {heap[nh - 1].first + cost[i], c};
                std::push_heap(heap, heap + nh, after);
            } else {
                --nh;
            }
        }
        qlen = std::max(qlen, qpos[x].size());
    }
    if (pad_items > 0) {
        const size_t padq = ((size_t)pad_items + XCDS - 1) / XCDS;
        if (qlen > padq)
            return fail(KVP_ERR_INVALID, "%s: the plan needs %zu items, more than pad_items=%d", who,
                        qlen * XCDS, pad_items);
        qlen = padq;
    }
    const long long n_image = (long long)qlen * XCDS;

    const size_t off_pb = align16((size_t)n_image * REC * 4);
    const size_t off_np = off_pb + align16((size_t)npairs * 4);
    const size_t off_rs = off_np + align16((size_t)npairs * 4);
    const size_t off_ids = off_rs + align16((size_t)B * 4);
    const size_t bytes = off_ids + align16(long_ids.size() * 4);
    if (image_bytes < bytes)
        return fail(KVP_ERR_INVALID, "%s: image buffer %zu bytes < %zu needed", who, image_bytes, bytes);
    int32_t *img = (int32_t *)h_image;
    std::memset((char *)h_image + off_pb, 0, bytes - off_pb); // records are written whole below
    for (size_t qi = 0; qi < qlen; ++qi)
        for (int x = 0; x < XCDS; ++x) {
            int32_t *dst = img + ((size_t)qi * XCDS + x) * REC;
            if (qi < qpos[x].size() && qpos[x][qi] >= 0) {
                std::memcpy(dst, recs.data() + (size_t)qpos[x][qi] * REC, REC * 4);
            } else {
                for (int j = 0; j < REC; ++j)
                    dst[j] = -1;
                dst[R_FLAGS] = F_EMPTY;
            }
        }
    std::memcpy((char *)h_image + off_pb, pair_base.data(), (size_t)npairs * 4);
    std::memcpy((char *)h_image + off_np, pair_nparts.data(), (size_t)npairs * 4);
    std::memcpy((char *)h_image + off_rs, E.data(), (size_t)B * 4);
    if (!long_ids.empty())
        std::memcpy((char *)h_image + off_ids, long_ids.data(), long_ids.size() * 4);

    plan->B = B;
    plan->num_kv_heads = hkv;
    plan->group = G;
    plan->num_blocks = num_blocks;
    plan->n_items = (int32_t)n_image;
    plan->n_shared = (int32_t)n_shared;
    plan->head_dim = dims->head_dim;
    // widest item: private items take G / 16 blocks when G > 16; shared items take
    // ceil(members / (16 / G)) blocks rounded up to 1, 2 or 4
    int widest = G <= 16 ? 1 : G / 16;
    for (const SubRun &sr : subs) {
        const int mpb = G <= 16 ? 16 / G : 1;
        const int ncb = (sr.n + mpb - 1) / mpb;
        widest = std::max(widest, ncb <= 1 ? 1 : (ncb <= 2 ? 2 : 4));
    }
    plan->col_blocks = std::min(widest, max_col_blocks(hd));
    plan->n_slots = slots;
    plan->bytes = (int64_t)bytes;
    plan->off_pair_base = (int64_t)off_pb;
    plan->off_pair_nparts = (int64_t)off_np;
    plan->off_req_shared = (int64_t)off_rs;
    plan->kv_blocks_read = blocks_read;
    plan->off_ids = (int64_t)off_ids;
    plan->n_ids = (int64_t)long_ids.size();
    return KVP_OK;
}

} // extern "C"
