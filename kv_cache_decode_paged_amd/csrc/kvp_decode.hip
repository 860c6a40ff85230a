// kvp_decode.hip -- host side of decode attention: argument checks, work decomposition
// sizes, workspace layout, and the C entry points.  The kernels live in kvp_decode_f16.hip
// (fp16, the hot path) and kvp_decode_f32.hip (fp32).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "kvp_decode_common.h"
#include "kvp_plan_format.h"

namespace kvp {

// wait bound of the fp16 split merge (polls of a pair's ticket)
static std::atomic<int> g_merge_polls{0};


using namespace dec;

static kvp_status check_dims(const kvp_dims *d, const char *who)
{
    if (!d)
        return fail(KVP_ERR_INVALID, "%s: dims is NULL", who);
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
        return fail(KVP_ERR_INVALID, "%s: num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                    who, d->num_q_heads, d->num_kv_heads);
    if (d->dtype != KVP_F16 && d->dtype != KVP_F32 && d->dtype != KVP_I8)
        return fail(KVP_ERR_INVALID, "%s: dtype=%d", who, d->dtype);
    if (d->head_dim != D && !(d->dtype != KVP_F32 && d->head_dim == 128))
        return fail(KVP_ERR_UNSUPPORTED, "%s: head_dim=%d (64, or 128 for fp16 / int8)", who, d->head_dim);
    const int group = d->num_q_heads / d->num_kv_heads;
    if (d->dtype == KVP_F32 && group > MAXG)
        return fail(KVP_ERR_UNSUPPORTED, "%s: %d query heads per KV head (fp32: 1..%d supported)", who, group, MAXG);
    if (d->dtype != KVP_F32 && !plan::group_supported(group, d->head_dim))
        return fail(KVP_ERR_UNSUPPORTED, "%s: %d query heads per KV head (1..16, or a multiple of 16 up to %d at head "
                    "dim %d)", who, group, 16 * plan::max_col_blocks(d->head_dim), d->head_dim);
    return KVP_OK;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------------------
// Static scratch of paged_decode_attention_noalloc: split counters (one int per request and
// KV head, in a fixed region so that partials of a larger call never land on counters of a
// later one) followed by the split partials.  Each GPU holds its own copy from the first
// use until the process ends; its device address is looked up once per device.
// ---------------------------------------------------------------------------------------
constexpr int NOALLOC_MAX_PAIRS = KVP_NOALLOC_MAX_PAIRS;
constexpr size_t NOALLOC_TICKET_BYTES = (size_t)KVP_NOALLOC_MAX_PAIRS * sizeof(int);
constexpr size_t NOALLOC_PART_BYTES = (size_t)KVP_NOALLOC_SCRATCH_BYTES - NOALLOC_TICKET_BYTES;
static_assert(NOALLOC_TICKET_BYTES % 256 == 0, "partials start 256-byte aligned");

static __device__ __align__(256) char scratch[KVP_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[SCRATCH_MAX_DEVICES]; // device address of `scratch`, per device

__global__ void clear_ints_kernel(int *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0;
}

// The current device's scratch address.  On the first use on a device: look the array up
// (hipGetSymbolAddress) and zero its counter region with a small kernel on `st` (stream-
// ordered before the caller's decode; the array also starts zeroed when the code object
// loads).  Every decode leaves the counters at zero again.
static kvp_status scratch_for_device(char **out, hipStream_t st, const char *who)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return fail(KVP_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", who, dev, SCRATCH_MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KVP_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
        hipLaunchKernelGGL(clear_ints_kernel, dim3(64), dim3(256), 0, st, (int *)p, NOALLOC_MAX_PAIRS);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(KVP_ERR_HIP, "%s: clearing the scratch counters: %s", who, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = (char *)g_scratch_ptr[dev];
    return KVP_OK;
}

static size_t part_bytes(const kvp_dims *d, int B, int max_context)
{
    if (d->dtype != KVP_F32) { // the fp16 kernel (fp16 or int8 caches)
        const int ipp = decode_f16_items_per_pair(max_context, d->dtype == KVP_I8, d->head_dim);
        return ipp > 1 ? decode_f16_part_bytes((long long)B * d->num_kv_heads * ipp, d->num_q_heads / d->num_kv_heads,
                                               d->head_dim)
                       : 0;
    }
    const int ms = decode_f32_max_splits(max_context);
    return ms > 1 ? decode_f32_part_bytes(B, d->num_q_heads, ms) : 0;
}

// workspace: [tickets: one int per (request, KV head), 256-byte aligned][partials]
static size_t ticket_bytes(int B, int hkv) { return align256((size_t)B * hkv * sizeof(int)); }

static size_t workspace_bytes(const kvp_dims *d, int B, int max_context)
{
    const size_t pb = part_bytes(d, B, max_context);
    if (pb == 0)
        return 0;
    return ticket_bytes(B, d->num_kv_heads) + pb;
}

// Where the split counters and partials live: the caller's workspace, or the library's
// static scratch array (paged_decode_attention_noalloc: counters in a fixed region, partials
// after it).  `dry` stops after the argument checks, before anything is launched.
struct WsMode {
    bool fixed = false;   // static scratch
    bool dry = false;
    int *tickets = nullptr;
    float *part = nullptr;
};

template <typename Addr>
static kvp_status decode_common(const kvp_dims *dims, void *out, const void *q, const void *kc,
                                const void *vc, const void *ksc, const void *vsc, const void *k_new,
                                const void *v_new, const Addr &A, int max_ctx, const int32_t *d_ctx,
                                int32_t B, float scale, void *ws, size_t ws_bytes, kvp_stream stream,
                                const char *who, const WsMode &wm = WsMode())
{
    kvp_status st = check_dims(dims, who);
    if (st != KVP_OK)
        return st;
    if (B < 0 || max_ctx < 0)
        return fail(KVP_ERR_INVALID, "%s: B=%d max_context=%d", who, B, max_ctx);
    if (B == 0)
        return KVP_OK;
    if (!out || !q || !kc || !vc || !d_ctx)
        return fail(KVP_ERR_INVALID, "%s: NULL pointer argument", who);
    if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)kc | (uintptr_t)vc | (uintptr_t)k_new |
         (uintptr_t)v_new) & 15)
        return fail(KVP_ERR_INVALID, "%s: q/out/cache/new-row pointers must be 16-byte aligned", who);
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(KVP_ERR_INVALID, "%s: k_new and v_new must both be given or both be NULL", who);
    if (k_new && dims->dtype == KVP_F32)
        return fail(KVP_ERR_UNSUPPORTED, "%s: the fused append is implemented for fp16 and int8", who);
    if (dims->dtype == KVP_I8 && (!ksc || !vsc))
        return fail(KVP_ERR_INVALID, "%s: an int8 cache needs its scale pools", who);
    DecodeParams P{};
    P.q = q;
    P.out = out;
    P.kc = kc;
    P.vc = vc;
    P.kc_w = const_cast<void *>(kc);
    P.vc_w = const_cast<void *>(vc);
    P.k_new = k_new;
    P.v_new = v_new;
    P.ksc = ksc;
    P.vsc = vsc;
    P.ksc_w = const_cast<void *>(ksc);
    P.vsc_w = const_cast<void *>(vsc);
    P.kv_i8 = dims->dtype == KVP_I8;
    P.ctx_lens = d_ctx;
    P.B = B;
    P.hq = dims->num_q_heads;
    P.hkv = dims->num_kv_heads;
    P.dim = dims->head_dim;
    P.group = dims->num_q_heads / dims->num_kv_heads;
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)P.dim);
    P.scale_log2 = scale * LOG2E;
    P.part = nullptr;
    P.tickets = nullptr;
    P.workers = dims->dtype != KVP_F32 ? 0 : decode_f32_max_splits(max_ctx);
    P.merge_polls = g_merge_polls.load(std::memory_order_relaxed);
    const size_t pb = part_bytes(dims, B, max_ctx);
    if (wm.fixed) {
        if ((long long)B * dims->num_kv_heads > NOALLOC_MAX_PAIRS || pb > NOALLOC_PART_BYTES)
            return fail(KVP_ERR_INVALID, "%s: %d requests x %d KV heads with contexts up to %d tokens need %zu bytes "
                        "of split partials; the static scratch holds %d (request, KV head) pairs and %zu bytes",
                        who, B, dims->num_kv_heads, max_ctx, pb, NOALLOC_MAX_PAIRS, (size_t)NOALLOC_PART_BYTES);
        P.tickets = wm.tickets;
        P.part = wm.part;
    } else if (pb > 0) {
        const size_t need = workspace_bytes(dims, B, max_ctx);
        if (!ws || ws_bytes < need)
            return fail(KVP_ERR_INVALID, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
        if ((uintptr_t)ws & 255)
            return fail(KVP_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
        P.tickets = (int *)ws;
        P.part = (float *)((char *)ws + ticket_bytes(B, dims->num_kv_heads));
    }
    if (wm.dry)
        return KVP_OK;
    const int group = P.hq / P.hkv;
    hipStream_t st_ = (hipStream_t)stream;
    return dims->dtype != KVP_F32 ? launch_decode_f16(P, A, group, max_ctx, st_)
                                  : launch_decode_f32(P, A, group, st_);
}

static kvp_status paged_common(const kvp_cache_desc *cache, int32_t layer, void *out,
                               const void *q, const void *k_new, const void *v_new,
                               const int32_t *d_block_table, int32_t max_blocks,
                               const int32_t *d_context_lens, int32_t B, float scale,
                               void *workspace, size_t ws_bytes, kvp_stream stream, const char *who,
                               const WsMode &wm = WsMode())
{
    if (!cache)
        return fail(KVP_ERR_INVALID, "%s: cache is NULL", who);
    kvp_status st0 = check_dims(&cache->dims, who);
    if (st0 != KVP_OK)
        return st0;
    if (cache->block_size != BS)
        return fail(KVP_ERR_UNSUPPORTED, "%s: block_size=%d (only 16)", who, cache->block_size);
    if (layer < 0 || layer >= cache->dims.num_layers)
        return fail(KVP_ERR_INVALID, "%s: layer %d out of range", who, layer);
    if (max_blocks <= 0 || cache->num_blocks <= 0 || !d_block_table)
        return fail(KVP_ERR_INVALID, "%s: max_blocks=%d num_blocks=%d table=%p", who, max_blocks,
                    cache->num_blocks, (const void *)d_block_table);
    if (!cache->k_pool || !cache->v_pool)
        return fail(KVP_ERR_INVALID, "%s: pool pointer is NULL", who);
    if ((long long)max_blocks * BS > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "%s: max_blocks too large", who);
    const int dt = cache->dims.dtype;
    const size_t esz = dt == KVP_F16 ? 2 : dt == KVP_F32 ? 4 : 1;
    const size_t layer_rows = (size_t)cache->num_blocks * cache->dims.num_kv_heads * BS;
    const size_t layer_elems = layer_rows * cache->dims.head_dim;
    const char *kc = (const char *)cache->k_pool + (size_t)layer * layer_elems * esz;
    const char *vc = (const char *)cache->v_pool + (size_t)layer * layer_elems * esz;
    const bool i8 = dt == KVP_I8;
    if (i8 && (!cache->k_scale || !cache->v_scale || (((uintptr_t)cache->k_scale | (uintptr_t)cache->v_scale) & 15)))
        return fail(KVP_ERR_INVALID, "%s: an int8 cache needs 16-byte aligned scale pools", who);
    const char *ksc = i8 ? (const char *)cache->k_scale + (size_t)layer * layer_rows * 2 : nullptr;
    const char *vsc = i8 ? (const char *)cache->v_scale + (size_t)layer * layer_rows * 2 : nullptr;
    PagedAddr A{d_block_table, max_blocks, cache->dims.num_kv_heads, cache->num_blocks, cache->dims.head_dim};
    return decode_common(&cache->dims, out, q, kc, vc, ksc, vsc, k_new, v_new, A, max_blocks * BS,
                         d_context_lens, B, scale, workspace, ws_bytes, stream, who, wm);
}

static size_t plan_workspace_bytes(const kvp_decode_plan *plan)
{
    if (plan->n_slots <= 0)
        return 0;
    return ticket_bytes(plan->B, plan->num_kv_heads) + decode_f16_part_bytes(plan->n_slots, plan->group, plan->head_dim);
}

} // namespace kvp

using namespace kvp;

extern "C" {

int32_t kvp_decode_merge_polls(int32_t polls)
{
    const int old = g_merge_polls.load(std::memory_order_relaxed);
    if (polls >= 0)
        g_merge_polls.store(polls, std::memory_order_relaxed);
    return old;
}

size_t decode_workspace_bytes(const kvp_dims *dims, int32_t B, int32_t max_context)
{
    if (check_dims(dims, "decode_workspace_bytes") != KVP_OK || B < 0 || max_context < 0)
        return 0;
    return workspace_bytes(dims, B, max_context);
}

kvp_status paged_decode_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                  const void *q, const int32_t *d_block_table,
                                  int32_t max_blocks, const int32_t *d_context_lens, int32_t B,
                                  float scale, void *workspace, size_t ws_bytes,
                                  kvp_stream stream)
{
    return paged_common(cache, layer, out, q, nullptr, nullptr, d_block_table, max_blocks,
                        d_context_lens, B, scale, workspace, ws_bytes, stream,
                        "paged_decode_attention");
}

kvp_status paged_decode_append_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                         const void *q, const void *k_new, const void *v_new,
                                         const int32_t *d_block_table, int32_t max_blocks,
                                         const int32_t *d_context_lens, int32_t B, float scale,
                                         void *workspace, size_t ws_bytes, kvp_stream stream)
{
    if (!k_new || !v_new)
        return fail(KVP_ERR_INVALID, "paged_decode_append_attention: k_new / v_new is NULL");
    return paged_common(cache, layer, out, q, k_new, v_new, d_block_table, max_blocks,
                        d_context_lens, B, scale, workspace, ws_bytes, stream,
                        "paged_decode_append_attention");
}

kvp_status paged_decode_attention_noalloc(const kvp_cache_desc *cache, int32_t layer, void *out, const void *q,
                                          const int32_t *d_block_table, int32_t max_blocks,
                                          const int32_t *d_context_lens, int32_t B, float scale, kvp_stream stream)
{
    const char *who = "paged_decode_attention_noalloc";
    WsMode wm;
    wm.fixed = true;
    wm.dry = true; // every argument and size check first: on error nothing is launched
    kvp_status st = paged_common(cache, layer, out, q, nullptr, nullptr, d_block_table, max_blocks, d_context_lens, B,
                                 scale, nullptr, 0, stream, who, wm);
    if (st != KVP_OK || B == 0)
        return st;
    char *base = nullptr;
    st = scratch_for_device(&base, (hipStream_t)stream, who);
    if (st != KVP_OK)
        return st;
    wm.dry = false;
    wm.tickets = (int *)base;
    wm.part = (float *)(base + NOALLOC_TICKET_BYTES);
    return paged_common(cache, layer, out, q, nullptr, nullptr, d_block_table, max_blocks, d_context_lens, B, scale,
                        nullptr, 0, stream, who, wm);
}

size_t decode_plan_workspace_bytes(const kvp_decode_plan *plan)
{
    return plan ? plan_workspace_bytes(plan) : 0;
}

kvp_status paged_decode_attention_planned(const kvp_cache_desc *cache, int32_t layer, void *out,
                                          const void *q, const void *k_new, const void *v_new,
                                          const kvp_decode_plan *plan, const void *d_plan, float scale,
                                          void *workspace, size_t ws_bytes, kvp_stream stream)
{
    const char *who = "paged_decode_attention_planned";
    if (!cache || !plan)
        return fail(KVP_ERR_INVALID, "%s: cache / plan is NULL", who);
    kvp_status st = check_dims(&cache->dims, who);
    if (st != KVP_OK)
        return st;
    if (cache->dims.dtype == KVP_F32)
        return fail(KVP_ERR_UNSUPPORTED, "%s: planned decode is implemented for fp16 and int8", who);
    const bool i8 = cache->dims.dtype == KVP_I8;
    if (i8 && (!cache->k_scale || !cache->v_scale || (((uintptr_t)cache->k_scale | (uintptr_t)cache->v_scale) & 15)))
        return fail(KVP_ERR_INVALID, "%s: an int8 cache needs 16-byte aligned scale pools", who);
    if (cache->block_size != BS)
        return fail(KVP_ERR_UNSUPPORTED, "%s: block_size=%d (only 16)", who, cache->block_size);
    if (layer < 0 || layer >= cache->dims.num_layers)
        return fail(KVP_ERR_INVALID, "%s: layer %d out of range", who, layer);
    const int hkv = cache->dims.num_kv_heads, group = cache->dims.num_q_heads / hkv;
    const int dim = cache->dims.head_dim;
    if (plan->num_kv_heads != hkv || plan->group != group || plan->head_dim != dim || plan->B < 0 ||
        plan->n_items < 0 || plan->num_blocks <= 0 || plan->num_blocks > cache->num_blocks)
        return fail(KVP_ERR_INVALID, "%s: plan (Hkv=%d group=%d d=%d num_blocks=%d) does not fit the cache "
                    "(Hkv=%d group=%d d=%d num_blocks=%d)", who, plan->num_kv_heads, plan->group,
                    plan->head_dim, plan->num_blocks, hkv, group, dim, cache->num_blocks);
    if (plan->n_ids < 0 || plan->off_ids < 0 || (plan->off_ids & 3) || plan->n_ids > 0x7fffffffLL)
        return fail(KVP_ERR_INVALID, "%s: plan id area (offset %lld, %lld ids) is not valid", who,
                    (long long)plan->off_ids, (long long)plan->n_ids);
    if (plan->B == 0 || plan->n_items == 0)
        return KVP_OK;
    if (!out || !q || !d_plan || !cache->k_pool || !cache->v_pool)
        return fail(KVP_ERR_INVALID, "%s: NULL pointer argument", who);
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(KVP_ERR_INVALID, "%s: k_new and v_new must both be given or both be NULL", who);
    if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)d_plan) & 15)
        return fail(KVP_ERR_INVALID, "%s: q/out/new-row/plan pointers must be 16-byte aligned", who);
    const size_t need = plan_workspace_bytes(plan);
    if (need > 0) {
        if (!workspace || ws_bytes < need)
            return fail(KVP_ERR_INVALID, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
        if ((uintptr_t)workspace & 255)
            return fail(KVP_ERR_INVALID, "%s: workspace must be 256-byte aligned", who);
    }
    const size_t layer_rows = (size_t)cache->num_blocks * hkv * BS;
    const size_t layer_bytes = layer_rows * dim * (i8 ? 1 : 2);
    DecodeParams P{};
    P.q = q;
    P.out = out;
    P.kc = (const char *)cache->k_pool + (size_t)layer * layer_bytes;
    P.vc = (const char *)cache->v_pool + (size_t)layer * layer_bytes;
    P.kc_w = const_cast<void *>(P.kc);
    P.vc_w = const_cast<void *>(P.vc);
    P.k_new = k_new;
    P.v_new = v_new;
    P.kv_i8 = i8;
    P.ksc = i8 ? (const char *)cache->k_scale + (size_t)layer * layer_rows * 2 : nullptr;
    P.vsc = i8 ? (const char *)cache->v_scale + (size_t)layer * layer_rows * 2 : nullptr;
    P.ksc_w = const_cast<void *>(P.ksc);
    P.vsc_w = const_cast<void *>(P.vsc);
    P.ctx_lens = nullptr;
    P.B = plan->B;
    P.hq = cache->dims.num_q_heads;
    P.hkv = hkv;
    P.dim = dim;
    P.group = group;
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)dim);
    P.scale_log2 = scale * LOG2E;
    P.workers = 0;
    P.merge_polls = g_merge_polls.load(std::memory_order_relaxed);
    // tickets first: the layout does not depend on the plan's slot count
    P.tickets = need > 0 ? (int *)workspace : nullptr;
    P.part = need > 0 ? (float *)((char *)workspace + ticket_bytes(plan->B, hkv)) : nullptr;
    PagedAddr A{nullptr, 0, hkv, plan->num_blocks, dim};
    return launch_decode_f16_planned(P, A, group, d_plan, *plan, (hipStream_t)stream);
}

kvp_status contiguous_decode_attention(const kvp_dims *dims, void *out, const void *q,
                                       const void *k_cache, const void *v_cache, int32_t Lmax,
                                       const int32_t *d_context_lens, int32_t B, float scale,
                                       void *workspace, size_t ws_bytes, kvp_stream stream)
{
    kvp_status st0 = check_dims(dims, "contiguous_decode_attention");
    if (st0 != KVP_OK)
        return st0;
    if (Lmax <= 0)
        return fail(KVP_ERR_INVALID, "contiguous_decode_attention: Lmax=%d", Lmax);
    if (dims->dtype == KVP_I8)
        return fail(KVP_ERR_UNSUPPORTED, "contiguous_decode_attention: int8 caches are paged only");
    ContigAddr A{dims->num_kv_heads, Lmax, dims->head_dim};
    return decode_common(dims, out, q, k_cache, v_cache, nullptr, nullptr, nullptr, nullptr, A, Lmax, d_context_lens,
                         B, scale, workspace, ws_bytes, stream, "contiguous_decode_attention");
}

} // extern "C"
