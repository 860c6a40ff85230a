// kvp_cache_ops.hip -- data movement of the paged KV cache on gfx950: append of new
// tokens into their slots, whole-block copies for copy-on-write, the paged -> contiguous
// gather, and the contiguous-layout append.  All are bit-exact 16-byte copies, except the
// append into an int8 cache, which quantizes each row (kvp_quant.h).
//
//   gustavoai "La cache de claves y valores", four-step token recipe, step 2: the new
//   token's k_t and v_t go to the end of each head's cache.
//   chatgpz.de "Aufmerksamkeit", paged-attention article, SECTION 2: the block table maps a
//   logical block of a request to a physical page; SECTION 3: copy-on-write gives a
//   diverging request a private copy of a shared page.
//
// Every kernel checks each computed index against the buffer it addresses and skips an
// out-of-range element instead of touching memory outside the caller's allocations.
#include <hip/hip_runtime.h>

#include "kvp_internal.h"
#include "kvp_quant.h"

namespace kvp {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BS = 16;

static bool head_dim_ok(int d) { return d == 64 || d == 128; }

static kvp_status check_cache(const kvp_cache_desc *c, const char *who)
{
    if (!c)
        return fail(KVP_ERR_INVALID, "%s: cache is NULL", who);
    const kvp_dims &d = c->dims;
    if (d.num_layers <= 0 || d.num_kv_heads <= 0 || d.num_q_heads <= 0 ||
        d.num_q_heads % d.num_kv_heads != 0)
        return fail(KVP_ERR_INVALID, "%s: bad dims (L=%d Hq=%d Hkv=%d)", who, d.num_layers,
                    d.num_q_heads, d.num_kv_heads);
    if (!head_dim_ok(d.head_dim))
        return fail(KVP_ERR_UNSUPPORTED, "%s: head_dim=%d (64 or 128)", who, d.head_dim);
    if (d.dtype != KVP_F16 && d.dtype != KVP_F32 && d.dtype != KVP_I8)
        return fail(KVP_ERR_INVALID, "%s: dtype=%d", who, d.dtype);
    if (d.dtype == KVP_I8 && (!c->k_scale || !c->v_scale || (((uintptr_t)c->k_scale | (uintptr_t)c->v_scale) & 15)))
        return fail(KVP_ERR_INVALID, "%s: an int8 cache needs 16-byte aligned scale pools", who);
    if (c->block_size != BS)
        return fail(KVP_ERR_UNSUPPORTED, "%s: block_size=%d (only 16)", who, c->block_size);
    if (c->num_blocks <= 0 || !c->k_pool || !c->v_pool)
        return fail(KVP_ERR_INVALID, "%s: empty pool", who);
    if (((uintptr_t)c->k_pool | (uintptr_t)c->v_pool) & 15)
        return fail(KVP_ERR_INVALID, "%s: pools must be 16-byte aligned", who);
    return KVP_OK;
}

// 16-byte chunks of one (token, head) row
static inline int elem_bytes(int dtype) { return dtype == KVP_F32 ? 4 : dtype == KVP_F16 ? 2 : 1; }
static inline int chunks_per_row(const kvp_dims &d) { return d.head_dim * elem_bytes(d.dtype) / 16; }

static kvp_status launched(const char *who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return KVP_OK;
}

// thread = one 16-byte chunk of one (token, head) row, for K and V
__global__ __launch_bounds__(256) void append_kernel(i32x4 *__restrict__ kpool,
                                                     i32x4 *__restrict__ vpool,
                                                     const i32x4 *__restrict__ k,
                                                     const i32x4 *__restrict__ v,
                                                     const int64_t *__restrict__ slots, int n,
                                                     int hkv, int nch, int64_t num_slots)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_tok = (int64_t)hkv * nch;
    if (idx >= (int64_t)n * per_tok)
        return;
    const int tok = (int)(idx / per_tok);
    const int rem = (int)(idx % per_tok);
    const int h = rem / nch, c = rem % nch;
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots)
        return;
    const int64_t blk = slot / BS, off = slot % BS;
    const int64_t dst = ((blk * hkv + h) * BS + off) * nch + c;
    kpool[dst] = k[idx];
    vpool[dst] = v[idx];
}

// int8 cache: thread = 8 values of one (token, head) row, for K and V; the CPR threads of a
// row are an aligned lane group that exchanges the row maximum.  K codes are stored
// row-major ([block][head][16][d]), V codes dim-major ([block][head][d][16]).
template <int CPR>
__global__ __launch_bounds__(256) void append_i8_kernel(char *__restrict__ kpool, char *__restrict__ vpool,
                                                        qf16 *__restrict__ kscale, qf16 *__restrict__ vscale,
                                                        const qf16 *__restrict__ k, const qf16 *__restrict__ v,
                                                        const int64_t *__restrict__ slots, int n, int hkv,
                                                        int64_t num_slots)
{
    constexpr int D = CPR * 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = idx / CPR; // (token, head)
    const int piece = (int)(idx % CPR);
    const bool valid = row < (int64_t)n * hkv;
    const int tok = valid ? (int)(row / hkv) : 0, h = valid ? (int)(row % hkv) : 0;
    const int64_t slot = valid ? slots[tok] : -1;
    const bool ok = slot >= 0 && slot < num_slots;
    const qf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    const size_t src = ((size_t)tok * hkv + h) * D + piece * 8;
    const qf16x8 xk = valid ? *(const qf16x8 *)(k + src) : z;
    const qf16x8 xv = valid ? *(const qf16x8 *)(v + src) : z;
    u32x2 ck, cvv;
    const qf16 sk = quantize_row_piece<CPR>(xk, ck); // every lane takes part in the exchange
    const qf16 sv = quantize_row_piece<CPR>(xv, cvv);
    if (!ok)
        return;
    const int64_t blk = slot / BS, off = slot % BS;
    const int64_t dst = (blk * hkv + h) * BS + off; // row index in the pool
    *(u32x2 *)(kpool + dst * D + piece * 8) = ck;
    char *vb = vpool + (blk * hkv + h) * BS * D + off; // dim-major block of this head
#pragma unroll
    for (int i = 0; i < 8; ++i)
        vb[(piece * 8 + i) * BS] = (char)((cvv[i >> 2] >> (8 * (i & 3))) & 0xff);
    if (piece == 0) {
        kscale[dst] = sk;
        vscale[dst] = sv;
    }
}

// grid = (pairs, layers, pools): pools 0 / 1 are K / V (block_chunks[0] chunks per block),
// 2 / 3 the int8 scale pools (block_chunks[1]); each workgroup copies one block of one layer
struct CopyPools {
    i32x4 *pool[4];
    int64_t block_chunks[2];
};
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyPools C, const int *__restrict__ pairs,
                                                          int num_blocks)
{
    const int p = blockIdx.x, layer = blockIdx.y;
    i32x4 *pool = C.pool[blockIdx.z];
    const int64_t block_chunks = C.block_chunks[blockIdx.z >> 1];
    const int64_t layer_chunks = block_chunks * num_blocks;
    const int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
        return;
    const i32x4 *s = pool + layer * layer_chunks + src * block_chunks;
    i32x4 *d = pool + layer * layer_chunks + dst * block_chunks;
    for (int64_t i = threadIdx.x; i < block_chunks; i += blockDim.x)
        d[i] = s[i];
}

// int8 cache, V codes: grid = (ceil(Lmax/16), Hkv, B), thread = one (token, dim) code of a
// dim-major block, written token-major
__global__ __launch_bounds__(256) void gather_v_i8_kernel(const char *__restrict__ vl,
                                                          const int *__restrict__ table, int max_blocks,
                                                          const int *__restrict__ ctx_lens, int hkv, int lmax,
                                                          int d, int num_blocks, char *__restrict__ vo)
{
    const int lb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int ctx = ctx_lens[b];
    if (ctx > max_blocks * BS)
        ctx = max_blocks * BS;
    if (ctx > lmax)
        ctx = lmax;
    if (lb * BS >= ctx)
        return;
    const int e = table[(size_t)b * max_blocks + lb];
    if (e < 0 || e >= num_blocks)
        return;
    for (int i = threadIdx.x; i < BS * d; i += blockDim.x) {
        const int r = i / d, c = i % d;
        const int t = lb * BS + r;
        if (t >= ctx)
            continue;
        vo[(((size_t)b * hkv + h) * lmax + t) * d + c] = vl[(((size_t)e * hkv + h) * d + c) * BS + r];
    }
}

// grid = (ceil(Lmax/16), Hkv, B): one 16-token block of one (request, head) per workgroup
__global__ __launch_bounds__(256) void gather_kernel(const i32x4 *__restrict__ kl,
                                                     const i32x4 *__restrict__ vl,
                                                     const int *__restrict__ table, int max_blocks,
                                                     const int *__restrict__ ctx_lens, int hkv,
                                                     int lmax, int nch, int num_blocks,
                                                     i32x4 *__restrict__ ko, i32x4 *__restrict__ vo)
{
    const int lb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    int ctx = ctx_lens[b];
    if (ctx > max_blocks * BS)
        ctx = max_blocks * BS;
    if (ctx > lmax)
        ctx = lmax;
    if (lb * BS >= ctx)
        return;
    const int e = table[(size_t)b * max_blocks + lb];
    if (e < 0 || e >= num_blocks)
        return;
    for (int i = threadIdx.x; i < BS * nch; i += blockDim.x) {
        const int r = i / nch, c = i % nch;
        const int t = lb * BS + r;
        if (t >= ctx)
            continue;
        const size_t src = (((size_t)e * hkv + h) * BS + r) * nch + c;
        const size_t dst = (((size_t)b * hkv + h) * lmax + t) * nch + c;
        ko[dst] = kl[src];
        vo[dst] = vl[src];
    }
}

// thread = one 16-byte chunk of (request, head) row written at position pos[b]
__global__ __launch_bounds__(256) void contig_append_kernel(i32x4 *__restrict__ kc,
                                                            i32x4 *__restrict__ vc,
                                                            const i32x4 *__restrict__ k,
                                                            const i32x4 *__restrict__ v,
                                                            const int *__restrict__ pos, int B,
                                                            int hkv, int lmax, int nch)
{
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * hkv * nch)
        return;
    const int b = idx / (hkv * nch);
    const int rem = idx % (hkv * nch);
    const int h = rem / nch, c = rem % nch;
    const int p = pos[b];
    if (p < 0 || p >= lmax)
        return;
    const size_t dst = (((size_t)b * hkv + h) * lmax + p) * nch + c;
    kc[dst] = k[idx];
    vc[dst] = v[idx];
}

} // namespace kvp

using namespace kvp;

extern "C" {

kvp_status kv_append(const kvp_cache_desc *cache, int32_t layer, const void *k, const void *v,
                     const int64_t *d_slots, int32_t n, kvp_stream stream)
{
    kvp_status st = check_cache(cache, "kv_append");
    if (st != KVP_OK)
        return st;
    if (layer < 0 || layer >= cache->dims.num_layers)
        return fail(KVP_ERR_INVALID, "kv_append: layer %d out of range", layer);
    if (n < 0)
        return fail(KVP_ERR_INVALID, "kv_append: n=%d", n);
    if (n == 0)
        return KVP_OK;
    if (!k || !v || !d_slots || (((uintptr_t)k | (uintptr_t)v) & 15))
        return fail(KVP_ERR_INVALID, "kv_append: k/v/slots must be non-NULL, k/v 16-byte aligned");
    const int nch = chunks_per_row(cache->dims);
    const int hkv = cache->dims.num_kv_heads;
    const int64_t layer_chunks = (int64_t)cache->num_blocks * hkv * BS * nch;
    if (cache->dims.dtype == KVP_I8) {
        const int d = cache->dims.head_dim;
        const int64_t rows = (int64_t)cache->num_blocks * hkv * BS; // rows per layer
        const int64_t total = (int64_t)n * hkv * (d / 8);
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7fffffff)
            return fail(KVP_ERR_UNSUPPORTED, "kv_append: n too large");
        char *kp = (char *)cache->k_pool + layer * rows * d;
        char *vp = (char *)cache->v_pool + layer * rows * d;
        qf16 *ks = (qf16 *)cache->k_scale + layer * rows;
        qf16 *vs = (qf16 *)cache->v_scale + layer * rows;
        const int64_t num_slots = (int64_t)cache->num_blocks * BS;
        if (d == 64)
            hipLaunchKernelGGL(append_i8_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, kp,
                               vp, ks, vs, (const qf16 *)k, (const qf16 *)v, d_slots, n, hkv, num_slots);
        else
            hipLaunchKernelGGL(append_i8_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, kp,
                               vp, ks, vs, (const qf16 *)k, (const qf16 *)v, d_slots, n, hkv, num_slots);
        return launched("kv_append");
    }
    i32x4 *kp = (i32x4 *)cache->k_pool + layer * layer_chunks;
    i32x4 *vp = (i32x4 *)cache->v_pool + layer * layer_chunks;
    const int64_t total = (int64_t)n * hkv * nch;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff)
        return fail(KVP_ERR_UNSUPPORTED, "kv_append: n too large");
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, kp,
                       vp, (const i32x4 *)k, (const i32x4 *)v, d_slots, n, hkv, nch,
                       (int64_t)cache->num_blocks * BS);
    return launched("kv_append");
}

kvp_status kv_copy_blocks(const kvp_cache_desc *cache, const int32_t *d_pairs, int32_t n,
                          kvp_stream stream)
{
    kvp_status st = check_cache(cache, "kv_copy_blocks");
    if (st != KVP_OK)
        return st;
    if (n < 0)
        return fail(KVP_ERR_INVALID, "kv_copy_blocks: n=%d", n);
    if (n == 0)
        return KVP_OK;
    if (!d_pairs)
        return fail(KVP_ERR_INVALID, "kv_copy_blocks: pairs is NULL");
    if (n > 0x7fffffff / 1 || cache->dims.num_layers > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "kv_copy_blocks: too many pairs or layers");
    const int nch = chunks_per_row(cache->dims);
    const bool i8 = cache->dims.dtype == KVP_I8;
    CopyPools C;
    C.pool[0] = (i32x4 *)cache->k_pool;
    C.pool[1] = (i32x4 *)cache->v_pool;
    C.pool[2] = i8 ? (i32x4 *)cache->k_scale : nullptr;
    C.pool[3] = i8 ? (i32x4 *)cache->v_scale : nullptr;
    C.block_chunks[0] = (int64_t)cache->dims.num_kv_heads * BS * nch;
    C.block_chunks[1] = (int64_t)cache->dims.num_kv_heads * BS * 2 / 16; // fp16 scales
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, cache->dims.num_layers, i8 ? 4 : 2), dim3(256), 0,
                       (hipStream_t)stream, C, d_pairs, cache->num_blocks);
    return launched("kv_copy_blocks");
}

kvp_status kv_gather(const kvp_cache_desc *cache, int32_t layer, const int32_t *d_block_table,
                     int32_t max_blocks, const int32_t *d_context_lens, int32_t B, int32_t Lmax,
                     void *k_out, void *v_out, kvp_stream stream)
{
    kvp_status st = check_cache(cache, "kv_gather");
    if (st != KVP_OK)
        return st;
    if (layer < 0 || layer >= cache->dims.num_layers)
        return fail(KVP_ERR_INVALID, "kv_gather: layer %d out of range", layer);
    if (B < 0 || Lmax <= 0 || max_blocks <= 0)
        return fail(KVP_ERR_INVALID, "kv_gather: B=%d Lmax=%d max_blocks=%d", B, Lmax, max_blocks);
    if (B == 0)
        return KVP_OK;
    if (!d_block_table || !d_context_lens || !k_out || !v_out ||
        (((uintptr_t)k_out | (uintptr_t)v_out) & 15))
        return fail(KVP_ERR_INVALID, "kv_gather: NULL or misaligned pointer");
    if (B > 65535 || cache->dims.num_kv_heads > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "kv_gather: B or H_kv too large");
    const int nch = chunks_per_row(cache->dims);
    const int hkv = cache->dims.num_kv_heads;
    const int64_t layer_chunks = (int64_t)cache->num_blocks * hkv * BS * nch;
    dim3 grid((Lmax + BS - 1) / BS, hkv, B);
    hipLaunchKernelGGL(gather_kernel, grid, dim3(128), 0, (hipStream_t)stream,
                       (const i32x4 *)cache->k_pool + layer * layer_chunks,
                       (const i32x4 *)cache->v_pool + layer * layer_chunks, d_block_table,
                       max_blocks, d_context_lens, hkv, Lmax, nch, cache->num_blocks,
                       (i32x4 *)k_out, (i32x4 *)v_out);
    if (cache->dims.dtype == KVP_I8) // V codes are stored dim-major: rewrite them token-major
        hipLaunchKernelGGL(gather_v_i8_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                           (const char *)cache->v_pool + layer * layer_chunks * 16, d_block_table, max_blocks,
                           d_context_lens, hkv, Lmax, cache->dims.head_dim, cache->num_blocks, (char *)v_out);
    return launched("kv_gather");
}

kvp_status contiguous_kv_append(const kvp_dims *dims, void *k_cache, void *v_cache, int32_t Lmax,
                                const void *k, const void *v, const int32_t *d_pos, int32_t B,
                                kvp_stream stream)
{
    if (!dims)
        return fail(KVP_ERR_INVALID, "contiguous_kv_append: dims is NULL");
    if (!head_dim_ok(dims->head_dim))
        return fail(KVP_ERR_UNSUPPORTED, "contiguous_kv_append: head_dim=%d (64 or 128)", dims->head_dim);
    if (dims->dtype == KVP_I8)
        return fail(KVP_ERR_UNSUPPORTED, "contiguous_kv_append: int8 caches are paged only");
    if ((dims->dtype != KVP_F16 && dims->dtype != KVP_F32) || dims->num_kv_heads <= 0 || B < 0 ||
        Lmax <= 0)
        return fail(KVP_ERR_INVALID, "contiguous_kv_append: bad arguments");
    if (B == 0)
        return KVP_OK;
    if (!k_cache || !v_cache || !k || !v || !d_pos ||
        (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k | (uintptr_t)v) & 15))
        return fail(KVP_ERR_INVALID, "contiguous_kv_append: NULL or misaligned pointer");
    const int nch = chunks_per_row(*dims);
    const int total = B * dims->num_kv_heads * nch;
    hipLaunchKernelGGL(contig_append_kernel, dim3((total + 255) / 256), dim3(256), 0,
                       (hipStream_t)stream, (i32x4 *)k_cache, (i32x4 *)v_cache, (const i32x4 *)k,
                       (const i32x4 *)v, d_pos, B, dims->num_kv_heads, Lmax, nch);
    return launched("contiguous_kv_append");
}

} // extern "C"
