/*
 * kvp.h -- C ABI of the MI355X (gfx950) paged key-value-cache attention library.
 *
 * What the library computes (pages cited by title and section):
 *   [CHAP]  neuralialabs "Tornar a inferencia barata: KV cache, batching e quantizacao":
 *           the KV cache (keys/values of earlier positions never change under the causal
 *           mask, so they are stored), prefill vs decode, the per-token cache size
 *           2*L*H_kv*d*bytes, grouped-query attention, PagedAttention (fixed-size blocks
 *           plus a per-sequence block table; shared-prefix blocks).
 *   [KVES]  gustavoai "La cache de claves y valores: cuanto cuesta cada token": the four
 *           steps of one cached token (append k_t, v_t to each head's cache, then attend
 *           over the whole cache including itself).
 *   [XF]    chatgpz.de "Aufmerksamkeit", xformers demo sections 4 (packed variable-length
 *           batch with a block-diagonal, optionally causal, mask) and 5 (grouped-query
 *           attention in the (B, M, G, Hq/G, K) layout).
 *   [PAGED] same feed, paged-attention article: SECTION 2 (page pool with a free list
 *           and reference counts, block table per request) and SECTION 3 (copy-on-write
 *           shared system prompts).
 *   [FLASH] same feed, FlashAttention post: blocks of keys/values processed on chip with
 *           a partial softmax, merged by rescaling with e^(block max - global max).
 *   [LIN]   same feed, linear-attention post: TraditionalAttention, softmax(QK^T/sqrt(d))V.
 *
 * Conventions for every call
 *   - Every function returns kvp_status (0 = KVP_OK, negative = error).  On error nothing
 *     has changed: no host state and no device memory; kvp_last_error() describes it.
 *   - Device memory is always owned by the caller.  Arguments documented "device" are
 *     device pointers (e.g. from torch tensors); the library never allocates device memory.
 *   - Work is enqueued asynchronously on the given stream (NULL = the null stream); the
 *     host returns before the kernels run.  Errors detected on the host are reported
 *     before anything is enqueued.
 *   - Host objects (kvp_pool) are owned by the library and freed by block_pool_destroy.
 *     A pool is not thread-safe: one owner thread at a time.
 *   - Layouts: head_dim d = 64, or 128 with fp16 or int8.  dtype is fp16 (KVP_F16), fp32
 *     (KVP_F32) or int8 codes with one fp16 scale per row (KVP_I8, paged caches only; q,
 *     out and appended rows are then fp16).
 *       paged K/V pool, one per K and V:  [num_layers][num_blocks][H_kv][block_size][d]
 *         (int8 V pool: dim-major blocks [num_layers][num_blocks][H_kv][d][block_size])
 *       int8 scale pool, one per K and V:   fp16 [num_layers][num_blocks][H_kv][block_size]
 *       contiguous cache (one layer):       [B][H_kv][Lmax][d]
 *       decode q / out:                     [B][H_q][d]
 *       packed prefill q / out:             [T][H_q][d];  k, v: [T][H_kv][d]
 *       block table:                        int32 [B][max_blocks], logical block -> block id
 *       slot:                               int64 block_id * block_size + offset
 *   - Query head h reads key-value head h / (H_q / H_kv)  ([CHAP] GQA passage, [XF] 5).
 */
#ifndef KVP_H
#define KVP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP stream handle without including the HIP headers (same type as hipStream_t). */
struct ihipStream_t;
typedef struct ihipStream_t *kvp_stream;

typedef int32_t kvp_status;
#define KVP_OK 0
#define KVP_ERR_INVALID (-1)     /* bad argument, shape or state                    */
#define KVP_ERR_OOM (-2)         /* block pool has no free block                    */
#define KVP_ERR_NOT_FOUND (-3)   /* unknown sequence id                             */
#define KVP_ERR_HIP (-4)         /* the HIP runtime reported an error on launch     */
#define KVP_ERR_UNSUPPORTED (-5) /* valid request this build does not implement     */

enum { KVP_F16 = 0, KVP_F32 = 1, KVP_I8 = 2 };

typedef struct {
    int32_t num_layers;
    int32_t num_q_heads;
    int32_t num_kv_heads; /* num_q_heads % num_kv_heads == 0            */
    int32_t head_dim;     /* 64, or 128 (fp16 / int8)                   */
    int32_t dtype;        /* KVP_F16, KVP_F32 or KVP_I8                  */
} kvp_dims;

/* Quantized cache rows (KVP_I8; [CHAP] quantization section, symmetric absmax, applied to
 * the cache): each (token, KV head) row x of d values of K, and separately of V, is stored
 * as int8 codes and one fp16 scale: scale = fp16(max|x| / 127) (fp32 quotient rounded to
 * nearest even), code = clamp(rint(x / scale), -128, 127) in fp32 with the stored scale
 * (round half to even), all codes 0 when the scale is 0.  Reconstruction: code * scale.
 * K codes are stored like fp16 rows; V codes dim-major within a block (byte j * 16 + r of
 * a (block, head) is dimension j of the block's row r), so that the decode kernel reads
 * the values of one dimension for consecutive tokens as consecutive bytes. */
typedef struct {
    kvp_dims dims;
    int32_t block_size; /* tokens per block: 16                          */
    int32_t num_blocks;
    void *k_pool; /* device [num_layers][num_blocks][H_kv][block_size][d] */
    void *v_pool; /* device, same shape (int8: [..][H_kv][d][block_size])  */
    void *k_scale; /* KVP_I8: device fp16 [num_layers][num_blocks][H_kv][block_size];
                      NULL otherwise                                      */
    void *v_scale; /* KVP_I8: same, for V                                 */
} kvp_cache_desc;

/* Thread-local description of the last error on this thread ("" if none). */
const char *kvp_last_error(void);
/* Library version string. */
const char *kvp_version(void);

/* ======================================================================================
 * Host block manager  ([PAGED] SECTION 2 and 3; [CHAP] PagedAttention passage)
 * ==================================================================================== */
typedef struct kvp_pool kvp_pool;

typedef struct {
    int32_t src; /* block copied from, -1 if no copy was needed */
    int32_t dst; /* block copied to,   -1 if no copy was needed */
} kvp_copy;

typedef struct {
    int32_t total_blocks;
    int32_t used_blocks;
    int32_t free_blocks;
    int32_t shared_blocks; /* blocks with reference count > 1 */
    int32_t num_seqs;
    double utilisation_pct; /* used / total * 100 ([PAGED] SECTION 2) */
} kvp_pool_stats;

/* Create a pool of num_blocks blocks of block_size tokens.  The free list starts as
 * 0..num_blocks-1; allocation takes the front, release appends to the back ([PAGED] 2).
 * INVALID if num_blocks <= 0 or block_size <= 0.  *out receives the pool. */
kvp_status block_pool_create(int32_t num_blocks, int32_t block_size, kvp_pool **out);
void block_pool_destroy(kvp_pool *pool);

/* Reorder the free list (only while every block is free): perm is a permutation of
 * 0..num_blocks-1 giving the new front-to-back order.  Used to obtain scattered tables.
 * INVALID if blocks are in use or perm is not a permutation. */
kvp_status block_pool_set_free_order(kvp_pool *pool, const int32_t *perm, int32_t n);

/* New sequence holding n_tokens tokens: ceil(n_tokens / block_size) fresh blocks, each
 * with reference count 1, taken from the front of the free list ([PAGED] SECTION 2: a new
 * request is given the pages its tokens need; [CHAP] PagedAttention passage: the cache is
 * allocated in fixed-size blocks on demand).  OOM (and no change) if too few blocks are
 * free. */
kvp_status block_table_alloc(kvp_pool *pool, int32_t n_tokens, int32_t *seq_id);

/* Reserve the position of sequence `seq`'s next token and return its slot.  At a block
 * boundary a new block is taken ([PAGED] 2, generate_token).  If the target block is
 * shared (reference count > 1) it is first made private by copy-on-write and *cow gets
 * {src, dst}: the caller must copy block src to dst on the device (kv_copy_blocks) before
 * writing the slot; otherwise *cow = {-1, -1}.  OOM / NOT_FOUND leave everything as is. */
kvp_status block_table_append_slot(kvp_pool *pool, int32_t seq, int64_t *slot, kvp_copy *cow);

/* One decode step for a batch: block_table_append_slot for seqs[0..n-1] in order (each id
 * at most once); slots[i] and cows[i] receive that call's results.  All or nothing:
 * capacity for every new and copied block is checked first, so OOM changes nothing. */
kvp_status block_table_append_slots(kvp_pool *pool, const int32_t *seqs, int32_t n,
                                    int64_t *slots, kvp_copy *cows);

/* Reserve the positions of the next n tokens of `seq` (e.g. a prompt appended after a
 * shared prefix) and write their slots to slots[n].  Same rules as n calls of
 * block_table_append_slot; at most the first, partially filled block can need
 * copy-on-write, reported in *cow as above.  All or nothing: OOM changes nothing. */
kvp_status block_table_reserve(kvp_pool *pool, int32_t seq, int32_t n, int64_t *slots,
                               kvp_copy *cow);

/* Fork: the child gets a copy of the parent's block table and token count, and every
 * block's reference count goes up by one ([PAGED] 3, share). */
kvp_status block_table_fork(kvp_pool *pool, int32_t parent, int32_t *child);

/* Copy-on-write of one logical block: if its block is shared, take a new block, release
 * the old one and point the table at the new one; *src and *dst report the pair to copy on the
 * device.  If the block is private, *src = *dst = that block (nothing to do). */
kvp_status block_table_cow(kvp_pool *pool, int32_t seq, int32_t logical_block, int32_t *src,
                           int32_t *dst);

/* Shorten a sequence to n_tokens (<= its current count): blocks past
 * ceil(n_tokens / block_size) are released; a kept block that is shared stays shared, so the
 * next append into it copies it first.  Used to give a forked request a shorter view of a
 * shared prefix, and to roll back tokens that were reserved but rejected. */
kvp_status block_table_truncate(kvp_pool *pool, int32_t seq, int32_t n_tokens);

/* Release every block of the sequence (a block returns to the free list when its
 * reference count reaches 0) and forget the sequence ([PAGED] SECTION 2: a finished
 * request hands its pages back, a page is free again once no table refers to it; SECTION
 * 3: a shared page survives while other requests hold it).  NOT_FOUND for an unknown id;
 * releasing a block that is already free is INVALID (nothing changes). */
kvp_status block_table_free(kvp_pool *pool, int32_t seq);

/* Host export of n sequences' tables into host_table [n][max_blocks] (unused entries -1)
 * and their token counts into context_lens [n] ([PAGED] SECTION 2: the per-request block
 * table maps logical block j / block_size to a physical page; [CHAP] PagedAttention
 * passage: the kernel reaches the cache through that table).  INVALID if a table is longer
 * than max_blocks; NOT_FOUND for an unknown id.  The caller uploads both to the device for
 * the attention calls. */
kvp_status block_table_export(const kvp_pool *pool, const int32_t *seqs, int32_t n,
                              int32_t max_blocks, int32_t *host_table, int32_t *context_lens);

/* Slots of tokens [start, start+n) of a sequence (all already reserved) into slots[n]. */
kvp_status block_table_slots(const kvp_pool *pool, int32_t seq, int32_t start, int32_t n,
                             int64_t *slots);

/* One sequence's table: *n_tokens, *n_blocks, and up to cap block ids into blocks. */
kvp_status block_table_get(const kvp_pool *pool, int32_t seq, int32_t *n_tokens,
                           int32_t *n_blocks, int32_t *blocks, int32_t cap);

kvp_status block_pool_stats(const kvp_pool *pool, kvp_pool_stats *stats);
/* Reference count of a block (0 if free). */
kvp_status block_pool_refcount(const kvp_pool *pool, int32_t block, int32_t *refcount);

/* Bytes of cache per token: 2 * L * H_kv * d * elem_bytes ([CHAP] cache-size passage). */
int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                           int32_t elem_bytes);

/* ======================================================================================
 * Batching over the block pool  ([CHAP] batching passage; [PAGED] SECTION 1, 2 and 4)
 * A step-by-step schedule of n requests on `slots` places, driving a private kvp_pool of
 * num_blocks blocks of block_size tokens:
 *   - all requests are queued at step 0, in index order;
 *   - at the start of a step, free places admit queued requests in order -- with
 *     KVP_SCHED_STATIC only when no place is occupied (the previous batch was returned),
 *     with KVP_SCHED_CONTINUOUS whenever a place is free; admission allocates the prompt
 *     (KVP_ALLOC_PAGED: ceil(prompt / block_size) blocks) or max_seq_len tokens
 *     (KVP_ALLOC_NAIVE, the contiguous worst-case reservation) and stops at the first
 *     request the pool cannot hold (a deferral);
 *   - in a step every admitted, unfinished request produces one token (paged: through
 *     block_table_append_slot; a request whose token needs a block the pool cannot give
 *     stalls for the step);
 *   - a request finishes in the step that produces its last token; continuous: it is
 *     returned at once and its place and blocks are free for the next step; static: the
 *     batch is returned, and its blocks freed, when its last member finishes (the others
 *     hold their places as padding until then);
 *   - latency[i] = number of the step that returns request i (from 1); service[i] = steps
 *     from its admission to its return; utilisation after a step = resident tokens /
 *     (blocks held * block_size), averaged over steps.
 * OOM when every admitted request waits for a block and nothing can be admitted (no
 * preemption); INVALID for bad arguments (output_lens >= 1, prompts >= 0, and with naive
 * allocation prompt + output <= max_seq_len).  latency / service: host int32 [n] or NULL.
 * ==================================================================================== */
#define KVP_SCHED_STATIC 0
#define KVP_SCHED_CONTINUOUS 1
#define KVP_ALLOC_PAGED 0
#define KVP_ALLOC_NAIVE 1

typedef struct {
    int32_t slots;       /* places in the batch                              */
    int32_t policy;      /* KVP_SCHED_STATIC or KVP_SCHED_CONTINUOUS          */
    int32_t alloc;       /* KVP_ALLOC_PAGED or KVP_ALLOC_NAIVE                */
    int32_t max_seq_len; /* naive reservation per request (tokens)            */
    int32_t block_size;  /* tokens per block                                  */
    int32_t num_blocks;  /* blocks in the pool                                */
} kvp_sched_config;

typedef struct {
    int64_t steps;              /* steps until every request was returned            */
    int64_t tokens;             /* tokens produced (sum of output_lens)              */
    int64_t busy_slot_steps;    /* tokens produced, i.e. places that did work        */
    int64_t padding_slot_steps; /* places held by finished members of a static batch */
    int64_t peak_blocks;        /* most blocks held at the end of a step             */
    int64_t deferrals;          /* admissions stopped by a full pool                 */
    int64_t stalls;             /* tokens delayed by a full pool                     */
    int64_t max_latency;
    double mean_latency;        /* steps, from arrival                               */
    double mean_service;        /* steps, from admission                             */
    double mean_utilisation;    /* mean over steps of resident / held tokens         */
} kvp_sched_result;

kvp_status sched_simulate(const kvp_sched_config *cfg, const int32_t *prompt_lens,
                          const int32_t *output_lens, int32_t n, int32_t *latency,
                          int32_t *service, kvp_sched_result *res);

/* ======================================================================================
 * Device operations (HIP kernels for gfx950)
 * ==================================================================================== */

/* Copy whole blocks for copy-on-write: for each pair p < n, block d_pairs[2p] is copied to
 * block d_pairs[2p+1] in every layer, in both K and V pools (and, for an int8 cache, in
 * both scale pools), bit for bit ([PAGED] 3).
 * d_pairs: device int32 [n][2].  n == 0 is a no-op. */
kvp_status kv_copy_blocks(const kvp_cache_desc *cache, const int32_t *d_pairs, int32_t n,
                          kvp_stream stream);

/* Write n new tokens' keys and values of one layer into their slots ([KVES] step 2:
 * k_t, v_t go to the end of each head's cache).  k, v: device [n][H_kv][d] in the cache
 * dtype (fp16 for an int8 cache); d_slots: device int64 [n] (slot = block * block_size +
 * offset, every slot < num_blocks * block_size, distinct).  Bit-exact copy; an int8 cache
 * stores each row's codes and scale (quantized as described at kvp_cache_desc). */
kvp_status kv_append(const kvp_cache_desc *cache, int32_t layer, const void *k, const void *v,
                     const int64_t *d_slots, int32_t n, kvp_stream stream);

/* Contiguous-layout append ([KVES] step 2: k_t, v_t go to the end of each head's cache;
 * [CHAP] allocator check: one contiguous (B, H_kv, L, d) tensor per layer): for each b < B,
 * writes k[b], v[b] ([B][H_kv][d], device) at position d_pos[b] (device int32 [B], each in
 * 0..Lmax-1, distinct per b) of k_cache / v_cache ([B][H_kv][Lmax][d], one layer, device),
 * bit for bit.  fp16 or fp32 (UNSUPPORTED for int8); INVALID for Lmax <= 0 or NULL
 * pointers. */
kvp_status contiguous_kv_append(const kvp_dims *dims, void *k_cache, void *v_cache,
                                int32_t Lmax, const void *k, const void *v,
                                const int32_t *d_pos, int32_t B, kvp_stream stream);

/* Workspace bytes for decode with B requests and contexts up to max_context tokens: one
 * counter per (request, KV head) and the split partials (m, l, o) that the [FLASH] rescale
 * merge combines (block softmaxes kept with their maximum and sum).  0 if the arguments are
 * invalid or no split is needed. */
size_t decode_workspace_bytes(const kvp_dims *dims, int32_t B, int32_t max_context);

/* Paged grouped-query decode attention for one layer ([CHAP] decode loop; [KVES] the new
 * position attends over every cached position and itself; [LIN] softmax(q k^T * scale) v;
 * [FLASH] block partials merged by rescaling).  For request b < B and query head h:
 *   out[b][h] = sum_j softmax_j(scale * q[b][h] . k_j) v_j over j < d_context_lens[b],
 * k_j / v_j read from block d_block_table[b][j / block_size], offset j % block_size, KV
 * head h / (H_q / H_kv).  The token of this step must already be appended.
 *   q, out: device [B][H_q][d] in the cache dtype (fp16 for an int8 cache, whose rows are
 *   reconstructed as code * scale inside the kernel).  d_block_table: device int32
 *   [B][max_blocks].  d_context_lens: device int32 [B], each in 1..max_blocks*block_size.
 *   scale: 0 means 1/sqrt(d).  workspace: device, at least
 *   decode_workspace_bytes(dims, B, max_blocks * block_size) bytes (may be NULL if that is
 *   0), 256-byte aligned and ZERO-FILLED before its first use; every call leaves its
 *   counters at zero again, so a workspace is reused without clearing.  Calls sharing a
 *   workspace must not overlap in time (one stream is fine).
 * Work split (fp16): each (request, KV head) pair is cut into splits of 32 blocks (512
 * tokens), one wave each; a pair with several splits is merged by the last of its waves in
 * split order, so results are deterministic and identical between the paged and
 * contiguous layouts.  fp32 softmax and accumulation; the softmax weights enter the value
 * product rounded once to fp16 (the normaliser sums the same rounded weights); one
 * rounding to the output dtype. */
kvp_status paged_decode_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                  const void *q, const int32_t *d_block_table,
                                  int32_t max_blocks, const int32_t *d_context_lens, int32_t B,
                                  float scale, void *workspace, size_t ws_bytes,
                                  kvp_stream stream);

/* paged_decode_attention fused with the append of this step's token ([KVES] step 2 then
 * step 3 in one pass): for every request b, k_new[b] / v_new[b] (device [B][H_kv][d], fp16)
 * are written into the cache at position d_context_lens[b] - 1 (through the block table; that
 * block must be private to the request, i.e. copy-on-write already done) and the attention
 * of the same call already sees them.  Equivalent to kv_append at those slots followed by
 * paged_decode_attention, in one kernel.  fp16 or int8 caches (the kernel quantizes the
 * new rows exactly as kv_append does); UNSUPPORTED for fp32. */
kvp_status paged_decode_append_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                         const void *q, const void *k_new, const void *v_new,
                                         const int32_t *d_block_table, int32_t max_blocks,
                                         const int32_t *d_context_lens, int32_t B, float scale,
                                         void *workspace, size_t ws_bytes, kvp_stream stream);

/* paged_decode_attention for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels, splits and
 * results (bit for bit), but no workspace argument -- the split counters and partials live
 * in a static device array of the library, KVP_NOALLOC_SCRATCH_BYTES per GPU (the first
 * KVP_NOALLOC_MAX_PAIRS * 4 bytes hold the counters), held by each GPU the library runs on
 * until the process ends.  The call itself allocates nothing.  INVALID (nothing launched)
 * when B * H_kv exceeds KVP_NOALLOC_MAX_PAIRS or the split partials of B requests with
 * contexts up to max_blocks * block_size tokens exceed the rest of the array (about 1000
 * requests with tables of up to 2048 tokens, or 64 of 32768, at 14q / 2kv, d = 64).  The first call on a device zeroes the
 * counters with a small kernel on `stream`; every call leaves them at zero.  Calls on one
 * GPU share the array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must not be issued; one stream at a time is fine. */
#define KVP_NOALLOC_SCRATCH_BYTES (16u << 20)
#define KVP_NOALLOC_MAX_PAIRS 65536
kvp_status paged_decode_attention_noalloc(const kvp_cache_desc *cache, int32_t layer, void *out,
                                          const void *q, const int32_t *d_block_table,
                                          int32_t max_blocks, const int32_t *d_context_lens,
                                          int32_t B, float scale, kvp_stream stream);

/* The same decode over a contiguous cache k_cache / v_cache [B][H_kv][Lmax][d] (one layer;
 * the layout of the cache tensors in [CHAP]'s allocator check).  Same kernels, same split
 * policy and the same arithmetic order as the paged call, so the outputs of the two are
 * bit-identical for the same logical data.  fp16 and fp32 (UNSUPPORTED for int8). */
kvp_status contiguous_decode_attention(const kvp_dims *dims, void *out, const void *q,
                                       const void *k_cache, const void *v_cache, int32_t Lmax,
                                       const int32_t *d_context_lens, int32_t B, float scale,
                                       void *workspace, size_t ws_bytes, kvp_stream stream);

/* --------------------------------------------------------------------------------------
 * Planned decode: a host-built work plan, built once per step from the host copy of the
 * block table and shared by every layer of that step.  Requests that are consecutive in
 * the batch and whose tables start with the same physical blocks (sequences forked from
 * one prefix, [PAGED] SECTION 3; [CHAP] PagedAttention passage on shared prefixes) get
 * that prefix read ONCE per KV head: one work item scores the K/V tiles of the shared
 * blocks against the query rows of every member (up to 16 members and 64 query rows),
 * each member up to its own limit, and the member's partial joins the partials of its
 * private blocks in the same merge as any other split.  Same result as
 * paged_decode_attention up to the order of the fp32 sums; without sharing
 * (flags = 0) the plan reproduces paged_decode_attention's splits exactly, bit for bit.
 * ------------------------------------------------------------------------------------ */
#define KVP_PLAN_SHARE_PREFIX 1u
/* Batches of long contexts: when the private blocks number far more than the waves the GPU
 * holds at once (about 1024 for fp16, 2048 for int8 caches, from dims->dtype), cut each
 * pair's private range into fewer, longer parts (up to 192 blocks; their block ids go to an
 * id area at the end of the image) so that the launch runs in about one generation of
 * waves.  Changes the splits, so the result equals the unplanned call's up to the order of
 * the fp32 sums only.  The plan's split sizes also follow dims->dtype: int8 caches at head
 * dim 64 are cut into 16-block parts (32 otherwise), as in the unplanned call. */
#define KVP_PLAN_LONG_ITEMS 2u
/* Width of shared items, in blocks of 16 query columns (a block holds 16 / G members of G
 * heads, G = H_q / H_kv <= 16).  By default a shared item is one block wide -- two blocks
 * when a block holds a single member (9 <= G <= 16) -- so a prefix is read once per run of
 * up to 16 / G members; KVP_PLAN_SHARE_WIDE2 / KVP_PLAN_SHARE_WIDE4 let one item serve 2 or
 * 4 blocks of members (at most 2 at head dim 128) and cut it to 16 or 8 blocks of the
 * prefix, so the prefix is read fewer times by more, shorter items.  Groups above 16 have
 * no shared items. */
#define KVP_PLAN_SHARE_WIDE2 4u
#define KVP_PLAN_SHARE_WIDE4 8u
/* Batches too small to fill the GPU (decode of one or a few requests): cut private ranges
 * into parts shorter than the default 32 blocks, down to 8 -- the shortest part length, in
 * whole 4-block tiles, at which the private items of every pair still fit the waves the GPU
 * holds at once (about 1024 for fp16, 2048 for int8 caches) beside the plan's shared items.
 * A split pair's parts are merged by the same rescale as any split (chatgpz.de
 * "Aufmerksamkeit", FlashAttention post: block softmaxes combined through their maxima), so
 * the chain of tiles one wave streams shortens while idle waves take the other parts.  A
 * batch whose 32-block parts already fill the waves keeps its plan.  Changes the splits, so
 * the result equals the unplanned call's up to the order of the fp32 sums only. */
#define KVP_PLAN_FILL 16u

typedef struct {
    int32_t B;            /* batch the plan was built for                            */
    int32_t num_kv_heads;
    int32_t group;        /* query heads per KV head                                 */
    int32_t num_blocks;   /* block ids in the plan are < num_blocks                  */
    int32_t n_items;      /* work items (one wave each)                              */
    int32_t n_shared;     /* of which read a shared prefix for several requests      */
    int32_t head_dim;     /* head dim of the cache the plan is for (64 or 128)       */
    int32_t col_blocks;   /* widest item, in blocks of 16 query columns (1, 2 or 4);
                           * launches of plans whose items are all one block wide use
                           * a kernel built for that width (0: up to 4)              */
    int64_t n_slots;      /* partial slots the workspace must hold                   */
    int64_t bytes;        /* bytes of the plan image (device copy)                   */
    int64_t off_pair_base, off_pair_nparts, off_req_shared; /* offsets in the image  */
    int64_t kv_blocks_read; /* (block, KV head) reads the plan performs               */
    int64_t off_ids, n_ids; /* id area of long items (offset in the image, int32 count);
                             * n_ids bounds the kernel's id reads, so a launch replayed
                             * for later plans may carry the device buffer's capacity  */
} kvp_decode_plan;

/* Upper bound of the plan image bytes for B requests of at most max_blocks blocks, or for
 * pad_items items if that is larger (0 if the arguments are invalid). */
size_t decode_plan_bytes(const kvp_dims *dims, int32_t B, int32_t max_blocks, int32_t pad_items);

/* Build a plan on the host.  h_block_table: host int32 [B][max_blocks]; h_context_lens:
 * host int32 [B] (the lengths the decode will use, i.e. with this step's token); entries
 * outside 0..num_blocks-1 are recorded as unusable (their rows are masked).  flags:
 * KVP_PLAN_SHARE_PREFIX to read shared prefixes once (0: plain per-request splits), plus
 * KVP_PLAN_LONG_ITEMS for long-context batches.
 * pad_items: 0, or a fixed item count (rounded up to a multiple of 8): the image then has
 * exactly that many items (the rest are empty) and offsets that depend only on pad_items,
 * B and the head shape, so that successive steps' plans launch identically (a captured
 * graph can be replayed with a new image in the same device buffer); INVALID if the step
 * needs more items.  h_image: host buffer of image_bytes >= decode_plan_bytes(...)
 * receiving the image; the caller copies plan->bytes of it to device memory (16-byte
 * aligned) before the decode.  UNSUPPORTED for fp32 (the planned kernel serves fp16 and
 * int8 caches), or a group size above 16 that is not a multiple of 16 or needs more than 4
 * column blocks (2 at head dim 128). */
kvp_status decode_plan_build(const kvp_dims *dims, const int32_t *h_block_table,
                             int32_t max_blocks, const int32_t *h_context_lens, int32_t B,
                             int32_t num_blocks, uint32_t flags, int32_t pad_items,
                             void *h_image, size_t image_bytes, kvp_decode_plan *plan);

/* Workspace bytes the planned decode needs for this plan (0 if it needs none).  The layout
 * (per-pair counters first, then partials) depends only on B and the head shape, so a
 * larger workspace serves later plans of the same batch. */
size_t decode_plan_workspace_bytes(const kvp_decode_plan *plan);

/* paged_decode_attention (k_new = v_new = NULL) or paged_decode_append_attention (both
 * given) following a plan.  d_plan: device copy of the plan image; the plan must have
 * been built from this step's block table and context lengths and for this cache
 * (num_blocks <= cache->num_blocks, same head shape).  The block table itself is not
 * read: its entries are in the plan.  workspace: decode_plan_workspace_bytes(plan) bytes,
 * same rules as paged_decode_attention.  The new token's block must be private (copy-on-
 * write done) -- the plan never treats a context's last block as shared. */
kvp_status paged_decode_attention_planned(const kvp_cache_desc *cache, int32_t layer,
                                          void *out, const void *q, const void *k_new,
                                          const void *v_new, const kvp_decode_plan *plan,
                                          const void *d_plan, float scale, void *workspace,
                                          size_t ws_bytes, kvp_stream stream);

/* Several new query rows per request against the paged cache: chunked prefill of a
 * suffix into an existing (possibly shared) prefix, or the verification pass over gamma
 * drafted tokens ([CHAP] speculative-decoding section: verifying gamma proposed tokens is
 * one forward pass over gamma positions; [PAGED] SECTION 3: requests continue from shared
 * prefix blocks with their own tokens).  Request b has m_b = d_cu_q[b+1] - d_cu_q[b] new
 * rows, packed rows d_cu_q[b] .. of q and out; they are the last m_b of its
 * d_context_lens[b] positions, whose K and V -- prefix and new rows -- are already in the
 * cache (kv_append into block_table_reserve slots), and row i attends to positions
 * 0 .. ctx_b - m_b + i (causal, aligned to the end of the context).
 *   q, out        device fp16 [T][H_q][64], T = d_cu_q[B]
 *   d_block_table device int32 [B][max_blocks]; entries outside [0, num_blocks) mask their
 *                 keys; max_blocks <= 4096
 *   d_cu_q        device int32 [B+1], non-decreasing from 0;  max_q >= every m_b
 * Requires m_b <= ctx_b (rows with no position of their own get zeros).  fp16 caches only
 * (UNSUPPORTED otherwise).  MFMA tiles with fp32 accumulation, as varlen_causal_prefill. */
kvp_status paged_prefill_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                   const void *q, const int32_t *d_block_table, int32_t max_blocks,
                                   const int32_t *d_context_lens, const int32_t *d_cu_q, int32_t B,
                                   int32_t max_q, float scale, kvp_stream stream);

/* Wait bound of the fp16 split merge.  A context split over several work items is merged
 * by the item that holds its final blocks: it polls the pair's counter until the others
 * have stored their partials, with a short sleep after each poll, and after `polls` polls
 * it falls back to the counted merge, in which the last of the pair's items to finish
 * merges every partial from memory.  Both merges combine the partials in the same order
 * with the same arithmetic, so results are bit-identical either way; 0 always takes the
 * counted merge.  Default 0.  Process-wide, for launches made after the call; returns
 * the previous bound (a negative argument only queries it). */
int32_t kvp_decode_merge_polls(int32_t polls);

/* Packed variable-length prefill ([XF] section 4, [XF] 5 for the head map).  Segment s
 * covers packed rows d_cu_seqlens[s] .. d_cu_seqlens[s+1]-1.  Row i of a segment attends
 * to rows j <= i of the same segment (causal = 1) or to every row of its segment
 * (causal = 0, block-diagonal mask).  q/out: device [T][H_q][d]; k, v: device [T][H_kv][d];
 * d_cu_seqlens: device int32 [nseg+1], non-decreasing, starting at 0; max_seqlen >= every
 * segment length (sizes the grid).  fp16 uses MFMA tiles with fp32 accumulation. */
kvp_status varlen_causal_prefill(const kvp_dims *dims, void *out, const void *q, const void *k,
                                 const void *v, const int32_t *d_cu_seqlens, int32_t nseg,
                                 int32_t max_seqlen, int32_t causal, float scale,
                                 kvp_stream stream);

/* Gather one layer of the paged cache back to the contiguous layout ([PAGED] SECTION 2:
 * logical token j of a request lives in page table[j / block_size] at offset
 * j % block_size; [CHAP] allocator check: the contiguous (B, H_kv, L, d) layout): positions
 * j < d_context_lens[b] of k_out / v_out [B][H_kv][Lmax][d] (device) receive the paged
 * rows, bit for bit; other positions are left untouched.  For an int8 cache the rows are
 * the codes (the scales stay in the scale pools).  A test aid: INVALID for bad sizes or
 * NULL pointers. */
kvp_status kv_gather(const kvp_cache_desc *cache, int32_t layer, const int32_t *d_block_table,
                     int32_t max_blocks, const int32_t *d_context_lens, int32_t B, int32_t Lmax,
                     void *k_out, void *v_out, kvp_stream stream);

/* --------------------------------------------------------------------------------------
 * Measurement aid: the achievable HBM read bandwidth, against which the decode kernels'
 * rates are set ([CHAP] decode is bound by the bytes read from memory).  Reads `bytes`
 * bytes of d_buf (device, 16-byte aligned, bytes a multiple of 16) once, with 16-byte
 * loads (8 in flight per lane) from `waves` wavefronts of 64 lanes (0: 8 per compute
 * unit) striding over the buffer, and stores nothing unless the data holds a bit pattern that decides it (into
 * d_sink, device int32 [1]); time it with events on `stream`.  INVALID for bad sizes.
 * ------------------------------------------------------------------------------------ */
kvp_status kvp_read_bandwidth_probe(const void *d_buf, size_t bytes, int32_t waves, int32_t *d_sink,
                                    kvp_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* KVP_H */
