// kvp_decode_f16.hip -- fp16 grouped-query decode attention for gfx950: one kernel per
// layer that (optionally) appends the step's new token, attends over the cache and merges
// split partitions.
//
// What is computed (pages cited by title and section):
//   neuralialabs "Tornar a inferencia barata: KV cache, batching e quantizacao": decode
//   feeds one token whose query attends over every cached key (a 1 x n score row);
//   grouped-query attention shares each key-value head among a group of query heads;
//   PagedAttention reaches the cache through a per-sequence table of fixed-size blocks,
//   and forked sequences share their prefix blocks (copy-on-write).
//   gustavoai "La cache de claves y valores", four-step token recipe: k_t, v_t are put at
//   the end of each head's cache (step 2) before the attention row over the whole cache
//   (step 3), so the new position sees itself.
//   chatgpz.de "Aufmerksamkeit", linear-attention post: TraditionalAttention,
//   softmax(q K^T / sqrt(d_k)) V.
//   same feed, FlashAttention post, "Was ist der mathematische Aspekt von Softmax?": block
//   softmaxes keep their maximum and exponential sum and are merged by rescaling with
//   e^(block max - global max) -- used across tiles and across split partitions.
//
// Work decomposition: one wave per work item.  An item is up to 32 consecutive 16-token
// blocks (8 tiles of 64 tokens at head dim 64, 16 tiles of 32 tokens at 128) of one KV head, either of one request ("private") or of a
// few requests that share those physical blocks ("shared": the query rows of every member,
// up to 16 rows, are scored against the same K/V tile).  The planner puts all shared items
// of one prefix on one XCD, so the prefix is fetched from HBM about once per step and
// served from that XCD's L2 to its other readers, and spreads each XCD's items over its
// CUs.  Items come from a host-built plan (paged_decode_attention_planned) or, without a
// plan, from the wave index: request pair (b, g), split k of ceil(blocks / 32).  A pair
// split over several items leaves one partial (m, l, o) per item; one of them merges the
// partials in slot order (merge_column), so results are deterministic.  Partials travel
// through 16-byte device-coherent stores and loads, ordered by a store-completion wait.
//
// Per wave: K and V tiles stream HBM -> LDS through global_load_lds_dwordx4 into a ring of
// NBUF slots (16 KB of K and V per tile, 16 loads); waits are explicit vmcnt counts.
//   scores  S^T = K Q^T       v_mfma_f32_16x16x32_f16, K rows from LDS (chunk-swizzled),
//                             query rows as one 16-column block
//   softmax fp32, hardware exp2 of one FMA (scale folded in), reference max moved only
//           when a row's maximum passes it by 2^8, p rounded once to fp16
//   values  O^T = V^T P^T     v_mfma_f32_16x16x32_f16; P^T is the score MFMA's own output
//                             layout (no data movement), V^T comes from transposing LDS
//                             reads (ds_read_b64_tr_b16); row sums from an all-ones operand
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "kvp_decode_common.h"
#include "kvp_gfx950.h"
#include "kvp_plan_format.h"
#include "kvp_quant.h"

namespace kvp {

using namespace dec;
using namespace plan;

// floats of one partial record of a head of dimension HD: o[HD], m, l and 2 of padding
// (16-byte records)
constexpr int part_floats(int HD) { return HD + 4; }
// tile length (tokens) and ring depth of the decode kernel at head dim 64: 64-token tiles in
// a 2-slot ring take 32 KB of LDS per wave, which leaves room for four waves per CU (head
// dim 128 takes 32-token tiles, the same 32 KB)
#ifndef DEC_TT
#define DEC_TT 64
#endif
#ifndef DEC_NBUF
#define DEC_NBUF 2
#endif

struct PlanView {
    const int *items;       // planned: [n_items][REC]
    const int *pair_base;   // planned: [B*Hkv]
    const int *pair_nparts; // planned: [B*Hkv]
    const int *req_shared;  // planned: [B]
    int ipp;                // unplanned: items per pair
    const int *ids;         // planned: id area of long items
    long long n_ids;        // planned: ints in the id area
};

struct Item {
    int b, g, nmem, blk0, nblk, end, slot, nparts, pbase;
};

// One step of the slot-order merge of partials (m, l, o): M, L, O absorb partial (m, l, o)
// over n output elements.  Both merge paths below go through it, in the same order, so a
// pair's result does not depend on which item merges it.
__device__ __forceinline__ void merge_step(float &M, float &L, float *O, int n, float m, float l, const float *o)
{
    const float mn = fmaxf(M, m);
    if (mn != -INFINITY) {
        const float a = fast_exp2(M - mn), c = fast_exp2(m - mn);
        L = fmaf(L, a, l * c);
        for (int k = 0; k < n; ++k)
            O[k] = fmaf(O[k], a, o[k] * c);
        M = mn;
    }
}

// 16- and 8-byte device-coherent accesses (agent scope, like coherent_store / _load: the
// write goes through to memory, the read misses the XCD's L2).  The loads are inline
// assembly: the caller waits for them (wait_stores) before it uses the results.
__device__ inline void coherent_store4(float *p, f32x4 v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ inline void coherent_store2(float *p, float a, float b)
{
    const float2 v = {a, b};
    asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
// Device-coherent reads of partials other items stored (sc1: past this XCD's L2), as
// relaxed agent-scope atomic loads of 8 bytes, so the compiler sees each load and waits for
// it before the first use of its value.
__device__ inline float2 coherent_load2(const float *p)
{
    const unsigned long long v =
        __hip_atomic_load((const unsigned long long *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return float2{__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32))};
}
__device__ inline f32x4 coherent_load4(const float *p)
{
    const float2 a = coherent_load2(p), b = coherent_load2(p + 2);
    return f32x4{a.x, a.y, b.x, b.y};
}

// Merge, for this lane's column, the np partials of its pair (slots pbase .. pbase+np-1) in
// slot order; the partial of slot own is this lane's registers (om, ol, oacc), the others are
// read from memory.  Lane (col, grp) holds output dims 16 db + 4 grp + i as O[4 db + i].
// Writes the normalised row to outp (this column's HD outputs).  The partials are read four
// at a time, every load of a batch issued before the first is used, so a batch costs one
// round trip.
template <int HD>
__device__ __forceinline__ void merge_column(const float *part, int G, int pbase, int np, int own, int hd, int grp,
                                             float om, float ol, const f32x4 (&oacc)[HD / 16], f16 *outp)
{
    constexpr int NDB = HD / 16;
    constexpr int NB = 4; // partials per batch (registers: NB (HD / 4 + 2))
    float M = -INFINITY, L = 0.f, O[4 * NDB];
#pragma unroll
    for (int k = 0; k < 4 * NDB; ++k)
        O[k] = 0.f;
    for (int j0 = 0; j0 < np; j0 += NB) {
        f32x4 ov[NB][NDB];
        float2 ml[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const int j = j0 + jj;
            if (j < np && j != own) {
                const float *src = part + ((size_t)(pbase + j) * G + hd) * part_floats(HD);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    ov[jj][db] = coherent_load4(src + 16 * db + 4 * grp);
                ml[jj] = coherent_load2(src + HD);
            } else {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    ov[jj][db] = oacc[db];
                ml[jj] = float2{om, ol};
            }
        }
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const int j = j0 + jj;
            if (j < np) {
                float o[4 * NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[4 * db + i] = ov[jj][db][i];
                merge_step(M, L, O, 4 * NDB, ml[jj].x, ml[jj].y, o);
            }
        }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        f16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = (f16)(L > 0.f ? O[4 * db + i] / L : 0.f);
        *(f16x4 *)(outp + 16 * db + 4 * grp) = o;
    }
}

// One work item.  rv: lane R_ENT + j holds the physical id of the item's block j; a long
// item (longi) has id j in lane j % 64 of rid[j / 64] instead.
//
// Tile t = TT tokens = blocks (TT / 16) t .. of the item.  Lane (col, grp) = (lane % 16,
// lane / 16).  MFMA column col is query row col of the item (member col / G, head col % G).
// fp16 cache: K and V tiles sit in LDS as TT rows of 2 HD bytes; 16-byte chunk c of row r
// is stored at chunk slot swz<HD>(c, r); the score MFMA's row m of 16-key block kb is tile
// row 16 kb + m, and V^T comes from transposing reads.
// int8 cache (I8): K rows of HD codes (16-byte chunk c of row r at slot swz8<HD>(c, r)), V
// blocks dim-major (HD rows of 16 codes per block, as the cache stores them), and the
// tile's row scales (K scales of tile row tt at byte 2 tt of the scale slot, V scales at
// 32 KB + 2 tt).  The score MFMA's row m of block kb is tile row 32 (kb / 2) + 8 (m / 4) +
// 4 (kb % 2) + m % 4, so that lane group grp's probabilities of k-step ks are the eight
// consecutive tokens 32 ks + 8 grp + s, whose V codes of one dimension are eight
// consecutive bytes.  K codes enter the score product as exact fp16 integers and each key's
// score is multiplied by its row scale in fp32; V codes become fp16 operands code * scale,
// rounded once.
template <int NCB, bool SHARED, int NBUF, int TT, int HD, bool I8, bool LONGI, typename Addr>
__device__ __forceinline__ void run_item(const DecodeParams &P, const Addr &A, const PlanView &PV,
                                         const Item &it, int rv, const int (&rid)[3], char *kring, char *vring,
                                         char *sring)
{
    static_assert(TT == 32 || TT == 64, "tiles of 32 or 64 tokens");
    static_assert(HD == 64 || HD == 128, "head dimension 64 or 128");
    constexpr int KB = TT / BS;      // blocks per tile
    constexpr int KS = TT / 32;      // k-steps of 32 tokens per tile (value product)
    constexpr int RB = 2 * HD;       // bytes of one K (or V) row
    constexpr int CPR = HD / 8;      // 16-byte chunks per row
    constexpr int RPI = 1024 / RB;   // rows per 1 KB DMA load
    constexpr int IPB = BS / RPI;    // 1 KB loads per block and tensor
    constexpr int KD = HD / 32;      // k-steps of 32 dims (score product)
    constexpr int NDB = HD / 16;     // 16-dim blocks (value product)
    constexpr int SLOT = TT * RB;    // bytes of one K (or V) fp16 tile
    // the cached rows as the ring holds them (int8: one byte per value)
    constexpr int RQ = I8 ? HD : RB;   // bytes of one cached row
    constexpr int CPQ = RQ / 16;       // 16-byte chunks per cached row
    constexpr int RPIQ = 1024 / RQ;    // cached rows per 1 KB DMA load
    constexpr int IPBQ = BS / RPIQ;    // 1 KB loads per block and tensor
    constexpr int SLOTQ = TT * RQ;     // bytes of one ring slot per tensor
    constexpr int NDMA = 2 * KB * IPBQ + (I8 ? 1 : 0); // loads per tile (+ the row scales)
    constexpr int VBLK = BS * HD;      // int8: bytes of one dim-major V block (per KV head)
    static_assert(!I8 || Addr::paged, "int8 caches are paged");
    static_assert(I8 || (RQ == RB && IPBQ == IPB), "fp16 ring = tile");
    const int lane = threadIdx.x;
    const int col = lane & 15, grp = lane >> 4;
    const int hkv = P.hkv;
    const char *kc = (const char *)P.kc;
    const char *vc = (const char *)P.vc;
    const float c = P.scale_log2;
    const float inv_c = 1.f / c;

    // ---- this lane's query rows, one per column block: q operand, token limit, slots ----
    // Group size G = Hq / Hkv.  G <= 16: column block cb holds members cb mpb .. (mpb =
    // 16 / G members of G columns each); column col is member cb mpb + col / G, head col % G,
    // and columns >= mpb G are unused.  G > 16 (a multiple of 16, private items only): block
    // cb holds heads 16 (cb % bpm) .. + 15 of member cb / bpm (bpm = G / 16).
    const int G = P.group;
    const int mpb = G <= 16 ? 16 / G : 1;
    const int bpm = G <= 16 ? 1 : G >> 4;
    const int jm = G <= 16 ? col / G : 0; // member of this column within its block
    int hdc[NCB], bm[NCB];
    bool cv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int mem = G <= 16 ? cb * mpb + jm : cb / bpm;
        hdc[cb] = G <= 16 ? col - jm * G : 16 * (cb % bpm) + col;
        cv[cb] = (G > 16 || jm < mpb) && mem < it.nmem;
        bm[cb] = it.b + (cv[cb] ? mem : 0);
    }
    f16x8 qop[NCB][KD];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const f16 *qp = (const f16 *)P.q + ((size_t)bm[cb] * P.hq + (size_t)it.g * G + hdc[cb]) * HD + grp * 8;
        const f16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
            const f16x8 qv = *(const f16x8 *)(qp + 32 * ks);
            qop[cb][ks] = cv[cb] ? qv : z;
        }
    }
    // the step's new K / V row (lanes 0 .. CPR-1: K chunks, CPR .. 2 CPR-1: V chunks)
    const bool app = !SHARED && P.k_new != nullptr;
    i32x4 nrow = {0, 0, 0, 0};
    if (app && lane < 2 * CPR) {
        // K or V row by lane, as masked arithmetic (a select of the two pointers is turned
        // into a table in scratch memory)
        const uintptr_t kb = (uintptr_t)P.k_new, vb = (uintptr_t)P.v_new;
        const uintptr_t base = kb + ((vb - kb) & (uintptr_t)(-(intptr_t)(lane >= CPR)));
        const size_t off = (((size_t)it.b * hkv + it.g) * HD + (lane & (CPR - 1)) * 8) * sizeof(f16);
        nrow = *(const __attribute__((address_space(1))) i32x4 *)(base + off);
    }
    const int nt = (it.nblk + KB - 1) / KB;
    auto ent = [&](int j) -> int {
        if constexpr (LONGI) {
            const int jj = min(j, LONG_BPI - 1);
            return jj < 64 ? lane_int(rid[0], jj) : (jj < 128 ? lane_int(rid[1], jj - 64) : lane_int(rid[2], jj - 128));
        } else {
            return lane_int(rv, R_ENT + min(j, BPI - 1));
        }
    };
    auto block_ok = [&](int j) -> bool { return (j < it.nblk) & A.valid(ent(j)); };

    // ---- DMA of tile t into ring slot t % NBUF: per block, IPB loads of RPI rows of K and V
    // (lane: row RPI h + lane / CPR, chunk lane % CPR of the LDS row) ----
    auto issue = [&](int t) {
        char *kd = kring + (t % NBUF) * SLOTQ;
        char *vd = vring + (t % NBUF) * SLOTQ;
        size_t brow[KB]; // row index of row 0 of each block (a readable block if unusable)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int j = KB * t + kb;
            const int e = ent(j);
            const bool ok = (j < it.nblk) & A.valid(e);
            const int lb = it.blk0 + j;
            brow[kb] = ok ? A.block_row(it.b, it.g, lb, e) : A.safe_row0(it.b, it.g);
#pragma unroll
            for (int h = 0; h < IPBQ; ++h) {
                const int r = RPIQ * h + lane / CPQ;
                const int sr = ok ? A.row(lb, r) : A.safe_row(r);
                size_t off, voff; // bytes
                if constexpr (I8) {
                    off = (brow[kb] + sr) * HD + swz8<HD>(lane % CPQ, 16 * kb + r) * 16;
                    voff = brow[kb] * HD + h * 1024 + lane * 16; // dim-major block, linear
                } else {
                    off = ((brow[kb] + sr) * HD + swz<HD>(lane & (CPR - 1), r) * 8) * sizeof(f16);
                    voff = off;
                }
                const int i = IPBQ * kb + h;
                __builtin_amdgcn_global_load_lds((const void *)(kc + off),
                                                 (__attribute__((address_space(3))) void *)(kd + i * 1024),
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const void *)(vc + voff),
                                                 (__attribute__((address_space(3))) void *)(vd + i * 1024),
                                                 16, 0, 0);
            }
        }
        if constexpr (I8) {
            // row scales: lane i < 2 KB takes half i % 2 of block i / 2's 16 K scales, the next
            // 2 KB lanes the V scales; the other lanes repeat them (their copies are unused)
            const int idx = lane % (4 * KB);
            const int sb = (idx >> 1) % KB, half = idx & 1;
            size_t rs = brow[0];
#pragma unroll
            for (int q = 1; q < KB; ++q)
                rs = sb == q ? brow[q] : rs;
            const uintptr_t kb_ = (uintptr_t)P.ksc, vb_ = (uintptr_t)P.vsc;
            const uintptr_t base = kb_ + ((vb_ - kb_) & (uintptr_t)(-(intptr_t)(idx >= 2 * KB)));
            __builtin_amdgcn_global_load_lds((const void *)(base + (rs + 8 * half) * sizeof(f16)),
                                             (__attribute__((address_space(3))) void *)(sring + (t % NBUF) * 1024),
                                             16, 0, 0);
        }
    };

    // shared items: each member's shared extent and slot range (loaded before the first DMA,
    // so that waiting for them does not also wait for the tile)
    int l0v[NCB], b0v[NCB], n0v[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        l0v[cb] = 0;
        b0v[cb] = 0;
        n0v[cb] = 0;
        if constexpr (SHARED) {
            const int pair = bm[cb] * hkv + it.g;
            l0v[cb] = PV.req_shared[bm[cb]];
            b0v[cb] = PV.pair_base[pair];
            n0v[cb] = PV.pair_nparts[pair];
        }
    }
    // The first NBUF tiles' DMA (one per ring slot) goes out as soon as the item's addresses
    // are known, before anything waits for a load: the column limits and the new row's
    // quantization are not needed before the first tile is computed.  The tiles are issued
    // even past the item's end (their rows then come from the readable block and are unused),
    // so that every path has the same loads in flight and one wait covers the loads issued
    // before them (q operands, the new row, the members' extents) without waiting for a tile.
#pragma unroll
    for (int k = 0; k < NBUF; ++k)
        issue(k);
    wait_vm<NBUF * NDMA>();
    __builtin_amdgcn_sched_barrier(0);

    // lim: tokens >= lim are masked for this row; rows whose results are not kept (padding
    // columns, members that do not take part) have no limit -- their columns of the MFMA
    // tiles are independent of the others and are never stored
    int lim[NCB], pb[NCB], np[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if constexpr (SHARED) {
            // a member takes part if its shared extent reaches into this item; its part index
            // inside the pair's slot range is the item's R_SLOT
            const int l0 = l0v[cb], b0 = b0v[cb], n0 = n0v[cb];
            const bool in = cv[cb] && l0 > BS * it.blk0;
            lim[cb] = in ? l0 : 0x7fffffff;
            pb[cb] = b0 + it.slot;
            np[cb] = in ? n0 : 0;
        } else {
            lim[cb] = cv[cb] ? it.end : 0x7fffffff;
            pb[cb] = it.slot;
            np[cb] = it.nparts;
        }
    }
    // tokens >= rend hold no data for any column of this item
    const int rend = SHARED ? BS * (it.blk0 + it.nblk) : it.end;
    // a tile ending at or before full_end needs no masking (when all its blocks are valid)
    int full_end = rend;
    if constexpr (SHARED) {
        // member cb mpb + j's limit sits in block cb, lane j G
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            for (int j = 0; j < mpb; ++j)
                if (cb * mpb + j < it.nmem)
                    full_end = min(full_end, lane_int(lim[cb], j * G));
    }

    // int8: the new rows' codes and scales (lanes of one row exchange its maximum)
    u32x2 ncodes = {0u, 0u};
    unsigned nscale = 0;
    if constexpr (I8) {
        if (app) {
            const f16 s16 = quantize_row_piece<CPR>(__builtin_bit_cast(f16x8, nrow), ncodes);
            nscale = __builtin_bit_cast(unsigned short, s16);
        }
    }

    // running state of this lane's column in each block: reference max (scaled, log2 units),
    // output O^T rows 16 db + 4 grp + i, and the row sum (every entry of accl holds it)
    float mref[NCB], thr[NCB]; // thr: rescale_threshold of mref (raw-score units)
    f32x4 acc[NCB][NDB], accl[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        mref[cb] = -INFINITY;
        thr[cb] = -INFINITY;
        accl[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};

    // fp16 cache: LDS byte addresses of this lane's operand reads in ring slot 0.  The
    // swizzle sees a row only through row % 8, which 16-row steps leave alone, so the K reads
    // of one 32-dim step and the V reads of one 16-dim block differ only by constants (the
    // instruction's offset field); the bases move to the tile's slot once per tile.
    //   K: row 16 kb + col, chunk 4 ks + grp              -> kbase[ks] + 16 kb RB
    //   V: row 16 (2 ks + h) + 4 grp + col / 4, chunk 2 db + (col % 4) / 2, half col % 2
    //                                                     -> vbase[db] + 16 (2 ks + h) RB
    unsigned kbase[KD], vbase[NDB];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
        kbase[ks] = lds_addr(kring) + col * RB + swz<HD>(4 * ks + grp, col) * 16;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int row = 4 * grp + (col >> 2);
        const int ch = 2 * db + ((col & 3) >> 1);
        vbase[db] = lds_addr(vring) + row * RB + swz<HD>(ch, row) * 16 + (col & 1) * 8;
    }

    auto compute = [&](int t) {
        char *kt = kring + (t % NBUF) * SLOT; // fp16 cache: the tiles read by the products
        char *vt = vring + (t % NBUF) * SLOT;
        const int tb = BS * (it.blk0 + KB * t); // position of tile row 0
        bool bok[KB];
        bool all_ok = true;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            bok[kb] = block_ok(KB * t + kb);
            all_ok = all_ok && bok[kb];
        }
        const bool full = all_ok && tb + TT <= full_end;
        // value row r of the tile holds data some column may use
        auto row_used = [&](int r) -> bool {
            const int kb = r >> 4;
            bool okb = bok[0];
#pragma unroll
            for (int q = 1; q < KB; ++q)
                okb = kb == q ? bok[q] : okb;
            return okb && tb + r < rend;
        };
        if constexpr (!I8) {
            // value rows that no column may use: zero them (the cache can hold NaN there)
            if (!full) {
#pragma unroll
                for (int k = 0; k < TT * CPR / 64; ++k) {
                    const int ch = lane + 64 * k, r = ch / CPR;
                    if (!row_used(r))
                        lds_store_b128(vt + ch * 16, i32x4{0, 0, 0, 0});
                }
            }
            // the new token of this step: into LDS (this tile) and into the cache
            if (app) {
                const int pos = it.end - 1, r = pos - tb;
                if (r >= 0 && r < TT) {
                    const int j = KB * t + (r >> 4);
                    const int e = ent(j);
                    if (lane < 2 * CPR && j < it.nblk && A.valid(e)) {
                        const int ch = lane & (CPR - 1);
                        const int lb = it.blk0 + j;
                        const size_t dst = A.block_off(it.b, it.g, lb, e) + (size_t)A.row(lb, r & 15) * HD + ch * 8;
                        lds_store_b128((lane < CPR ? kt : vt) + r * RB + swz<HD>(ch, r) * 16, nrow);
                        const uintptr_t kb = (uintptr_t)P.kc_w, vb = (uintptr_t)P.vc_w;
                        const uintptr_t base = kb + ((vb - kb) & (uintptr_t)(-(intptr_t)(lane >= CPR)));
                        *(__attribute__((address_space(1))) i32x4 *)(base + dst * sizeof(f16)) = nrow;
                    }
                }
            }
        } else {
            char *kq = kring + (t % NBUF) * SLOTQ;
            char *vq = vring + (t % NBUF) * SLOTQ;
            char *sq = sring + (t % NBUF) * 1024;
            // the new token of this step: codes and scale into the ring slot and the cache
            // (K row-major, V dim-major: one byte per dimension)
            if (app) {
                const int pos = it.end - 1, r = pos - tb;
                if (r >= 0 && r < TT) {
                    const int j = KB * t + (r >> 4);
                    const int e = ent(j);
                    if (lane < 2 * CPR && j < it.nblk && A.valid(e)) {
                        const int ch = lane & (CPR - 1); // dims 8 ch .. 8 ch + 7
                        const int lb = it.blk0 + j;
                        const size_t brow = A.block_row(it.b, it.g, lb, e);
                        if (lane < CPR) {
                            lds_store_b64(kq + r * RQ + swz8<HD>(ch >> 1, r) * 16 + (ch & 1) * 8, ncodes);
                            *(__attribute__((address_space(1))) u32x2 *)((uintptr_t)P.kc_w + (brow + (r & 15)) * HD +
                                                                          ch * 8) = ncodes;
                        } else {
                            char *vg = (char *)P.vc_w + brow * HD + (r & 15);
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                const unsigned b = (ncodes[i >> 2] >> (8 * (i & 3))) & 0xff;
                                lds_store_b8(vq + (r >> 4) * VBLK + (8 * ch + i) * BS + (r & 15), b);
                                *(__attribute__((address_space(1))) unsigned char *)(vg + (8 * ch + i) * BS) =
                                    (unsigned char)b;
                            }
                        }
                        if (ch == 0) {
                            lds_store_b16(sq + (lane < CPR ? 0 : 32 * KB) + 2 * r, nscale);
                            const uintptr_t ks = (uintptr_t)P.ksc_w, vs = (uintptr_t)P.vsc_w;
                            const uintptr_t sb = ks + ((vs - ks) & (uintptr_t)(-(intptr_t)(lane >= CPR)));
                            *(__attribute__((address_space(1))) unsigned short *)(sb + (brow + (r & 15)) * sizeof(f16)) =
                                (unsigned short)nscale;
                        }
                    }
                }
            }
        }
        wave_lds_sync();

        f16x8 kop[KB][KD]; // A of the score MFMA
        f16x8 vop[KS][NDB]; // A of the value MFMA (V^T)
        float kscale[KB][4]; // int8: the K row scales of this lane's score rows
        if constexpr (I8) {
            char *kq = kring + (t % NBUF) * SLOTQ;
            char *vq = vring + (t % NBUF) * SLOTQ;
            char *sq = sring + (t % NBUF) * 1024;
            // K: lane (col, grp) of block kb reads tile row 32 (kb/2) + 8 (col/4) + 4 (kb%2) +
            // col%4, dims 32 ks + 8 grp .. (8 bytes); the codes enter the score product as
            // exact fp16 integers and the row scales multiply the fp32 scores afterwards.
            // The lane's score rows 4 grp + i of block kb are the consecutive tile rows
            // 32 (kb/2) + 8 grp + 4 (kb%2) + i: their four scales are one 8-byte read.
            constexpr int NK = KB * KD + KB; // K codes and their row scales: one group of reads
            unsigned ka[NK];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int rt = 32 * (kb >> 1) + 8 * (col >> 2) + 4 * (kb & 1) + (col & 3);
#pragma unroll
                for (int ks = 0; ks < KD; ++ks)
                    ka[kb * KD + ks] = lds_addr(kq + rt * RQ + swz8<HD>(2 * ks + (grp >> 1), rt) * 16 + (grp & 1) * 8);
                ka[KB * KD + kb] = lds_addr(sq + 2 * (32 * (kb >> 1) + 8 * grp + 4 * (kb & 1)));
            }
            u32x2 kr[NK];
            lds_read_b64<NK>(kr, ka);
            u32x2 kraw[KB][KD];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KD; ++ks)
                    kraw[kb][ks] = kr[kb * KD + ks];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned w = kr[KB * KD + kb][i >> 1];
                    kscale[kb][i] = (float)__builtin_bit_cast(f16, (unsigned short)(i & 1 ? w >> 16 : w & 0xffffu));
                }
            // V^T: lane (col, grp) of k-step ks reads dimension 16 db + col of tokens 32 ks +
            // 8 grp .. + 7 (8 consecutive bytes of the dim-major block), and their 8 scales
            static_assert(KS * NDB == 8, "8 V reads per int8 tile");
            unsigned va[8], sa[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sa[ks] = lds_addr(sq + 32 * KB + 2 * (32 * ks + 8 * grp));
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    va[ks * NDB + db] = lds_addr(vq + (2 * ks + (grp >> 1)) * VBLK + (16 * db + col) * BS + 8 * (grp & 1));
            }
            u32x2 vr[8];
            i32x4 vsc[KS];
            lds_read_v_i8<KS>(vr, vsc, va, sa);
            u32x2 vraw8[KS][NDB];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vraw8[ks][db] = vr[ks * NDB + db];
            // value rows no column may use: their scales (which can be anything) become 0
            if (!full) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int tb0 = 32 * ks + 8 * grp; // tile row of slot 0
                    bool okb = bok[0];
#pragma unroll
                    for (int q = 1; q < KB; ++q)
                        okb = (tb0 >> 4) == q ? bok[q] : okb;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        unsigned m = 0;
                        if (okb && tb + tb0 + 2 * w < rend)
                            m |= 0xffffu;
                        if (okb && tb + tb0 + 2 * w + 1 < rend)
                            m |= 0xffff0000u;
                        vsc[ks][w] = (int)((unsigned)vsc[ks][w] & m);
                    }
                }
            }
            // codes -> fp16: code + 128 as the low byte of the fp16 number 1024 + byte, minus
            // 1152 (exact), times the scale (one rounding)
            typedef f16 f16x2_ __attribute__((ext_vector_type(2)));
            const f16x2_ bias = {(f16)1152.f, (f16)1152.f};
            // the codes alone, as exact fp16 integers
            auto codes8 = [&](u32x2 code) -> f16x8 {
                unsigned h[4];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const unsigned x = code[w] ^ 0x80808080u;
                    const unsigned lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
                    const unsigned hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
                    h[2 * w] = __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2_, lo) - bias);
                    h[2 * w + 1] = __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2_, hi) - bias);
                }
                return __builtin_bit_cast(f16x8, i32x4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
            };
            auto dequant8 = [&](u32x2 code, const unsigned (&sc)[4]) -> f16x8 {
                unsigned h[4];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const unsigned x = code[w] ^ 0x80808080u;
                    const unsigned lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
                    const unsigned hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
                    h[2 * w] = __builtin_bit_cast(
                        unsigned, (__builtin_bit_cast(f16x2_, lo) - bias) * __builtin_bit_cast(f16x2_, sc[2 * w]));
                    h[2 * w + 1] = __builtin_bit_cast(
                        unsigned, (__builtin_bit_cast(f16x2_, hi) - bias) * __builtin_bit_cast(f16x2_, sc[2 * w + 1]));
                }
                return __builtin_bit_cast(f16x8, i32x4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
            };
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KD; ++ks)
                    kop[kb][ks] = codes8(kraw[kb][ks]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const unsigned sc[4] = {(unsigned)vsc[ks][0], (unsigned)vsc[ks][1], (unsigned)vsc[ks][2],
                                        (unsigned)vsc[ks][3]};
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vop[ks][db] = dequant8(vraw8[ks][db], sc);
            }
        } else {
        // K rows (A of the score MFMA): row 16 kb + col, dims 32 ks + 8 grp .. (chunk 4 ks + grp)
        const unsigned soff = (unsigned)((t % NBUF) * SLOT);
        unsigned kb_t[KD], vb_t[NDB]; // the operand bases in this tile's ring slot
#pragma unroll
        for (int ks = 0; ks < KD; ++ks)
            kb_t[ks] = kbase[ks] + soff;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vb_t[db] = vbase[db] + soff;
        lds_read_k<KB, KD, 0, 16 * RB>(kop, kb_t);
        // V^T (A of the value MFMA) of k-step ks and dims 16 db ..: lane (col, grp) needs
        // V[token][16 db + col] for its k-slots s, token 16 (2 ks + s / 4) + 4 grp + s % 4.
        // A transposing read hands lane i of a 16-lane group half i % 4 of the 8 bytes
        // addressed by lane 4 j + i / 4 as its element j; so lane L of the group addresses
        // token row 16 (2 ks + h) + 4 grp + L / 4, dims 16 db + 4 (L % 4) .. + 3, and the two
        // reads h = 0, 1 give slots 0-3 and 4-7.
        f16x4 vraw[KS][NDB][2];
        lds_read_vt<KS, NDB, 0, 16 * RB>(vraw, vb_t);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                vop[ks][db] = __builtin_shufflevector(vraw[ks][db][0], vraw[ks][db][1], 0, 1, 2, 3, 4, 5, 6, 7);
        }

        // per column block: scores, softmax, values (the K and V operands serve every block)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
        // scores: sacc[kb][i] = S[token of MFMA row 4 grp + i of block kb][column col] (unscaled)
        f32x4 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb][0], qop[cb][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int ks = 1; ks < KD; ++ks)
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb][ks], qop[cb][ks], s, 0, 0, 0);
            sacc[kb] = s;
        }
        if constexpr (I8) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sacc[kb][i] *= kscale[kb][i];
        }
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                // tile row of sacc[kb][0] and its block
                const int r0 = I8 ? 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) : 16 * kb + 4 * grp;
                bool okb = bok[0];
#pragma unroll
                for (int q = 1; q < KB; ++q)
                    okb = (r0 >> 4) == q ? bok[q] : okb;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sacc[kb][i] = (okb && tb + r0 + i < lim[cb]) ? sacc[kb][i] : -INFINITY;
            }
        }
        float mt;
        if constexpr (KB == 4) {
            mt = max16(sacc);
        } else {
            mt = max3(sacc[0][0], sacc[0][1], sacc[0][2]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = kb == 0 ? 3 : 0; i < 4; ++i)
                    mt = max3(mt, sacc[kb][i], sacc[kb][i]);
        }
        // a column's reference max moves only when the column's own maximum passes it by more
        // than 2^8: between moves p = 2^(s c - mref) stays below 256, exact in fp16 range, and
        // the output and row sum need no rescaling.  Columns that do not move scale by exactly
        // 1, so no query row depends on another's keys.  The lane's own maximum is first held
        // against thr; only when some lane passes it does the wave reduce the columns' maxima
        // across lanes and apply the exact test.
        if (__ballot(mt > thr[cb]) != 0) {
            mt = group_max(mt) * c;
            const bool need = mt > mref[cb] + RESCALE_LOG2;
            if (__ballot(need) != 0) {
                const float mn = need ? mt : mref[cb];
                const float alpha = need ? (mref[cb] == -INFINITY ? 0.f : fast_exp2(mref[cb] - mn)) : 1.f;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[cb][db] *= alpha;
                accl[cb] *= alpha;
                mref[cb] = mn;
                thr[cb] = rescale_threshold(mref[cb], c, inv_c);
            }
        }
        const float mc = mref[cb] == -INFINITY ? 0.f : mref[cb];
        // P^T operand of k-step ks, slot s = sacc[2 ks + s / 4][s % 4] -- already in this lane
        // (tile row 16 (2 ks + s / 4) + 4 grp + s % 4 for an fp16 cache, 32 ks + 8 grp + s for
        // int8); rounded once to fp16
        f16x8 pop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int s = 0; s < 8; s += 2) {
                const float p0 = fast_exp2(fmaf(sacc[2 * ks + (s >> 2)][s & 3], c, -mc));
                const float p1 = fast_exp2(fmaf(sacc[2 * ks + (s >> 2)][(s & 3) + 1], c, -mc));
                pop[ks][s] = (f16)p0;
                pop[ks][s + 1] = (f16)p1;
            }
        // values: acc[db][i] = O[column col][dim 16 db + 4 grp + i]; row sums from a ones operand
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[ks][db], pop[ks], acc[cb][db], 0, 0, 0);
            accl[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[ks], accl[cb], 0, 0, 0);
        }
        } // column blocks
        wait_lds(); // this slot is refilled by a later DMA
        wave_lds_sync();
    };

    // ---- stream the item's tiles, NBUF-1 ahead (tiles 0 .. NBUF-1 are already issued) ----
    for (int t = 0; t < nt; ++t) {
        if (t >= 1 && t + NBUF - 1 < nt)
            issue(t + NBUF - 1);
        const int ahead = min(nt - 1 - t, NBUF - 1); // tiles issued after this one
        if (ahead >= 3)
            wait_vm<(NBUF > 3 ? 3 : 0) * NDMA>();
        else if (ahead == 2)
            wait_vm<(NBUF > 2 ? 2 : 0) * NDMA>();
        else if (ahead == 1)
            wait_vm<NDMA>();
        else
            wait_vm<0>();
        compute(t);
    }
    if (nt == 0)
        wait_vm<0>(); // the unused tiles have landed before the wave goes on

    // ---- results ----
    // Rows of an unsplit pair are normalised and written.  A pair split over several items
    // (np > 1) leaves one partial (m, l, o) per item in its slot range and is merged in slot
    // order by one of them: normally the item that counts last on the pair's ticket after
    // storing its partial; with merge polls enabled, the private item of the pair's last
    // slot instead waits (bounded) for the others' count and merges without storing its
    // own.  Every merge goes through merge_column, so the result does not depend on which
    // item merges.
    f16 *outp[NCB];
    bool split_col[NCB];
    bool any_split = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        outp[cb] = (f16 *)P.out + ((size_t)bm[cb] * P.hq + (size_t)it.g * G + hdc[cb]) * HD;
        if (cv[cb] && np[cb] == 1) {
            const float lsum = accl[cb][0];
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const f16x4 o = {(f16)(acc[cb][db][0] * inv), (f16)(acc[cb][db][1] * inv),
                                 (f16)(acc[cb][db][2] * inv), (f16)(acc[cb][db][3] * inv)};
                *(f16x4 *)(outp[cb] + 16 * db + 4 * grp) = o;
            }
        }
        split_col[cb] = cv[cb] && np[cb] > 1;
        any_split = any_split || split_col[cb];
    }
    if (__ballot(any_split) == 0)
        return;
    // each column's pair: first slot and this item's part index in it
    int pbase[NCB], own;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
        pbase[cb] = SHARED ? b0v[cb] : it.pbase; // shared: loaded with the member extents
    own = SHARED ? it.slot : it.slot - it.pbase;
    if constexpr (!SHARED) {
        if (P.merge_polls > 0 && own == np[0] - 1) {
            const int pair = it.b * hkv + it.g;
            int ready = 0;
            if (lane == 0) {
                for (int k = 0; k < P.merge_polls; ++k) {
                    if (coherent_load_int(&P.tickets[pair]) >= np[0] - 1) {
                        ready = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            if (__builtin_amdgcn_readfirstlane(ready)) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    if (cv[cb])
                        merge_column<HD>(P.part, G, pbase[cb], np[cb], own, hdc[cb], grp, mref[cb], accl[cb][0],
                                         acc[cb], outp[cb]);
                if (lane == 0)
                    reset_ticket(&P.tickets[pair]);
                return;
            }
        }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if (split_col[cb]) {
            float *dst = P.part + ((size_t)pb[cb] * G + hdc[cb]) * part_floats(HD);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                coherent_store4(dst + 16 * db + 4 * grp, acc[cb][db]);
            if (grp == 0)
                coherent_store2(dst + HD, mref[cb], accl[cb][0]);
        }
    }
    wait_stores(); // every partial store has completed before a ticket publishes it
    // one ticket per member pair, taken by the lane of the member's first column (G <= 16:
    // head 0 of the member in its block; G > 16: the item's single member, block 0, lane 0)
    int tk[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        int t = -1;
        const bool first = G <= 16 ? hdc[cb] == 0 : (cb == 0 && col == 0);
        if (split_col[cb] && first && grp == 0)
            t = take_ticket(&P.tickets[bm[cb] * hkv + it.g]);
        tk[cb] = t;
    }
    bool last[NCB];
    bool any_last = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int t = G <= 16 ? __shfl(tk[cb], jm * G, 64) : __builtin_amdgcn_readfirstlane(tk[0]);
        last[cb] = split_col[cb] && t == np[cb] - 1;
        any_last = any_last || last[cb];
    }
    if (__ballot(any_last) == 0)
        return;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if (last[cb]) {
            merge_column<HD>(P.part, G, pbase[cb], np[cb], own, hdc[cb], grp, mref[cb], accl[cb][0], acc[cb],
                             outp[cb]);
            const bool first = G <= 16 ? hdc[cb] == 0 : (cb == 0 && col == 0);
            if (first && grp == 0)
                reset_ticket(&P.tickets[bm[cb] * hkv + it.g]);
        }
    }
}

// Private items of a pair take G / 16 column blocks when G > 16 (else one); shared items
// take ceil(members / (16 / G)) blocks, rounded up to 1, 2 or 4.  At most 4 blocks at head
// dim 64 and 2 at 128 (the accumulators of 4 blocks of 128 dims would not fit the VGPRs).
template <int NCB, int NBUF, int TT, int HD, bool I8, bool LONGI, typename Addr>
__device__ __forceinline__ void run_private(const DecodeParams &P, const Addr &A, const PlanView &PV,
                                            const Item &it, int rv, const int (&rid)[3], char *kring, char *vring,
                                            char *sring)
{
    run_item<NCB, false, NBUF, TT, HD, I8, LONGI>(P, A, PV, it, rv, rid, kring, vring, sring);
}

// MAXNCB: the widest item a kernel build serves (1, or 4): the wider paths hold more
// accumulators, and a kernel carrying them allocates more registers for every item (fewer
// resident waves), so launches whose items are all one block wide use the MAXNCB = 1 build.
template <int MAXNCB, int NBUF, int TT, int HD, bool I8, bool LONGI, typename Addr>
__device__ __forceinline__ void dispatch_private(const DecodeParams &P, const Addr &A, const PlanView &PV,
                                                 const Item &it, int rv, const int (&rid)[3], char *kring,
                                                 char *vring, char *sring)
{
    const int bpm = P.group <= 16 ? 1 : P.group >> 4;
    if (bpm == 1)
        run_private<1, NBUF, TT, HD, I8, LONGI>(P, A, PV, it, rv, rid, kring, vring, sring);
    else if constexpr (MAXNCB >= 2) {
        if (bpm == 2)
            run_private<2, NBUF, TT, HD, I8, LONGI>(P, A, PV, it, rv, rid, kring, vring, sring);
        else if constexpr (HD == 64 && MAXNCB >= 4) {
            if (bpm == 4)
                run_private<4, NBUF, TT, HD, I8, LONGI>(P, A, PV, it, rv, rid, kring, vring, sring);
        }
    }
}

template <int MAXNCB, int NBUF, int TT, int HD, bool I8, bool PLANNED, typename Addr>
// items0 = PV.items, passed first so that the dispatcher preloads it into SGPRs (built with
// kernel-argument preloading): a wave's plan record load is its first instruction.
__global__ __launch_bounds__(64) void decode_f16_kernel(const int *items0, DecodeParams P, Addr A, PlanView PV)
{
    static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
    constexpr int EB = I8 ? 1 : 2; // bytes per cached value
    __shared__ __attribute__((aligned(16))) char kring[NBUF * TT * EB * HD];
    __shared__ __attribute__((aligned(16))) char vring[NBUF * TT * EB * HD];
    // int8 only: the tile's row scales per ring slot
    __shared__ __attribute__((aligned(16))) char sring[I8 ? NBUF * 1024 : 16];
    const int lane = threadIdx.x;
    Item it;
    int rv;
    if constexpr (PLANNED) {
        const int *rec = items0 + (size_t)blockIdx.x * REC;
        rv = rec[min(lane, REC - 1)]; // every lane loads (no branch); lanes >= REC are unused
        rv = lane < REC ? rv : -1;
        // the scalar parameters the item needs before its first DMA, fetched while the record
        // is in flight (the compiler would fetch each batch where it is first used, after the
        // record has arrived)
        asm volatile("" ::"s"(P.B), "s"(P.hkv), "s"(P.hq), "s"(P.group), "s"(P.q), "s"(P.kc), "s"(P.vc),
                     "s"(P.k_new), "s"(P.v_new), "s"(A.num_blocks), "s"(A.hkv), "s"(P.scale_log2));
        const int flags = lane_int(rv, R_FLAGS);
        it.b = lane_int(rv, R_B);
        it.g = lane_int(rv, R_G);
        it.nmem = lane_int(rv, R_NMEM);
        it.blk0 = lane_int(rv, R_BLK0);
        it.nblk = lane_int(rv, R_NBLK);
        it.end = lane_int(rv, R_END);
        it.slot = lane_int(rv, R_SLOT);
        it.nparts = lane_int(rv, R_NPARTS);
        it.pbase = lane_int(rv, R_PBASE);
        const bool longi = (flags & F_LONG) != 0;
        // a record that does not fit this call is skipped rather than trusted
        if (it.b < 0 || it.g < 0 || it.g >= P.hkv || it.nmem < 1 || it.b + it.nmem > P.B ||
            it.nblk < 0 || it.nblk > (longi ? LONG_BPI : BPI) || it.blk0 < 0)
            return;
        if (flags & F_EMPTY)
            return;
        if (flags & F_SHARED) {
            const int G = P.group;
            if (G > 16 || it.slot < 0 || longi)
                return;
            const int mpb = 16 / G;
            const int ncb = (it.nmem + mpb - 1) / mpb;
            if (ncb <= 1)
                run_item<1, true, NBUF, TT, HD, I8, false>(P, A, PV, it, rv, {-1, -1, -1}, kring, vring, sring);
            else if constexpr (MAXNCB >= 2) {
                if (ncb <= 2)
                    run_item<2, true, NBUF, TT, HD, I8, false>(P, A, PV, it, rv, {-1, -1, -1}, kring, vring, sring);
                else if constexpr (HD == 64 && MAXNCB >= 4) {
                    if (ncb <= 4)
                        run_item<4, true, NBUF, TT, HD, I8, false>(P, A, PV, it, rv, {-1, -1, -1}, kring, vring,
                                                                   sring);
                }
            }
            return;
        }
        if (it.nmem != 1)
            return;
        // a long item's block ids: from the id area into three registers, lane j holding ids
        // j, 64 + j and 128 + j
        int rid[3] = {-1, -1, -1};
        if (longi) {
            const int off = lane_int(rv, R_IDS);
            if (off < 0 || (long long)off + it.nblk > PV.n_ids)
                return;
#pragma unroll
            for (int k = 0; k < 3; ++k)
                if (64 * k + lane < it.nblk)
                    rid[k] = PV.ids[off + 64 * k + lane];
        }
        if (longi)
            dispatch_private<MAXNCB, NBUF, TT, HD, I8, true>(P, A, PV, it, rv, rid, kring, vring, sring);
        else
            dispatch_private<MAXNCB, NBUF, TT, HD, I8, false>(P, A, PV, it, rv, rid, kring, vring, sring);
    } else {
        const int pair = blockIdx.x / PV.ipp;
        const int k = blockIdx.x - pair * PV.ipp;
        it.b = pair / P.hkv;
        it.g = pair - it.b * P.hkv;
        const int maxc = A.max_ctx();
        int ctx = P.ctx_lens[it.b];
        ctx = ctx < 0 ? 0 : (ctx > maxc ? maxc : ctx);
        const int nbt = (ctx + BS - 1) / BS;
        // one item up to unsplit_blocks blocks, else ceil(blocks / split_blocks) parts; the last
        // (the pair's merging item) up to SPLIT_SLACK tiles longer than the others
        const int n = nbt <= unsplit_blocks(I8, HD) ? 1 : (nbt + split_blocks(I8, HD) - 1) / split_blocks(I8, HD);
        if (k >= n)
            return;
        const int T = (nbt + 3) >> 2;
        it.blk0 = min(nbt, 4 * part_tile_begin(T, n, k, SPLIT_SLACK));
        it.nmem = 1;
        it.nblk = max(0, min(4 * part_tile_begin(T, n, k + 1, SPLIT_SLACK), nbt) - it.blk0);
        it.end = ctx;
        it.nparts = n;
        it.pbase = pair * PV.ipp;
        it.slot = it.pbase + k;
        const int j = lane - R_ENT;
        rv = (j >= 0 && j < it.nblk) ? A.entry(it.b, it.blk0 + j) : -1;
        dispatch_private<MAXNCB, NBUF, TT, HD, I8, false>(P, A, PV, it, rv, {-1, -1, -1}, kring, vring, sring);
    }
}

// ---------------------------------------------------------------------------------------
template <int MAXNCB, bool PLANNED, typename Addr>
static void launch_width(const DecodeParams &P, const Addr &A, const PlanView &PV, dim3 g, hipStream_t st)
{
    dim3 block(64);
    // head_dim 64: 64-token tiles; 128: 32-token tiles (the same 32 KB of LDS for the rings)
    if (P.kv_i8) {
        if constexpr (Addr::paged) {
            if (P.dim == 64)
                hipLaunchKernelGGL((decode_f16_kernel<MAXNCB, DEC_NBUF, DEC_TT, 64, true, PLANNED, Addr>), g, block, 0,
                                   st, PV.items, P, A, PV);
            else
                hipLaunchKernelGGL((decode_f16_kernel<MAXNCB, 2, 32, 128, true, PLANNED, Addr>), g, block, 0, st, PV.items, P, A,
                                   PV);
        }
    } else {
        if (P.dim == 64)
            hipLaunchKernelGGL((decode_f16_kernel<MAXNCB, DEC_NBUF, DEC_TT, 64, false, PLANNED, Addr>), g, block, 0, st,
                               PV.items, P, A, PV);
        else
            hipLaunchKernelGGL((decode_f16_kernel<MAXNCB, 2, 32, 128, false, PLANNED, Addr>), g, block, 0, st, PV.items, P, A,
                               PV);
    }
}

// width: the widest item of the launch in column blocks (1, 2 or 4)
template <bool PLANNED, typename Addr>
static kvp_status launch_f16(const DecodeParams &P, const Addr &A, const PlanView &PV, long long grid, int width,
                             hipStream_t st)
{
    if (grid <= 0)
        return KVP_OK;
    if (grid > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "decode: %lld work items", grid);
    dim3 g((unsigned)grid);
    if (P.dim != 64 && P.dim != 128)
        return fail(KVP_ERR_UNSUPPORTED, "decode: head_dim=%d (64 or 128)", P.dim);
    if (!group_supported(P.group, P.dim))
        return fail(KVP_ERR_UNSUPPORTED, "decode: %d query heads per KV head (1..16, or a multiple of 16 up to %d "
                    "at head dim %d)", P.group, P.dim == 64 ? 64 : 32, P.dim);
    if (P.kv_i8 && !Addr::paged)
        return fail(KVP_ERR_UNSUPPORTED, "decode: int8 caches are paged only");
    if (width <= 1)
        launch_width<1, PLANNED>(P, A, PV, g, st);
    else
        launch_width<4, PLANNED>(P, A, PV, g, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return KVP_OK;
}

int decode_f16_items_per_pair(int max_context, bool i8, int dim)
{
    const int nb = (std::max(max_context, 1) + BS - 1) / BS;
    return nb <= unsplit_blocks(i8, dim) ? 1 : (nb + split_blocks(i8, dim) - 1) / split_blocks(i8, dim);
}

size_t decode_f16_part_bytes(long long slots, int group, int dim)
{
    return (size_t)slots * group * part_floats(dim) * sizeof(float);
}

kvp_status launch_decode_f16(const DecodeParams &P, const PagedAddr &A, int group, int max_context,
                             hipStream_t st)
{
    PlanView PV{nullptr, nullptr, nullptr, nullptr, decode_f16_items_per_pair(max_context, P.kv_i8 != 0, P.dim), nullptr,
                0};
    return launch_f16<false>(P, A, PV, (long long)P.B * P.hkv * PV.ipp, P.group <= 16 ? 1 : P.group / 16, st);
}
kvp_status launch_decode_f16(const DecodeParams &P, const ContigAddr &A, int group, int max_context,
                             hipStream_t st)
{
    PlanView PV{nullptr, nullptr, nullptr, nullptr, decode_f16_items_per_pair(max_context, P.kv_i8 != 0, P.dim), nullptr,
                0};
    return launch_f16<false>(P, A, PV, (long long)P.B * P.hkv * PV.ipp, P.group <= 16 ? 1 : P.group / 16, st);
}
kvp_status launch_decode_f16_planned(const DecodeParams &P, const PagedAddr &A, int group,
                                     const void *d_image, const kvp_decode_plan &plan, hipStream_t st)
{
    const char *img = (const char *)d_image;
    PlanView PV{(const int *)img, (const int *)(img + plan.off_pair_base),
                (const int *)(img + plan.off_pair_nparts), (const int *)(img + plan.off_req_shared), 0,
                (const int *)(img + plan.off_ids), plan.n_ids};
    // plans of an older layout carry 0: every width
    return launch_f16<true>(P, A, PV, plan.n_items, plan.col_blocks > 0 ? plan.col_blocks : 4, st);
}

} // namespace kvp
