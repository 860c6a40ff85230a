// kvp_decode_f16.hip -- fp16 grouped-query decode attention for gfx950: one fused kernel
// per layer (optional append of the new token, attention over the whole cache, merge of
// split partitions).
//
// What is computed (pages cited by title and section):
//   neuralialabs "Tornar a inferencia barata: KV cache, batching e quantizacao": decode
//   feeds one token whose query attends over every cached key (a 1 x n score row);
//   grouped-query attention shares each key-value head among a group of query heads;
//   PagedAttention reaches the cache through a per-sequence table of fixed-size blocks.
//   gustavoai "La cache de claves y valores", four-step token recipe: k_t, v_t are put at
//   the end of each head's cache (step 2) before the attention row over the whole cache
//   (step 3), so the new position sees itself.
//   chatgpz.de "Aufmerksamkeit", linear-attention post: TraditionalAttention,
//   softmax(q K^T / sqrt(d_k)) V.
//   same feed, FlashAttention post, "Was ist der mathematische Aspekt von Softmax?": block
//   softmaxes keep their maximum and exponential sum and are merged by rescaling with
//   e^(block max - global max) -- used across tiles and across split partitions.
//
// Work decomposition (stream-K): every (request, KV head) pair is cut into 64-token tiles
// (4 blocks of 16); the tiles of all pairs, in pair order, form one sequence that is cut
// into equal contiguous chunks, one per worker wave (4 per CU).  Load balance is within
// one tile whatever the mix of context lengths.  A pair lying inside one chunk is finished
// by that wave; a pair spread over several chunks leaves one partial (m, l, o) per chunk
// and the last wave to finish (device-scope ticket) merges them in chunk order, so the
// result is deterministic.  Partials travel through relaxed device-scope atomics (sc1
// stores / loads) ordered by a store-completion wait: no L2 write-back is needed.
//
// Per wave: K, V and q tiles stream HBM -> LDS through global_load_lds_dwordx4 into a ring
// of NBUF slots (16 KB per tile); waits are explicit vmcnt counts (17 loads per tile).
// Scores S^T = K Q^T run on the matrix cores (v_mfma_f32_16x16x32_f16, exact fp16 products,
// fp32 sums); softmax in fp32 with the hardware exp2; p*v on the vector ALUs in fp32 with
// v_fma_mix_f32 reading fp16 values straight from LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "kvp_decode_common.h"

namespace kvp {

using namespace dec;

constexpr int QB = MAXG * D * 2; // bytes of one q slot
constexpr int TB = TILE * D * 2; // bytes of one K (or V) tile
constexpr int PART_FLOATS = D + 2; // o[64], m, l
constexpr int DMA_PER_TILE = 18;   // 8 K + 8 V + 1 q + 1 new-token row

__device__ inline int wave_sum_i(int x)
{
    x += __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(x, x, 0x140, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false);
    return __builtin_amdgcn_readlane(x, 63);
}

// inclusive prefix sum over the 64 lanes (row_shr steps inside rows, then row broadcasts)
__device__ inline int wave_incl_scan_i(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false); // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false); // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false); // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false); // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31
    return x;
}

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima); issued through the builtin so
// that the compiler's own wait insertion knows about it
template <int N> __device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
    __builtin_amdgcn_s_waitcnt(imm);
}

// number of tiles of a request (context clamped to [1, max_ctx])
__device__ inline int tiles_of(int ctx, int maxc)
{
    ctx = ctx < 1 ? 1 : (ctx > maxc ? maxc : ctx);
    return (ctx + TILE - 1) / TILE;
}

// worker owning flattened tile x: chunks are [floor(w T / W), floor((w+1) T / W))
__device__ inline int owner_of(long long x, long long T, int W)
{
    return (int)(((x + 1) * W + T - 1) / T) - 1;
}
__device__ inline long long chunk_begin(int w, long long T, int W) { return (long long)w * T / W; }

template <int G, int NBUF, typename Addr>
__global__ __launch_bounds__(64) void decode_f16_kernel(DecodeParams P, Addr A)
{
    static_assert(G >= 1 && G <= MAXG, "group size");
    static_assert(NBUF == 2 || NBUF == 3, "ring depth");
    __shared__ __attribute__((aligned(16))) char kring[NBUF][TB];
    __shared__ __attribute__((aligned(16))) char vring[NBUF][TB];
    __shared__ __attribute__((aligned(16))) char qring[NBUF][QB];
    __shared__ __attribute__((aligned(16))) char nring[NBUF][1024]; // new-token K (lanes 0-7), V (8-15)
    __shared__ __attribute__((aligned(16))) float pbuf[TILE * MAXG];

    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    const int hkv = P.hkv;
    const int maxc = A.max_ctx();

    // ---- 1. total number of tiles ----
    long long T = 0;
    for (int b0 = 0; b0 < P.B; b0 += 64) {
        const int b = b0 + lane;
        const int nt = b < P.B ? tiles_of(P.ctx_lens[b], maxc) : 0;
        T += wave_sum_i(nt);
    }
    T *= hkv;
    // with fewer tiles than workers only the first T workers take part, so every chunk is
    // non-empty and the workers sharing a pair are exactly its tiles' owners
    const int W = (int)std::min<long long>(gridDim.x, T);
    if (w >= W)
        return;
    const long long c0 = chunk_begin(w, T, W), c1 = chunk_begin(w + 1, T, W);

    // ---- 2. request holding tile c0: the last b with hkv * prefix(b) <= c0 ----
    int rb = 0;
    long long rbase = 0; // tiles before request rb (all heads)
    {
        long long run = 0;
        for (int b0 = 0; b0 < P.B; b0 += 64) {
            const int b = b0 + lane;
            const int nt = b < P.B ? tiles_of(P.ctx_lens[b], maxc) : 0;
            const int incl = wave_incl_scan_i(nt);
            const long long excl = run + (incl - nt);
            const bool le = b < P.B && (long long)hkv * excl <= c0;
            const unsigned long long bal = __ballot(le);
            if (bal) {
                const int hi = 63 - __builtin_clzll(bal);
                rb = b0 + hi;
                const int ex_lo = __builtin_amdgcn_readlane((int)(excl & 0xffffffff), hi);
                const int ex_hi = __builtin_amdgcn_readlane((int)(excl >> 32), hi);
                rbase = (long long)hkv * (((long long)ex_hi << 32) | (unsigned)ex_lo);
            }
            run += __builtin_amdgcn_readlane(incl, 63);
        }
    }

    const f16 *kc = (const f16 *)P.kc;
    const f16 *vc = (const f16 *)P.vc;
    const int hl = lane & 15, grp = lane >> 4; // MFMA layout: head / token column, lane group
    const int tg = lane >> 3, cv = lane & 7;   // value layout: token group, 16-byte chunk

    // a cursor over the chunk: pair (b, g) with nt tiles starting at flattened index
    // pstart; current tile t of the pair; the chunk's part of this pair ends at tile te
    struct Cur {
        int b, g, nt, ctx, t, te;
        long long pstart;
    };
    auto cur_at = [&](int b, long long bbase, long long pos) -> Cur {
        Cur c;
        c.b = b;
        const int ctx = P.ctx_lens[b];
        c.ctx = ctx < 0 ? 0 : (ctx > maxc ? maxc : ctx);
        c.nt = tiles_of(ctx, maxc);
        const long long off = pos - bbase;
        c.g = (int)(off / c.nt);
        c.t = (int)(off - (long long)c.g * c.nt);
        c.pstart = bbase + (long long)c.g * c.nt;
        c.te = (int)std::min<long long>(c.nt, c.t + (c1 - pos));
        return c;
    };
    // first tile of the next pair after the part of c that lies in the chunk
    auto cur_next_pair = [&](const Cur &c) -> Cur {
        const long long pos = c.pstart + c.nt;
        if (c.g + 1 < hkv) {
            Cur n = c;
            n.g = c.g + 1;
            n.pstart = pos;
            n.t = 0;
            n.te = (int)std::min<long long>(n.nt, c1 - pos);
            return n;
        }
        return cur_at(c.b + 1, pos, pos);
    };
    const Cur first = cur_at(rb, rbase, c0);

    // ---- 3. table entries of the whole chunk, flat: entry f = 4 * (tile - c0) + block ----
    const int nflat = (int)std::min<long long>(4 * (c1 - c0), 256);
    int ent[4] = {-1, -1, -1, -1};
    if (A.paged) {
        Cur c = first;
        for (;;) {
            const long long xs = c.pstart + c.t, xe = c.pstart + c.te; // chunk tiles of c
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int f = lane + 64 * j;
                const long long x = c0 + f / 4;
                if (f < nflat && x >= xs && x < xe)
                    ent[j] = A.entry(c.b, (int)(4 * (x - c.pstart)) + (f & 3));
            }
            if (xe >= c1)
                break;
            c = cur_next_pair(c);
        }
        wait_vm<0>(); // entries in registers before the stream starts
    }
    auto ent_flat = [&](int f) -> int { // f uniform
        if (f >= nflat)
            return -1;
        const int j = f >> 6, l = f & 63;
        const int v = j == 0 ? ent[0] : (j == 1 ? ent[1] : (j == 2 ? ent[2] : ent[3]));
        return __builtin_amdgcn_readlane(v, l);
    };

    // ---- DMA of one tile (17 instructions, no lane masked off) ----
    auto issue_tile = [&](const Cur &c, long long x, int slot) {
        const int t = c.t;
        const int fb = (int)(4 * (x - c0));
        const int t0 = t * TILE; // first token of the tile in the pair
        // an unusable block is read from a known-good one (its rows are masked later)
        const int e0 = ent_flat(fb);
        char *kdst = kring[slot];
        char *vdst = vring[slot];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kb = i >> 1; // block of rows 8i .. 8i+7
            const int e = ent_flat(fb + kb);
            const int bi = 4 * t + kb;
            const bool ok = t0 + kb * BS < c.ctx && A.valid(e);
            const bool ok0 = A.valid(e0);
            const size_t base = ok ? A.block_off(c.b, c.g, bi, e)
                                   : (ok0 ? A.block_off(c.b, c.g, 4 * t, e0) : A.block_off(c.b, c.g, 0, 0));
            const int bir = ok ? bi : (ok0 ? 4 * t : 0);
            const int r = i * 8 + (lane >> 3);   // tile row of this lane
            const int rr = A.row(bir, r & 15);
            const int cg = (lane & 7) ^ (r & 7); // K chunk kept at this LDS slot
            __builtin_amdgcn_global_load_lds((const void *)(kc + base + (size_t)rr * D + cg * 8),
                                             (__attribute__((address_space(3))) void *)(kdst + i * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(vc + base + (size_t)rr * D + (lane & 7) * 8),
                                             (__attribute__((address_space(3))) void *)(vdst + i * 1024),
                                             16, 0, 0);
        }
        // q rows of the group: lane 8h + c carries head h, chunk c (rows past G repeat row 0)
        const int qh = (lane >> 3) < G ? (lane >> 3) : 0;
        const f16 *qs = (const f16 *)P.q + ((size_t)c.b * P.hq + (size_t)c.g * G + qh) * D + (lane & 7) * 8;
        __builtin_amdgcn_global_load_lds((const void *)qs, (__attribute__((address_space(3))) void *)qring[slot],
                                         16, 0, 0);
        // the step's new K / V row of this pair (read for every tile so that every tile
        // costs the same number of loads; used only on the pair's last tile)
        const void *ns = qs;
        if (P.k_new) {
            const size_t src = ((size_t)c.b * hkv + c.g) * D + (lane & 7) * 8;
            ns = ((lane >> 3) & 1) ? (const void *)((const f16 *)P.v_new + src)
                                   : (const void *)((const f16 *)P.k_new + src);
        }
        __builtin_amdgcn_global_load_lds(ns, (__attribute__((address_space(3))) void *)nring[slot], 16, 0, 0);
    };

    float m = -INFINITY, lsum = 0.f;
    float o[G][8];
    auto reset_acc = [&]() {
        m = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[h][e] = 0.f;
    };
    reset_acc();

    // ---- one tile: fix-ups, scores, softmax, p*v ----
    auto compute_tile = [&](const Cur &c, long long x, int slot) {
        const int t = c.t;
        const int fb = (int)(4 * (x - c0));
        const int t0 = t * TILE;
        char *kt = kring[slot];
        char *vt = vring[slot];
        // rows that must not contribute: past the context, or in an unusable block
        const int valid_rows = min(TILE, c.ctx - t0);
        bool bad_block = false;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            if (t0 + kb * BS < c.ctx && !A.valid(ent_flat(fb + kb)))
                bad_block = true;
        if (valid_rows < TILE || bad_block) {
            // zero the value rows that get p = 0 (the cache may hold NaN there)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int ch = lane + 64 * k, r = ch >> 3;
                if (r >= valid_rows || !A.valid(ent_flat(fb + (k >> 1))))
                    *(i32x4 *)(vt + ch * 16) = i32x4{0, 0, 0, 0};
            }
        }
        // the new token of this step: into LDS (this tile) and into the cache
        if (P.k_new && c.ctx >= 1 && t == c.nt - 1) {
            const int pos = c.ctx - 1, r = pos - t0;
            const int e = ent_flat(fb + (r >> 4));
            if (lane < 8 && A.valid(e)) {
                const i32x4 kn = *(const i32x4 *)(nring[slot] + lane * 16);
                const i32x4 vn = *(const i32x4 *)(nring[slot] + 128 + lane * 16);
                *(i32x4 *)(kt + r * 128 + ((lane ^ (r & 7)) * 16)) = kn;
                *(i32x4 *)(vt + r * 128 + lane * 16) = vn;
                const int bi = pos / BS;
                const size_t dst = A.block_off(c.b, c.g, bi, e) + (size_t)A.row(bi, pos % BS) * D + lane * 8;
                *(i32x4 *)((f16 *)P.kc_w + dst) = kn;
                *(i32x4 *)((f16 *)P.vc_w + dst) = vn;
            }
        }
        wave_lds_sync();
        // scores on the matrix cores: lane holds S[16kb + 4grp + i][head hl]
        const char *qt = qring[slot];
        f16x8 qop[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const f16x8 qv = *(const f16x8 *)(qt + (hl < G ? hl : 0) * 128 + (st * 4 + grp) * 16);
            qop[st] = hl < G ? qv : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        f32x4 sacc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int r = kb * 16 + hl;
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int ch = st * 4 + grp;
                const f16x8 kop = *(const f16x8 *)(kt + r * 128 + ((ch ^ (r & 7)) * 16));
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[st], sacc[kb], 0, 0, 0);
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bool okb = A.valid(ent_flat(fb + kb));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = kb * BS + grp * 4 + i;
                const float xs = (okb && r < valid_rows) ? sacc[kb][i] * P.scale_log2 : -INFINITY;
                sacc[kb][i] = xs;
                mt = fmaxf(mt, xs);
            }
        }
        mt = fmaxf(mt, lane_xor(mt, 16));
        mt = fmaxf(mt, lane_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
        m = mn;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = mn == -INFINITY ? 0.f : fast_exp2(sacc[kb][i] - mn);
                sacc[kb][i] = p;
                ps += p;
            }
        lsum = lsum * alpha + ps;
        if (hl < MAXG) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pbuf[(kb * BS + grp * 4 + i) * MAXG + hl] = sacc[kb][i];
        }
        float al[G];
        bool any = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            al[h] = uniform_lane(alpha, h);
            any |= al[h] != 1.f;
        }
        if (any) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[h][e] *= al[h];
        }
        wave_lds_sync();
        // p * v: rows 8i + tg, dims 8cv .. 8cv+7
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = i * 8 + tg;
            const f32x4 p0 = *(const f32x4 *)&pbuf[r * MAXG];
            const f32x4 p1 = *(const f32x4 *)&pbuf[r * MAXG + 4];
            const float pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            const f16x8 vh = *(const f16x8 *)(vt + r * 128 + cv * 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ve = (float)vh[e];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    o[h][e] = fmaf(pr[h], ve, o[h][e]);
            }
        }
        wave_lds_sync(); // pbuf and this slot are rewritten later
    };

    Cur pend = first; // a pair whose partial was stored and whose ticket is not yet taken
    bool has_pend = false;
    // ---- end of the chunk's part of a pair: a complete pair is written, otherwise a
    // partial is stored (its ticket is taken after the next wait, see settle) ----
    auto finish_pair = [&](const Cur &c, bool first_of_chunk) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float xv = o[h][e];
                xv += dpp<0x128>(xv); // row_ror:8: lane ^ 8 inside 16-lane rows
                xv += lane_xor(xv, 16);
                xv += lane_xor(xv, 32);
                o[h][e] = xv;
            }
        float lt = lsum;
        lt += lane_xor(lt, 16);
        lt += lane_xor(lt, 32);
        // head h: max and sum sit in lane h; lanes with tg == h write head h
        float mh = -INFINITY, lh = 0.f;
        float oh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            oh[e] = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mu = uniform_lane(m, h), lu = uniform_lane(lt, h);
            if (tg == h) {
                mh = mu;
                lh = lu;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    oh[e] = o[h][e];
            }
        }
        const int pair = c.b * hkv + c.g;
        f16 *outp = (f16 *)P.out + ((size_t)c.b * P.hq + (size_t)c.g * G) * D;
        const bool whole = c.pstart >= c0 && c.pstart + c.nt <= c1;
        if (whole) {
            if (tg < G) {
                const float inv = lh > 0.f ? 1.f / lh : 0.f;
                f16x8 r;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    r[e] = (f16)(oh[e] * inv);
                *(f16x8 *)(outp + tg * D + cv * 8) = r;
            }
            return;
        }
        const int slotp = first_of_chunk ? 0 : 1;
        float *mine = P.part + ((size_t)w * 2 + slotp) * MAXG * PART_FLOATS;
        if (tg < G) {
            float *dst = mine + tg * PART_FLOATS;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                coherent_store(dst + cv * 8 + e, oh[e]);
            if (cv == 0) {
                coherent_store(dst + D, mh);
                coherent_store(dst + D + 1, lh);
            }
        }
        pend = c;
        has_pend = true;
    };
    // Ticket of a pair whose partial is known to be complete (every store issued before the
    // last wait has finished: vector memory operations complete in order); the pair's last
    // worker merges the partials in chunk order, lane = dim.
    auto settle = [&](const Cur &c) {
        const int pair = c.b * hkv + c.g;
        f16 *outp = (f16 *)P.out + ((size_t)c.b * P.hq + (size_t)c.g * G) * D;
        const int wf = owner_of(c.pstart, T, W), wl = owner_of(c.pstart + c.nt - 1, T, W);
        int tk = 0;
        if (lane == 0)
            tk = take_ticket(&P.tickets[pair]);
        tk = __builtin_amdgcn_readfirstlane(tk);
        if (tk != wl - wf)
            return;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = -INFINITY;
            for (int ww = wf; ww <= wl; ++ww) {
                const int sl = chunk_begin(ww, T, W) >= c.pstart ? 0 : 1;
                M = fmaxf(M, coherent_load(P.part + (((size_t)ww * 2 + sl) * MAXG + h) * PART_FLOATS + D));
            }
            float L = 0.f, O = 0.f;
            for (int ww = wf; ww <= wl; ++ww) {
                const int sl = chunk_begin(ww, T, W) >= c.pstart ? 0 : 1;
                const float *src = P.part + (((size_t)ww * 2 + sl) * MAXG + h) * PART_FLOATS;
                const float f = M == -INFINITY ? 0.f : fast_exp2(coherent_load(src + D) - M);
                L = fmaf(coherent_load(src + D + 1), f, L);
                O = fmaf(coherent_load(src + lane), f, O);
            }
            outp[h * D + lane] = (f16)(L > 0.f ? O / L : 0.f);
        }
        if (lane == 0)
            reset_ticket(&P.tickets[pair]);
    };

    // ---- 4. stream the chunk: the issue cursor runs NBUF-1 tiles ahead ----
    const long long ntot = c1 - c0;
    Cur ic = first; // issue cursor (tile ic.t of its pair, flattened c0 + issued)
    long long issued = 0;
    auto issue_next = [&]() {
        issue_tile(ic, c0 + issued, (int)(issued % NBUF));
        ++issued;
        if (issued < ntot) {
            ++ic.t;
            if (ic.t >= ic.te)
                ic = cur_next_pair(ic);
        }
    };
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
        if (issued < ntot)
            issue_next();
    Cur cc = first; // compute cursor
    bool first_pair = true;
    for (long long done = 0; done < ntot; ++done) {
        if (issued < ntot)
            issue_next();
        const long long ahead = issued - done - 1; // tiles issued after this one
        if (ahead >= 2)
            wait_vm<2 * DMA_PER_TILE>();
        else if (ahead == 1)
            wait_vm<DMA_PER_TILE>();
        else
            wait_vm<0>();
        if (has_pend) { // its partial stores were issued before this tile's successor
            settle(pend);
            has_pend = false;
        }
        compute_tile(cc, c0 + done, (int)(done % NBUF));
        ++cc.t;
        if (cc.t >= cc.te) {
            finish_pair(cc, first_pair);
            first_pair = false;
            if (done + 1 < ntot) {
                cc = cur_next_pair(cc);
                reset_acc();
            }
        }
    }
    if (has_pend) {
        wait_vm<0>();
        settle(pend);
    }
}

// ---------------------------------------------------------------------------------------
template <typename Addr>
static kvp_status launch_f16(const DecodeParams &P, const Addr &A, int group, hipStream_t st)
{
    dim3 grid(P.workers), block(64);
    switch (group) {
#define KVP_G(GG)                                                                              \
    case GG:                                                                                   \
        hipLaunchKernelGGL((decode_f16_kernel<GG, 2, Addr>), grid, block, 0, st, P, A);       \
        break;
        KVP_G(1) KVP_G(2) KVP_G(3) KVP_G(4) KVP_G(5) KVP_G(6) KVP_G(7) KVP_G(8)
#undef KVP_G
    default:
        return fail(KVP_ERR_UNSUPPORTED, "decode: %d query heads per KV head (1..8 supported)", group);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return KVP_OK;
}

kvp_status launch_decode_f16(const DecodeParams &P, const PagedAddr &A, int group, hipStream_t st)
{
    return launch_f16(P, A, group, st);
}
kvp_status launch_decode_f16(const DecodeParams &P, const ContigAddr &A, int group, hipStream_t st)
{
    return launch_f16(P, A, group, st);
}

size_t decode_f16_part_bytes(int workers)
{
    return (size_t)workers * 2 * MAXG * PART_FLOATS * sizeof(float);
}

} // namespace kvp
