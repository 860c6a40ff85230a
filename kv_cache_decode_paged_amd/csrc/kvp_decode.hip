// kvp_decode.hip -- grouped-query decode attention over a paged or contiguous KV cache,
// split-K partitions and their merge, for gfx950 (MI355X, wave64).
//
// What is computed (pages cited by title and section):
//   neuralialabs "Tornar a inferencia barata: KV cache, batching e quantizacao": in decode
//   the query of the one new token attends over every cached key; a 1 x n score row
//   replaces the n x n matrix; grouped-query attention shares each key-value head among a
//   group of query heads; PagedAttention stores the cache in fixed-size blocks reached
//   through a per-sequence block table.
//   gustavoai "La cache de claves y valores": the new position attends to all earlier
//   positions and to itself (its k, v are appended before the attention row).
//   chatgpz.de "Aufmerksamkeit", linear-attention post: TraditionalAttention, scores
//   divided by sqrt(d_k), softmax, weighted sum of values.
//   same feed, FlashAttention post, "Was ist der mathematische Aspekt von Softmax?": each
//   block keeps its maximum and its sum of exponentials; blocks are merged by rescaling
//   with e^(block max - global max).  Used twice: across 64-token tiles (online softmax)
//   and across split-K partitions (the merge done by the last partition to finish).
//
// fp16 kernel (the hot path), designed for gfx950:
//   * one workgroup = one wave64 = one (request, KV head, split of <= 256..1024 tokens);
//     it serves all G query heads of the group, so each K/V byte is read once per group;
//   * the split is walked in 64-token tiles (4 blocks of 16 tokens) with the next tile's
//     K and V loads in flight (register double buffer) while the current one computes;
//   * scores S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_f16: 16 tokens x 16
//     padded heads per instruction, fp32 accumulation; q and k are fp16 so every product
//     is exact in fp32).  K rows go straight from HBM into the MFMA A operand;
//   * online softmax in fp32 with the hardware exp2 on log2e-prescaled scores; the
//     probabilities stay fp32 and pass through 2 KB of LDS to the value layout;
//   * p*v on the vector ALUs in fp32 (v_fma_mix_f32 reads the fp16 values directly),
//     values loaded coalesced (1 KB per instruction) into VGPRs;
//   * 1-D grid ordered so consecutive workgroups (which the dispatcher deals round-robin
//     to the 8 XCDs) rotate over (request, head) pairs and splits: work is even across
//     XCDs whatever the context-length mix;
//   * a request whose context needs several splits writes (m, l, o) partials; the last
//     split to finish (device-scope ticket) merges them in split order, so the result is
//     deterministic and no second kernel is launched.
// fp32 kernel (single-head fp32 workloads): the same split/merge scheme with a VALU score
// path (lane = token, 4 waves per workgroup).
// Paged and contiguous layouts differ only in the address of a 16-token block; arithmetic
// and its order are identical, so their outputs are bit-identical.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "kvp_internal.h"

namespace kvp {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 64;     // head dim
constexpr int BS = 16;    // tokens per block
constexpr int TILE = 64;  // tokens per tile
constexpr int MAXG = 8;   // query heads per group handled by one workgroup
constexpr int SPEC = 16;  // table entries fetched before the context length is known
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------
// split policy: a pure function of the context length (an optional override applies to
// every layout alike), so the paged and contiguous calls split identically.
// ---------------------------------------------------------------------------------------
__host__ __device__ inline int split_tokens(int ctx, int override_tokens)
{
    if (override_tokens > 0)
        return override_tokens;
    if (ctx <= 4096)
        return 256;
    if (ctx <= 16384)
        return 512;
    return 1024;
}

__host__ __device__ inline int num_splits(int ctx, int override_tokens)
{
    if (ctx <= 0)
        return 1;
    int s = split_tokens(ctx, override_tokens);
    return (ctx + s - 1) / s;
}

int max_splits_for(int max_context, int override_tokens)
{
    if (max_context <= 0)
        return 1;
    if (override_tokens > 0)
        return (max_context + override_tokens - 1) / override_tokens;
    // the worst case of each tier of split_tokens() sits at its upper end
    int best = num_splits(std::min(max_context, 4096), 0);
    if (max_context > 4096)
        best = std::max(best, num_splits(std::min(max_context, 16384), 0));
    if (max_context > 16384)
        best = std::max(best, num_splits(max_context, 0));
    return best;
}

int split_override_from_env()
{
    const char *e = getenv("KVP_SPLIT_TOKENS");
    if (!e || !*e)
        return 0;
    int v = atoi(e);
    if (v <= 0 || v % 256 != 0 || v > 1024)
        return 0; // ignored: must be a positive multiple of 256, at most 1024
    return v;
}

// ---------------------------------------------------------------------------------------
// address of a 16-token block
// ---------------------------------------------------------------------------------------
struct PagedAddr {
    const int *table; // [B][max_blocks]
    int max_blocks;
    int hkv;
    int num_blocks;
    static constexpr bool paged = true;
    __device__ int entry(int b, int idx) const
    {
        return idx < max_blocks ? table[(size_t)b * max_blocks + idx] : -1;
    }
    __device__ bool valid(int e) const { return e >= 0 && e < num_blocks; }
    // element offset of row 0 of the block (b, kv head g, logical block idx -> entry e)
    __device__ size_t block_off(int, int g, int, int e) const
    {
        return ((size_t)e * hkv + g) * (BS * D);
    }
    __device__ int max_ctx() const { return max_blocks * BS; }
    // row of logical block idx to read for in-block row r (blocks always hold 16 rows)
    __device__ int row(int, int r) const { return r; }
};

struct ContigAddr {
    int hkv;
    int lmax;
    static constexpr bool paged = false;
    __device__ int entry(int, int) const { return 0; }
    __device__ bool valid(int) const { return true; }
    __device__ size_t block_off(int b, int g, int idx, int) const
    {
        return (((size_t)b * hkv + g) * lmax + (size_t)idx * BS) * D;
    }
    __device__ int max_ctx() const { return lmax; }
    // the last 16-row group of a slice may run past Lmax: clamp (such rows are masked)
    __device__ int row(int idx, int r) const { return min(idx * BS + r, lmax - 1) - idx * BS; }
};

// ---------------------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND = false>
__device__ inline float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                         CTRL, ROW_MASK, BANK_MASK, BOUND));
}

// max / sum over all 64 lanes, result uniform (DPP butterflies inside 16-lane rows, row
// broadcasts across rows, then lane 63)
__device__ inline float wave_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    x = fmaxf(x, dpp<0x142, 0xa>(x));
    x = fmaxf(x, dpp<0x143, 0xc>(x));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ inline float wave_sum(float x)
{
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    x = x + dpp<0x141>(x);
    x = x + dpp<0x140>(x);
    x = x + dpp<0x142, 0xa>(x);
    x = x + dpp<0x143, 0xc>(x);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ inline float lane_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ inline float uniform_lane(float x, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ inline T from_f32(float x) { return (T)x; }

struct DecodeParams {
    const void *q;
    void *out;
    const void *kc; // layer base of the K pool / cache
    const void *vc;
    const int *ctx_lens;
    int B;
    int hq;
    int hkv;
    float scale_log2;
    int split_override;
    int max_splits;
    float *part_o;  // [B][Hq][max_splits][D]
    float *part_ml; // [B][Hq][max_splits][2]
    int *tickets;   // [B][Hkv], zero between calls
};

// (linear workgroup id) -> (pair = b*hkv + g, split s); consecutive ids rotate over pairs
// and, from one split to the next, shift by one pair so a request's splits land on
// different XCDs.
__device__ inline void decode_work_item(int L, int npairs, int &pair, int &s)
{
    s = L / npairs;
    int j = L - s * npairs;
    pair = j + (s % npairs);
    if (pair >= npairs)
        pair -= npairs;
}

// Final merge of the split partials of (b, g), in split order; lane = dim.
template <typename T, int G>
__device__ inline void merge_splits(const DecodeParams &P, int b, int g, int nsplit, int lane)
{
    T *outg = (T *)P.out + ((size_t)b * P.hq + (size_t)g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t base = ((size_t)b * P.hq + (size_t)g * G + h) * P.max_splits;
        float M = -INFINITY;
        for (int i = 0; i < nsplit; ++i)
            M = fmaxf(M, P.part_ml[(base + i) * 2]);
        float L = 0.f, O = 0.f;
        for (int i = 0; i < nsplit; ++i) {
            const float f = M == -INFINITY ? 0.f : fast_exp2(P.part_ml[(base + i) * 2] - M);
            L = fmaf(P.part_ml[(base + i) * 2 + 1], f, L);
            O = fmaf(P.part_o[(base + i) * D + lane], f, O);
        }
        outg[h * D + lane] = from_f32<T>(L > 0.f ? O / L : 0.f);
    }
}

// After a split has written its partial: take a ticket; the last split merges.
template <typename T, int G>
__device__ inline void finish_split(const DecodeParams &P, int b, int g, int nsplit, int lane)
{
    __threadfence(); // partial visible device-wide before the ticket
    int t = 0;
    if (lane == 0)
        t = atomicAdd(&P.tickets[b * P.hkv + g], 1);
    t = __shfl(t, 0, 64);
    if (t != nsplit - 1)
        return;
    __threadfence(); // see every other split's partial
    merge_splits<T, G>(P, b, g, nsplit, lane);
    if (lane == 0)
        atomicExch(&P.tickets[b * P.hkv + g], 0); // ready for the next call
}

// ---------------------------------------------------------------------------------------
// fp16 decode kernel.  grid = (max_splits * B * Hkv), block = 64.
// ---------------------------------------------------------------------------------------
struct KTile {
    f16x8 k[4][2]; // MFMA A operand: token 16*kb + lane%16, dims 32*st + 8*(lane/16) + e
};
struct VTile {
    i32x4 v[8]; // value rows 8*i + lane/8, dims 8*(lane%8) + e
};

template <int G, typename Addr>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_f16_kernel(DecodeParams P, Addr A)
{
    static_assert(G >= 1 && G <= MAXG, "group size");
    __shared__ __attribute__((aligned(16))) float pbuf[TILE * MAXG];

    const int lane = threadIdx.x;
    const int npairs = P.B * P.hkv;
    int pair, s;
    decode_work_item(blockIdx.x, npairs, pair, s);
    const int b = pair / P.hkv, g = pair - (pair / P.hkv) * P.hkv;

    // ---- prologue: context length, speculative table entries, query operand ----
    int ctx = P.ctx_lens[b];
    int spec = -1;
    if (A.paged && lane < SPEC)
        spec = A.entry(b, s * (256 / BS) + lane); // valid if this split is 256 tokens
    const int hl = lane & 15, grp = lane >> 4;
    f16x8 qop[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        if (hl < G)
            qop[st] = *(const f16x8 *)((const f16 *)P.q + ((size_t)b * P.hq + (size_t)g * G + hl) * D +
                                       st * 32 + grp * 8);
        else
            qop[st] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (ctx > A.max_ctx())
        ctx = A.max_ctx();
    const int S = split_tokens(ctx, P.split_override);
    const int nsplit = num_splits(ctx, P.split_override);
    if (s >= nsplit)
        return;
    f16 *outg = (f16 *)P.out + ((size_t)b * P.hq + (size_t)g * G) * D;
    if (ctx <= 0) { // invalid length: defined output (zeros), no cache read
        for (int i = lane; i < G * D; i += 64)
            outg[i] = (f16)0.f;
        return;
    }
    const int t_begin = s * S;
    const int t_end = min(ctx, t_begin + S);
    const int blk0 = t_begin / BS;
    int ent = spec;
    if (A.paged && S != 256) // other tier: fetch this split's entries (<= 64)
        ent = lane < S / BS ? A.entry(b, blk0 + lane) : -1;
    const int ntiles = (t_end - t_begin + TILE - 1) / TILE;

    const f16 *kc = (const f16 *)P.kc;
    const f16 *vc = (const f16 *)P.vc;
    const int tg = lane >> 3, cv = lane & 7; // value layout: token group, 16-byte chunk

    // block base and in-block rows of block kb of tile tt (unusable blocks read the
    // split's first block instead, always in bounds; their rows are masked out)
    auto block_base = [&](int tt, int kb, int &bi) -> size_t {
        const int t0 = t_begin + tt * TILE;
        const int e = __builtin_amdgcn_readlane(ent, tt * 4 + kb);
        const bool ok = (t0 + kb * BS < t_end) && A.valid(e);
        const int e0 = __builtin_amdgcn_readlane(ent, 0);
        bi = ok ? blk0 + tt * 4 + kb : blk0;
        return ok ? A.block_off(b, g, bi, e) : (A.valid(e0) ? A.block_off(b, g, bi, e0) : 0);
    };
    auto load_k = [&](KTile &T, int tt) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            int bi;
            const size_t base = block_base(tt, kb, bi);
            const int rk = A.row(bi, hl);
#pragma unroll
            for (int st = 0; st < 2; ++st)
                T.k[kb][st] = *(const f16x8 *)(kc + base + (size_t)rk * D + st * 32 + grp * 8);
        }
    };
    auto load_v = [&](VTile &T, int tt) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            int bi;
            const size_t base = block_base(tt, kb, bi);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int rv = A.row(bi, h2 * 8 + tg);
                T.v[kb * 2 + h2] = *(const i32x4 *)(vc + base + (size_t)rv * D + cv * 8);
            }
        }
    };

    float m = -INFINITY; // running max of head hl (valid in lanes with hl < G)
    float lsum = 0.f;    // running sum of head hl over this lane's tokens
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[h][e] = 0.f;

    auto scores_softmax = [&](KTile &T, int tt) {
        const int t0 = t_begin + tt * TILE;
        // ---- scores on the matrix cores: lane holds S[16kb + 4grp + i][head hl] ----
        f32x4 sacc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(T.k[kb][0], qop[0], sacc[kb], 0, 0, 0);
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(T.k[kb][1], qop[1], sacc[kb], 0, 0, 0);
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int e = __builtin_amdgcn_readlane(ent, tt * 4 + kb);
            const bool okb = A.valid(e);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + kb * BS + grp * 4 + i;
                const float x = (okb && t < t_end) ? sacc[kb][i] * P.scale_log2 : -INFINITY;
                sacc[kb][i] = x;
                mt = fmaxf(mt, x);
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
        // probabilities -> LDS, row = token, column = head
        if (hl < MAXG) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pbuf[(kb * BS + grp * 4 + i) * MAXG + hl] = sacc[kb][i];
        }
        // rescale of the value accumulators (alpha of head h sits in lane h)
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
    };
    auto pv = [&](VTile &T, int tt) {
        const int t0 = t_begin + tt * TILE;
        // ---- p * v on the vector ALUs: rows 8i + tg of the tile ----
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = i * 8 + tg;
            const int kb = i >> 1;
            const int e = __builtin_amdgcn_readlane(ent, tt * 4 + kb);
            const bool okr = A.valid(e) && (t0 + r < t_end);
            const f32x4 p0 = *(const f32x4 *)&pbuf[r * MAXG];
            const f32x4 p1 = *(const f32x4 *)&pbuf[r * MAXG + 4];
            const float pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            const f16x8 vh = __builtin_bit_cast(f16x8, T.v[i]);
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                // rows past the end are zeroed: their p is 0 but the cache may hold NaN
                const float ve = okr ? (float)vh[e2] : 0.f;
#pragma unroll
                for (int h = 0; h < G; ++h)
                    o[h][e2] = fmaf(pr[h], ve, o[h][e2]);
            }
        }
        wave_lds_sync(); // the next tile overwrites pbuf
    };

    // ---- software pipeline: the next tile's K is in flight during this tile's scores,
    // its V during this tile's p*v ----
    KTile ka, kb2;
    VTile va, vb;
    load_k(ka, 0);
    load_v(va, 0);
    for (int tt = 0; tt < ntiles; tt += 2) {
        const bool n1 = tt + 1 < ntiles, n2 = tt + 2 < ntiles;
        if (n1)
            load_k(kb2, tt + 1);
        scores_softmax(ka, tt);
        if (n1)
            load_v(vb, tt + 1);
        pv(va, tt);
        if (!n1)
            break;
        if (n2)
            load_k(ka, tt + 2);
        scores_softmax(kb2, tt + 1);
        if (n2)
            load_v(va, tt + 2);
        pv(vb, tt + 1);
    }

    // ---- end of split: sum the 8 token groups (lanes cv, cv+8, ..., cv+56) ----
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = o[h][e];
            x += dpp<0x128>(x);  // row_ror:8 -> lane ^ 8 inside 16-lane rows
            x += lane_xor(x, 16);
            x += lane_xor(x, 32);
            o[h][e] = x;
        }
    lsum += lane_xor(lsum, 16);
    lsum += lane_xor(lsum, 32);
    // head h statistics live in lane h
    float mh[G], lh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        mh[h] = uniform_lane(m, h);
        lh[h] = uniform_lane(lsum, h);
    }
    if (nsplit == 1) {
        if (lane < 8) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = lh[h] > 0.f ? 1.f / lh[h] : 0.f;
                f16x8 r;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    r[e] = (f16)(o[h][e] * inv);
                *(f16x8 *)(outg + h * D + lane * 8) = r;
            }
        }
        return;
    }
    if (lane < 8) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const size_t pi = ((size_t)b * P.hq + (size_t)g * G + h) * P.max_splits + s;
            float *dst = P.part_o + pi * D + lane * 8;
            *(f32x4 *)dst = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
            *(f32x4 *)(dst + 4) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
            if (lane == 0) {
                P.part_ml[pi * 2 + 0] = mh[h];
                P.part_ml[pi * 2 + 1] = lh[h];
            }
        }
    }
    finish_split<f16, G>(P, b, g, nsplit, lane);
}

// ---------------------------------------------------------------------------------------
// fp32 decode kernel (VALU).  grid = (max_splits * B * Hkv), block = 256 (4 waves, each
// owning 64 tokens of every 256-token step of the split).
// ---------------------------------------------------------------------------------------
constexpr int NW = 4;

template <int G, typename Addr>
__global__ __launch_bounds__(NW * 64) void decode_f32_kernel(DecodeParams P, Addr A)
{
    constexpr int CH = 4, NCH = 16, RPI = 4, NLD = 16; // 16-byte chunks of fp32 rows
    constexpr int ROWB = D * 4;
    __shared__ __attribute__((aligned(16))) char kbuf[NW * TILE * ROWB]; // 64 KB
    __shared__ __attribute__((aligned(16))) float pbuf[NW * TILE * MAXG];
    __shared__ __attribute__((aligned(16))) float qbuf[MAXG * D];
    __shared__ float mlbuf[NW * MAXG * 2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int pair, s;
    decode_work_item(blockIdx.x, P.B * P.hkv, pair, s);
    const int b = pair / P.hkv, g = pair - (pair / P.hkv) * P.hkv;
    const float *qg = (const float *)P.q + ((size_t)b * P.hq + (size_t)g * G) * D;
    float *outg = (float *)P.out + ((size_t)b * P.hq + (size_t)g * G) * D;

    int ctx = P.ctx_lens[b];
    if (ctx > A.max_ctx())
        ctx = A.max_ctx();
    const int S = split_tokens(ctx, P.split_override);
    const int nsplit = num_splits(ctx, P.split_override);
    if (s >= nsplit)
        return;
    if (ctx <= 0) {
        for (int i = threadIdx.x; i < G * D; i += NW * 64)
            outg[i] = 0.f;
        return;
    }
    const int t_begin = s * S;
    const int t_end = min(ctx, t_begin + S);
    for (int i = threadIdx.x; i < G * D; i += NW * 64)
        qbuf[i] = qg[i];
    const int blk0 = t_begin / BS;
    const int nblk = (t_end - t_begin + BS - 1) / BS;
    int my_entry = 0;
    if (lane < nblk)
        my_entry = A.entry(b, blk0 + lane);
    __syncthreads();

    const float *kc = (const float *)P.kc;
    const float *vc = (const float *)P.vc;
    char *kl = kbuf + wave * (TILE * ROWB);
    float *pl = pbuf + wave * (TILE * MAXG);
    float m[G], lsum[G], o[G][CH];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < CH; ++e)
            o[h][e] = 0.f;
    }
    const int tg = lane / NCH, cv = lane % NCH;
    const int nit = (t_end - t_begin + NW * TILE - 1) / (NW * TILE);
    for (int it = 0; it < nit; ++it) {
        const int r0 = it * NW * TILE + wave * TILE;
        const int t0 = t_begin + r0;
        if (t0 >= t_end)
            continue;
        int ent[TILE / BS];
        bool ok[TILE / BS];
#pragma unroll
        for (int k = 0; k < TILE / BS; ++k) {
            const int li = r0 / BS + k;
            ent[k] = __builtin_amdgcn_readlane(my_entry, li < 64 ? li : 63);
            ok[k] = (t0 + k * BS < t_end) && A.valid(ent[k]);
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int k = (i * RPI) / BS;
            const int r = i * RPI + lane / NCH;
            const int cg = (lane % NCH) ^ (r % NCH);
            const int t = t0 + r;
            if (ok[k] && t < t_end) {
                const float *src = kc + A.block_off(b, g, blk0 + r0 / BS + k, ent[k]) +
                                   (size_t)(r % BS) * D + cg * CH;
                __builtin_amdgcn_global_load_lds((const void *)src,
                                                 (__attribute__((address_space(3))) void *)(kl + i * 1024),
                                                 16, 0, 0);
            }
        }
        f32x4 vreg[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int k = (i * RPI) / BS;
            const int r = i * RPI + tg;
            const int t = t0 + r;
            if (ok[k] && t < t_end)
                vreg[i] = *(const f32x4 *)(vc + A.block_off(b, g, blk0 + r0 / BS + k, ent[k]) +
                                           (size_t)(r % BS) * D + cv * CH);
            else
                vreg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        wave_lds_sync();
        const int j = lane;
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            sc[h] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const f32x4 kv = *(const f32x4 *)(kl + j * ROWB + ((c ^ (j % NCH)) * 16));
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const f32x4 qv = *(const f32x4 *)&qbuf[h * D + c * CH];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sc[h] = fmaf(kv[e], qv[e], sc[h]);
            }
        }
        const int tj = t0 + j;
        bool valid_j = tj < t_end;
#pragma unroll
        for (int k = 0; k < TILE / BS; ++k)
            if (k == j / BS)
                valid_j = valid_j && ok[k];
        float alpha[G];
        bool rescale = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float x = valid_j ? sc[h] * P.scale_log2 : -INFINITY;
            const float mt = wave_max(x);
            const float mn = fmaxf(m[h], mt);
            alpha[h] = mn == -INFINITY ? 1.f : fast_exp2(m[h] - mn);
            rescale |= (mn != m[h]);
            m[h] = mn;
            const float pj = mn == -INFINITY ? 0.f : fast_exp2(x - mn);
            lsum[h] = lsum[h] * alpha[h] + pj;
            pl[j * MAXG + h] = pj;
        }
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < CH; ++e)
                    o[h][e] *= alpha[h];
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int r = i * RPI + tg;
#pragma unroll
            for (int e = 0; e < CH; ++e)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    o[h][e] = fmaf(pl[r * MAXG + h], vreg[i][e], o[h][e]);
        }
        wave_lds_sync();
    }

    // merge the 4 token groups of each wave (one per 16-lane row) and the 4 waves
    __syncthreads();
    float *mbuf = (float *)kbuf; // [NW][4 rows][MAXG][D]
    const int row = lane >> 4;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float *dst = mbuf + (((wave * 4 + row) * MAXG + h) * D) + cv * CH;
#pragma unroll
        for (int e = 0; e < CH; ++e)
            dst[e] = o[h][e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float lw = wave_sum(lsum[h]);
        if (lane == 0) {
            mlbuf[(wave * MAXG + h) * 2 + 0] = m[h];
            mlbuf[(wave * MAXG + h) * 2 + 1] = lw;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int h = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, mlbuf[(w * MAXG + h) * 2]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = M == -INFINITY ? 0.f : fast_exp2(mlbuf[(w * MAXG + h) * 2] - M);
            L = fmaf(mlbuf[(w * MAXG + h) * 2 + 1], f, L);
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc += mbuf[((w * 4 + r) * MAXG + h) * D + c];
            O = fmaf(acc, f, O);
        }
        if (nsplit == 1) {
            outg[h * D + c] = L > 0.f ? O / L : 0.f;
        } else {
            const size_t pi = ((size_t)b * P.hq + (size_t)g * G + h) * P.max_splits + s;
            P.part_o[pi * D + c] = O;
            if (c == 0) {
                P.part_ml[pi * 2 + 0] = M;
                P.part_ml[pi * 2 + 1] = L;
            }
        }
    }
    if (nsplit == 1)
        return;
    // every thread's partial stores are done before one ticket is taken for the workgroup
    __threadfence();
    __syncthreads();
    __shared__ int is_last;
    if (threadIdx.x == 0)
        is_last = atomicAdd(&P.tickets[b * P.hkv + g], 1) == nsplit - 1;
    __syncthreads();
    if (!is_last || wave != 0)
        return;
    __threadfence();
    merge_splits<float, G>(P, b, g, nsplit, lane);
    if (lane == 0)
        atomicExch(&P.tickets[b * P.hkv + g], 0);
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static kvp_status check_dims(const kvp_dims *d, const char *who)
{
    if (!d)
        return fail(KVP_ERR_INVALID, "%s: dims is NULL", who);
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0)
        return fail(KVP_ERR_INVALID, "%s: num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                    who, d->num_q_heads, d->num_kv_heads);
    if (d->head_dim != D)
        return fail(KVP_ERR_UNSUPPORTED, "%s: head_dim=%d (only 64 is implemented)", who, d->head_dim);
    if (d->dtype != KVP_F16 && d->dtype != KVP_F32)
        return fail(KVP_ERR_INVALID, "%s: dtype=%d", who, d->dtype);
    return KVP_OK;
}

static size_t ws_partial_floats(int B, int hq, int ms) { return (size_t)B * hq * ms * (D + 2); }

size_t workspace_bytes(const kvp_dims *d, int B, int max_context)
{
    int ms = max_splits_for(max_context, split_override_from_env());
    if (ms <= 1)
        return 0;
    size_t fl = ws_partial_floats(B, d->num_q_heads, ms);
    size_t tickets = ((size_t)B * d->num_kv_heads * sizeof(int) + 255) / 256 * 256;
    return fl * sizeof(float) + tickets;
}

} // namespace kvp

namespace kvp {

template <typename Addr>
static kvp_status launch_decode(const DecodeParams &P, const Addr &A, int dtype, int group,
                                hipStream_t st)
{
    const long long nwg = (long long)P.max_splits * P.B * P.hkv;
    if (nwg > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "decode: grid of %lld workgroups too large", nwg);
    dim3 grid((unsigned)nwg);
    if (dtype == KVP_F16) {
        switch (group) {
#define KVP_G(GG)                                                                              \
    case GG:                                                                                   \
        hipLaunchKernelGGL((decode_f16_kernel<GG, Addr>), grid, dim3(64), 0, st, P, A);       \
        break;
            KVP_G(1) KVP_G(2) KVP_G(3) KVP_G(4) KVP_G(5) KVP_G(6) KVP_G(7) KVP_G(8)
#undef KVP_G
        default:
            return fail(KVP_ERR_UNSUPPORTED, "decode: %d query heads per KV head (1..8 supported)", group);
        }
    } else {
        switch (group) {
#define KVP_G(GG)                                                                              \
    case GG:                                                                                   \
        hipLaunchKernelGGL((decode_f32_kernel<GG, Addr>), grid, dim3(NW * 64), 0, st, P, A);  \
        break;
            KVP_G(1) KVP_G(2) KVP_G(3) KVP_G(4) KVP_G(5) KVP_G(6) KVP_G(7) KVP_G(8)
#undef KVP_G
        default:
            return fail(KVP_ERR_UNSUPPORTED, "decode: %d query heads per KV head (1..8 supported)", group);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return KVP_OK;
}

template <typename Addr>
static kvp_status decode_common(const kvp_dims *dims, void *out, const void *q, const void *kc,
                                const void *vc, const Addr &A, int max_ctx,
                                const int32_t *d_ctx, int32_t B, float scale, void *ws,
                                size_t ws_bytes, kvp_stream stream, const char *who)
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
    if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)kc | (uintptr_t)vc) & 15)
        return fail(KVP_ERR_INVALID, "%s: q/out/cache pointers must be 16-byte aligned", who);
    DecodeParams P;
    P.q = q;
    P.out = out;
    P.kc = kc;
    P.vc = vc;
    P.ctx_lens = d_ctx;
    P.B = B;
    P.hq = dims->num_q_heads;
    P.hkv = dims->num_kv_heads;
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)D);
    P.scale_log2 = scale * LOG2E;
    P.split_override = split_override_from_env();
    P.max_splits = max_splits_for(max_ctx, P.split_override);
    P.part_o = nullptr;
    P.part_ml = nullptr;
    P.tickets = nullptr;
    if (P.max_splits > 1) {
        const size_t fl = ws_partial_floats(B, P.hq, P.max_splits);
        const size_t need = workspace_bytes(dims, B, max_ctx);
        if (!ws || ws_bytes < need)
            return fail(KVP_ERR_INVALID, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
        if ((uintptr_t)ws & 15)
            return fail(KVP_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
        P.part_o = (float *)ws;
        P.part_ml = (float *)ws + (size_t)B * P.hq * P.max_splits * D;
        P.tickets = (int *)((float *)ws + fl);
    }
    return launch_decode(P, A, dims->dtype, dims->num_q_heads / dims->num_kv_heads,
                         (hipStream_t)stream);
}

} // namespace kvp

using namespace kvp;

extern "C" {

size_t decode_workspace_bytes(const kvp_dims *dims, int32_t B, int32_t max_context)
{
    if (check_dims(dims, "decode_workspace_bytes") != KVP_OK || B < 0 || max_context < 0)
        return 0;
    return workspace_bytes(dims, B, max_context);
}

int32_t decode_num_splits(int32_t context_len)
{
    return num_splits(context_len, split_override_from_env());
}

kvp_status paged_decode_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                  const void *q, const int32_t *d_block_table,
                                  int32_t max_blocks, const int32_t *d_context_lens, int32_t B,
                                  float scale, void *workspace, size_t ws_bytes,
                                  kvp_stream stream)
{
    if (!cache)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: cache is NULL");
    kvp_status st0 = check_dims(&cache->dims, "paged_decode_attention");
    if (st0 != KVP_OK)
        return st0;
    if (cache->block_size != BS)
        return fail(KVP_ERR_UNSUPPORTED, "paged_decode_attention: block_size=%d (only 16)", cache->block_size);
    if (layer < 0 || layer >= cache->dims.num_layers)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: layer %d out of range", layer);
    if (max_blocks <= 0 || cache->num_blocks <= 0 || !d_block_table)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: max_blocks=%d num_blocks=%d table=%p",
                    max_blocks, cache->num_blocks, (const void *)d_block_table);
    if (!cache->k_pool || !cache->v_pool)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: pool pointer is NULL");
    if ((long long)max_blocks * BS > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "paged_decode_attention: max_blocks too large");
    const size_t esz = cache->dims.dtype == KVP_F16 ? 2 : 4;
    const size_t layer_elems = (size_t)cache->num_blocks * cache->dims.num_kv_heads * BS * D;
    const char *kc = (const char *)cache->k_pool + (size_t)layer * layer_elems * esz;
    const char *vc = (const char *)cache->v_pool + (size_t)layer * layer_elems * esz;
    PagedAddr A{d_block_table, max_blocks, cache->dims.num_kv_heads, cache->num_blocks};
    return decode_common(&cache->dims, out, q, kc, vc, A, max_blocks * BS, d_context_lens, B, scale,
                         workspace, ws_bytes, stream, "paged_decode_attention");
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
    ContigAddr A{dims->num_kv_heads, Lmax};
    return decode_common(dims, out, q, k_cache, v_cache, A, Lmax, d_context_lens, B, scale,
                         workspace, ws_bytes, stream, "contiguous_decode_attention");
}

} // extern "C"
