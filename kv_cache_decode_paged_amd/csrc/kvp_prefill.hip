// kvp_prefill.hip -- packed variable-length prefill attention (causal or block-diagonal)
// for gfx950.
//
//   chatgpz.de "Aufmerksamkeit", xformers demo section 4: sequences of different lengths
//   are packed on one token axis without padding; the block-diagonal mask keeps attention
//   inside each sequence and its causal variant also hides later tokens.  Section 5: the
//   grouped-query head map (B, M, G, Hq/G, K).
//   same feed, FlashAttention post: keys/values are processed block by block on chip and
//   the n x n score matrix is never written; block softmaxes are merged by rescaling with
//   e^(old max - new max).
//   neuralialabs chapter: prefill is one pass over the whole prompt, a matrix-matrix
//   product, so this is where the matrix cores pay off.
//
// fp16: one workgroup = 4 wave64 = 64 NQB query rows of one (segment, query head).  Wave w
// owns NQB blocks of 16 rows, rows q0 + 64 nb + 16 w, so the four waves reach the causal
// diagonal together and share every K/V tile.  K and V stream HBM -> LDS through
// global_load_lds in ring tiles of two compute tiles of KT keys, 2 slots, the next ring tile
// in flight while one is computed (paged keys whose block table is too wide for its staged
// ids to fit beside that ring: ring tiles of one compute tile in 3 slots); one barrier per
// ring tile.  Each wave reads a compute tile's K rows and its transposed V once and uses
// them for all of its blocks.  Head dim
// 64: NQB = 4, KT = 64; head dim 128: NQB = 2, KT = 32 (the operands of twice the width in
// the same register budget, and the same 8 KB K or V tile):
//   scores  S^T = K Q^T       v_mfma_f32_16x16x32_f16, one query row per MFMA column
//   softmax fp32, exp2 of one FMA (scale folded in), reference max moved only when a row's
//           maximum passes it by 2^8, masks only on the diagonal and ragged tiles
//   values  O^T = V^T P^T     P^T is the score MFMA's own output layout; V^T comes from
//                             transposing LDS reads; row sums from an all-ones operand
// Tiles entirely above a block's causal diagonal are skipped; the longest (last) query
// tiles are launched first.
// fp32: a plain VALU kernel (wave = one query row), exact fp32 throughout.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "kvp_gfx950.h"
#include "kvp_internal.h"

namespace kvp {

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

namespace pf {
constexpr int D = 64;        // head dim of the fp32 kernel
constexpr int BS = 16;       // tokens per cache block
constexpr float LOG2E = 1.4426950408889634f;

// tiling of the fp16 kernel by head dim HD
template <int HD> struct Tiles {
    static_assert(HD == 64 || HD == 128, "head dim 64 or 128");
    static constexpr int NQB = HD == 64 ? 4 : 2; // 16-row query blocks per wave
    static constexpr int QB = 64 * NQB;         // query rows per workgroup
    static constexpr int KT = HD == 64 ? 64 : 32; // keys per tile
    static constexpr int RB = 2 * HD;           // bytes of one K (or V) row
    static constexpr int SLOT = KT * RB;        // bytes of one K (or V) tile
    static constexpr int LPW = SLOT / 1024 / 4; // 1 KB loads per wave per tile, each of K and V
    static constexpr int NDMA = 2 * LPW;
};
// query rows per workgroup of the fp16 kernel
inline int query_rows_per_workgroup(int hd) { return hd == 64 ? Tiles<64>::QB : Tiles<128>::QB; }
} // namespace pf

__device__ inline float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Query rows and keys of one workgroup's sequence.  Packed (varlen prefill): segment s is
// rows cu[s] .. cu[s+1]-1 of q and of k / v, every row a query and a key.  Paged (several
// new rows against the cache): request s has rows cu[s] .. cu[s+1]-1 of q, the last of
// its ctx[s] cached positions, whose keys are reached through the block table.
struct PrefillArgs {
    const f16 *q;
    const f16 *k;      // packed k [T][Hkv][d], or the layer's K pool [blocks][Hkv][16][d]
    const f16 *v;
    f16 *out;
    const int *cu;     // [nseg + 1] query-row offsets (packed: also key rows)
    const int *ctx;    // paged: context length per request
    const int *table;  // paged: block table [nseg][max_blocks]
    int max_blocks;
    int num_blocks;
    int hq;
    int hkv;
    float scale_log2;
    int causal;
};

// block ids of one request staged in LDS (paged): contexts of up to MAX_IDS blocks
constexpr int MAX_IDS = 4096;
// LDS of one workgroup when two share a CU (160 KB): the paged kernel takes the wide ring
// (64 KB) when the staged ids of the table's width fit beside it
constexpr int LDS_TWO_PER_CU = 80 * 1024;
constexpr int WIDE_RING_LDS = 64 * 1024 + 16; // both rings + the bad-id flag

// grid = (Hq, nseg, ceil(max query rows / QB)), block = 256; paged: dynamic LDS of
// max_blocks ints for the staged block ids
template <bool PAGED, int D, int SUB>
__global__ __launch_bounds__(256) void prefill_mfma_f16_kernel(PrefillArgs P)
{
    using namespace pf;
    using T_ = Tiles<D>;
    constexpr int NQB = T_::NQB, QB = T_::QB, KT = T_::KT, RB = T_::RB, SLOT = T_::SLOT;
    // ring: ring tiles of SUB compute tiles; two compute tiles through 2 slots (64 KB of K
    // and V), or, where a paged table's staged block ids leave no room for that beside a
    // second workgroup, single compute tiles through 3 slots (48 KB)
    constexpr int NB = SUB == 2 ? 2 : 3; // ring slots
    constexpr int RT = SUB * KT, RSLOT = SUB * SLOT; // keys and bytes (K or V) of a ring tile
    constexpr int LPW = SUB * T_::LPW, NDMA = 2 * LPW; // 1 KB loads per wave per ring tile (K or V); both
    constexpr int CPR = D / 8;    // 16-byte chunks per row
    constexpr int RPI = 1024 / RB; // rows per 1 KB load
    constexpr int KB = KT / 16;   // 16-key blocks per tile
    constexpr int KS = KT / 32;   // 32-key steps per tile (value product)
    constexpr int KD = D / 32;    // 32-dim steps (score product)
    constexpr int NDB = D / 16;   // 16-dim blocks of the output
    // one barrier per ring tile: the DMA of ring tile t + NB - 1 refills the slot of ring tile
    // t - 1, which every wave has finished at the barrier; either ring takes 64 KB of K and V
    // (two workgroups per CU), the paged one 16 KB of block ids besides
    static_assert((SUB == 1 || SUB == 2) && (PAGED || SUB == 2), "ring shape");
    __shared__ __attribute__((aligned(16))) char kring[NB * RSLOT];
    __shared__ __attribute__((aligned(16))) char vring[NB * RSLOT];
    extern __shared__ int ids[]; // paged: [max_blocks] staged block ids (dynamic LDS)
    __shared__ int ids_bad;

    // the query tile is the slowest grid dimension: workgroups are dispatched x fastest, so
    // with causal masking every head's and segment's last (longest) tiles go first
    const int qtile = P.causal ? (int)gridDim.z - 1 - (int)blockIdx.z : (int)blockIdx.z;
    const int h = blockIdx.x, seg = blockIdx.y;
    const int hq = P.hq, hkv = P.hkv, causal = P.causal;
    const int a = P.cu[seg];             // first query row
    const int n = P.cu[seg + 1] - a;     // query rows
    int nk = n;                          // keys
    if constexpr (PAGED) {
        const int c = P.ctx[seg];
        nk = c < 0 ? 0 : (c > P.max_blocks * BS ? P.max_blocks * BS : c);
    }
    const int off = nk - n; // row i attends to keys 0 .. off + i (the rows end the context)
    const int q0 = qtile * QB;
    if (q0 >= n || n <= 0)
        return;
    const int g_kv = h / (hq / hkv);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15; // query row within a 16-row block (MFMA column)
    const int grp = lane >> 4; // lane group 0..3
    const float c = P.scale_log2;
    const float inv_c = 1.f / c;

    // ---- this wave's query blocks: Q^T operands and each row's key limit ----
    f16x8 qop[NQB][KD];
    int r0[NQB], lim[NQB];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        r0[nb] = q0 + 64 * nb + 16 * wave;
        const int row = r0[nb] + col;
        const f16 *qp = P.q + ((size_t)(a + min(row, n - 1)) * hq + h) * D + grp * 8;
        const f16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
            const f16x8 qv = *(const f16x8 *)(qp + 32 * ks);
            qop[nb][ks] = row < n ? qv : z;
        }
        lim[nb] = causal ? max(0, min(off + row + 1, nk)) : nk; // keys >= lim are masked for this row
    }
    const int kend = causal ? max(0, min(nk, off + q0 + QB)) : nk; // keys any row of the workgroup sees
    // first key no row of block nb sees from (-1: the block holds no row; with causal masking
    // its last row sees up to off + r0 + 15), and the largest over the wave's blocks: a
    // compute tile starting at key k0 has work for block nb when k0 < kvis[nb]
    int kvis[NQB], kvis_any = -1;
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        kvis[nb] = __builtin_amdgcn_readfirstlane(r0[nb] < n ? (causal ? off + r0[nb] + 16 : INT_MAX) : -1);
        kvis_any = max(kvis_any, kvis[nb]);
    }
    const int nt = (kend + RT - 1) / RT;
    // paged: the request's block ids for keys < kend, an unusable entry (-1) masks its keys
    bool all_ok = true;
    if constexpr (PAGED) {
        if (threadIdx.x == 0)
            ids_bad = 0;
        __syncthreads();
        const int nids = (kend + BS - 1) / BS;
        int bad = 0;
        for (int j = threadIdx.x; j < nids; j += 256) {
            const int e = P.table[(size_t)seg * P.max_blocks + j];
            const bool ok = e >= 0 && e < P.num_blocks;
            ids[j] = ok ? e : -1;
            bad |= !ok;
        }
        if (bad)
            ids_bad = 1;
        __syncthreads();
        all_ok = ids_bad == 0;
    }

    // ---- DMA of tile t into ring slot t % NB: wave w loads the tile's 1 KB pieces
    // LPW w .. LPW w + LPW - 1 of K and of V (RPI rows each; LDS row r, chunk slot
    // swz(c, r) holds chunk c); rows past the workgroup's last visible key re-read that
    // key's row (they are masked; its block id is staged), an unusable block reads block 0
    // (masked too) ----
    // lane part of an interior tile's packed K/V offsets: row r of the tile is key t KT + r,
    // at element (a + t KT) hkv D + (r hkv + g) D + 8 chunk, whose first term is the same for
    // every lane of the workgroup
    int lane_off[LPW];
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
        const int r = RPI * (LPW * wave + ii) + lane / CPR;
        lane_off[ii] = (r * hkv + g_kv) * D + swz<D>(lane & (CPR - 1), r) * 8;
    }
    auto issue = [&](int t) {
        char *kd = kring + (t % NB) * RSLOT;
        char *vd = vring + (t % NB) * RSLOT;
        if (!PAGED && (t + 1) * RT <= kend) {
            // every row of the tile is a key the workgroup sees: no clamp, no block ids
            const size_t tb = (size_t)(a + t * RT) * hkv * D;
            const f16 *kt = P.k + tb, *vt = P.v + tb;
#pragma unroll
            for (int ii = 0; ii < LPW; ++ii) {
                const int i = LPW * wave + ii;
                __builtin_amdgcn_global_load_lds((const void *)(kt + lane_off[ii]),
                                                 (__attribute__((address_space(3))) void *)(kd + i * 1024), 16, 0,
                                                 0);
                __builtin_amdgcn_global_load_lds((const void *)(vt + lane_off[ii]),
                                                 (__attribute__((address_space(3))) void *)(vd + i * 1024), 16, 0,
                                                 0);
            }
            return;
        }
        int kk[LPW], e[LPW];
        unsigned ea[LPW];
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) {
            const int r = RPI * (LPW * wave + ii) + lane / CPR;
            kk[ii] = min(t * RT + r, kend - 1); // beyond kend every row of the workgroup masks the key
            e[ii] = 0;
            ea[ii] = 0;
            if constexpr (PAGED)
                ea[ii] = lds_addr((const char *)&ids[kk[ii] >> 4]);
        }
        if constexpr (PAGED)
            lds_read_b32<LPW>(e, ea);
#pragma unroll
        for (int ii = 0; ii < LPW; ++ii) {
            const int i = LPW * wave + ii;
            const int r = RPI * i + lane / CPR;
            size_t off_e;
            if constexpr (PAGED)
                off_e = (((size_t)max(e[ii], 0) * hkv + g_kv) * BS + (kk[ii] & (BS - 1))) * D;
            else
                off_e = ((size_t)(a + kk[ii]) * hkv + g_kv) * D;
            const size_t o = off_e + swz<D>(lane & (CPR - 1), r) * 8;
            __builtin_amdgcn_global_load_lds((const void *)(P.k + o),
                                             (__attribute__((address_space(3))) void *)(kd + i * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(P.v + o),
                                             (__attribute__((address_space(3))) void *)(vd + i * 1024), 16, 0, 0);
        }
    };

    // running state per block: reference max (scaled, log2 units), O^T rows 16 db + 4 grp + i
    // of column col, and the row sum (every entry of accl holds it)
    float mref[NQB];
    // nmc[nb]: the exponent offset -mref (0 while the row has no reference yet, so that
    // masked scores give exp2(-inf) = 0 rather than NaN), kept beside mref
    float nmc[NQB];
    // thr[nb]: raw-score level below which no key of a tile can move row block nb's reference
    // (rescale_threshold: a little under (mref + 8) / c, so every tile the exact test would
    // move is seen)
    float thr[NQB];
    f32x4 acc[NQB][NDB], accl[NQB];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        mref[nb] = -INFINITY;
        nmc[nb] = -0.f;
        thr[nb] = -INFINITY;
        accl[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            acc[nb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    asm volatile("" : "+v"(ones)); // held in registers, not rebuilt from scalars per block

    // LDS byte addresses of this lane's operand reads in ring slot 0.  The swizzle depends
    // on a row only through row % 8, which the 16-row steps leave alone, so K reads of one
    // 32-dim step and V reads of one 16-dim block differ only by constants (the offset
    // field): KD + NDB base registers per lane, moved to the tile's slot once per tile.
    //   K: key 16 kb + col, chunk 4 ks + grp        -> kbase[ks] + 16 kb RB
    //   V: key row 16 (2 ks + hh) + 4 grp + col / 4, chunk 2 db + (col % 4) / 2, half col % 2
    //                                               -> vbase[db] + 16 (2 ks + hh) RB
    unsigned kbase[KD], vbase[NDB];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
        kbase[ks] = lds_addr(kring) + col * RB + swz<D>(4 * ks + grp, col) * 16;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int row = 4 * grp + (col >> 2);
        const int ch = 2 * db + ((col & 3) >> 1);
        vbase[db] = lds_addr(vring) + row * RB + swz<D>(ch, row) * 16 + (col & 1) * 8;
    }

    for (int k = 0; k < NB - 1 && k < nt; ++k)
        issue(k);
    for (int t = 0; t < nt; ++t) {
        // this wave's loads of ring tile t have landed; after the barrier every wave's have,
        // and every wave has finished reading ring tile t - 1, whose slot the next DMA refills
        const int ahead = min(nt - 1 - t, NB - 2); // ring tiles issued after ring tile t
        if (ahead >= 2)
            wait_vm<2 * NDMA>();
        else if (ahead == 1)
            wait_vm<NDMA>();
        else
            wait_vm<0>();
        block_barrier();
        if (t + NB - 1 < nt)
            issue(t + NB - 1);
#pragma unroll 1
        for (int sub = 0; sub < SUB; ++sub) {
            const int k0 = t * RT + sub * KT;
            if (k0 >= kvis_any)
                continue; // no key of this tile is visible to any of the wave's blocks
            const unsigned soff = (unsigned)((t % NB) * RSLOT + sub * SLOT);
            unsigned kb_t[KD], vb_t[NDB]; // the operand bases in this tile's ring slot
#pragma unroll
            for (int ks = 0; ks < KD; ++ks)
                kb_t[ks] = kbase[ks] + soff;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                vb_t[db] = vbase[db] + soff;
            // K rows (A of the score MFMA): key 16 kb + col, dims 32 ks + 8 grp .. (chunk 4 ks + grp)
            f16x8 kop[KB][KD];
            lds_read_k<KB, KD, 0, 16 * RB>(kop, kb_t);
            // V^T (A of the value MFMA), k-step ks, dims 16 db ..: lane L of group grp addresses
            // key row 16 (2 ks + h) + 4 grp + L / 4, dims 16 db + 4 (L % 4); the transposing
            // read hands lane i element j = half i % 4 of lane 4 j + i / 4's 8 bytes
            f16x4 vraw[KS][NDB][2];
            lds_read_vt<KS, NDB, 0, 16 * RB>(vraw, vb_t);
            f16x8 vop[KS][NDB];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vop[ks][db] = __builtin_shufflevector(vraw[ks][db][0], vraw[ks][db][1], 0, 1, 2, 3, 4, 5, 6, 7);

#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) {
                if (k0 >= kvis[nb])
                    continue; // wave-uniform: no key of this tile is visible to the block
                // scores: sacc[kb][i] = S[key k0 + 16 kb + 4 grp + i][row r0 + col] (unscaled)
                f32x4 sacc[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb][0], qop[nb][0], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0);
#pragma unroll
                    for (int ks = 1; ks < KD; ++ks)
                        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb][ks], qop[nb][ks], s, 0, 0, 0);
                    sacc[kb] = s;
                }
                const bool full = all_ok && (!causal || k0 + KT - 1 <= off + r0[nb]) && k0 + KT <= nk;
                if (!full) {
                    bool bok[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        bok[kb] = true;
                    if constexpr (PAGED) {
                        if (!all_ok) { // keys of unusable blocks are masked
                            int e4[KB];
                            unsigned a4[KB];
#pragma unroll
                            for (int kb = 0; kb < KB; ++kb)
                                a4[kb] = lds_addr((const char *)&ids[min((k0 >> 4) + kb, max(P.max_blocks - 1, 0))]);
                            lds_read_b32<KB>(e4, a4);
#pragma unroll
                            for (int kb = 0; kb < KB; ++kb)
                                bok[kb] = e4[kb] >= 0;
                        }
                    }
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sacc[kb][i] = (bok[kb] && k0 + 16 * kb + 4 * grp + i < lim[nb]) ? sacc[kb][i] : -INFINITY;
                }
                // a row's reference max moves only when the row's own maximum passes it by more
                // than 2^8; between moves p = 2^(s c - mref) < 256 and nothing needs rescaling.
                // Rows that do not move scale by exactly 1, so no row depends on another's keys.
                // The lane's own maximum is first held against thr; only when some lane passes it
                // does the wave reduce the rows' maxima across lanes and apply the exact test.
                const float lmax = max_scores<KB>(sacc);
                if (__ballot(lmax > thr[nb]) != 0) {
                    const float mt = group_max(lmax) * c;
                    const bool need = mt > mref[nb] + RESCALE_LOG2;
                    if (__ballot(need) != 0) {
                        const float mn = need ? mt : mref[nb];
                        const float alpha = need ? (mref[nb] == -INFINITY ? 0.f : pf_exp2(mref[nb] - mn)) : 1.f;
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            acc[nb][db] *= alpha;
                        accl[nb] *= alpha;
                        mref[nb] = mn;
                        nmc[nb] = mn == -INFINITY ? -0.f : -mn;
                        thr[nb] = rescale_threshold(mref[nb], c, inv_c);
                    }
                }
                // P^T operand of k-step ks, slot s: key 16 (2 ks + s / 4) + 4 grp + s % 4 =
                // sacc[2 ks + s / 4][s % 4], rounded once to fp16
                f16x8 pop[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int s = 0; s < 8; ++s)
                        pop[ks][s] = (f16)pf_exp2(fmaf(sacc[2 * ks + (s >> 2)][s & 3], c, nmc[nb]));
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        acc[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[ks][db], pop[ks], acc[nb][db], 0, 0, 0);
                    accl[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[ks], accl[nb], 0, 0, 0);
                }
            }
        }
    }

    // ---- normalise and store: lane holds O^T[d = 16 db + 4 grp + i][row r0 + col] ----
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        const int row = r0[nb] + col;
        if (row >= n)
            continue;
        const float l = accl[nb][0];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        f16 *dst = P.out + ((size_t)(a + row) * hq + h) * D + grp * 4;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const f16x4 o4 = {(f16)(acc[nb][db][0] * inv), (f16)(acc[nb][db][1] * inv), (f16)(acc[nb][db][2] * inv),
                              (f16)(acc[nb][db][3] * inv)};
            *(f16x4 *)(dst + 16 * db) = o4;
        }
    }
}

// fp32: one wave per (query row, head); lane = key for the scores, lane = dim for p*v.
// grid = (max_seqlen, Hq, nseg), block = 64
__global__ __launch_bounds__(64) void prefill_valu_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ out, const int *__restrict__ cu, int hq, int hkv, float scale_log2,
    int causal)
{
    using namespace pf;
    __shared__ float qs[D];
    __shared__ float ps[64];
    const int i = blockIdx.x, h = blockIdx.y, seg = blockIdx.z;
    const int a = cu[seg];
    const int n = cu[seg + 1] - a;
    if (i >= n || n <= 0)
        return;
    const int g_kv = h / (hq / hkv);
    const int lane = threadIdx.x;
    qs[lane] = q[((size_t)(a + i) * hq + h) * D + lane];
    __syncthreads();
    const int kend = causal ? i + 1 : n;
    float m_run = -INFINITY, l_run = 0.f, o = 0.f;
    for (int k0 = 0; k0 < kend; k0 += 64) {
        const int kk = k0 + lane;
        float s = -INFINITY;
        if (kk < kend) {
            const float *kr = k + ((size_t)(a + kk) * hkv + g_kv) * D;
            float acc = 0.f;
            for (int c = 0; c < D; ++c)
                acc = fmaf(qs[c], kr[c], acc);
            s = acc * scale_log2;
        }
        float tmax = s;
        for (int msk = 32; msk >= 1; msk >>= 1)
            tmax = fmaxf(tmax, __shfl_xor(tmax, msk, 64));
        const float mn = fmaxf(m_run, tmax);
        const float alpha = pf_exp2(m_run - mn);
        const float p = kk < kend ? pf_exp2(s - mn) : 0.f;
        float psum = p;
        for (int msk = 32; msk >= 1; msk >>= 1)
            psum += __shfl_xor(psum, msk, 64);
        l_run = l_run * alpha + psum;
        m_run = mn;
        ps[lane] = p;
        __syncthreads();
        o *= alpha;
        const int cnt = min(64, kend - k0);
        for (int j = 0; j < cnt; ++j)
            o = fmaf(ps[j], v[((size_t)(a + k0 + j) * hkv + g_kv) * D + lane], o);
        __syncthreads();
    }
    out[((size_t)(a + i) * hq + h) * D + lane] = o / l_run;
}

} // namespace kvp

using namespace kvp;

extern "C" kvp_status varlen_causal_prefill(const kvp_dims *dims, void *out, const void *q,
                                            const void *k, const void *v,
                                            const int32_t *d_cu_seqlens, int32_t nseg,
                                            int32_t max_seqlen, int32_t causal, float scale,
                                            kvp_stream stream)
{
    if (!dims)
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: dims is NULL");
    if (dims->num_q_heads <= 0 || dims->num_kv_heads <= 0 ||
        dims->num_q_heads % dims->num_kv_heads != 0)
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: num_q_heads=%d, num_kv_heads=%d",
                    dims->num_q_heads, dims->num_kv_heads);
    if (dims->dtype != KVP_F16 && dims->dtype != KVP_F32)
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: dtype=%d", dims->dtype);
    const int hd = dims->head_dim;
    if (hd != pf::D && !(dims->dtype == KVP_F16 && hd == 128))
        return fail(KVP_ERR_UNSUPPORTED, "varlen_causal_prefill: head_dim=%d (64, or 128 for fp16)", hd);
    const int QB = pf::query_rows_per_workgroup(hd);
    if (nseg < 0 || max_seqlen < 0 || (causal != 0 && causal != 1))
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: nseg=%d max_seqlen=%d causal=%d", nseg,
                    max_seqlen, causal);
    if (nseg == 0 || max_seqlen == 0)
        return KVP_OK;
    if (!out || !q || !k || !v || !d_cu_seqlens ||
        (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15))
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: NULL or misaligned pointer");
    if (nseg > 65535 || dims->num_q_heads > 65535 || (max_seqlen + QB - 1) / QB > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "varlen_causal_prefill: nseg, H_q or max_seqlen too large");
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)hd);
    const float sl2 = scale * pf::LOG2E;
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == KVP_F16) {
        dim3 grid(dims->num_q_heads, nseg, (max_seqlen + QB - 1) / QB);
        PrefillArgs A{(const f16 *)q, (const f16 *)k, (const f16 *)v, (f16 *)out, d_cu_seqlens, nullptr, nullptr,
                      0, 0, dims->num_q_heads, dims->num_kv_heads, sl2, causal};
        if (hd == 64)
            hipLaunchKernelGGL((prefill_mfma_f16_kernel<false, 64, 2>), grid, dim3(256), 0, st, A);
        else
            hipLaunchKernelGGL((prefill_mfma_f16_kernel<false, 128, 2>), grid, dim3(256), 0, st, A);
    } else {
        dim3 grid(max_seqlen, dims->num_q_heads, nseg);
        hipLaunchKernelGGL(prefill_valu_f32_kernel, grid, dim3(64), 0, st, (const float *)q,
                           (const float *)k, (const float *)v, (float *)out, d_cu_seqlens,
                           dims->num_q_heads, dims->num_kv_heads, sl2, causal);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "varlen_causal_prefill: launch failed: %s", hipGetErrorString(e));
    return KVP_OK;
}

extern "C" kvp_status paged_prefill_attention(const kvp_cache_desc *cache, int32_t layer, void *out,
                                              const void *q, const int32_t *d_block_table,
                                              int32_t max_blocks, const int32_t *d_context_lens,
                                              const int32_t *d_cu_q, int32_t B, int32_t max_q,
                                              float scale, kvp_stream stream)
{
    const char *who = "paged_prefill_attention";
    if (!cache)
        return fail(KVP_ERR_INVALID, "%s: cache is NULL", who);
    const kvp_dims &d = cache->dims;
    if (d.num_layers <= 0 || d.num_q_heads <= 0 || d.num_kv_heads <= 0 || d.num_q_heads % d.num_kv_heads != 0)
        return fail(KVP_ERR_INVALID, "%s: num_q_heads=%d, num_kv_heads=%d", who, d.num_q_heads, d.num_kv_heads);
    const int hd = d.head_dim;
    if (hd != 64 && hd != 128)
        return fail(KVP_ERR_UNSUPPORTED, "%s: head_dim=%d (64 or 128)", who, hd);
    const int QB = pf::query_rows_per_workgroup(hd);
    if (d.dtype != KVP_F16)
        return fail(KVP_ERR_UNSUPPORTED, "%s: dtype=%d (fp16 only)", who, d.dtype);
    if (cache->block_size != pf::BS)
        return fail(KVP_ERR_UNSUPPORTED, "%s: block_size=%d (only 16)", who, cache->block_size);
    if (cache->num_blocks <= 0 || !cache->k_pool || !cache->v_pool ||
        (((uintptr_t)cache->k_pool | (uintptr_t)cache->v_pool) & 15))
        return fail(KVP_ERR_INVALID, "%s: empty or misaligned pool", who);
    if (layer < 0 || layer >= d.num_layers)
        return fail(KVP_ERR_INVALID, "%s: layer %d of %d", who, layer, d.num_layers);
    if (B < 0 || max_q < 0 || max_blocks < 0)
        return fail(KVP_ERR_INVALID, "%s: B=%d max_q=%d max_blocks=%d", who, B, max_q, max_blocks);
    if (B == 0 || max_q == 0)
        return KVP_OK;
    if (!out || !q || !d_block_table || !d_context_lens || !d_cu_q || (((uintptr_t)out | (uintptr_t)q) & 15))
        return fail(KVP_ERR_INVALID, "%s: NULL or misaligned pointer", who);
    if (max_blocks > MAX_IDS)
        return fail(KVP_ERR_UNSUPPORTED, "%s: max_blocks=%d (at most %d)", who, max_blocks, MAX_IDS);
    if (B > 65535 || d.num_q_heads > 65535 || (max_q + QB - 1) / QB > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "%s: B, H_q or max_q too large", who);
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)hd);
    const size_t layer_elems = (size_t)cache->num_blocks * d.num_kv_heads * pf::BS * hd;
    PrefillArgs A{(const f16 *)q, (const f16 *)cache->k_pool + (size_t)layer * layer_elems,
                  (const f16 *)cache->v_pool + (size_t)layer * layer_elems, (f16 *)out, d_cu_q, d_context_lens,
                  d_block_table, max_blocks, cache->num_blocks, d.num_q_heads, d.num_kv_heads,
                  scale * pf::LOG2E, 1};
    dim3 grid(d.num_q_heads, B, (max_q + QB - 1) / QB);
    const size_t ids_bytes = 4 * (size_t)std::max(max_blocks, 1);
    const bool wide = WIDE_RING_LDS + ids_bytes <= (size_t)LDS_TWO_PER_CU;
    hipStream_t st = (hipStream_t)stream;
    if (hd == 64 && wide)
        hipLaunchKernelGGL((prefill_mfma_f16_kernel<true, 64, 2>), grid, dim3(256), ids_bytes, st, A);
    else if (hd == 64)
        hipLaunchKernelGGL((prefill_mfma_f16_kernel<true, 64, 1>), grid, dim3(256), ids_bytes, st, A);
    else if (wide)
        hipLaunchKernelGGL((prefill_mfma_f16_kernel<true, 128, 2>), grid, dim3(256), ids_bytes, st, A);
    else
        hipLaunchKernelGGL((prefill_mfma_f16_kernel<true, 128, 1>), grid, dim3(256), ids_bytes, st, A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return KVP_OK;
}
