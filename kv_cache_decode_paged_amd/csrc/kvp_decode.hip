// kvp_decode.hip -- grouped-query decode attention over a paged or contiguous KV cache,
// split-K partials and their merge, for gfx950 (MI355X, wave64).
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
//   with e^(block max - global max).  Used twice: across the 64-token tiles inside a
//   workgroup (online softmax) and across split-K partitions (the merge kernel).
//
// Design for gfx950 (not a translation of any other GPU's kernel):
//   * one workgroup = 4 wave64 = one (request, KV head, split); it serves all G query
//     heads of the group, so every K/V byte is read from HBM once per group;
//   * each wave owns a 64-token tile per iteration (4 blocks of 16 tokens); K rows are
//     moved HBM -> LDS with global_load_lds_dwordx4 (16 B per lane, 1 KB per instruction,
//     fully coalesced), with an XOR swizzle of the 16-byte chunk so that the transposed
//     per-token read (lane = token) is free of bank conflicts;
//   * scores: lane = token, full 64-dim dot products with v_dot2_f32_f16 (fp16) or FMA
//     (fp32) against the query held in LDS; no cross-lane reduction needed;
//   * tile max per head by a DPP wave reduction; p = exp2(s*scale*log2e - m) with the
//     hardware exp2; p goes through a small LDS buffer;
//   * values: loaded straight into VGPRs in the coalesced layout (lane = 16-byte chunk x
//     token group), p*v accumulated in fp32 (mixed fp16 x fp32 FMA);
//   * the 4 waves keep independent online-softmax states and are merged once at the end.
//   * paged and contiguous layouts differ only in the address of a 16-token block; the
//     arithmetic and its order are identical, so their outputs are bit-identical.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "kvp_internal.h"

namespace kvp {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 64;      // head dim
constexpr int BS = 16;     // tokens per block
constexpr int NW = 4;      // waves per workgroup
constexpr int TILE = 64;   // tokens per wave per iteration
constexpr int ITER = NW * TILE;
constexpr int MAXG = 8;    // query heads per group handled by one workgroup
constexpr float LOG2E = 1.4426950408889634f;

template <typename T> struct Elem;
template <> struct Elem<f16> {
    static constexpr int CH = 8; // elements per 16-byte chunk
};
template <> struct Elem<float> {
    static constexpr int CH = 4;
};

// ---------------------------------------------------------------------------------------
// split policy: a pure function of the context length (and an optional override that the
// host applies identically to every layout), so the paged and contiguous calls agree.
// ---------------------------------------------------------------------------------------
__host__ __device__ inline int split_tokens(int ctx, int override_tokens)
{
    if (override_tokens > 0)
        return override_tokens;
    if (ctx <= 4096)
        return 256;
    if (ctx <= 8192)
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
    // tiers of split_tokens(): the worst case in each tier is at its upper end
    int best = num_splits(std::min(max_context, 4096), 0);
    if (max_context > 4096)
        best = std::max(best, num_splits(std::min(max_context, 8192), 0));
    if (max_context > 8192)
        best = std::max(best, num_splits(max_context, 0));
    return best;
}

int split_override_from_env()
{
    const char *e = getenv("KVP_SPLIT_TOKENS");
    if (!e || !*e)
        return 0;
    int v = atoi(e);
    if (v <= 0 || v % ITER != 0 || v > 1024)
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
    __device__ int entry(int b, int idx) const { return table[(size_t)b * max_blocks + idx]; }
    __device__ bool valid(int e) const { return e >= 0 && e < num_blocks; }
    // element offset of row 0 of the block for (b, kv head g, logical block idx)
    __device__ size_t block_off(int b, int g, int idx, int e) const
    {
        (void)b;
        (void)idx;
        return ((size_t)e * hkv + g) * (BS * D);
    }
    __device__ int max_ctx() const { return max_blocks * BS; }
};

struct ContigAddr {
    int hkv;
    int lmax;
    __device__ int entry(int, int) const { return 0; }
    __device__ bool valid(int) const { return true; }
    __device__ size_t block_off(int b, int g, int idx, int) const
    {
        return (((size_t)b * hkv + g) * lmax + (size_t)idx * BS) * D;
    }
    __device__ int max_ctx() const { return lmax; }
};

// ---------------------------------------------------------------------------------------
// wave64 reductions with DPP (gfx9 encodings) and a final readlane
// ---------------------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND = false>
__device__ inline float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                         CTRL, ROW_MASK, BANK_MASK, BOUND));
}

__device__ inline float wave_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));  // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));  // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x)); // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x)); // row_mirror: every lane holds its row's max
    x = fmaxf(x, dpp<0x142, 0xa>(x)); // row_bcast:15 into rows 1, 3
    x = fmaxf(x, dpp<0x143, 0xc>(x)); // row_bcast:31 into rows 2, 3
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

__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// dot of a 16-byte chunk of K with the same chunk of q, accumulated in fp32
__device__ inline float chunk_dot(const i32x4 &k, const i32x4 &q, float acc, f16)
{
    const f16x8 kh = __builtin_bit_cast(f16x8, k);
    const f16x8 qh = __builtin_bit_cast(f16x8, q);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        f16x2 a = {kh[e], kh[e + 1]};
        f16x2 b = {qh[e], qh[e + 1]};
        acc = __builtin_amdgcn_fdot2(a, b, acc, false);
    }
    return acc;
}

__device__ inline float chunk_dot(const i32x4 &k, const i32x4 &q, float acc, float)
{
    const f32x4 kf = __builtin_bit_cast(f32x4, k);
    const f32x4 qf = __builtin_bit_cast(f32x4, q);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        acc = fmaf(kf[e], qf[e], acc);
    return acc;
}

__device__ inline float elem_to_f32(const i32x4 &v, int e, f16)
{
    return (float)__builtin_bit_cast(f16x8, v)[e];
}
__device__ inline float elem_to_f32(const i32x4 &v, int e, float)
{
    return __builtin_bit_cast(f32x4, v)[e];
}

template <typename T> __device__ inline T from_f32(float x) { return (T)x; }

// ---------------------------------------------------------------------------------------
// The decode kernel.  grid = (max_splits, H_kv, B), block = 256.
// ---------------------------------------------------------------------------------------
template <typename T> struct DecodeSmem {
    static constexpr int KBYTES = NW * TILE * D * (int)sizeof(T);
    static constexpr int PBYTES = NW * TILE * MAXG * 4;
    static constexpr int QBYTES = MAXG * D * (int)sizeof(T);
    static constexpr int MBYTES = NW * 4 * MAXG * D * 4; // merge: waves x rows x heads x d
    static constexpr int ML = NW * MAXG * 2 * 4;
    static constexpr int BYTES = (KBYTES > MBYTES ? KBYTES : MBYTES) + PBYTES + QBYTES + ML;
};

struct DecodeParams {
    const void *q;
    void *out;
    const void *kc; // layer base of the K pool / cache
    const void *vc;
    const int *ctx_lens;
    int hq;
    int hkv;
    float scale_log2;
    int split_override;
    int max_splits;
    float *part_o;  // [B][Hq][max_splits][D]
    float *part_ml; // [B][Hq][max_splits][2]
};

template <typename T, int G, typename Addr>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(DecodeParams P, Addr A)
{
    constexpr int CH = Elem<T>::CH;     // elements per 16-byte chunk
    constexpr int NCH = D / CH;         // chunks per row (8 fp16, 16 fp32)
    constexpr int RPI = 64 / NCH;       // rows per load instruction (8, 4)
    constexpr int NLD = TILE / RPI;     // load instructions per tile (8, 16)
    constexpr int ROWB = D * sizeof(T); // bytes per row
    using SM = DecodeSmem<T>;

    __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];
    char *kbuf = smem;
    float *pbuf = (float *)(smem + (SM::KBYTES > SM::MBYTES ? SM::KBYTES : SM::MBYTES));
    T *qbuf = (T *)((char *)pbuf + SM::PBYTES);
    float *mlbuf = (float *)((char *)qbuf + SM::QBYTES);

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const T *qg = (const T *)P.q + ((size_t)b * P.hq + (size_t)g * G) * D;
    T *outg = (T *)P.out + ((size_t)b * P.hq + (size_t)g * G) * D;

    int ctx = P.ctx_lens[b];
    if (ctx > A.max_ctx())
        ctx = A.max_ctx();
    const int S = split_tokens(ctx, P.split_override);
    const int nsplit = num_splits(ctx, P.split_override);
    if (s >= nsplit)
        return;
    if (ctx <= 0) { // invalid length: defined output (zeros), no memory read
        for (int i = threadIdx.x; i < G * D; i += NW * 64)
            outg[i] = from_f32<T>(0.f);
        return;
    }
    const int t_begin = s * S;
    const int t_end = min(ctx, t_begin + S);

    // query rows of the group -> LDS
    for (int i = threadIdx.x; i < G * NCH; i += NW * 64)
        ((i32x4 *)qbuf)[i] = ((const i32x4 *)qg)[i];

    // block-table entries of this split: lane i holds entry (t_begin/16 + i); a split
    // has at most 1024 tokens = 64 blocks
    const int blk0 = t_begin / BS;
    const int nblk = (t_end - t_begin + BS - 1) / BS;
    int my_entry = 0;
    if (lane < nblk)
        my_entry = A.entry(b, blk0 + lane);
    __syncthreads();

    const T *kc = (const T *)P.kc;
    const T *vc = (const T *)P.vc;
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

    const int tg = lane / NCH; // token group of this lane in the value layout
    const int cv = lane % NCH; // 16-byte chunk of this lane in the value layout
    const int nit = (t_end - t_begin + ITER - 1) / ITER;

    for (int it = 0; it < nit; ++it) {
        const int r0 = it * ITER + wave * TILE; // first row of this wave's tile, rel. to split
        const int t0 = t_begin + r0;
        if (t0 >= t_end)
            continue; // wave-uniform
        // block ids of the tile's 4 blocks (wave-uniform)
        int ent[TILE / BS];
        bool ok[TILE / BS];
#pragma unroll
        for (int k = 0; k < TILE / BS; ++k) {
            int li = r0 / BS + k;
            ent[k] = __builtin_amdgcn_readlane(my_entry, li < 64 ? li : 63);
            ok[k] = (t0 + k * BS < t_end) && A.valid(ent[k]);
        }
        // ---- K: HBM -> LDS, coalesced 1 KB per instruction, chunk-swizzled ----
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int k = (i * RPI) / BS;
            const int r = i * RPI + lane / NCH;     // row in the tile
            const int cg = (lane % NCH) ^ (r % NCH); // global chunk stored at this LDS slot
            const int t = t0 + r;
            if (ok[k] && t < t_end) {
                const T *src = kc + A.block_off(b, g, blk0 + r0 / BS + k, ent[k]) +
                               (size_t)(r % BS) * D + cg * CH;
                __builtin_amdgcn_global_load_lds((const void *)src,
                                                 (__attribute__((address_space(3))) void *)(kl + i * 1024),
                                                 16, 0, 0);
            }
        }
        // ---- V: HBM -> VGPRs, lane = (token group, chunk) ----
        i32x4 vreg[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int k = (i * RPI) / BS;
            const int r = i * RPI + tg;
            const int t = t0 + r;
            if (ok[k] && t < t_end)
                vreg[i] = *(const i32x4 *)(vc + A.block_off(b, g, blk0 + r0 / BS + k, ent[k]) +
                                           (size_t)(r % BS) * D + cv * CH);
            else
                vreg[i] = i32x4{0, 0, 0, 0};
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        wave_lds_sync();

        // ---- scores: lane = token ----
        const int j = lane;
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            sc[h] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const i32x4 kv = *(const i32x4 *)(kl + j * ROWB + ((c ^ (j % NCH)) * 16));
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const i32x4 qv = ((const i32x4 *)qbuf)[h * NCH + c];
                sc[h] = chunk_dot(kv, qv, sc[h], T());
            }
        }
        const int tj = t0 + j;
        const int kj = (tj - t0) / BS;
        bool valid_j = tj < t_end;
#pragma unroll
        for (int k = 0; k < TILE / BS; ++k)
            if (k == kj)
                valid_j = valid_j && ok[k];
        float pj[G];
        bool rescale = false;
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float x = valid_j ? sc[h] * P.scale_log2 : -INFINITY;
            const float mt = wave_max(x);
            const float mn = fmaxf(m[h], mt);
            // mn is -inf only if no token so far was readable (bad table entries)
            alpha[h] = mn == -INFINITY ? 1.f : fast_exp2(m[h] - mn);
            rescale |= (mn != m[h]);
            m[h] = mn;
            pj[h] = mn == -INFINITY ? 0.f : fast_exp2(x - mn);
            lsum[h] = lsum[h] * alpha[h] + pj[h];
        }
        // p of this token -> LDS row j
#pragma unroll
        for (int h = 0; h < G; ++h)
            pl[j * MAXG + h] = pj[h];
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < CH; ++e)
                    o[h][e] *= alpha[h];
        }
        wave_lds_sync();

        // ---- p * v: lane = (token group tg, chunk cv) ----
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int r = i * RPI + tg;
            float pr[G];
#pragma unroll
            for (int h = 0; h < G; ++h)
                pr[h] = pl[r * MAXG + h];
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const float ve = elem_to_f32(vreg[i], e, T());
#pragma unroll
                for (int h = 0; h < G; ++h)
                    o[h][e] = fmaf(pr[h], ve, o[h][e]);
            }
        }
        wave_lds_sync(); // the next tile overwrites kl and pl
    }

    // ---- end of split: merge token groups, then waves ----
    // fp16: token groups 2r and 2r+1 share DPP row r; add lane c and c+8 (row_ror:8)
    if constexpr (NCH == 8) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < CH; ++e)
                o[h][e] += dpp<0x128>(o[h][e]);
    }
    __syncthreads(); // everyone is done with kbuf; reuse it for the merge
    float *mbuf = (float *)kbuf; // [NW][4 rows][MAXG][D]
    const int row = lane >> 4;
    const int cl = lane & 15;
    if (cl < NCH) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float *dst = mbuf + (((wave * 4 + row) * MAXG + h) * D) + cl * CH;
#pragma unroll
            for (int e = 0; e < CH; ++e)
                dst[e] = o[h][e];
        }
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
            outg[h * D + c] = from_f32<T>(L > 0.f ? O / L : 0.f);
        } else {
            const size_t pi = ((size_t)b * P.hq + (size_t)g * G + h) * P.max_splits + s;
            P.part_o[pi * D + c] = O;
            if (c == 0) {
                P.part_ml[pi * 2 + 0] = M;
                P.part_ml[pi * 2 + 1] = L;
            }
        }
    }
}

// Merge of split partials, in split order.  grid = (H_q, B), block = 64 (lane = dim).
template <typename T>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeParams P, int max_ctx)
{
    const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    int ctx = P.ctx_lens[b];
    if (ctx > max_ctx)
        ctx = max_ctx;
    const int nsplit = num_splits(ctx, P.split_override);
    if (nsplit <= 1 || ctx <= 0)
        return; // written directly by the partial kernel
    const size_t base = ((size_t)b * P.hq + h) * P.max_splits;
    float M = -INFINITY;
    for (int i = 0; i < nsplit; ++i)
        M = fmaxf(M, P.part_ml[(base + i) * 2]);
    float L = 0.f, O = 0.f;
    for (int i = 0; i < nsplit; ++i) {
        const float f = M == -INFINITY ? 0.f : fast_exp2(P.part_ml[(base + i) * 2] - M);
        L = fmaf(P.part_ml[(base + i) * 2 + 1], f, L);
        O = fmaf(P.part_o[(base + i) * D + c], f, O);
    }
    ((T *)P.out)[((size_t)b * P.hq + h) * D + c] = from_f32<T>(L > 0.f ? O / L : 0.f);
}

// ---------------------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------------------
template <typename T, typename Addr>
static kvp_status launch_decode_t(const DecodeParams &P, const Addr &A, int B, int group,
                                  int max_ctx, hipStream_t st)
{
    dim3 grid(P.max_splits, P.hkv, B), block(NW * 64);
    switch (group) {
#define KVP_G(GG)                                                                              \
    case GG:                                                                                   \
        hipLaunchKernelGGL((decode_partial_kernel<T, GG, Addr>), grid, block, 0, st, P, A);   \
        break;
        KVP_G(1) KVP_G(2) KVP_G(3) KVP_G(4) KVP_G(5) KVP_G(6) KVP_G(7) KVP_G(8)
#undef KVP_G
    default:
        return fail(KVP_ERR_UNSUPPORTED, "decode: query heads per KV head = %d (1..8 supported)", group);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(KVP_ERR_HIP, "decode partial launch: %s", hipGetErrorString(e));
    if (P.max_splits > 1) {
        hipLaunchKernelGGL((decode_reduce_kernel<T>), dim3(P.hq, B), dim3(64), 0, st, P, max_ctx);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(KVP_ERR_HIP, "decode reduce launch: %s", hipGetErrorString(e));
    }
    return KVP_OK;
}

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

size_t workspace_bytes(const kvp_dims *d, int B, int max_context)
{
    int ms = max_splits_for(max_context, split_override_from_env());
    if (ms <= 1)
        return 0;
    return (size_t)B * d->num_q_heads * ms * (D + 2) * sizeof(float);
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
    if (B > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "%s: B=%d > 65535", who, B);
    const int group = dims->num_q_heads / dims->num_kv_heads;
    DecodeParams P;
    P.q = q;
    P.out = out;
    P.kc = kc;
    P.vc = vc;
    P.ctx_lens = d_ctx;
    P.hq = dims->num_q_heads;
    P.hkv = dims->num_kv_heads;
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)D);
    P.scale_log2 = scale * LOG2E;
    P.split_override = split_override_from_env();
    P.max_splits = max_splits_for(max_ctx, P.split_override);
    P.part_o = nullptr;
    P.part_ml = nullptr;
    if (P.max_splits > 1) {
        size_t need = (size_t)B * P.hq * P.max_splits * (D + 2) * sizeof(float);
        if (!ws || ws_bytes < need)
            return fail(KVP_ERR_INVALID, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
        if ((uintptr_t)ws & 15)
            return fail(KVP_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
        P.part_o = (float *)ws;
        P.part_ml = (float *)ws + (size_t)B * P.hq * P.max_splits * D;
    }
    hipStream_t st_ = (hipStream_t)stream;
    if (dims->dtype == KVP_F16)
        return launch_decode_t<f16>(P, A, B, group, max_ctx, st_);
    return launch_decode_t<float>(P, A, B, group, max_ctx, st_);
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
    if (cache->block_size != BS)
        return fail(KVP_ERR_UNSUPPORTED, "paged_decode_attention: block_size=%d (only 16)", cache->block_size);
    if (layer < 0 || layer >= cache->dims.num_layers)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: layer %d out of range", layer);
    if (max_blocks <= 0 || cache->num_blocks <= 0 || !d_block_table)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: max_blocks=%d num_blocks=%d table=%p",
                    max_blocks, cache->num_blocks, (const void *)d_block_table);
    kvp_status st0 = check_dims(&cache->dims, "paged_decode_attention");
    if (st0 != KVP_OK)
        return st0;
    const size_t esz = cache->dims.dtype == KVP_F16 ? 2 : 4;
    const size_t layer_elems = (size_t)cache->num_blocks * cache->dims.num_kv_heads * BS * D;
    const char *kc = (const char *)cache->k_pool + (size_t)layer * layer_elems * esz;
    const char *vc = (const char *)cache->v_pool + (size_t)layer * layer_elems * esz;
    if (!cache->k_pool || !cache->v_pool)
        return fail(KVP_ERR_INVALID, "paged_decode_attention: pool pointer is NULL");
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
