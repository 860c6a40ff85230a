// kvp_decode_f32.hip -- fp32 grouped-query decode attention (single-head fp32 workloads)
// for gfx950.
//
// Same definition as the fp16 path (pages cited there and in kvp.h): the new token's query
// attends over every cached key including its own (gustavoai "La cache de claves y
// valores", four-step token recipe), softmax(q K^T / sqrt(d)) V (chatgpz.de linear-
// attention post, TraditionalAttention), split partitions merged by rescaling with
// e^(block max - global max) (chatgpz.de FlashAttention post).
//
// Kernel: one workgroup of 4 waves per (request, KV head, split); K rows go HBM -> LDS with
// global_load_lds (chunk-swizzled) and each lane scores one token against the query in
// LDS with exact fp32 FMAs; p*v in fp32 with values held in VGPRs; the 4 waves' softmax
// states are merged in LDS.  A request split over several workgroups leaves fp32 partials
// (device-coherent stores) and the last workgroup to finish merges them in split order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "kvp_decode_common.h"

namespace kvp {

using namespace dec;

// split policy: a pure function of the context length (an optional override applies to
// every layout alike), so the paged and contiguous calls split identically
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
    const int s = split_tokens(ctx, override_tokens);
    return (ctx + s - 1) / s;
}

static int split_override_from_env()
{
    const char *e = getenv("KVP_SPLIT_TOKENS");
    if (!e || !*e)
        return 0;
    const int v = atoi(e);
    return (v > 0 && v % 256 == 0 && v <= 1024) ? v : 0; // otherwise ignored
}

int decode_f32_max_splits(int max_context)
{
    const int ov = split_override_from_env();
    if (max_context <= 0)
        return 1;
    if (ov > 0)
        return (max_context + ov - 1) / ov;
    // the worst case of each tier of split_tokens() sits at its upper end
    int best = num_splits(std::min(max_context, 4096), 0);
    if (max_context > 4096)
        best = std::max(best, num_splits(std::min(max_context, 16384), 0));
    if (max_context > 16384)
        best = std::max(best, num_splits(max_context, 0));
    return best;
}

size_t decode_f32_part_bytes(int B, int hq, int max_splits)
{
    return (size_t)B * hq * max_splits * (D + 2) * sizeof(float);
}

// (linear workgroup id) -> (pair = b*hkv + g, split s), rotating pairs across XCDs
__device__ inline void f32_work_item(int L, int npairs, int &pair, int &s)
{
    s = L / npairs;
    int j = L - s * npairs;
    pair = j + (s % npairs);
    if (pair >= npairs)
        pair -= npairs;
}

struct F32Extra {
    int split_override;
};

// ---------------------------------------------------------------------------------------
// fp32 decode kernel (VALU).  grid = (max_splits * B * Hkv), block = 256 (4 waves, each
// owning 64 tokens of every 256-token step of the split).
// ---------------------------------------------------------------------------------------
constexpr int NW = 4;

template <int G, typename Addr>
__global__ __launch_bounds__(NW * 64) void decode_f32_kernel(DecodeParams P, Addr A, F32Extra X)
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
    f32_work_item(blockIdx.x, P.B * P.hkv, pair, s);
    const int b = pair / P.hkv, g = pair - (pair / P.hkv) * P.hkv;
    const float *qg = (const float *)P.q + ((size_t)b * P.hq + (size_t)g * G) * D;
    float *outg = (float *)P.out + ((size_t)b * P.hq + (size_t)g * G) * D;

    int ctx = P.ctx_lens[b];
    if (ctx > A.max_ctx())
        ctx = A.max_ctx();
    const int S = split_tokens(ctx, X.split_override);
    const int nsplit = num_splits(ctx, X.split_override);
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
            const size_t pi = ((size_t)b * P.hq + (size_t)g * G + h) * P.workers + s;
            coherent_store(P.part + pi * (D + 2) + c, O);
            if (c == 0) {
                coherent_store(P.part + pi * (D + 2) + D, M);
                coherent_store(P.part + pi * (D + 2) + D + 1, L);
            }
        }
    }
    if (nsplit == 1)
        return;
    // every thread's partial stores are complete before one ticket is taken for the
    // workgroup; the partials went out as device-coherent stores
    wait_stores();
    __syncthreads();
    __shared__ int is_last;
    if (threadIdx.x == 0)
        is_last = take_ticket(&P.tickets[b * P.hkv + g]) == nsplit - 1;
    __syncthreads();
    if (!is_last || wave != 0)
        return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t base = ((size_t)b * P.hq + (size_t)g * G + h) * P.workers;
        float M = -INFINITY;
        for (int i = 0; i < nsplit; ++i)
            M = fmaxf(M, coherent_load(P.part + (base + i) * (D + 2) + D));
        float L = 0.f, O = 0.f;
        for (int i = 0; i < nsplit; ++i) {
            const float *pp = P.part + (base + i) * (D + 2);
            const float f = M == -INFINITY ? 0.f : fast_exp2(coherent_load(pp + D) - M);
            L = fmaf(coherent_load(pp + D + 1), f, L);
            O = fmaf(coherent_load(pp + lane), f, O);
        }
        outg[h * D + lane] = L > 0.f ? O / L : 0.f;
    }
    if (lane == 0)
        reset_ticket(&P.tickets[b * P.hkv + g]);
}


template <typename Addr>
static kvp_status launch_f32(const DecodeParams &P, const Addr &A, int group, hipStream_t st)
{
    const long long nwg = (long long)P.workers * P.B * P.hkv;
    if (nwg > 0x7fffffffLL)
        return fail(KVP_ERR_UNSUPPORTED, "decode: grid of %lld workgroups too large", nwg);
    F32Extra X{split_override_from_env()};
    dim3 grid((unsigned)nwg), block(NW * 64);
    switch (group) {
#define KVP_G(GG)                                                                              \
    case GG:                                                                                   \
        hipLaunchKernelGGL((decode_f32_kernel<GG, Addr>), grid, block, 0, st, P, A, X);       \
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

kvp_status launch_decode_f32(const DecodeParams &P, const PagedAddr &A, int group, hipStream_t st)
{
    return launch_f32(P, A, group, st);
}
kvp_status launch_decode_f32(const DecodeParams &P, const ContigAddr &A, int group, hipStream_t st)
{
    return launch_f32(P, A, group, st);
}

} // namespace kvp
