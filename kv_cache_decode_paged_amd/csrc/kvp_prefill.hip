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
// fp16: MFMA v_mfma_f32_16x16x32_f16 tiles with fp32 accumulation.  One workgroup = 4
// wave64 = 64 query rows of one (segment, query head); each wave owns 16 rows.  Per
// 64-key tile it computes S^T = K Q^T (keys as MFMA rows, so the result lands with one
// query per lane column), runs the online softmax on S^T in registers, and accumulates
// O^T = V^T P^T where P^T is the fp16-rounded probability tile taken straight from the
// S^T accumulator registers.  K goes HBM -> LDS with global_load_lds (chunk-swizzled);
// V is stored transposed in LDS for the A operand of the second product.  Tiles entirely
// above the causal diagonal are skipped.
// fp32: a plain VALU kernel (wave = one query row), exact fp32 throughout.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kvp_internal.h"

namespace kvp {

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

namespace pf {
constexpr int D = 64;
constexpr int QT = 64;  // query rows per workgroup
constexpr int KT = 64;  // keys per iteration
constexpr int NW = 4;
constexpr int VTS = KT + 4; // padded row (in halfs) of the transposed V tile
constexpr float LOG2E = 1.4426950408889634f;
} // namespace pf

__device__ inline float pf_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float xor_shfl(float x, int m)
{
    return __shfl_xor(x, m, 64);
}

// grid = (ceil(max_seqlen/64), Hq, nseg), block = 256
__global__ __launch_bounds__(256) void prefill_mfma_f16_kernel(
    const f16 *__restrict__ q, const f16 *__restrict__ k, const f16 *__restrict__ v,
    f16 *__restrict__ out, const int *__restrict__ cu, int hq, int hkv, float scale_log2,
    int causal)
{
    using namespace pf;
    __shared__ __attribute__((aligned(16))) char klds[KT * D * 2];      // [key][64] swizzled
    __shared__ __attribute__((aligned(16))) f16 vt[D * VTS];            // [d][key] padded

    const int qtile = blockIdx.x, h = blockIdx.y, seg = blockIdx.z;
    const int a = cu[seg];
    const int n = cu[seg + 1] - a;
    const int q0 = qtile * QT;
    if (q0 >= n || n <= 0)
        return;
    const int g_kv = h / (hq / hkv);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15; // query row within the wave's 16 (MFMA column)
    const int grp = lane >> 4; // lane group 0..3
    const int qi = q0 + wave * 16 + col; // query index within the segment

    // Q^T operand: lane holds Q[qi][8*grp .. +8] (step 0) and [32 + 8*grp ..] (step 1)
    f16x8 qop[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        if (qi < n)
            qop[st] = *(const f16x8 *)(q + ((size_t)(a + qi) * hq + h) * D + st * 32 + grp * 8);
        else
            qop[st] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    f32x4 acc[4]; // O^T tiles: d = 16*dt + 4*grp + i, query col
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int kend = causal ? min(n, q0 + QT) : n; // keys needed by this workgroup
    const int ntiles = (kend + KT - 1) / KT;
    const int wq_hi = q0 + wave * 16 + 15; // last query row of this wave

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * KT;
        // ---- K tile -> LDS (2 instructions of 1 KB per wave), chunk swizzled ----
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int inst = wave * 2 + i;           // 0..7, rows 8*inst .. 8*inst+7
            const int r = inst * 8 + (lane >> 3);
            const int cg = (lane & 7) ^ (r & 7);
            const int kk = k0 + r;
            if (kk < kend) {
                const f16 *src = k + ((size_t)(a + kk) * hkv + g_kv) * D + cg * 8;
                __builtin_amdgcn_global_load_lds((const void *)src,
                                                 (__attribute__((address_space(3))) void *)(klds + inst * 1024),
                                                 16, 0, 0);
            }
        }
        // ---- V tile -> LDS transposed: thread loads 16 B of one key row ----
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = threadIdx.x + i * 256; // 0..511 = 64 rows x 8 chunks
            const int r = idx >> 3, c = idx & 7;
            const int kk = k0 + r;
            f16x8 vv = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (kk < kend)
                vv = *(const f16x8 *)(v + ((size_t)(a + kk) * hkv + g_kv) * D + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vt[(c * 8 + e) * VTS + r] = vv[e];
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        if (!(causal && k0 > wq_hi)) { // wave-uniform: tile has keys this wave can see
            // ---- S^T = K Q^T : 4 key tiles of 16 ----
            f32x4 sacc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int r = kt * 16 + col; // key row used as MFMA row
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int c = st * 4 + grp;
                    const f16x8 kop = *(const f16x8 *)(klds + r * 128 + ((c ^ (r & 7)) * 16));
                    sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[st], sacc[kt], 0, 0, 0);
                }
            }
            // lane holds S^T[key = 16*kt + 4*grp + i][query col]
            float tmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kk = k0 + kt * 16 + grp * 4 + i;
                    const bool ok = kk < kend && (!causal || kk <= qi);
                    const float x = ok ? sacc[kt][i] * scale_log2 : -INFINITY;
                    sacc[kt][i] = x;
                    tmax = fmaxf(tmax, x);
                }
            tmax = fmaxf(tmax, xor_shfl(tmax, 16));
            tmax = fmaxf(tmax, xor_shfl(tmax, 32));
            const float mn = fmaxf(m_run, tmax);
            const float alpha = mn == -INFINITY ? 1.f : pf_exp2(m_run - mn);
            m_run = mn;
            float psum = 0.f;
            f16x8 pop[2];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = mn == -INFINITY ? 0.f : pf_exp2(sacc[kt][i] - mn);
                    const f16 ph = (f16)p;
                    psum += (float)ph; // normaliser from the same rounded weights
                    pop[kt >> 1][(kt & 1) * 4 + i] = ph;
                }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                acc[dt] *= alpha;
            // ---- O^T += V^T P^T : per 32-key step, k slot (grp, e) -> key
            //      32*ks + (e < 4 ? 4*grp + e : 16 + 4*grp + e - 4) ----
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const int dr = dt * 16 + col;
                    const f16 *row = vt + dr * VTS + ks * 32 + grp * 4;
                    const f16x4 lo = *(const f16x4 *)(row);
                    const f16x4 hi = *(const f16x4 *)(row + 16);
                    const f16x8 vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[ks], acc[dt], 0, 0, 0);
                }
            }
        }
        __syncthreads(); // before the next tile overwrites klds / vt
    }

    // ---- normalise and store: lane holds O^T[d = 16*dt + 4*grp + i][query col] ----
    float lt = l_run;
    lt += xor_shfl(lt, 16);
    lt += xor_shfl(lt, 32);
    if (qi < n) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        f16 *dst = out + ((size_t)(a + qi) * hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            f16x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o4[i] = (f16)(acc[dt][i] * inv);
            *(f16x4 *)(dst + dt * 16 + grp * 4) = o4;
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
    if (dims->head_dim != pf::D)
        return fail(KVP_ERR_UNSUPPORTED, "varlen_causal_prefill: head_dim=%d (only 64)", dims->head_dim);
    if (dims->dtype != KVP_F16 && dims->dtype != KVP_F32)
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: dtype=%d", dims->dtype);
    if (nseg < 0 || max_seqlen < 0 || (causal != 0 && causal != 1))
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: nseg=%d max_seqlen=%d causal=%d", nseg,
                    max_seqlen, causal);
    if (nseg == 0 || max_seqlen == 0)
        return KVP_OK;
    if (!out || !q || !k || !v || !d_cu_seqlens ||
        (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15))
        return fail(KVP_ERR_INVALID, "varlen_causal_prefill: NULL or misaligned pointer");
    if (nseg > 65535 || dims->num_q_heads > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "varlen_causal_prefill: nseg or H_q too large");
    if (scale == 0.f)
        scale = 1.0f / sqrtf((float)pf::D);
    const float sl2 = scale * pf::LOG2E;
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == KVP_F16) {
        dim3 grid((max_seqlen + pf::QT - 1) / pf::QT, dims->num_q_heads, nseg);
        hipLaunchKernelGGL(prefill_mfma_f16_kernel, grid, dim3(256), 0, st, (const f16 *)q,
                           (const f16 *)k, (const f16 *)v, (f16 *)out, d_cu_seqlens,
                           dims->num_q_heads, dims->num_kv_heads, sl2, causal);
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
