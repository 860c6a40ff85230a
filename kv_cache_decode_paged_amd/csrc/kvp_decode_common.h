// kvp_decode_common.h -- device helpers and parameter blocks shared by the decode kernels
// (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "kvp_internal.h"

namespace kvp {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

namespace dec {
constexpr int D = 64;    // head dim of the fp32 kernel (fp16: 64 or 128, a template argument)
constexpr int BS = 16;   // tokens per block
constexpr int TILE = 64; // tokens per tile (4 blocks)
constexpr int MAXG = 8;  // fp32 kernel: query heads per group handled by one wave
constexpr float LOG2E = 1.4426950408889634f;
} // namespace dec

// ---------------------------------------------------------------------------------------
// address of a 16-token block of one (request, KV head) in one layer
// ---------------------------------------------------------------------------------------
struct PagedAddr {
    const int *table; // [B][max_blocks]
    int max_blocks;
    int hkv;
    int num_blocks;
    int dim;          // head dim
    static constexpr bool paged = true;
    __device__ int entry(int b, int idx) const
    {
        return (idx >= 0 && idx < max_blocks) ? table[(size_t)b * max_blocks + idx] : -1;
    }
    __device__ bool valid(int e) const { return e >= 0 && e < num_blocks; }
    // row index (rows of dim elements) of row 0 of the block (request b, kv head g,
    // logical block idx, table entry e), and its element offset
    __device__ size_t block_row(int, int g, int, int e) const { return ((size_t)e * hkv + g) * dec::BS; }
    __device__ size_t block_off(int b, int g, int idx, int e) const { return block_row(b, g, idx, e) * dim; }
    __device__ int max_ctx() const { return max_blocks * dec::BS; }
    // row to read for in-block row r (blocks always hold 16 rows)
    __device__ int row(int, int r) const { return r; }
    // a block that is always readable (block 0 of KV head g), for rows that are masked
    __device__ size_t safe_row0(int, int g) const { return (size_t)g * dec::BS; }
    __device__ size_t safe_off(int b, int g) const { return safe_row0(b, g) * dim; }
    __device__ int safe_row(int r) const { return r; }
};

struct ContigAddr {
    int hkv;
    int lmax;
    int dim;          // head dim
    static constexpr bool paged = false;
    __device__ int entry(int, int) const { return 0; }
    __device__ bool valid(int) const { return true; }
    __device__ size_t block_row(int b, int g, int idx, int) const
    {
        return ((size_t)b * hkv + g) * lmax + (size_t)idx * dec::BS;
    }
    __device__ size_t block_off(int b, int g, int idx, int e) const { return block_row(b, g, idx, e) * dim; }
    __device__ int max_ctx() const { return lmax; }
    // the last 16-row group of a slice may run past Lmax: clamp (such rows are masked)
    __device__ int row(int idx, int r) const { return min(idx * dec::BS + r, lmax - 1) - idx * dec::BS; }
    __device__ size_t safe_row0(int b, int g) const { return ((size_t)b * hkv + g) * lmax; }
    __device__ size_t safe_off(int b, int g) const { return safe_row0(b, g) * dim; }
    __device__ int safe_row(int r) const { return min(r, lmax - 1); }
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

// max / sum over all 64 lanes, result uniform: DPP butterflies inside 16-lane rows, row
// broadcasts across rows, then lane 63 holds the total
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

// Device-coherent exchange between workgroups without a cache write-back: relaxed
// agent-scope atomic stores and loads bypass the per-XCD L2's non-coherent state; a
// wait for every outstanding store orders them before the ticket that publishes them.
__device__ inline void coherent_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float coherent_load(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int coherent_load_int(const int *p)
{
    return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ inline int take_ticket(int *t)
{
    return __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void reset_ticket(int *t)
{
    __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------
// parameters
// ---------------------------------------------------------------------------------------
struct DecodeParams {
    const void *q;     // [B][Hq][dim]
    void *out;         // [B][Hq][dim]
    const void *kc;    // layer base of the K pool / cache
    const void *vc;
    void *kc_w;        // same as kc, writable (fused append)
    void *vc_w;
    const void *k_new; // [B][Hkv][dim] or NULL: new token written at position ctx-1
    const void *v_new;
    const void *ksc;   // int8 cache: layer base of the K / V scale pools (fp16 per row)
    const void *vsc;
    void *ksc_w;       // same, writable (fused append)
    void *vsc_w;
    const int *ctx_lens;
    int B;
    int hq;
    int hkv;
    int dim;           // head dim: 64 (fp32, fp16) or 128 (fp16, int8)
    int group;         // query heads per KV head (hq / hkv)
    int kv_i8;         // the cache holds int8 codes and fp16 row scales
    float scale_log2;
    int workers;       // fp32: max splits per pair
    float *part;       // partial results
    int *tickets;      // [B][Hkv], zero between calls
    int merge_polls;   // fp16: polls of a pair's ticket by its merging item before it falls
                       // back to the counted merge
};

// launchers (one translation unit per kernel family)
kvp_status launch_decode_f16(const DecodeParams &P, const PagedAddr &A, int group, int max_context,
                             hipStream_t st);
kvp_status launch_decode_f16(const DecodeParams &P, const ContigAddr &A, int group, int max_context,
                             hipStream_t st);
kvp_status launch_decode_f16_planned(const DecodeParams &P, const PagedAddr &A, int group,
                                     const void *d_image, const kvp_decode_plan &plan, hipStream_t st);
kvp_status launch_decode_f32(const DecodeParams &P, const PagedAddr &A, int group, hipStream_t st);
kvp_status launch_decode_f32(const DecodeParams &P, const ContigAddr &A, int group, hipStream_t st);

// workspace layout helpers (bytes), shared by the launchers and the size queries
size_t decode_f16_part_bytes(long long slots, int group, int dim);
int decode_f16_items_per_pair(int max_context, bool i8, int dim);
size_t decode_f32_part_bytes(int B, int hq, int max_splits);
int decode_f32_max_splits(int max_context);

} // namespace kvp
