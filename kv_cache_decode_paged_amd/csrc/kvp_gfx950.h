// kvp_gfx950.h -- gfx950 device helpers shared by the attention kernels (internal to the
// library): explicit memory-counter waits, LDS reads and writes of DMA-filled tiles as
// inline assembly, the transposing LDS read, and a cross-row maximum by lane swaps.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace kvp {

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N> __device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
    __builtin_amdgcn_s_waitcnt(imm);
}
// s_waitcnt lgkmcnt(0): every LDS access of the wave has completed
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

__device__ inline int lane_int(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// LDS reads of the DMA-filled ring, issued as inline assembly.  The compiler's wait
// insertion cannot tell these reads from reads of the slot a DMA is still filling, so for a
// plain LDS read it waits for every outstanding vector-memory operation -- the prefetched
// tiles included.  The ring is ordered by the explicit vmcnt waits instead; the results
// are tied to an explicit lgkmcnt(0) before use.
__device__ inline unsigned lds_addr(const char *p)
{
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
__device__ inline f16x8 lds_b128(const char *p)
{
    f16x8 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}
__device__ inline int lds_b32(const void *p)
{
    int r;
    asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(lds_addr((const char *)p)));
    return r;
}
__device__ inline f16x4 lds_tr16_b64(const char *p)
{
    f16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}
// the same reads at an LDS byte address plus an immediate offset (the instruction's own
// 16-bit offset field): one base register serves every read that differs by a constant
template <int OFF> __device__ inline f16x8 lds_b128_at(unsigned addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    f16x8 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF> __device__ inline f16x4 lds_tr16_b64_at(unsigned addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    f16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
// compile-time loop: f(integral_constant<int, I>) for I = B .. E - 1
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
__device__ inline void lds_store_b128(char *p, i32x4 v)
{
    asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ inline void lds_store_b64(char *p, u32x2 v)
{
    asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ inline void lds_store_b16(char *p, unsigned v)
{
    asm volatile("ds_write_b16 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ inline void lds_store_b8(char *p, unsigned v)
{
    asm volatile("ds_write_b8 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ inline u32x2 lds_b64(const char *p)
{
    u32x2 r;
    asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}
__device__ inline i32x4 lds_i128(const char *p)
{
    i32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}
__device__ inline unsigned lds_u16(const char *p)
{
    unsigned r;
    asm volatile("ds_read_u16 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}

// maximum of three as one v_max3_f32 (fmaxf would first quiet each operand, a
// canonicalising v_max per input; the scores here are never signalling NaNs)
__device__ inline float max3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// maximum of the 16 scores a lane holds for one MFMA column (four 4-row accumulators)
typedef float f32x4_ __attribute__((ext_vector_type(4)));
__device__ inline float max16(const f32x4_ (&s)[4])
{
    const float a = max3(s[0][0], s[0][1], s[0][2]), b = max3(s[0][3], s[1][0], s[1][1]);
    const float c = max3(s[1][2], s[1][3], s[2][0]), d = max3(s[2][1], s[2][2], s[2][3]);
    const float e = max3(s[3][0], s[3][1], s[3][2]);
    return max3(max3(a, b, c), max3(d, e, s[3][3]), a);
}
// the same for 8 scores (two 4-row accumulators)
__device__ inline float max8(const f32x4_ (&s)[2])
{
    const float a = max3(s[0][0], s[0][1], s[0][2]), b = max3(s[0][3], s[1][0], s[1][1]);
    return max3(a, b, max3(s[1][2], s[1][3], s[1][3]));
}
// maximum of the scores of KB 16-key blocks (KB = 2 or 4)
template <int KB> __device__ inline float max_scores(const f32x4_ (&s)[KB])
{
    static_assert(KB == 2 || KB == 4, "2 or 4 key blocks");
    if constexpr (KB == 4)
        return max16(s);
    else
        return max8(s);
}

// LDS slot of 16-byte chunk c of tile row r, for rows of HD fp16 values (128 or 256 bytes):
// an XOR swizzle under which 8 consecutive rows read at one chunk, and 4 consecutive rows
// read at two neighbouring chunks (the transposing reads of V), fall on distinct banks.
// 128-byte rows alternate between the two bank halves, so XOR with r mod 8 suffices;
// 256-byte rows all start at bank 0, so the XOR keeps the chunk's low bit and moves the
// other bits with r mod 8.
template <int HD> __device__ inline int swz(int c, int r)
{
    static_assert(HD == 64 || HD == 128, "rows of 64 or 128 values");
    return HD == 64 ? c ^ (r & 7) : c ^ ((r & 7) << 1);
}

// The same for int8 rows of HD bytes (64 or 128), read 8 bytes per lane by 16 lanes at one
// 8-byte piece of rows 8 (c / 4) + 4 h + c % 4 (c = 0..15; the score operand's row order):
// 64-byte rows fall on four bank quarters by r mod 4, and XOR with (r / 8) mod 4 spreads
// the four row groups; 128-byte rows fall on two bank halves by r mod 2, and the XOR with
// a 3-bit value of r / 2 and r / 8 spreads the eight rows of each half.
template <int HD> __device__ inline int swz8(int c, int r)
{
    static_assert(HD == 64 || HD == 128, "rows of 64 or 128 bytes");
    return HD == 64 ? c ^ ((r >> 3) & 3) : c ^ (((r >> 1) & 1) | ((r >> 2) & 6));
}

// max over lanes col, col + 16, col + 32, col + 48 (the k-groups of one MFMA column): swap
// odd and even 16-lane rows, then the two 32-lane halves, without an LDS round trip
__device__ inline float group_max(float x)
{
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float x1 = __builtin_bit_cast(float, (unsigned)a[0]), x2 = __builtin_bit_cast(float, (unsigned)a[1]);
    x = max3(x1, x2, x2);
    const unsigned w = __builtin_bit_cast(unsigned, x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    const float y1 = __builtin_bit_cast(float, (unsigned)b[0]), y2 = __builtin_bit_cast(float, (unsigned)b[1]);
    return max3(y1, y2, y2);
}

// growth of a column's maximum (log2 units) that moves its softmax reference
constexpr float RESCALE_LOG2 = 8.f;
// The per-lane pre-check of that growth compares raw scores (before the scale c > 0) with
// the level (mref + RESCALE_LOG2) / c lowered by a relative 2e-5, far more than the few ulps
// of rounding in that level, so it passes every tile the exact test (max * c > mref +
// RESCALE_LOG2) would move; a scale <= 0 disables it (the exact test runs on every tile).
__device__ inline float rescale_threshold(float mref, float c, float inv_c)
{
    if (!(c > 0.f) || mref == -INFINITY)
        return -INFINITY;
    const float x = (mref + RESCALE_LOG2) * inv_c;
    return x - fabsf(x) * 2e-5f;
}

// workgroup execution barrier without a memory fence: the callers order their LDS and
// LDS-DMA traffic with explicit counter waits, so the barrier must not also drain the
// prefetch still in flight (as the fenced __syncthreads would)
__device__ inline void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

} // namespace kvp
