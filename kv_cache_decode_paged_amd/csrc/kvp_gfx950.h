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
// tiles included.  The ring is ordered by the explicit vmcnt waits instead.
__device__ inline unsigned lds_addr(const char *p)
{
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
// Groups of LDS reads issued back to back and waited for inside one asm statement, so that
// every result is complete when the statement ends: the compiler never holds a register
// that a read in flight is still to write (it takes an asm output as written when the
// statement ends).  The outputs are early-clobber, so every address stays intact until
// the group's last read has been issued.  (Reads of LDS through the compiler would each wait
// for every load in flight, the LDS-DMA prefetch of the next tiles included.)
// K operands of a tile: k[kb][ks] = the 16 bytes at LDS byte address base[ks] + OFF + kb STRIDE
template <int KB, int KD, int OFF, int STRIDE>
__device__ inline void lds_read_k(f16x8 (&k)[KB][KD], const unsigned (&base)[KD])
{
    static_assert((KB == 4 && KD == 2) || (KB == 2 && KD == 4), "tile shapes of head dim 64 and 128");
    static_assert(OFF >= 0 && OFF + (KB - 1) * STRIDE < 65536, "ds offset field");
    if constexpr (KB == 4 && KD == 2)
        asm volatile(
            "ds_read_b128 %0, %8 offset:%10\n\t"
            "ds_read_b128 %1, %8 offset:%11\n\t"
            "ds_read_b128 %2, %8 offset:%12\n\t"
            "ds_read_b128 %3, %8 offset:%13\n\t"
            "ds_read_b128 %4, %9 offset:%10\n\t"
            "ds_read_b128 %5, %9 offset:%11\n\t"
            "ds_read_b128 %6, %9 offset:%12\n\t"
            "ds_read_b128 %7, %9 offset:%13\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0][0]), "=&v"(k[1][0]), "=&v"(k[2][0]), "=&v"(k[3][0]), "=&v"(k[0][1]), "=&v"(k[1][1]), "=&v"(k[2][1]), "=&v"(k[3][1])
            : "v"(base[0]), "v"(base[1]), "i"(OFF + 0 * STRIDE), "i"(OFF + 1 * STRIDE), "i"(OFF + 2 * STRIDE), "i"(OFF + 3 * STRIDE));
    if constexpr (KB == 2 && KD == 4)
        asm volatile(
            "ds_read_b128 %0, %8 offset:%12\n\t"
            "ds_read_b128 %1, %8 offset:%13\n\t"
            "ds_read_b128 %2, %9 offset:%12\n\t"
            "ds_read_b128 %3, %9 offset:%13\n\t"
            "ds_read_b128 %4, %10 offset:%12\n\t"
            "ds_read_b128 %5, %10 offset:%13\n\t"
            "ds_read_b128 %6, %11 offset:%12\n\t"
            "ds_read_b128 %7, %11 offset:%13\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0][0]), "=&v"(k[1][0]), "=&v"(k[0][1]), "=&v"(k[1][1]), "=&v"(k[0][2]), "=&v"(k[1][2]), "=&v"(k[0][3]), "=&v"(k[1][3])
            : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "i"(OFF + 0 * STRIDE), "i"(OFF + 1 * STRIDE));
}

// transposed V operands: v[ks][db][h] = ds_read_b64_tr_b16 at base[db] + OFF + (2 ks + h) STRIDE
template <int KS, int NDB, int OFF, int STRIDE>
__device__ inline void lds_read_vt(f16x4 (&v)[KS][NDB][2], const unsigned (&base)[NDB])
{
    static_assert((KS == 2 && NDB == 4) || (KS == 1 && NDB == 8), "tile shapes of head dim 64 and 128");
    static_assert(OFF >= 0 && OFF + (2 * KS - 1) * STRIDE < 65536, "ds offset field");
    if constexpr (KS == 2 && NDB == 4)
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
            "ds_read_b64_tr_b16 %1, %16 offset:%21\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:%22\n\t"
            "ds_read_b64_tr_b16 %3, %16 offset:%23\n\t"
            "ds_read_b64_tr_b16 %4, %17 offset:%20\n\t"
            "ds_read_b64_tr_b16 %5, %17 offset:%21\n\t"
            "ds_read_b64_tr_b16 %6, %17 offset:%22\n\t"
            "ds_read_b64_tr_b16 %7, %17 offset:%23\n\t"
            "ds_read_b64_tr_b16 %8, %18 offset:%20\n\t"
            "ds_read_b64_tr_b16 %9, %18 offset:%21\n\t"
            "ds_read_b64_tr_b16 %10, %18 offset:%22\n\t"
            "ds_read_b64_tr_b16 %11, %18 offset:%23\n\t"
            "ds_read_b64_tr_b16 %12, %19 offset:%20\n\t"
            "ds_read_b64_tr_b16 %13, %19 offset:%21\n\t"
            "ds_read_b64_tr_b16 %14, %19 offset:%22\n\t"
            "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1]), "=&v"(v[0][2][0]), "=&v"(v[0][2][1]), "=&v"(v[1][2][0]), "=&v"(v[1][2][1]), "=&v"(v[0][3][0]), "=&v"(v[0][3][1]), "=&v"(v[1][3][0]), "=&v"(v[1][3][1])
            : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "i"(OFF + 0 * STRIDE), "i"(OFF + 1 * STRIDE), "i"(OFF + 2 * STRIDE), "i"(OFF + 3 * STRIDE));
    if constexpr (KS == 1 && NDB == 8)
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
            "ds_read_b64_tr_b16 %1, %16 offset:%25\n\t"
            "ds_read_b64_tr_b16 %2, %17 offset:%24\n\t"
            "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
            "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
            "ds_read_b64_tr_b16 %5, %18 offset:%25\n\t"
            "ds_read_b64_tr_b16 %6, %19 offset:%24\n\t"
            "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
            "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
            "ds_read_b64_tr_b16 %9, %20 offset:%25\n\t"
            "ds_read_b64_tr_b16 %10, %21 offset:%24\n\t"
            "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
            "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
            "ds_read_b64_tr_b16 %13, %22 offset:%25\n\t"
            "ds_read_b64_tr_b16 %14, %23 offset:%24\n\t"
            "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]), "=&v"(v[0][2][0]), "=&v"(v[0][2][1]), "=&v"(v[0][3][0]), "=&v"(v[0][3][1]), "=&v"(v[0][4][0]), "=&v"(v[0][4][1]), "=&v"(v[0][5][0]), "=&v"(v[0][5][1]), "=&v"(v[0][6][0]), "=&v"(v[0][6][1]), "=&v"(v[0][7][0]), "=&v"(v[0][7][1])
            : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "v"(base[4]), "v"(base[5]), "v"(base[6]), "v"(base[7]), "i"(OFF + 0 * STRIDE), "i"(OFF + 1 * STRIDE));
}

// N reads of 8 bytes: r[i] at LDS byte address a[i]
template <int N> __device__ inline void lds_read_b64(u32x2 (&r)[N], const unsigned (&a)[N])
{
    static_assert(N == 10 || N == 12, "group sizes of the int8 tiles");
    if constexpr (N == 10)
        asm volatile(
            "ds_read_b64 %0, %10\n\t"
            "ds_read_b64 %1, %11\n\t"
            "ds_read_b64 %2, %12\n\t"
            "ds_read_b64 %3, %13\n\t"
            "ds_read_b64 %4, %14\n\t"
            "ds_read_b64 %5, %15\n\t"
            "ds_read_b64 %6, %16\n\t"
            "ds_read_b64 %7, %17\n\t"
            "ds_read_b64 %8, %18\n\t"
            "ds_read_b64 %9, %19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]));
    if constexpr (N == 12)
        asm volatile(
            "ds_read_b64 %0, %12\n\t"
            "ds_read_b64 %1, %13\n\t"
            "ds_read_b64 %2, %14\n\t"
            "ds_read_b64 %3, %15\n\t"
            "ds_read_b64 %4, %16\n\t"
            "ds_read_b64 %5, %17\n\t"
            "ds_read_b64 %6, %18\n\t"
            "ds_read_b64 %7, %19\n\t"
            "ds_read_b64 %8, %20\n\t"
            "ds_read_b64 %9, %21\n\t"
            "ds_read_b64 %10, %22\n\t"
            "ds_read_b64 %11, %23\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]));
}

// int8 V tile: r[i] = 8 bytes at a[i] (i < 8), s[j] = 16 bytes at b[j] (j < KS)
template <int KS> __device__ inline void lds_read_v_i8(u32x2 (&r)[8], i32x4 (&s)[KS], const unsigned (&a)[8],
                                                     const unsigned (&b)[KS])
{
    static_assert(KS == 1 || KS == 2, "k-steps of an int8 tile");
    if constexpr (KS == 1)
        asm volatile(
            "ds_read_b64 %0, %9\n\t"
            "ds_read_b64 %1, %10\n\t"
            "ds_read_b64 %2, %11\n\t"
            "ds_read_b64 %3, %12\n\t"
            "ds_read_b64 %4, %13\n\t"
            "ds_read_b64 %5, %14\n\t"
            "ds_read_b64 %6, %15\n\t"
            "ds_read_b64 %7, %16\n\t"
            "ds_read_b128 %8, %17\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(s[0])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(b[0]));
    if constexpr (KS == 2)
        asm volatile(
            "ds_read_b64 %0, %10\n\t"
            "ds_read_b64 %1, %11\n\t"
            "ds_read_b64 %2, %12\n\t"
            "ds_read_b64 %3, %13\n\t"
            "ds_read_b64 %4, %14\n\t"
            "ds_read_b64 %5, %15\n\t"
            "ds_read_b64 %6, %16\n\t"
            "ds_read_b64 %7, %17\n\t"
            "ds_read_b128 %8, %18\n\t"
            "ds_read_b128 %9, %19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(s[0]), "=&v"(s[1])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(b[0]), "v"(b[1]));
}

// N reads of 4 bytes: r[i] at LDS byte address a[i]
template <int N> __device__ inline void lds_read_b32(int (&r)[N], const unsigned (&a)[N])
{
    static_assert(N == 2 || N == 4, "group sizes of the block-id reads");
    if constexpr (N == 2)
        asm volatile(
            "ds_read_b32 %0, %2\n\t"
            "ds_read_b32 %1, %3\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1])
            : "v"(a[0]), "v"(a[1]));
    if constexpr (N == 4)
        asm volatile(
            "ds_read_b32 %0, %4\n\t"
            "ds_read_b32 %1, %5\n\t"
            "ds_read_b32 %2, %6\n\t"
            "ds_read_b32 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
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
