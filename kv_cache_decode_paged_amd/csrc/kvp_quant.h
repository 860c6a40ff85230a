// kvp_quant.h -- symmetric absmax quantization of one cache row into int8 codes and an
// fp16 scale, for the append kernel and the decode kernel's fused append (internal).
//
//   neuralialabs "Tornar a inferencia barata", quantization section: with qmax =
//   2^(bits-1) - 1 the scale maps the largest magnitude to qmax; values are divided by the
//   scale, rounded, clamped to [-qmax-1, qmax] and stored with the scale; the
//   reconstruction multiplies back.  Applied per (token, KV head) row of K and of V, bits 8.
//
// The scale is the fp32 quotient max|x| / 127 rounded to fp16; the codes divide by that
// stored scale in fp32 (correctly rounded division) and round half to even; a zero scale
// gives zero codes.  Inputs are finite.
#pragma once

#include <hip/hip_runtime.h>

namespace kvp {

typedef _Float16 qf16;
typedef qf16 qf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One row is held by W consecutive lanes (an aligned group of a wave), 8 values each.
// Every lane of the group returns the row's scale and its own 8 codes, packed little-endian
// (code i in byte i).  All lanes of the wave must call it (the maximum is exchanged).
template <int W>
__device__ inline qf16 quantize_row_piece(const qf16x8 &x, u32x2 &codes)
{
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "power-of-two lane group");
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        a = fmaxf(a, fabsf((float)x[i]));
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1)
        a = fmaxf(a, __shfl_xor(a, m, 64));
    const qf16 s16 = (qf16)(a / 127.0f);
    const float s = (float)s16;
    unsigned lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q = s > 0.f ? __builtin_rintf((float)x[i] / s) : 0.f;
        q = fminf(fmaxf(q, -128.f), 127.f);
        const unsigned b = (unsigned)((int)q & 0xff);
        if (i < 4)
            lo |= b << (8 * i);
        else
            hi |= b << (8 * (i - 4));
    }
    codes = u32x2{lo, hi};
    return s16;
}

} // namespace kvp
