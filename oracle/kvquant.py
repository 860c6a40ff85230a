"""Symmetric absmax quantization of cache rows -- TEST INFRASTRUCTURE ONLY (oracle).

Recipe (neuralialabs "Tornar a inferencia barata", quantization section: symmetric
quantization by the absolute maximum): with qmax = 2^(bits-1) - 1, a scale maps the
largest magnitude to qmax, each value is divided by the scale, rounded, clamped to
[-qmax-1, qmax] and stored as an integer together with the scale; the reconstruction
multiplies back.  The same section shrinks the scale's territory (one scale per output
row, then per group) to cut the error.

Applied here to the key/value cache (a reading: the page applies it to weights), one
scale per row -- one (token, KV head) row of d values of K, and separately of V -- with:
  * bits = 8, so codes lie in [-128, 127] and qmax = 127;
  * the scale computed as the fp32 quotient max|x| / 127 and stored as fp16 (rounded to
    nearest even); the codes are computed against that stored fp16 scale, so that
    reconstruction uses exactly the scale that quantized;
  * the division x / scale in fp32 and rounding half to even (torch.round's rule, which
    the page's listing uses);
  * a row of zeros (or one whose scale rounds to 0 in fp16) gets scale 0 and all-zero codes
    (the listing would divide by zero there).
Reconstruction is exact in fp64: code * scale.

Pinned by tests/test_oracle_kvquant.py against an exact rational brute force (the nearest
code to x / scale among all 256, ties to even), closed-form special cases and bounds, and
planted mutants.
"""
import numpy as np

BITS = 8


def qmax(bits=BITS):
    return 2 ** (bits - 1) - 1


def absmax_quantize_rows(x, bits=BITS):
    """x: array [..., d] (any float dtype; values are taken as fp32, as a cache row in fp16
    converts exactly).  Returns (codes int16 [..., d] in [-qmax-1, qmax], scales float16
    [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    q = np.float32(qmax(bits))
    absmax = np.max(np.abs(x32), axis=-1)
    scale16 = (absmax / q).astype(np.float16)          # fp32 quotient, rounded to fp16
    s32 = scale16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = x32 / s32                              # fp32 division
    codes = np.rint(ratio)                             # round half to even
    codes = np.clip(codes, -q - 1, q)
    codes = np.where(s32 > 0, codes, 0.0)
    return codes.astype(np.int16), scale16


def dequantize_rows(codes, scales):
    """codes [..., d], scales [...] -> float64 [..., d] = code * scale (exact in fp64)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def kv_bytes_per_token_int8(L, Hkv, d, scale_bytes=2):
    """Cache bytes per token with int8 codes and one fp16 scale per row: for K and V, in
    every layer and KV head, d one-byte codes plus one scale (the page's cache-size
    formula with one byte per element, plus the scales' bookkeeping)."""
    return 2 * L * Hkv * (d * 1 + scale_bytes)
