"""Pins of the absmax row quantizer of the oracle (oracle/kvquant.py) against things other
than itself: an exact rational brute force of the nearest code, closed forms (the row's
largest magnitude maps to +-127, exact multiples reconstruct exactly, ties go to even),
the reconstruction bound |x - code * scale| <= scale / 2, sign symmetry, the per-row
granularity, and the byte formula.  Planted mutants of the quantizer (on the CPU) must
each fail at least one pin.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvquant as KQ

QMAX = 127


def _rows(seed, n=64, d=64):
    """fp16 rows of mixed magnitudes (normal, tiny, large, sparse)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32)
    x[: n // 4] *= 1e-3
    x[n // 4: n // 2] *= 300.0
    x[n // 2: n // 2 + 4, 5:] = 0.0
    return x.astype(np.float16)


def _nearest_code_exact(x, s):
    """Nearest integer in [-128, 127] to x / s in exact rational arithmetic, ties to even;
    0 when s == 0."""
    if s == 0:
        return 0, False
    r = Fraction(float(x)) / Fraction(float(s))
    fl = r.numerator // r.denominator
    frac = r - fl
    if frac > Fraction(1, 2):
        c = fl + 1
    elif frac < Fraction(1, 2):
        c = fl
    else:
        c = fl if fl % 2 == 0 else fl + 1
    near_tie = abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 5)
    return max(-128, min(127, c)), near_tie


def _check_nearest(quantize, x):
    codes, scales = quantize(x)
    mism = 0
    ties = 0
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            c, near = _nearest_code_exact(x[i, j], scales[i])
            if near:
                ties += 1
                continue
            mism += int(codes[i, j] != c)
    return mism, ties


def _check_max_maps_to_qmax(quantize, x):
    codes, scales = quantize(x)
    bad = 0
    for i in range(x.shape[0]):
        j = int(np.argmax(np.abs(x[i].astype(np.float32))))
        if scales[i] > 0 and abs(int(codes[i, j])) != QMAX:
            bad += 1
    return bad


def _check_bound(quantize, x):
    codes, scales = quantize(x)
    rec = KQ.dequantize_rows(codes, scales)
    err = np.abs(rec - x.astype(np.float64))
    lim = scales.astype(np.float64)[:, None] / 2 * (1 + 2.0 ** -10)
    return int(np.sum(err > lim))


def test_codes_are_the_exact_nearest_codes():
    x = _rows(1)
    mism, ties = _check_nearest(KQ.absmax_quantize_rows, x)
    assert mism == 0
    assert ties < 4  # near-ties (within 1e-5 of .5) are skipped; random rows have almost none


def test_largest_magnitude_maps_to_qmax_in_every_row():
    x = _rows(2)
    assert _check_max_maps_to_qmax(KQ.absmax_quantize_rows, x) == 0
    codes, _ = KQ.absmax_quantize_rows(x)
    assert codes.min() >= -128 and codes.max() <= 127


def test_reconstruction_within_half_a_step():
    x = _rows(3)
    assert _check_bound(KQ.absmax_quantize_rows, x) == 0


def test_sign_symmetry():
    x = _rows(4)
    c1, s1 = KQ.absmax_quantize_rows(x)
    c2, s2 = KQ.absmax_quantize_rows(-x)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c2, -c1)


def test_zero_row_and_single_nonzero():
    x = np.zeros((2, 64), np.float16)
    x[1, 7] = -3.5
    c, s = KQ.absmax_quantize_rows(x)
    assert s[0] == 0 and not c[0].any()
    assert c[1, 7] == -127 and np.count_nonzero(c[1]) == 1
    assert s[1] == np.float16(np.float32(3.5) / np.float32(127))


def test_exact_multiples_reconstruct_exactly():
    # scale 2^-7 exactly: x = k 2^-7 with the row's maximum 127 2^-7
    k = np.arange(-127, 128, dtype=np.float32)[:64]
    k[0] = 127
    x = (k * 2.0 ** -7).astype(np.float16)[None]
    c, s = KQ.absmax_quantize_rows(x)
    assert s[0] == np.float16(2.0 ** -7)
    assert np.array_equal(c[0], k.astype(np.int16))
    assert np.array_equal(KQ.dequantize_rows(c, s)[0], x[0].astype(np.float64))


def _check_ties(quantize):
    """Exact half-way values (scale 2^-7) must round to the even code."""
    step = 2.0 ** -7
    vals = [127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5]
    x = (np.array(vals + [0] * 56, np.float32) * step).astype(np.float16)[None]
    c, _ = quantize(x)
    return int(np.sum(np.array(c[0, :8].tolist()) != np.array([127, 2, 4, -2, -4, 0, 0, 2])))


def test_ties_round_to_even():
    assert _check_ties(KQ.absmax_quantize_rows) == 0


def test_one_scale_per_row():
    x = np.ones((2, 64), np.float16)
    x[0] *= np.float16(0.01)
    x[1] *= np.float16(100.0)
    c, s = KQ.absmax_quantize_rows(x)
    assert (c == 127).all()
    assert s[0] < s[1]


def test_int8_bytes_per_token():
    # the page's fp16 formula, 2 L Hkv d 2 bytes, at one byte per code plus one 2-byte scale
    # per (layer, K/V, KV head) row; the 7B-class shape's 128 KB per token in fp16
    assert 2 * 32 * 8 * 128 * 2 == 131072
    assert KQ.kv_bytes_per_token_int8(32, 8, 128) == 131072 // 2 + 2 * 32 * 8 * 2
    assert KQ.kv_bytes_per_token_int8(24, 2, 64) == 6336


# ---- planted mutants: each must fail at least one pin ----
def _mut_half_away(x):
    x32 = np.asarray(x, np.float32)
    s = (np.max(np.abs(x32), -1) / np.float32(127)).astype(np.float16)
    r = x32 / s.astype(np.float32)[:, None]
    c = np.sign(r) * np.floor(np.abs(r) + 0.5)
    return np.clip(c, -128, 127).astype(np.int16), s


def _mut_qmax_255(x):
    x32 = np.asarray(x, np.float32)
    s = (np.max(np.abs(x32), -1) / np.float32(255)).astype(np.float16)
    c = np.rint(x32 / s.astype(np.float32)[:, None])
    return np.clip(c, -128, 127).astype(np.int16), s


def _mut_per_tensor(x):
    x32 = np.asarray(x, np.float32)
    s1 = np.float16(np.max(np.abs(x32)) / np.float32(127))
    s = np.full(x32.shape[0], s1, np.float16)
    c = np.rint(x32 / np.float32(s1))
    return np.clip(c, -128, 127).astype(np.int16), s


def _mut_fp32_scale_codes(x):
    # codes from the unrounded fp32 scale, stored scale rounded to fp16
    x32 = np.asarray(x, np.float32)
    s32 = np.max(np.abs(x32), -1) / np.float32(127)
    c = np.rint(x32 / s32[:, None])
    return np.clip(c, -128, 127).astype(np.int16), s32.astype(np.float16)


def _mut_truncate(x):
    x32 = np.asarray(x, np.float32)
    s = (np.max(np.abs(x32), -1) / np.float32(127)).astype(np.float16)
    c = np.trunc(x32 / s.astype(np.float32)[:, None])
    return np.clip(c, -128, 127).astype(np.int16), s


@pytest.mark.parametrize("mutant", [_mut_half_away, _mut_qmax_255, _mut_per_tensor, _mut_fp32_scale_codes,
                                    _mut_truncate])
def test_mutants_fail_a_pin(mutant):
    x = _rows(5)
    failed = (_check_nearest(mutant, x)[0] > 0 or _check_max_maps_to_qmax(mutant, x) > 0
              or _check_bound(mutant, x) > 0 or _check_ties(mutant) > 0)
    assert failed
