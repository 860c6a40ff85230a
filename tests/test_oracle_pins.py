"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Nothing here compares the oracle with itself under the same code path: every check is a
value printed on the pages (tests/golden), a closed form, an invariant, an independent
library routine (scipy / torch SDPA in float64), or a second code path of the oracle that
a plausible mistake would make disagree (decode row vs full recompute, partial + merge vs
direct).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from conftest import golden, golden_kv

RNG = np.random.default_rng(42)
TOL = dict(rtol=1e-12, atol=1e-12)


def _sdpa64(q, k, v, causal, scale):
    """torch SDPA in float64 on the CPU: q [H, n, d], k/v [H, m, d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=causal, scale=scale)[0].numpy()


# --------------------------------------------------------------------------------------
# KV bytes per token and whole-cache sizes (golden values printed on the pages)
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("row", golden("kv_bytes.txt"))
def test_kv_bytes_per_token_matches_pages(row):
    L, hkv, d, b, want = map(int, row)
    assert oracle.kv_bytes_per_token(L, hkv, d, b) == want


@pytest.mark.parametrize("row", golden("kv_totals.txt"))
def test_kv_totals_match_pages(row):
    per_tok, tokens, want = map(int, row)
    assert per_tok * tokens == want


def test_kv_bytes_mha_is_seven_times_gqa():
    # 14 query heads over 2 KV heads: the GQA cache is exactly 1/7 of the MHA cache
    assert oracle.kv_bytes_per_token(24, 14, 64, 2) == 7 * oracle.kv_bytes_per_token(24, 2, 64, 2)


def test_kv_bytes_mini_gpt_cache():
    g = golden_kv("opcount_minigpt.txt")
    # mini-GPT: 2 layers, 4 heads of d_k 16 (d_model 64), fp64, full window of 64 tokens
    per_tok = oracle.kv_bytes_per_token(2, 4, 16, 8)
    assert per_tok * 64 == int(g["cache_kib_fp64"][0]) * 1024
    assert per_tok * 64 // 8 == int(g["cache_numbers"][0])


def test_kv_bytes_per_layer_tensor_shape():
    # neuralialabs chapter: per-layer K and V tensors of shape (1, 2, 295, 64) in fp16,
    # 24 layers, 3,624,960 bytes in total
    per_layer = 2 * (1 * 2 * 295 * 64) * 2
    assert per_layer * 24 == 3624960 == oracle.kv_bytes_per_token(24, 2, 64, 2) * 295


# --------------------------------------------------------------------------------------
# attention row: normalisation, special cases, closed forms, library routine
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("n,d", [(1, 64), (7, 4), (33, 64), (300, 64)])
def test_softmax_row_sums_to_one(n, d):
    q, K, V = RNG.standard_normal(d), RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    _, p = oracle.attention_row(q, K, V, return_p=True)
    assert abs(math.fsum(p) - 1.0) <= 1e-12
    assert (p >= 0).all()


def test_context_one_returns_value_exactly():
    q, K, V = RNG.standard_normal(64), RNG.standard_normal((1, 64)), RNG.standard_normal((1, 64))
    out = oracle.attention_row(q, K, V)
    assert np.array_equal(out, V[0])


def test_zero_query_is_mean_of_values():
    n, d = 37, 64
    K, V = RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    out = oracle.attention_row(np.zeros(d), K, V)
    np.testing.assert_allclose(out, V.mean(axis=0), **TOL)


def test_equal_keys_is_mean_of_values():
    n, d = 19, 64
    k = RNG.standard_normal(d)
    K, V = np.tile(k, (n, 1)), RNG.standard_normal((n, d))
    out = oracle.attention_row(RNG.standard_normal(d), K, V)
    np.testing.assert_allclose(out, V.mean(axis=0), **TOL)


def test_two_keys_closed_form():
    d = 8
    q, K, V = RNG.standard_normal(d), RNG.standard_normal((2, d)), RNG.standard_normal((2, d))
    s = K @ q / math.sqrt(d)
    sig = 1.0 / (1.0 + math.exp(-(s[1] - s[0])))
    np.testing.assert_allclose(oracle.attention_row(q, K, V), V[0] + (V[1] - V[0]) * sig, **TOL)


@pytest.mark.parametrize("n,alpha", [(5, 0.7), (64, 0.3), (40, -1.1)])
def test_geometric_weights_one_hot_values(n, alpha):
    # q = e_0, k_j = j*alpha*e_0 -> s_j = j*alpha/sqrt(d); V = identity rows -> out = p row
    d = 64
    q = np.zeros(d); q[0] = 1.0
    K = np.zeros((n, d)); K[:, 0] = alpha * np.arange(n)
    V = np.eye(n, d)
    r = math.exp(alpha / math.sqrt(d))
    want = np.array([r ** j for j in range(n)]) * (1 - r) / (1 - r ** n)
    out = oracle.attention_row(q, K, V)
    np.testing.assert_allclose(out[:n], want, **TOL)
    assert np.all(out[n:] == 0)


def test_scale_argument_and_default():
    d, n = 64, 20
    q, K, V = RNG.standard_normal(d), RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    np.testing.assert_allclose(oracle.attention_row(q, K, V),
                               oracle.attention_row(q, K, V, scale=0.125), rtol=0, atol=0)
    s = 0.37 * (K @ q)
    np.testing.assert_allclose(oracle.attention_row(q, K, V, scale=0.37),
                               scipy.special.softmax(s) @ V, **TOL)


@pytest.mark.parametrize("n", [1, 2, 17, 256, 1025])
def test_row_matches_library_softmax(n):
    d = 64
    q, K, V = RNG.standard_normal(d) * 3, RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    want = scipy.special.softmax(K @ q / 8.0) @ V
    np.testing.assert_allclose(oracle.attention_row(q, K, V), want, **TOL)


def test_row_is_stable_for_large_scores():
    # scores of several hundred: the max subtraction must keep exp finite
    d, n = 64, 50
    q, K, V = RNG.standard_normal(d) * 40, RNG.standard_normal((n, d)) * 40, RNG.standard_normal((n, d))
    out = oracle.attention_row(q, K, V)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, scipy.special.softmax(K @ q / 8.0) @ V, **TOL)


# --------------------------------------------------------------------------------------
# GQA head map
# --------------------------------------------------------------------------------------
def test_kv_head_map_contiguous_groups():
    assert [oracle.kv_head(h, 14, 2) for h in range(14)] == [0] * 7 + [1] * 7
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    assert [oracle.kv_head(h, 6, 1) for h in range(6)] == [0] * 6


def test_gqa_decode_equals_mha_on_repeated_kv_library():
    # xformers demo section 5: k/v broadcast over the query-head axis of each group.
    B, Hq, Hkv, d, L = 3, 14, 2, 64, 29
    q = RNG.standard_normal((B, Hq, d))
    K, V = RNG.standard_normal((B, Hkv, L, d)), RNG.standard_normal((B, Hkv, L, d))
    ctx = np.array([29, 1, 13])
    out = oracle.decode_gqa(q, K, V, ctx)
    Kr = np.repeat(K, Hq // Hkv, axis=1)
    Vr = np.repeat(V, Hq // Hkv, axis=1)
    for b in range(B):
        n = ctx[b]
        want = _sdpa64(q[b][:, None, :], Kr[b, :, :n], Vr[b, :, :n], False, 1 / 8)[:, 0]
        np.testing.assert_allclose(out[b], want, **TOL)


# --------------------------------------------------------------------------------------
# cached decode == full recompute (the single-head fp32 workload, in fp64 here)
# --------------------------------------------------------------------------------------
def test_cached_decode_equals_full_recompute_last_row():
    # neuralialabs chapter: the cache changes nothing in the output; gustavoai lesson:
    # cached and full-forward logits differ only by summation order (4e-15 in fp64).
    n_prompt, steps, d = 40, 48, 64
    n = n_prompt + steps
    q = RNG.standard_normal((n, 1, d))
    k = RNG.standard_normal((n, 1, d))
    v = RNG.standard_normal((n, 1, d))
    full = oracle.full_causal(q, k, v)
    K = k.transpose(1, 0, 2)[None]  # [1, 1, n, d]
    V = v.transpose(1, 0, 2)[None]
    for t in range(n_prompt, n):
        dec = oracle.decode_gqa(q[t][None], K, V, np.array([t + 1]))[0]
        np.testing.assert_allclose(dec, full[t], **TOL)
        # the row really is the cached decode, not a copy of an earlier row
        assert not np.allclose(dec, full[t - 1])


def test_full_causal_matches_library_sdpa():
    n, Hq, Hkv, d = 23, 4, 2, 64
    q = RNG.standard_normal((n, Hq, d))
    k, v = RNG.standard_normal((n, Hkv, d)), RNG.standard_normal((n, Hkv, d))
    out = oracle.full_causal(q, k, v)
    kr = np.repeat(k, Hq // Hkv, axis=1)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    want = _sdpa64(q.transpose(1, 0, 2).copy(), kr.transpose(1, 0, 2).copy(),
                   vr.transpose(1, 0, 2).copy(), True, 1 / 8).transpose(1, 0, 2)
    np.testing.assert_allclose(out, want, **TOL)


def test_full_causal_first_row_is_first_value():
    n, d = 9, 64
    q, k, v = (RNG.standard_normal((n, 1, d)) for _ in range(3))
    out = oracle.full_causal(q, k, v)
    assert np.array_equal(out[0, 0], v[0, 0])


def test_causality_future_rows_do_not_change_past():
    n, d = 16, 64
    q, k, v = (RNG.standard_normal((n, 2, d)) for _ in range(3))
    base = oracle.full_causal(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[10:] += 5.0
    v2[10:] -= 3.0
    pert = oracle.full_causal(q, k2, v2)
    assert np.array_equal(base[:10], pert[:10])
    assert not np.allclose(base[10:], pert[10:])


# --------------------------------------------------------------------------------------
# packed varlen prefill
# --------------------------------------------------------------------------------------
def _varlen_case(seqlens, Hq, Hkv, d=64):
    T = sum(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    return (RNG.standard_normal((T, Hq, d)), RNG.standard_normal((T, Hkv, d)),
            RNG.standard_normal((T, Hkv, d)), cu)


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_equals_per_segment_library(causal):
    seqlens = (37, 120, 8, 200)
    q, k, v, cu = _varlen_case(seqlens, 8, 8)
    out = oracle.varlen_prefill(q, k, v, cu, causal=causal)
    for s in range(len(seqlens)):
        a, e = cu[s], cu[s + 1]
        want = _sdpa64(q[a:e].transpose(1, 0, 2).copy(), k[a:e].transpose(1, 0, 2).copy(),
                       v[a:e].transpose(1, 0, 2).copy(), causal, 1 / 8).transpose(1, 0, 2)
        np.testing.assert_allclose(out[a:e], want, **TOL)


def test_varlen_causal_equals_full_causal_per_segment():
    seqlens = (5, 1, 12)
    q, k, v, cu = _varlen_case(seqlens, 4, 2)
    out = oracle.varlen_prefill(q, k, v, cu, causal=True)
    for s in range(len(seqlens)):
        a, e = cu[s], cu[s + 1]
        np.testing.assert_allclose(out[a:e], oracle.full_causal(q[a:e], k[a:e], v[a:e]), **TOL)


def test_varlen_block_diagonal_isolation():
    seqlens = (37, 120, 8, 200)
    q, k, v, cu = _varlen_case(seqlens, 8, 2)
    base = oracle.varlen_prefill(q, k, v, cu, causal=False)
    k2, v2 = k.copy(), v.copy()
    k2[cu[2]:cu[3]] *= -2.0
    v2[cu[2]:cu[3]] += 1.0
    pert = oracle.varlen_prefill(q, k2, v2, cu, causal=False)
    keep = np.r_[0:cu[2], cu[3]:cu[4]]
    assert np.array_equal(base[keep], pert[keep])
    assert not np.allclose(base[cu[2]:cu[3]], pert[cu[2]:cu[3]])


def test_varlen_gqa_bmghk_noncausal_library():
    # xformers demo section 5: B=2, M=256, 8 query heads over 2 KV heads, no mask
    B, M, Hq, Hkv, d = 2, 256, 8, 2, 64
    q, k, v, cu = _varlen_case((M,) * B, Hq, Hkv)
    out = oracle.varlen_prefill(q, k, v, cu, causal=False)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    for b in range(B):
        a, e = cu[b], cu[b + 1]
        want = _sdpa64(q[a:e].transpose(1, 0, 2).copy(), kr[a:e].transpose(1, 0, 2).copy(),
                       vr[a:e].transpose(1, 0, 2).copy(), False, 1 / 8).transpose(1, 0, 2)
        np.testing.assert_allclose(out[a:e], want, **TOL)
    # output in the (B, M, G, Hq/G, K) layout of the demo
    assert out.reshape(B, M, Hkv, Hq // Hkv, d).shape == (2, 256, 2, 4, 64)


# --------------------------------------------------------------------------------------
# block partials and their merge (online softmax rescale rule)
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("cuts", [[0, 300], [0, 1, 300], [0, 64, 128, 256, 300], [0, 299, 300],
                                  list(range(0, 301, 16)) + [300]])
def test_merge_of_partials_equals_direct(cuts):
    cuts = sorted(set(cuts))
    n, d = 300, 64
    q, K, V = RNG.standard_normal(d) * 2, RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    parts = [oracle.partial(q, K, V, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    ms = [p[0] for p in parts]
    ls = [p[1] for p in parts]
    os_ = np.stack([p[2] for p in parts])
    np.testing.assert_allclose(oracle.merge(ms, ls, os_), oracle.attention_row(q, K, V), **TOL)


def test_partial_closed_form_single_key():
    d = 16
    q, K, V = RNG.standard_normal(d), RNG.standard_normal((3, d)), RNG.standard_normal((3, d))
    m, l, o = oracle.partial(q, K, V, 1, 2)
    assert m == pytest.approx(float(K[1] @ q) / 4.0, rel=1e-15)
    assert l == 1.0
    assert np.array_equal(o, V[1])


def test_merge_rescale_with_far_apart_maxima():
    # one block dominates by ~200 in score: the other must be scaled by e^(m_i - M)
    d, n = 64, 40
    q = RNG.standard_normal(d)
    K = RNG.standard_normal((n, d))
    K[20:] += 30 * q / np.linalg.norm(q)
    V = RNG.standard_normal((n, d))
    parts = [oracle.partial(q, K, V, 0, 20), oracle.partial(q, K, V, 20, 40)]
    out = oracle.merge([p[0] for p in parts], [p[1] for p in parts], np.stack([p[2] for p in parts]))
    np.testing.assert_allclose(out, scipy.special.softmax(K @ q / 8.0) @ V, **TOL)
