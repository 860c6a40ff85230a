"""The C oracle against the independent pure-Python brute force on tiny shapes (CPU)."""
import itertools

import numpy as np
import pytest

import oracle
from oracle import brute

TOL = dict(rtol=1e-12, atol=1e-12)


def _cases():
    for B, (Hq, Hkv), n, d in itertools.product((1, 2), ((1, 1), (2, 1), (4, 2), (4, 4)),
                                                (1, 2, 5, 9), (4, 8, 64)):
        yield B, Hq, Hkv, n, d


@pytest.mark.parametrize("B,Hq,Hkv,n,d", list(_cases()))
def test_decode_matches_brute(B, Hq, Hkv, n, d):
    rng = np.random.default_rng(B * 1000 + Hq * 100 + n * 10 + d)
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    ctx = np.array([n - (b % n) for b in range(B)], dtype=np.int32)  # ragged
    scale = 1 / np.sqrt(d)
    got = oracle.decode_gqa(q, K, V, ctx, scale)
    want = np.array(brute.decode_gqa(q.tolist(), K.tolist(), V.tolist(), ctx.tolist(), scale))
    np.testing.assert_allclose(got, want, **TOL)


@pytest.mark.parametrize("seqlens", [(1,), (3, 1, 4), (9, 2), (5, 5, 5)])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (4, 1)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [4, 64])
def test_varlen_matches_brute(seqlens, Hq, Hkv, causal, d):
    rng = np.random.default_rng(sum(seqlens) * 7 + Hq + d)
    T = sum(seqlens)
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    scale = 1 / np.sqrt(d)
    got = oracle.varlen_prefill(q, k, v, cu, causal, scale)
    want = np.array(brute.varlen_prefill(q.tolist(), k.tolist(), v.tolist(), cu.tolist(), causal, scale))
    np.testing.assert_allclose(got, want, **TOL)


@pytest.mark.parametrize("n,d", [(1, 4), (6, 8), (9, 64)])
def test_full_causal_matches_brute(n, d):
    rng = np.random.default_rng(n + d)
    q, k, v = (rng.standard_normal((n, 2, d)) for _ in range(3))
    scale = 1 / np.sqrt(d)
    got = oracle.full_causal(q, k, v, scale)
    want = np.array(brute.varlen_prefill(q.tolist(), k.tolist(), v.tolist(), [0, n], True, scale))
    np.testing.assert_allclose(got, want, **TOL)
