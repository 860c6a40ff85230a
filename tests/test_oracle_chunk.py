"""Pins of oracle.chunk_attention: several new query rows per request against its cache
(chunked prefill into a cached prefix, verification of gamma drafted tokens).

Pages: [CHAP] speculative-decoding section -- verifying gamma proposed tokens is one
forward pass over gamma positions; [KVES] prompt paragraph -- a stretch of known tokens is
computed in one pass under the causal mask and leaves one cached row per token.  The rows
are the last m positions of the context and each attends up to its own position.

Pinned by: the independent brute force on tiny shapes; m = 1 is the decode row (already
pinned); an empty prefix is the causal prefill of the chunk (already pinned); and any
split of a sequence into a prefix and a chunk reproduces the rows of the full causal
recompute, whatever the split point (a misaligned mask -- rows counted from the start of
the cache instead of from its end -- fails all but the last of these).
"""
import numpy as np
import pytest

import oracle
from oracle import brute

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _case(rng, B, Hq, Hkv, d, Lmax, ms=None):
    ctx = rng.integers(1, Lmax + 1, size=B)
    m = np.array([rng.integers(1, c + 1) for c in ctx]) if ms is None else np.minimum(np.array(ms), ctx)
    cu = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    q = _rand((int(cu[-1]), Hq, d), rng)
    K = _rand((B, Hkv, Lmax, d), rng)
    V = _rand((B, Hkv, Lmax, d), rng)
    return q, K, V, ctx.astype(np.int32), cu.astype(np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_chunk_matches_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    q, K, V, ctx, cu = _case(rng, B=2, Hq=4, Hkv=2, d=8, Lmax=9)
    got = oracle.chunk_attention(q, K, V, ctx, cu)
    want = np.array(brute.chunk_attention(q.tolist(), K.tolist(), V.tolist(), ctx.tolist(), cu.tolist(),
                                          1 / np.sqrt(8)))
    assert np.abs(got - want).max() <= 1e-13


def test_single_new_row_is_the_decode_row():
    rng = np.random.default_rng(7)
    q, K, V, ctx, cu = _case(rng, B=5, Hq=14, Hkv=2, d=64, Lmax=90, ms=[1] * 5)
    got = oracle.chunk_attention(q, K, V, ctx, cu)
    want = oracle.decode_gqa(q, K, V, ctx)
    assert np.abs(got - want).max() <= 1e-12


def test_empty_prefix_is_the_causal_prefill_of_the_chunk():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, d, Lmax = 3, 8, 2, 64, 40
    ctx = np.array([40, 17, 33], np.int32)
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)  # m = ctx: nothing cached before
    q = _rand((int(cu[-1]), Hq, d), rng)
    K = _rand((B, Hkv, Lmax, d), rng)
    V = _rand((B, Hkv, Lmax, d), rng)
    got = oracle.chunk_attention(q, K, V, ctx, cu)
    # the same rows packed on one token axis for the varlen prefill
    k = np.concatenate([K[b, :, :ctx[b]].transpose(1, 0, 2) for b in range(B)])
    v = np.concatenate([V[b, :, :ctx[b]].transpose(1, 0, 2) for b in range(B)])
    want = oracle.varlen_prefill(q, k, v, cu, causal=True)
    assert np.abs(got - want).max() <= 1e-12


@pytest.mark.parametrize("split", [0, 1, 13, 39])
def test_prefix_plus_chunk_equals_full_recompute(split):
    rng = np.random.default_rng(9)
    n, Hq, Hkv, d = 40, 4, 2, 64
    qf = _rand((n, Hq, d), rng)
    kf = _rand((n, Hkv, d), rng)
    vf = _rand((n, Hkv, d), rng)
    full = oracle.full_causal(qf, kf, vf)
    K = kf.transpose(1, 0, 2)[None]
    V = vf.transpose(1, 0, 2)[None]
    ctx = np.array([n], np.int32)
    cu = np.array([0, n - split], np.int32)
    got = oracle.chunk_attention(qf[split:], K, V, ctx, cu)
    assert np.abs(got - full[split:]).max() <= 1e-12
