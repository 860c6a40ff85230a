"""Host-side byte accounting of bench.py: the unique and logical K/V tokens of one decode call
against a brute-force count, and the per-call byte formula at sizes past 2^31 bytes per
layer (the long-context batch at head dim 128), which must not wrap."""
import numpy as np

import bench


def _brute(table, ctx):
    seen = {}
    for i, c in enumerate(ctx):
        for t in range(int(c)):
            blk = int(table[i, t // 16])
            seen[blk] = max(seen.get(blk, 0), t % 16 + 1)
    return sum(seen.values()), int(sum(int(c) for c in ctx))


def test_unique_tokens_match_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(20):
        B = int(rng.integers(1, 9))
        ctx = rng.integers(0, 80, size=B).astype(np.int32)
        nb = max(1, int((ctx.max() + 15) // 16))
        # shared prefixes: rows draw their blocks from a small pool, so blocks repeat
        table = rng.integers(0, 6, size=(B, nb)).astype(np.int32)
        assert bench.unique_and_logical_tokens(table, ctx) == _brute(table, ctx)


def test_call_bytes_past_two_gib_per_layer():
    saved = (bench.HQ, bench.HKV, bench.D, bench.KV_TOKEN_LAYER_BYTES)
    try:
        bench.set_shape("32q8kv_d128")
        B, C = 32, 32790
        nb = (C + 15) // 16
        table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
        ctx = np.full(B, C, dtype=np.int32)
        got, uniq, logical = bench.decode_call_bytes(table, ctx, B)
        kv = B * C * 2 * 8 * 128 * 2           # K and V, 8 KV heads of 128 fp16 values
        qo = 2 * B * 32 * 128 * 2              # q in and out, 32 query heads
        assert uniq == logical == B * C
        assert got == kv + qo + 4 * B * nb + 4 * B
        assert got > 2 ** 32
    finally:
        bench.HQ, bench.HKV, bench.D, bench.KV_TOKEN_LAYER_BYTES = saved
