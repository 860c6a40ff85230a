"""Bit-exact data movement on the GPU: append, gather, copy-on-write block copies."""
import pytest
import torch

import workloads as W
from gpu_support import GPU, PagedStep, need_gpu, say

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_append_then_gather_is_bit_exact(dtype):
    need_gpu()
    pb = W.paged_batch(12, lo=1, hi=300, prefix=64, group_size=4, seed=7)
    say("append/gather", dtype, pb.ctx_before)
    step = PagedStep(kvp, pb, layers=3, hq=4, hkv=2, dtype=dtype, seed=11)
    for l in range(3):
        kg, vg = kvp.kv_gather(step.cache, l, step.table, step.ctx, step.lmax)
        torch.cuda.synchronize()
        K, V = step.logical[l]
        assert torch.equal(_bits(kg.cpu()), _bits(K)), f"layer {l} K"
        assert torch.equal(_bits(vg.cpu()), _bits(V)), f"layer {l} V"


def test_copy_on_write_keeps_parent_and_extends_child():
    need_gpu()
    say("cow block copy")
    dtype, hkv, layers = torch.float16, 2, 4
    pool = kvp.BlockPool(32)
    pool.set_free_order(W.free_list_permutation(32, 5).tolist())
    cache = kvp.PagedKVCache(layers, 32, 14, hkv, dtype)
    cache.k_pool.fill_(float("nan"))
    cache.v_pool.fill_(float("nan"))
    parent = pool.alloc(40)
    rows_k = [W.randn((40, hkv, 64), 100 + l) for l in range(layers)]
    rows_v = [W.randn((40, hkv, 64), 200 + l) for l in range(layers)]
    sl = pool.slots(parent, 0, 40).cuda()
    for l in range(layers):
        kvp.kv_append(cache, l, rows_k[l].cuda(), rows_v[l].cuda(), sl)
    child = pool.fork(parent)
    slot, cp = pool.append_slot(child)
    assert cp is not None and cp[0] == pool.table(parent)[2]
    kvp.kv_copy_blocks(cache, torch.tensor([cp], dtype=torch.int32, device="cuda"))
    newk = [W.randn((1, hkv, 64), 300 + l) for l in range(layers)]
    newv = [W.randn((1, hkv, 64), 400 + l) for l in range(layers)]
    for l in range(layers):
        kvp.kv_append(cache, l, newk[l].cuda(), newv[l].cuda(), torch.tensor([slot], device="cuda"))
    table, ctx = pool.export([parent, child], 4)
    table, ctx = table.cuda(), ctx.cuda()
    for l in range(layers):
        kg, vg = kvp.kv_gather(cache, l, table, ctx, 48)
        torch.cuda.synchronize()
        kg, vg = kg.cpu(), vg.cpu()
        want_k = rows_k[l].transpose(0, 1)
        want_v = rows_v[l].transpose(0, 1)
        assert torch.equal(_bits(kg[0, :, :40]), _bits(want_k))  # parent unchanged
        assert torch.equal(_bits(vg[0, :, :40]), _bits(want_v))
        assert torch.equal(_bits(kg[1, :, :40]), _bits(want_k))  # child = parent ...
        assert torch.equal(_bits(kg[1, :, 40]), _bits(newk[l][0]))  # ... + the new row
        assert torch.equal(_bits(vg[1, :, 40]), _bits(newv[l][0]))
    # the parent's own next append goes in place now (its block is private again)
    slot2, cp2 = pool.append_slot(parent)
    assert cp2 is None and slot2 == pool.table(parent)[2] * 16 + 8


def test_contiguous_append_writes_rows():
    need_gpu()
    say("contiguous append")
    B, hkv, lmax = 3, 2, 37
    kc = torch.zeros((B, hkv, lmax, 64), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    k = W.randn((B, hkv, 64), 1, torch.float32).cuda()
    v = W.randn((B, hkv, 64), 2, torch.float32).cuda()
    pos = torch.tensor([0, 36, 17], dtype=torch.int32, device="cuda")
    kvp.contiguous_kv_append(kc, vc, k, v, pos)
    torch.cuda.synchronize()
    for b, p in enumerate([0, 36, 17]):
        assert torch.equal(kc[b, :, p], k[b]) and torch.equal(vc[b, :, p], v[b])
    assert int((kc != 0).sum()) == int((k != 0).sum())


def test_append_skips_out_of_range_slots():
    need_gpu()
    say("append bounds")
    cache = kvp.PagedKVCache(1, 4, 2, 2, torch.float16)
    cache.k_pool.zero_()
    cache.v_pool.zero_()
    k = torch.ones((2, 2, 64), dtype=torch.float16, device="cuda")
    slots = torch.tensor([5, 4 * 16 + 3], dtype=torch.int64, device="cuda")  # 2nd beyond pool
    kvp.kv_append(cache, 0, k, k, slots)
    torch.cuda.synchronize()
    assert int(cache.k_pool.float().sum()) == 2 * 64
