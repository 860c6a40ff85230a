"""Decode attention on the GPU against the fp64 oracle, paged vs contiguous identity,
special cases and the long-context split-K path."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, PagedStep, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32)


# ---------------------------------------------------------------------------------------
# single head, fp32: 40-token prompt then 48 decode steps; cached decode == full recompute
# ---------------------------------------------------------------------------------------
def test_single_head_fp32_decode_equals_full_recompute():
    need_gpu()
    say("single head fp32 40+48")
    q, k, v = W.single_head_sequence()
    n = q.shape[0]
    full = oracle.full_causal(to64(q), to64(k), to64(v))
    dev = "cuda"
    # contiguous cache [1, 1, 88, 64]
    kc = torch.zeros((1, 1, n, 64), dtype=torch.float32, device=dev)
    vc = torch.zeros_like(kc)
    # paged cache through a scrambled table
    pool = kvp.BlockPool(16)
    pool.set_free_order(W.free_list_permutation(16, 3).tolist())
    cache = kvp.PagedKVCache(1, 16, 1, 1, torch.float32, dev)
    cache.k_pool.fill_(float("nan"))
    cache.v_pool.fill_(float("nan"))
    seq = pool.alloc(0)
    worst = 0.0
    for t in range(n):
        kt, vt = k[t].to(dev)[None], v[t].to(dev)[None]  # [1, 1, 64]
        kvp.contiguous_kv_append(kc, vc, kt, vt, torch.tensor([t], dtype=torch.int32, device=dev))
        slot, cp = pool.append_slot(seq)
        assert cp is None
        kvp.kv_append(cache, 0, kt, vt, torch.tensor([slot], device=dev))
        if t < W.SINGLE_PROMPT:
            continue
        ctx = torch.tensor([t + 1], dtype=torch.int32, device=dev)
        qt = q[t].to(dev)[None]
        oc = kvp.contiguous_decode_attention(qt, kc, vc, ctx)
        table, _ = pool.export([seq], math.ceil(n / 16))
        op = kvp.paged_decode_attention(cache, 0, qt, table.to(dev), ctx)
        torch.cuda.synchronize()
        assert torch.equal(_bits(oc.cpu()), _bits(op.cpu())), f"step {t}: paged != contiguous"
        err = max_abs(to64(oc)[0], full[t])
        worst = max(worst, err)
        assert err <= TOL[torch.float32], f"step {t}: {err}"
    say("single head worst err", worst)


def test_single_head_page_count_steps():
    # the page's own run: 40 prompt tokens then 47 steps; only the last row is checked here
    need_gpu()
    q, k, v = W.single_head_sequence()
    n = W.SINGLE_PROMPT + 47
    full = oracle.full_causal(to64(q[:n]), to64(k[:n]), to64(v[:n]))
    kc = k[:n].transpose(0, 1)[None].contiguous().cuda()
    vc = v[:n].transpose(0, 1)[None].contiguous().cuda()
    out = kvp.contiguous_decode_attention(q[n - 1].cuda()[None], kc, vc,
                                          torch.tensor([n], dtype=torch.int32, device="cuda"))
    assert max_abs(to64(out)[0], full[n - 1]) <= 1e-5


# ---------------------------------------------------------------------------------------
# 24 layers, 14 q / 2 kv heads, fp16, batch 1, contexts 16 / 64 / 256 / 1024
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("C", [16, 64, 256, 1024])
def test_gqa_24_layers_batch1(C):
    need_gpu()
    say("24-layer batch-1 context", C)
    pb = W.uniform_batch(1, C)
    step = PagedStep(kvp, pb, layers=24, hq=14, hkv=2, dtype=torch.float16, seed=1000 + C)
    ws = kvp.make_workspace(14, 2, torch.float16, 1, step.max_blocks * 16)
    for l in range(24):
        q = step.q(l).cuda()
        op = kvp.paged_decode_attention(step.cache, l, q, step.table, step.ctx, workspace=ws)
        K, V = step.logical[l]
        oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
        torch.cuda.synchronize()
        assert torch.equal(_bits(op.cpu()), _bits(oc.cpu())), f"layer {l}: paged != contiguous"
        err = max_abs(to64(op), step.oracle(l))
        assert err <= TOL[torch.float16], f"layer {l}: {err}"


# ---------------------------------------------------------------------------------------
# paged batches with shared prefixes (copy-on-write on the step), all rows vs the oracle
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("B", [10, 50, 100])
def test_paged_batch_matches_oracle(B):
    need_gpu()
    pb = W.paged_batch(B)
    say("paged batch", B, "ctx", min(pb.ctx_before), max(pb.ctx_before))
    step = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=2000 + B)
    assert any(c < pb.prefix for c in pb.ctx_before) == (len(step.cow_pairs) > 0)
    for l in range(2):
        q = step.q(l).cuda()
        op = kvp.paged_decode_attention(step.cache, l, q, step.table, step.ctx)
        K, V = step.logical[l]
        oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
        torch.cuda.synchronize()
        assert torch.equal(_bits(op.cpu()), _bits(oc.cpu())), "paged != contiguous"
        err = max_abs(to64(op), step.oracle(l))
        say("paged batch", B, "layer", l, "max err", err)
        assert err <= TOL[torch.float16]


def test_paged_batch_full_size_b200():
    need_gpu()
    pb = W.paged_batch(200)
    say("paged batch 200 (24-layer pool, data in layers 0 and 23)")
    step = PagedStep(kvp, pb, layers=24, hq=14, hkv=2, dtype=torch.float16, seed=3000,
                     layers_with_data=[0, 23])
    for l in (0, 23):
        q = step.q(l).cuda()
        op = kvp.paged_decode_attention(step.cache, l, q, step.table, step.ctx)
        torch.cuda.synchronize()
        err = max_abs(to64(op), step.oracle(l))
        say("b200 layer", l, "max err", err)
        assert err <= TOL[torch.float16]


def test_ragged_edges_and_tile_boundaries():
    need_gpu()
    ctxs = [0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 1023, 1024, 1025, 4095, 4096, 4100, 8193]
    pb = W.PagedBatch(ctx_before=ctxs, group=list(range(len(ctxs))), prefix=0, group_size=1)
    say("ragged edges", ctxs)
    for dtype in (torch.float16, torch.float32):
        step = PagedStep(kvp, pb, layers=1, hq=7, hkv=1, dtype=dtype, seed=4000)
        q = step.q(0).cuda()
        op = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
        K, V = step.logical[0]
        oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
        torch.cuda.synchronize()
        assert torch.equal(_bits(op.cpu()), _bits(oc.cpu()))
        err = max_abs(to64(op), step.oracle(0))
        say("ragged", dtype, "max err", err)
        assert err <= TOL[dtype]


# groups 1..16 fill one block of 16 MFMA columns; 14 query heads on one KV head is the
# chapter's model as multi-query attention, 32 and 64 take two and four column blocks
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2), (6, 2), (8, 1), (12, 4), (16, 2), (18, 2), (14, 1),
                                    (16, 1), (32, 1), (64, 2)])
def test_head_groupings(hq, hkv):
    need_gpu()
    say("grouping", hq, hkv)
    pb = W.paged_batch(6, lo=1, hi=700, prefix=0, group_size=1, seed=31)
    step = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=torch.float16, seed=5000 + hq)
    q = step.q(0).cuda()
    op = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    K, V = step.logical[0]
    oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(op.cpu()), _bits(oc.cpu())), "paged != contiguous"
    err = max_abs(to64(op), step.oracle(0))
    say("grouping", hq, hkv, "max err", err)
    assert err <= TOL[torch.float16]


def test_groups_beyond_the_column_blocks_are_refused():
    need_gpu()
    pb = W.paged_batch(2, lo=10, hi=40, prefix=0, group_size=1, seed=32)
    step = PagedStep(kvp, pb, layers=1, hq=20, hkv=1, dtype=torch.float16, seed=5100)
    with pytest.raises(kvp.KvpError) as e:  # group 20: above 16 and not a multiple of 16
        kvp.paged_decode_attention(step.cache, 0, step.q(0).cuda(), step.table, step.ctx)
    assert e.value.status == kvp.KVP_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------------------
# special cases fixed by the definition
# ---------------------------------------------------------------------------------------
def test_values_all_one_give_exactly_one():
    need_gpu()
    B, L = 5, 777
    k = W.randn((B, 2, L, 64), 1).cuda()
    v = torch.ones_like(k)
    q = W.randn((B, 14, 64), 2).cuda()
    ctx = torch.tensor([1, 2, 300, 700, 777], dtype=torch.int32, device="cuda")
    out = kvp.contiguous_decode_attention(q, k, v, ctx)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.ones((B, 14, 64), dtype=torch.float16))


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_context_one_returns_first_value_bit_exact(dtype):
    need_gpu()
    k = W.randn((3, 2, 8, 64), 3, dtype).cuda()
    v = W.randn((3, 2, 8, 64), 4, dtype).cuda()
    q = W.randn((3, 14, 64), 5, dtype).cuda()
    ctx = torch.ones((3,), dtype=torch.int32, device="cuda")
    out = kvp.contiguous_decode_attention(q, k, v, ctx)
    torch.cuda.synchronize()
    want = v[:, :, 0].repeat_interleave(7, dim=1)
    assert torch.equal(_bits(out.cpu()), _bits(want.cpu()))


def test_zero_query_is_mean_of_values():
    need_gpu()
    L = 300
    k = W.randn((1, 2, L, 64), 6).cuda()
    v = W.randn((1, 2, L, 64), 7).cuda()
    q = torch.zeros((1, 14, 64), dtype=torch.float16, device="cuda")
    out = kvp.contiguous_decode_attention(q, k, v, torch.tensor([L], dtype=torch.int32, device="cuda"))
    want = to64(v)[0].mean(axis=1).repeat(7, axis=0)
    assert max_abs(to64(out)[0], want) <= 2e-3


def test_one_hot_values_give_probability_row():
    # v_j = e_j (j < 64): the output is the softmax row itself, so it sums to 1
    need_gpu()
    L = 64
    k = W.randn((1, 1, L, 64), 8).cuda()
    v = torch.eye(64, dtype=torch.float16).reshape(1, 1, L, 64).cuda()
    q = W.randn((1, 1, 64), 9).cuda()
    out = kvp.contiguous_decode_attention(q, k, v, torch.tensor([L], dtype=torch.int32, device="cuda"))
    _, p = oracle.attention_row(to64(q)[0, 0], to64(k)[0, 0], to64(v)[0, 0], return_p=True)
    got = to64(out)[0, 0]
    assert max_abs(got, p) <= 2e-3
    assert abs(got.sum() - 1.0) <= 64 * 2e-3


def test_rows_beyond_context_are_never_read():
    need_gpu()
    B, L = 4, 600
    k = W.randn((B, 2, L, 64), 10).cuda()
    v = W.randn((B, 2, L, 64), 11).cuda()
    q = W.randn((B, 14, 64), 12).cuda()
    ctx = torch.tensor([1, 100, 599, 257], dtype=torch.int32, device="cuda")
    base = kvp.contiguous_decode_attention(q, k, v, ctx)
    k2, v2 = k.clone(), v.clone()
    for b, c in enumerate([1, 100, 599, 257]):
        k2[b, :, c:] = float("nan")
        v2[b, :, c:] = float("inf")
    pert = kvp.contiguous_decode_attention(q, k2, v2, ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(base.cpu()), _bits(pert.cpu()))


def test_deterministic_repeat():
    need_gpu()
    pb = W.paged_batch(20, seed=77)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=torch.float16, seed=6000)
    q = step.q(0).cuda()
    a = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    b = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a.cpu()), _bits(b.cpu()))


def test_counted_merge_matches_polled_merge():
    """A split context is merged by the item holding its final blocks, which polls for the
    others' partials; with zero polls every pair takes the counted merge (the last item to
    finish merges from memory).  Both combine in slot order with the same arithmetic, so the
    outputs must be bit-identical."""
    need_gpu()
    pb = W.paged_batch(50, seed=78)
    say("polled vs counted merge, B", pb.batch)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=torch.float16, seed=6100)
    q = step.q(0).cuda()
    old = kvp.decode_merge_polls(1 << 14)
    try:
        a = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
        kvp.decode_merge_polls(0)
        b = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
        c = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    finally:
        kvp.decode_merge_polls(old)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a.cpu()), _bits(b.cpu()))
    assert torch.equal(_bits(b.cpu()), _bits(c.cpu()))
    err = max_abs(to64(a), step.oracle(0))
    assert err <= TOL[torch.float16]


def test_fused_append_matches_separate_append():
    need_gpu()
    pb = W.paged_batch(40, seed=91)
    say("fused append", pb.batch)
    # two identical caches; the step's new rows are appended by the fused call in one and
    # by kv_append in the other
    a = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=8000)
    b = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=8000)
    kn = W.randn((pb.batch, 2, 64), 8101).cuda()
    vn = W.randn((pb.batch, 2, 64), 8102).cuda()
    # overwrite the new-token slots of cache a with garbage: the fused call must rewrite them
    blk, row = a.new_slots // 16, a.new_slots % 16
    a.cache.k_pool[1][blk, :, row] = float("nan")
    a.cache.v_pool[1][blk, :, row] = float("nan")
    q = a.q(1).cuda()
    oa = kvp.paged_decode_append_attention(a.cache, 1, q, kn, vn, a.table, a.ctx)
    kvp.kv_append(b.cache, 1, kn, vn, b.new_slots)
    ob = kvp.paged_decode_attention(b.cache, 1, q, b.table, b.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa.cpu()), _bits(ob.cpu()))
    assert torch.equal(_bits(a.cache.k_pool[1].cpu()), _bits(b.cache.k_pool[1].cpu()))
    assert torch.equal(_bits(a.cache.v_pool[1].cpu()), _bits(b.cache.v_pool[1].cpu()))


# ---------------------------------------------------------------------------------------
# long context: batch 32 x 32,768 tokens, split-K, sampled rows vs the oracle
# ---------------------------------------------------------------------------------------
def test_long_context_split_k_sampled():
    need_gpu()
    B, C, hkv, hq = 32, 32768, 2, 14
    L = C + 1
    say("long context", B, "x", C)
    dev = "cuda"
    K = W.randn_device((B, hkv, L, 64), 9001, torch.float16, dev)
    V = W.randn_device((B, hkv, L, 64), 9002, torch.float16, dev)
    q = W.randn_device((B, hq, 64), 9003, torch.float16, dev)
    nb_per = math.ceil(L / 16)
    pool = kvp.BlockPool(B * nb_per)
    pool.set_free_order(W.free_list_permutation(B * nb_per, 9004).tolist())
    cache = kvp.PagedKVCache(1, B * nb_per, hq, hkv, torch.float16, dev)
    seqs = []
    for b in range(B):
        s = pool.alloc(0)
        sl, _ = pool.reserve(s, L)
        kvp.kv_append(cache, 0, K[b].transpose(0, 1).contiguous(), V[b].transpose(0, 1).contiguous(), sl.to(dev))
        seqs.append(s)
    table, ctx = pool.export(seqs, nb_per)
    out = kvp.paged_decode_attention(cache, 0, q, table.to(dev), ctx.to(dev))
    oc = kvp.contiguous_decode_attention(q, K, V, ctx.to(dev))
    old = kvp.decode_merge_polls(1 << 14)  # 65 parts per pair through the polled merge
    try:
        ocount = kvp.paged_decode_attention(cache, 0, q, table.to(dev), ctx.to(dev))
    finally:
        kvp.decode_merge_polls(old)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out.cpu()), _bits(oc.cpu()))
    assert torch.equal(_bits(out.cpu()), _bits(ocount.cpu()))
    # every request against the oracle, one request per host thread
    import concurrent.futures as cf
    rows = list(range(B))

    def one(b):
        return oracle.decode_gqa(to64(q[b:b + 1]), to64(K[b:b + 1]), to64(V[b:b + 1]), np.array([L]))[0]
    with cf.ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        want = np.stack(list(ex.map(one, rows)))
    err = max_abs(to64(out[rows]), want)
    say("long context max err", err)
    assert err <= TOL[torch.float16]
    # the planned decode with long items: 16 parts of up to 132 blocks per pair (one wave
    # each, 1024 in all), ids from the plan's id area; counted and polled merges agree
    plan, image = kvp.decode_plan_build(hq, hkv, table, ctx, B * nb_per, share_prefix=False, long_items=True)
    assert plan.n_ids == B * hkv * nb_per
    dp = kvp.upload_plan(plan, image)
    ws = kvp.make_plan_workspace(plan)
    olong = kvp.paged_decode_attention_planned(cache, 0, q, plan, dp, workspace=ws)
    old = kvp.decode_merge_polls(1 << 14)
    try:
        olong_p = kvp.paged_decode_attention_planned(cache, 0, q, plan, dp, workspace=ws)
    finally:
        kvp.decode_merge_polls(old)
    torch.cuda.synchronize()
    assert torch.equal(_bits(olong.cpu()), _bits(olong_p.cpu()))
    err = max_abs(to64(olong[rows]), want)
    say("long context, long items: items", plan.n_items, "max err", err)
    assert err <= TOL[torch.float16]
    assert (olong.float() - out.float()).abs().max().item() <= 2 * TOL[torch.float16]
