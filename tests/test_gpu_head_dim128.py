"""Head dim 128 on the GPU: the 7B-class head shape (8 KV heads of d = 128 with 32 query
heads, group 4), multi-head (32 / 32) and multi-query (hkv = 1) limits of the grouped
layout ([CHAP] grouped-query passage: GQA shares each key-value head among a group of
query heads; MHA and MQA are its two ends), through every kernel: cache appends and
copies, paged / contiguous / planned decode, the fused append, packed prefill and the
paged multi-row call.  Expected values come from the fp64 oracle; never-written cache rows
hold NaN, so a read of one shows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, ChunkStep, PagedStep, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp

D = 128


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32)


def _plan(step, share=True, long_items=False):
    plan, image = kvp.decode_plan_build(step.hq, step.hkv, step.table.cpu(), step.ctx.cpu(), step.num_blocks,
                                        share_prefix=share, head_dim=D, long_items=long_items,
                                        kv_dtype=step.dtype)
    assert plan.head_dim == D
    return plan, kvp.upload_plan(plan, image)


def test_append_gather_and_copy_on_write_are_bit_exact():
    need_gpu()
    pb = W.paged_batch(12, lo=1, hi=300, prefix=64, group_size=4, seed=7)
    say("d128 append/gather", pb.ctx_before)
    step = PagedStep(kvp, pb, layers=2, hq=8, hkv=2, dtype=torch.float16, seed=21, head_dim=D)
    assert step.cow_pairs, "the batch should copy at least one shared block on write"
    for l in range(2):
        kg, vg = kvp.kv_gather(step.cache, l, step.table, step.ctx, step.lmax)
        torch.cuda.synchronize()
        K, V = step.logical[l]
        assert torch.equal(_bits(kg.cpu()), _bits(K)), f"layer {l} K"
        assert torch.equal(_bits(vg.cpu()), _bits(V)), f"layer {l} V"


@pytest.mark.parametrize("hq,hkv", [(32, 8), (32, 32), (8, 1), (14, 2), (14, 1), (32, 1)])
def test_paged_decode_matches_oracle_and_contiguous(hq, hkv):
    need_gpu()
    pb = W.paged_batch(10)
    say("d128 paged decode", hq, hkv, "ctx", min(pb.ctx_before), max(pb.ctx_before))
    step = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=torch.float16, seed=22000 + hq + hkv, head_dim=D)
    q = step.q(0).cuda()
    op = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    K, V = step.logical[0]
    oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(op.cpu()), _bits(oc.cpu())), "paged != contiguous"
    err = max_abs(to64(op), step.oracle(0))
    say("d128", hq, hkv, "max err", err)
    assert err <= TOL[torch.float16]


def test_ragged_edges_and_tile_boundaries():
    need_gpu()
    # 32-token tiles at d = 128: edges at 31 / 32 / 33 as well as the block and split edges
    ctxs = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1025, 4095, 4100, 8193]
    pb = W.PagedBatch(ctx_before=ctxs, group=list(range(len(ctxs))), prefix=0, group_size=1)
    say("d128 ragged edges", ctxs)
    step = PagedStep(kvp, pb, layers=1, hq=4, hkv=1, dtype=torch.float16, seed=22100, head_dim=D)
    q = step.q(0).cuda()
    op = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    K, V = step.logical[0]
    oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(op.cpu()), _bits(oc.cpu()))
    err = max_abs(to64(op), step.oracle(0))
    say("d128 ragged max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("hq,hkv", [(32, 8), (14, 2)])
def test_planned_decode_bit_identical_without_sharing_and_oracle_with_sharing(hq, hkv):
    need_gpu()
    pb = W.paged_batch(24, seed=91)
    say("d128 planned", pb.batch, hq, hkv)
    step = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=torch.float16, seed=22200, head_dim=D)
    q = step.q(0).cuda()
    o_plain = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    plan0, dp0 = _plan(step, share=False)
    o_plan0 = kvp.paged_decode_attention_planned(step.cache, 0, q, plan0, dp0)
    plan1, dp1 = _plan(step, share=True)
    assert plan1.n_shared > 0
    o_plan1 = kvp.paged_decode_attention_planned(step.cache, 0, q, plan1, dp1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_plan0.cpu()), _bits(o_plain.cpu()))
    want = step.oracle(0)
    err = max_abs(to64(o_plan1), want)
    say("d128 planned shared max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("dtype", [torch.float16, torch.int8])
def test_planned_long_items_match_oracle(dtype):
    # 32q/8kv: batch 200 has about 57000 private blocks (fp16: more than 1024 waves x 32),
    # batch 80 of 3000-4000 tokens about 120000 (int8: more than 2048 x 32), so the private
    # ranges become long items of 32-token tiles (two blocks a tile); every 13th request is
    # compared with the oracle
    need_gpu()
    pb = W.paged_batch(200) if dtype == torch.float16 else W.paged_batch(80, lo=3000, hi=4000, seed=62)
    say("d128 planned long items", dtype)
    step = PagedStep(kvp, pb, layers=1, hq=32, hkv=8, dtype=dtype, seed=22300, head_dim=D)
    plan, dp = _plan(step, long_items=True)
    assert plan.n_ids > 0
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp, workspace=kvp.make_plan_workspace(plan))
    torch.cuda.synchronize()
    rows = list(range(0, pb.batch, 13))
    err = max_abs(to64(o[rows]), step.oracle(0, rows))
    say("d128 long items", dtype, "items", plan.n_items, "ids", plan.n_ids, "max err", err)
    assert err <= TOL[torch.float16]


def test_planned_fused_append_matches_separate_append():
    need_gpu()
    pb = W.paged_batch(16, seed=95)
    say("d128 planned fused append", pb.batch)
    a = PagedStep(kvp, pb, layers=1, hq=32, hkv=8, dtype=torch.float16, seed=22300, head_dim=D)
    b = PagedStep(kvp, pb, layers=1, hq=32, hkv=8, dtype=torch.float16, seed=22300, head_dim=D)
    kn = W.randn((pb.batch, 8, D), 22301).cuda()
    vn = W.randn((pb.batch, 8, D), 22302).cuda()
    blk, row = a.new_slots // 16, a.new_slots % 16
    a.cache.k_pool[0][blk, :, row] = float("nan")
    a.cache.v_pool[0][blk, :, row] = float("nan")
    plan, dp = _plan(a)
    q = a.q(0).cuda()
    oa = kvp.paged_decode_attention_planned(a.cache, 0, q, plan, dp, k_new=kn, v_new=vn)
    kvp.kv_append(b.cache, 0, kn, vn, b.new_slots)
    ob = kvp.paged_decode_attention_planned(b.cache, 0, q, plan, dp)
    # the unplanned fused call writes the same rows and gives the unplanned result
    c = PagedStep(kvp, pb, layers=1, hq=32, hkv=8, dtype=torch.float16, seed=22300, head_dim=D)
    oc = kvp.paged_decode_append_attention(c.cache, 0, q, kn, vn, c.table, c.ctx)
    od = kvp.paged_decode_attention(b.cache, 0, q, b.table, b.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa.cpu()), _bits(ob.cpu()))
    assert torch.equal(_bits(a.cache.k_pool.cpu()), _bits(b.cache.k_pool.cpu()))
    assert torch.equal(_bits(a.cache.v_pool.cpu()), _bits(b.cache.v_pool.cpu()))
    assert torch.equal(_bits(oc.cpu()), _bits(od.cpu()))
    assert torch.equal(_bits(c.cache.k_pool.cpu()), _bits(b.cache.k_pool.cpu()))


def test_values_all_one_give_exactly_one():
    need_gpu()
    B, L = 3, 300
    k = W.randn((B, 8, L, D), 22400).cuda()
    v = torch.ones((B, 8, L, D), dtype=torch.float16, device="cuda")
    q = W.randn((B, 32, D), 22401).cuda()
    ctx = torch.tensor([1, 77, 300], dtype=torch.int32, device="cuda")
    out = kvp.contiguous_decode_attention(q, k, v, ctx)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.ones((B, 32, D), dtype=torch.float16))


@pytest.mark.parametrize("seqlens", [(37, 120, 8, 200), (1,), (63, 64, 65), (129, 7, 300, 1, 64), (1000,)])
@pytest.mark.parametrize("causal", [True, False])
def test_packed_prefill_matches_oracle(seqlens, causal):
    need_gpu()
    say("d128 prefill", seqlens, "causal", causal)
    q, k, v, cu = W.varlen_inputs(seqlens, 32, 8, seed=22500, head_dim=D)
    out = kvp.varlen_causal_prefill(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(seqlens), causal=causal)
    torch.cuda.synchronize()
    want = oracle.varlen_prefill(to64(q), to64(k), to64(v), cu.numpy(), causal=causal)
    err = max_abs(to64(out), want)
    say("d128 prefill max err", err)
    assert err <= TOL[torch.float16]


def test_causal_prefill_never_reads_future_rows():
    need_gpu()
    # changing keys and values after row i must not change row i's output, bit for bit
    seqlens = (300,)
    q, k, v, cu = W.varlen_inputs(seqlens, 8, 2, seed=22600, head_dim=D)
    a = kvp.varlen_causal_prefill(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), 300, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[150:] = W.randn((150, 2, D), 22601)
    v2[150:] = W.randn((150, 2, D), 22602)
    b = kvp.varlen_causal_prefill(q.cuda(), k2.cuda(), v2.cuda(), cu.cuda(), 300, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a[:150].cpu()), _bits(b[:150].cpu()))


def test_paged_multi_row_call_matches_oracle():
    need_gpu()
    prefixes = [0, 17, 300, 511, 1000, 2047]
    chunks = [64, 100, 1, 257, 300, 5]
    say("d128 chunked prefill", list(zip(prefixes, chunks)))
    st = ChunkStep(kvp, prefixes, chunks, seed=22700, hq=32, hkv=8, head_dim=D)
    out = st.run()
    torch.cuda.synchronize()
    err = max_abs(to64(out), st.oracle())
    say("d128 chunked prefill max err", err)
    assert err <= TOL[torch.float16]


def test_paged_multi_row_call_after_shared_prefix_and_one_row_equals_decode():
    need_gpu()
    st = ChunkStep(kvp, [512, 512, 512, 200], [33, 1, 300, 7], seed=22800, hq=32, hkv=8,
                   share_groups=[[0, 1, 2]], head_dim=D)
    out = st.run()
    torch.cuda.synchronize()
    assert max_abs(to64(out), st.oracle()) <= TOL[torch.float16]
    one = ChunkStep(kvp, [15, 16, 200, 1023, 1500], [1] * 5, seed=22900, hq=32, hkv=8, head_dim=D)
    a = one.run()
    b = kvp.paged_decode_attention(one.cache, 0, one.q.cuda(), one.table, one.ctxd)
    torch.cuda.synchronize()
    assert max_abs(to64(a), to64(b)) <= TOL[torch.float16]
    assert max_abs(to64(a), one.oracle()) <= TOL[torch.float16]


def test_long_context_split_sampled():
    need_gpu()
    # one 32k-token context per request: 64 parts merged per (request, KV head)
    B, hq, hkv, L = 2, 32, 8, 32768
    say("d128 long context", B, L)
    dev = "cuda"
    K = W.randn_device((B, hkv, L, D), 23000, torch.float16, dev)
    V = W.randn_device((B, hkv, L, D), 23001, torch.float16, dev)
    q = W.randn((B, hq, D), 23002).to(dev)
    ctx = torch.tensor([L, L - 1000], dtype=torch.int32, device=dev)
    out = kvp.contiguous_decode_attention(q, K, V, ctx)
    torch.cuda.synchronize()
    got = to64(out)
    for b, h in ((0, 0), (0, 31), (1, 5), (1, 17)):
        g = h // (hq // hkv)
        n = int(ctx[b])
        want = oracle.attention_row(to64(q[b, h]), to64(K[b, g, :n]), to64(V[b, g, :n]))
        assert max_abs(got[b, h], want) <= TOL[torch.float16]
