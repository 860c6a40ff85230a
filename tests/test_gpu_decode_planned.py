"""Planned decode (decode_plan_build + paged_decode_attention_planned) on the GPU.

Without prefix sharing the plan reproduces paged_decode_attention's splits, so the outputs
must be bit-identical.  With sharing, requests forked from one prefix ([PAGED] paged-
attention article, SECTION 3) have the shared blocks read once per item for several
members; the attention is the same, so the result must match the fp64 oracle within the
fp16 tolerance."""
import pytest
import torch

import workloads as W
from gpu_support import GPU, TOL, PagedStep, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp


def _bits(t):
    return t.contiguous().view(torch.int16)


def _plan(step, share=True, long_items=False, fill=False):
    plan, image = kvp.decode_plan_build(step.hq, step.hkv, step.table.cpu(), step.ctx.cpu(), step.num_blocks,
                                        share_prefix=share, head_dim=step.head_dim, long_items=long_items,
                                        kv_dtype=step.dtype, fill=fill)
    return plan, kvp.upload_plan(plan, image)


def test_planned_without_sharing_is_bit_identical():
    need_gpu()
    pb = W.paged_batch(50, seed=77)
    say("planned, no sharing, B", pb.batch)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=torch.float16, seed=9100)
    plan, dp = _plan(step, share=False)
    assert plan.n_shared == 0
    q = step.q(0).cuda()
    o_plain = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    o_plan = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_plan.cpu()), _bits(o_plain.cpu()))


@pytest.mark.parametrize("dtype", ["float16", "int8"])
def test_planned_ragged_edges_are_bit_identical(dtype):
    """Contexts at and around tile and part boundaries, an empty one included (its item has no
    tile of its own to stream): a plan without sharing reproduces the unplanned call's splits,
    so the outputs are equal bit for bit, and they match the oracle."""
    need_gpu()
    ctxs = [0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1025, 2049]
    pb = W.PagedBatch(ctx_before=ctxs, group=list(range(len(ctxs))), prefix=0, group_size=1)
    say("planned ragged edges", dtype, ctxs)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=getattr(torch, dtype), seed=9150)
    plan, dp = _plan(step, share=False)
    q = step.q(0).cuda()
    o_plain = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    o_plan = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_plan.cpu()), _bits(o_plain.cpu()))
    err = max_abs(to64(o_plan), step.oracle(0))
    say("planned ragged", dtype, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("B", [10, 50, 100])
def test_planned_shared_prefix_matches_oracle(B):
    need_gpu()
    pb = W.paged_batch(B)
    say("planned shared prefix, B", B)
    step = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=9200 + B)
    plan, dp = _plan(step)
    assert plan.n_shared > 0
    ws = kvp.make_plan_workspace(plan)
    for l in range(2):
        q = step.q(l).cuda()
        o = kvp.paged_decode_attention_planned(step.cache, l, q, plan, dp, workspace=ws)
        torch.cuda.synchronize()
        err = max_abs(to64(o), step.oracle(l))
        say("planned B", B, "layer", l, "max err", err)
        assert err <= TOL[torch.float16]


def test_planned_full_size_b200():
    need_gpu()
    pb = W.paged_batch(200)
    say("planned batch 200 (24-layer pool, data in layers 0 and 23)")
    step = PagedStep(kvp, pb, layers=24, hq=14, hkv=2, dtype=torch.float16, seed=9300,
                     layers_with_data=[0, 23])
    plan, dp = _plan(step)
    ws = kvp.make_plan_workspace(plan)
    for l in (0, 23):
        q = step.q(l).cuda()
        o = kvp.paged_decode_attention_planned(step.cache, l, q, plan, dp, workspace=ws)
        o2 = kvp.paged_decode_attention_planned(step.cache, l, q, plan, dp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o.cpu()), _bits(o2.cpu())), "repeat with the same workspace differs"
        old = kvp.decode_merge_polls(1 << 14)  # split pairs merged by their last item, polling
        try:
            o3 = kvp.paged_decode_attention_planned(step.cache, l, q, plan, dp, workspace=ws)
        finally:
            kvp.decode_merge_polls(old)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o.cpu()), _bits(o3.cpu())), "polled merge differs from the counted merge"
        err = max_abs(to64(o), step.oracle(l))
        say("planned b200 layer", l, "max err", err)
        assert err <= TOL[torch.float16]


# shared items serve 16 / G members per column block (up to 4 blocks); groups above 16
# (multi-query with 32 or 64 heads) read every request privately
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (8, 1), (14, 2), (16, 2), (4, 4), (2, 2), (14, 1), (12, 1),
                                    (32, 1), (64, 1)])
def test_planned_head_groupings(hq, hkv):
    need_gpu()
    say("planned grouping", hq, hkv)
    pb = W.paged_batch(20, lo=1, hi=900, prefix=160, group_size=5, seed=41)
    step = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=torch.float16, seed=9400 + hq * 10 + hkv)
    plan, dp = _plan(step)
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp)
    torch.cuda.synchronize()
    err = max_abs(to64(o), step.oracle(0))
    say("planned grouping", hq, hkv, "shared items", plan.n_shared, "max err", err)
    assert err <= TOL[torch.float16]


def test_planned_fused_append_matches_separate_append():
    need_gpu()
    pb = W.paged_batch(40, seed=93)
    say("planned fused append", pb.batch)
    a = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=9500)
    b = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=9500)
    kn = W.randn((pb.batch, 2, 64), 9501).cuda()
    vn = W.randn((pb.batch, 2, 64), 9502).cuda()
    blk, row = a.new_slots // 16, a.new_slots % 16
    a.cache.k_pool[1][blk, :, row] = float("nan")
    a.cache.v_pool[1][blk, :, row] = float("nan")
    plan, dp = _plan(a)
    assert plan.n_shared > 0
    q = a.q(1).cuda()
    oa = kvp.paged_decode_attention_planned(a.cache, 1, q, plan, dp, k_new=kn, v_new=vn)
    kvp.kv_append(b.cache, 1, kn, vn, b.new_slots)
    ob = kvp.paged_decode_attention_planned(b.cache, 1, q, plan, dp)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa.cpu()), _bits(ob.cpu()))
    assert torch.equal(_bits(a.cache.k_pool[1].cpu()), _bits(b.cache.k_pool[1].cpu()))
    assert torch.equal(_bits(a.cache.v_pool[1].cpu()), _bits(b.cache.v_pool[1].cpu()))


def test_planned_rejects_mismatched_plan():
    need_gpu()
    pb = W.paged_batch(10, seed=95)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=torch.float16, seed=9600)
    plan, dp = _plan(step)
    q = step.q(0).cuda()
    with pytest.raises(ValueError):  # batch differs from the plan's
        kvp.paged_decode_attention_planned(step.cache, 0, q[:5], plan, dp)
    small = kvp.PagedKVCache(1, plan.num_blocks - 1, 14, 2, torch.float16, "cuda")
    with pytest.raises(kvp.KvpError):
        kvp.paged_decode_attention_planned(small, 0, q, plan, dp)


@pytest.mark.parametrize("dtype", [torch.float16, torch.int8])
def test_planned_long_items_match_oracle(dtype):
    # 200 requests of 3000-4000 tokens in sharing groups: about 75000 private blocks, more
    # than the resident waves x 32 blocks (1024 fp16 waves, 2048 int8 waves), so the private
    # ranges become long items (ids in the id area); the shared prefixes stay 32-block items
    need_gpu()
    pb = W.paged_batch(200, lo=3000, hi=4000, seed=61)
    say("planned long items", dtype, "B", pb.batch)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=dtype, seed=9700)
    plan, dp = _plan(step, long_items=True)
    assert plan.n_ids > 0 and plan.n_shared > 0
    ws = kvp.make_plan_workspace(plan)
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp, workspace=ws)
    o2 = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o.cpu()), _bits(o2.cpu())), "repeat with the same workspace differs"
    err = max_abs(to64(o), step.oracle(0))
    say("planned long items", dtype, "items", plan.n_items, "ids", plan.n_ids, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("B,dtype", [(1, torch.float16), (10, torch.float16), (100, torch.float16),
                                     (10, torch.int8)])
def test_planned_fill_matches_oracle(B, dtype):
    # KVP_PLAN_FILL: batches that leave resident waves idle are cut into parts of 8 to 28
    # blocks; the parts of a pair merge through the same rescale, so every request still
    # matches the oracle (a lone request: every 8 blocks its own item)
    need_gpu()
    pb = W.paged_batch(B) if B > 1 else W.uniform_batch(1, 1500)
    say("planned fill", dtype, "B", B)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=dtype, seed=9800 + B)
    plan, dp = _plan(step, fill=True)
    default, _ = _plan(step)
    assert plan.n_slots > default.n_slots  # shorter parts: more of them
    ws = kvp.make_plan_workspace(plan)
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp, workspace=ws)
    o2 = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o.cpu()), _bits(o2.cpu())), "repeat with the same workspace differs"
    err = max_abs(to64(o), step.oracle(0))
    say("planned fill B", B, dtype, "items", plan.n_items, "slots", plan.n_slots, "max err", err)
    assert err <= TOL[torch.float16]
