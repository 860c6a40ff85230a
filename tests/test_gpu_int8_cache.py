"""int8 paged cache on the GPU: rows quantized on append (symmetric absmax, one fp16 scale
per (token, KV head) row, [CHAP] quantization section applied to K and V), reconstructed in
the decode kernel.

The codes and scales the kernels write must equal the oracle's quantization of the same
fp16 rows bit for bit (oracle/kvquant.py); the attention must match the fp64 oracle run on
the oracle's reconstruction (code * scale) within the fp16 tolerance.  Never-written scale
rows hold NaN, so a read of one shows.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_support import GPU, TOL, PagedStep, max_abs, need_gpu, say, to64
from oracle import kvquant as KQ

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp

I8 = torch.int8


def _bits(t):
    return t.contiguous().view(torch.int16)


def _paged_rows(step, layer):
    """Codes [B, hkv, lmax, d] (gathered) and scales [B, hkv, lmax] of one layer, read back
    through the block table; positions at or beyond a context are zero."""
    kc, vc = kvp.kv_gather(step.cache, layer, step.table, step.ctx, step.lmax)
    table = step.table.cpu()
    B, hkv = step.pb.batch, step.hkv
    ks = torch.zeros((B, hkv, step.lmax), dtype=torch.float16)
    vs = torch.zeros_like(ks)
    ksp, vsp = step.cache.k_scale[layer].cpu(), step.cache.v_scale[layer].cpu()
    for b in range(B):
        n = step.ctx_host[b]
        j = torch.arange(n)
        blk = table[b, j // 16].long()
        ks[b, :, :n] = ksp[blk, :, j % 16].t()
        vs[b, :, :n] = vsp[blk, :, j % 16].t()
    return kc.cpu(), vc.cpu(), ks, vs


def _check_codes(step, layer):
    kc, vc, ks, vs = _paged_rows(step, layer)
    K, V = step.logical[layer]
    for got_c, got_s, X in ((kc, ks, K), (vc, vs, V)):
        want_c, want_s = KQ.absmax_quantize_rows(X.numpy())
        for b in range(step.pb.batch):
            n = step.ctx_host[b]
            assert np.array_equal(got_c[b, :, :n].numpy().astype(np.int16), want_c[b, :, :n]), f"codes of {b}"
            assert np.array_equal(got_s[b, :, :n].numpy().view(np.uint16), want_s[b, :, :n].view(np.uint16)), \
                f"scales of {b}"


@pytest.mark.parametrize("d", [64, 128])
def test_append_writes_the_oracle_codes_and_scales(d):
    need_gpu()
    pb = W.paged_batch(12, lo=1, hi=300, prefix=64, group_size=4, seed=7)
    say("int8 append d", d, pb.ctx_before)
    step = PagedStep(kvp, pb, layers=2, hq=8, hkv=2, dtype=I8, seed=31000 + d, head_dim=d)
    assert step.cow_pairs, "the batch should copy at least one shared block on write"
    for l in range(2):
        _check_codes(step, l)


@pytest.mark.parametrize("B", [10, 50])
def test_paged_decode_matches_oracle(B):
    need_gpu()
    pb = W.paged_batch(B)
    say("int8 paged decode B", B)
    step = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=I8, seed=31100 + B)
    for l in range(2):
        op = kvp.paged_decode_attention(step.cache, l, step.q(l).cuda(), step.table, step.ctx)
        torch.cuda.synchronize()
        err = max_abs(to64(op), step.oracle(l))
        say("int8 B", B, "layer", l, "max err", err)
        assert err <= TOL[torch.float16]


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (32, 32, 128), (8, 1, 64), (4, 4, 64), (16, 2, 128),
                                      (14, 1, 64), (32, 1, 64), (32, 1, 128)])
def test_head_shapes(hq, hkv, d):
    need_gpu()
    pb = W.paged_batch(6, lo=1, hi=900, prefix=0, group_size=1, seed=33)
    say("int8 shape", hq, hkv, d)
    step = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=I8, seed=31200 + hq + hkv + d, head_dim=d)
    op = kvp.paged_decode_attention(step.cache, 0, step.q(0).cuda(), step.table, step.ctx)
    torch.cuda.synchronize()
    assert max_abs(to64(op), step.oracle(0)) <= TOL[torch.float16]


@pytest.mark.parametrize("d", [64, 128])
def test_ragged_edges_and_tile_boundaries(d):
    need_gpu()
    ctxs = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 511, 512, 513, 1025, 4100, 8193]
    pb = W.PagedBatch(ctx_before=ctxs, group=list(range(len(ctxs))), prefix=0, group_size=1)
    say("int8 ragged d", d)
    step = PagedStep(kvp, pb, layers=1, hq=7, hkv=1, dtype=I8, seed=31300 + d, head_dim=d)
    op = kvp.paged_decode_attention(step.cache, 0, step.q(0).cuda(), step.table, step.ctx)
    torch.cuda.synchronize()
    err = max_abs(to64(op), step.oracle(0))
    say("int8 ragged max err", err)
    assert err <= TOL[torch.float16]


def _plan(step, share=True):
    plan, image = kvp.decode_plan_build(step.hq, step.hkv, step.table.cpu(), step.ctx.cpu(), step.num_blocks,
                                        share_prefix=share, head_dim=step.head_dim, kv_dtype=I8)
    return plan, kvp.upload_plan(plan, image)


def test_planned_decode():
    need_gpu()
    pb = W.paged_batch(50, seed=77)
    say("int8 planned", pb.batch)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=I8, seed=31400)
    q = step.q(0).cuda()
    o_plain = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    plan0, dp0 = _plan(step, share=False)
    o_plan0 = kvp.paged_decode_attention_planned(step.cache, 0, q, plan0, dp0)
    plan1, dp1 = _plan(step, share=True)
    assert plan1.n_shared > 0
    o_plan1 = kvp.paged_decode_attention_planned(step.cache, 0, q, plan1, dp1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_plan0.cpu()), _bits(o_plain.cpu()))
    err = max_abs(to64(o_plan1), step.oracle(0))
    say("int8 planned shared max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("d", [64, 128])
def test_fused_append_quantizes_like_kv_append(d):
    need_gpu()
    pb = W.paged_batch(24, seed=93)
    hq, hkv = (14, 2) if d == 64 else (32, 8)
    say("int8 fused append d", d)
    a = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=I8, seed=31500 + d, head_dim=d)
    b = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=I8, seed=31500 + d, head_dim=d)
    c = PagedStep(kvp, pb, layers=1, hq=hq, hkv=hkv, dtype=I8, seed=31500 + d, head_dim=d)
    kn = W.randn((pb.batch, hkv, d), 31501).cuda()
    vn = W.randn((pb.batch, hkv, d), 31502).cuda()
    for st in (a, c):  # the new rows are written by the kernels under test
        blk, row = st.new_slots // 16, st.new_slots % 16
        st.cache.k_pool[0][blk, :, row] = 0
        st.cache.k_scale[0][blk, :, row] = float("nan")
        st.cache.v_scale[0][blk, :, row] = float("nan")
    q = a.q(0).cuda()
    plan, dp = _plan(a)
    oa = kvp.paged_decode_attention_planned(a.cache, 0, q, plan, dp, k_new=kn, v_new=vn)
    kvp.kv_append(b.cache, 0, kn, vn, b.new_slots)
    ob = kvp.paged_decode_attention_planned(b.cache, 0, q, plan, dp)
    oc = kvp.paged_decode_append_attention(c.cache, 0, q, kn, vn, c.table, c.ctx)
    od = kvp.paged_decode_attention(b.cache, 0, q, b.table, b.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa.cpu()), _bits(ob.cpu()))
    assert torch.equal(_bits(oc.cpu()), _bits(od.cpu()))
    for st in (a, c):
        assert torch.equal(st.cache.k_pool.cpu(), b.cache.k_pool.cpu())
        assert torch.equal(st.cache.v_pool.cpu(), b.cache.v_pool.cpu())
        assert torch.equal(_bits(st.cache.k_scale.cpu()), _bits(b.cache.k_scale.cpu()))
        assert torch.equal(_bits(st.cache.v_scale.cpu()), _bits(b.cache.v_scale.cpu()))
    # and the appended rows are the oracle's quantization of kn / vn
    blk, row = b.new_slots.cpu() // 16, b.new_slots.cpu() % 16
    want_c, want_s = KQ.absmax_quantize_rows(kn.cpu().numpy())
    got_c = b.cache.k_pool[0].cpu()[blk, :, row]
    got_s = b.cache.k_scale[0].cpu()[blk, :, row]
    assert np.array_equal(got_c.numpy().astype(np.int16), want_c)
    assert np.array_equal(got_s.numpy().view(np.uint16), want_s.view(np.uint16))


def test_zero_and_extreme_rows():
    need_gpu()
    # rows of zeros (scale 0, codes 0) and rows with one large and many tiny values
    B, hkv, hq, d, n = 2, 2, 4, 64, 40
    pool = kvp.BlockPool(16)
    cache = kvp.PagedKVCache(1, 16, hq, hkv, I8, "cuda")
    K = W.randn((B, hkv, n, d), 31600)
    V = W.randn((B, hkv, n, d), 31601)
    K[0, :, 3] = 0
    V[0, :, 5] = 0
    K[1, 0, 7] = 1e-4
    K[1, 0, 7, 9] = 30.0
    V[1, 1, 2] = -2e-3
    V[1, 1, 2, 0] = 50.0
    seqs = []
    for b in range(B):
        s = pool.alloc(0)
        slots, _ = pool.reserve(s, n)
        kvp.kv_append(cache, 0, K[b].transpose(0, 1).contiguous().cuda(), V[b].transpose(0, 1).contiguous().cuda(),
                      slots.cuda())
        seqs.append(s)
    table, ctx = pool.export(seqs, math.ceil(n / 16))
    q = W.randn((B, hq, d), 31602)
    out = kvp.paged_decode_attention(cache, 0, q.cuda(), table.cuda(), ctx.cuda())
    torch.cuda.synchronize()
    import oracle
    Kd = PagedStep.dequantized(K)
    Vd = PagedStep.dequantized(V)
    want = oracle.decode_gqa(to64(q), Kd, Vd, np.array([n, n]))
    assert max_abs(to64(out), want) <= TOL[torch.float16]
    kc, vc = kvp.kv_gather(cache, 0, table.cuda(), ctx.cuda(), n)
    torch.cuda.synchronize()
    assert not kc.cpu()[0, :, 3].any() and not vc.cpu()[0, :, 5].any()
    assert kc.cpu()[1, 0, 7, 9].item() == 127


def test_planned_full_size_b200():
    # the batch-200 step of the benchmark over an int8 cache: 24-layer pool (data in layers 0
    # and 23), shared prefixes, the graph-style padded plan; all rows against the oracle
    need_gpu()
    pb = W.paged_batch(200)
    say("int8 planned batch 200 (24-layer pool, data in layers 0 and 23)")
    step = PagedStep(kvp, pb, layers=24, hq=14, hkv=2, dtype=I8, seed=31700, layers_with_data=[0, 23])
    plan0, _ = kvp.decode_plan_build(14, 2, step.table.cpu(), step.ctx.cpu(), step.num_blocks, share_prefix=True,
                                     kv_dtype=I8)
    plan, image = kvp.decode_plan_build(14, 2, step.table.cpu(), step.ctx.cpu(), step.num_blocks, share_prefix=True,
                                        pad_items=plan0.n_items + 256, kv_dtype=I8)
    dp = kvp.upload_plan(plan, image)
    ws = kvp.make_plan_workspace(plan)
    for l in (0, 23):
        q = step.q(l).cuda()
        o = kvp.paged_decode_attention_planned(step.cache, l, q, plan, dp, workspace=ws)
        o2 = kvp.paged_decode_attention(step.cache, l, q, step.table, step.ctx)
        torch.cuda.synchronize()
        err = max_abs(to64(o), step.oracle(l))
        say("int8 planned b200 layer", l, "max err", err)
        assert err <= TOL[torch.float16]
        assert max_abs(to64(o), to64(o2)) <= TOL[torch.float16]
