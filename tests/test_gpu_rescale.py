"""The online-softmax rescale on the GPU: inputs whose scores make every kernel move its
per-row reference maximum in the middle of a row, and merge split partials whose maxima
lie tens of log2 units apart (chatgpz.de "Aufmerksamkeit", FlashAttention post: block
softmaxes are combined by rescaling each with e^(block max - global max)).

The shapes (tests/gpu_support.ScoreShaper): keys ramped along the context (gently, steeply,
and mirrored), one late dominant key, and queries scaled by 40.  Every path -- unplanned
paged decode (counted and polled merges), planned decode with shared prefixes, planned
long items, the int8 cache, packed varlen prefill and several rows against the paged cache
-- is compared with the fp64 oracle at the fp16 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, ChunkStep, PagedStep, ScoreShaper, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp

KINDS = ScoreShaper.KINDS


def _bits(t):
    return t.contiguous().view(torch.int16)


def _batch():
    # 6 requests of 1500..2100 tokens (3 to 5 split parts of 512 tokens), groups of 3 forked
    # from a 512-token prefix
    return W.paged_batch(6, lo=1500, hi=2100, prefix=512, group_size=3, seed=314)


@pytest.mark.parametrize("kind", KINDS)
def test_unplanned_decode_rescale(kind):
    need_gpu()
    say("rescale: unplanned decode", kind)
    step = PagedStep(kvp, _batch(), layers=1, hq=14, hkv=2, dtype=torch.float16, seed=7100,
                     shaper=ScoreShaper(kind))
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    K, V = step.logical[0]
    oc = kvp.contiguous_decode_attention(q, K.cuda(), V.cuda(), step.ctx)
    old = kvp.decode_merge_polls(1 << 14)  # the polled merge of the same splits
    try:
        op = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    finally:
        kvp.decode_merge_polls(old)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o.cpu()), _bits(oc.cpu())), "paged != contiguous"
    assert torch.equal(_bits(o.cpu()), _bits(op.cpu())), "polled merge != counted merge"
    err = max_abs(to64(o), step.oracle(0))
    say("rescale: unplanned", kind, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("kind", KINDS)
def test_planned_shared_decode_rescale(kind):
    need_gpu()
    say("rescale: planned shared decode", kind)
    step = PagedStep(kvp, _batch(), layers=1, hq=14, hkv=2, dtype=torch.float16, seed=7200,
                     shaper=ScoreShaper(kind))
    plan, image = kvp.decode_plan_build(14, 2, step.table.cpu(), step.ctx.cpu(), step.num_blocks)
    assert plan.n_shared > 0
    dp = kvp.upload_plan(plan, image)
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp)
    torch.cuda.synchronize()
    err = max_abs(to64(o), step.oracle(0))
    say("rescale: planned shared", kind, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("kind", ["steep", "big_q"])
def test_planned_long_items_rescale(kind):
    # 200 requests of 3000..4000 tokens: long private items of up to ~90 blocks (22 tiles),
    # so the steep ramp moves the reference many times inside one item
    need_gpu()
    pb = W.paged_batch(200, lo=3000, hi=4000, seed=62)
    say("rescale: long items", kind)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=torch.float16, seed=7300, shaper=ScoreShaper(kind))
    plan, image = kvp.decode_plan_build(14, 2, step.table.cpu(), step.ctx.cpu(), step.num_blocks, long_items=True)
    assert plan.n_ids > 0
    dp = kvp.upload_plan(plan, image)
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, dp)
    torch.cuda.synchronize()
    rows = list(range(0, 200, 7))
    err = max_abs(to64(o[rows]), step.oracle(0, rows))
    say("rescale: long items", kind, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("kind", ["ramp_up", "steep", "late_peak", "big_q"])
def test_int8_decode_rescale(kind):
    need_gpu()
    say("rescale: int8 decode", kind)
    step = PagedStep(kvp, _batch(), layers=1, hq=14, hkv=2, dtype=torch.int8, seed=7400,
                     shaper=ScoreShaper(kind))
    q = step.q(0).cuda()
    o = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    plan, image = kvp.decode_plan_build(14, 2, step.table.cpu(), step.ctx.cpu(), step.num_blocks,
                                        kv_dtype=torch.int8)
    op = kvp.paged_decode_attention_planned(step.cache, 0, q, plan, kvp.upload_plan(plan, image))
    torch.cuda.synchronize()
    want = step.oracle(0)
    err = max(max_abs(to64(o), want), max_abs(to64(op), want))
    say("rescale: int8", kind, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kind", KINDS)
def test_varlen_prefill_rescale(kind, causal):
    need_gpu()
    say("rescale: varlen prefill", kind, "causal", causal)
    seqlens = (1000, 300, 2048)
    q, k, v, cu = W.varlen_inputs(seqlens, 8, 2, seed=7500)
    sh = ScoreShaper(kind)
    q = sh.query(q)
    for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()):
        # positions counted from each segment's start; the peak 3 rows before its end
        ks, vs = sh.keys(k[a:b].transpose(0, 1), v[a:b].transpose(0, 1), 0, b - a - 3)
        k[a:b], v[a:b] = ks.transpose(0, 1), vs.transpose(0, 1)
    out = kvp.varlen_causal_prefill(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(seqlens), causal=causal)
    torch.cuda.synchronize()
    want = oracle.varlen_prefill(to64(q), to64(k), to64(v), cu.numpy(), causal=causal)
    err = max_abs(to64(out), want)
    say("rescale: varlen", kind, causal, "max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("kind", KINDS)
def test_paged_prefill_rescale(kind):
    need_gpu()
    say("rescale: rows against the paged cache", kind)
    # a chunk after a long prefix, a short chunk, and two requests sharing a prefix
    st = ChunkStep(kvp, [1500, 600, 1024, 1024], [300, 100, 200, 64], seed=7600, share_groups=[[2, 3]],
                   shaper=ScoreShaper(kind))
    out = st.run()
    torch.cuda.synchronize()
    err = max_abs(to64(out), st.oracle())
    say("rescale: paged prefill", kind, "max err", err)
    assert err <= TOL[torch.float16]
