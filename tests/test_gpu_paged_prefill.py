"""Several new query rows per request against the paged cache (paged_prefill_attention) on
the GPU, against the fp64 oracle (oracle.chunk_attention).

The rows of request b are the last m_b of its ctx_b positions and row i attends to
positions 0 .. ctx_b - m_b + i: a chunk of a prompt prefilled into an existing prefix, or
the verification pass over gamma drafted tokens ([CHAP] speculative-decoding section: one
forward pass over gamma positions).  Prefixes may be shared between requests forked from
one prompt ([PAGED] SECTION 3).  Never-written cache rows hold NaN, so a read of one shows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, ChunkStep, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp

def test_chunked_prefill_into_prefixes():
    need_gpu()
    prefixes = [0, 17, 300, 511, 1000, 2047]
    chunks = [64, 100, 1, 257, 300, 5]
    say("chunked prefill", list(zip(prefixes, chunks)))
    st = ChunkStep(kvp, prefixes, chunks, seed=12000)
    out = st.run()
    torch.cuda.synchronize()
    err = max_abs(to64(out), st.oracle())
    say("chunked prefill max err", err)
    assert err <= TOL[torch.float16]


def test_draft_verification_rows():
    need_gpu()
    rng = np.random.default_rng(5)
    prefixes = [int(x) for x in rng.integers(100, 2000, size=32)]
    say("verification of 4 drafts + 1, B", len(prefixes))
    st = ChunkStep(kvp, prefixes, [5] * 32, seed=12100)
    out = st.run()
    torch.cuda.synchronize()
    err = max_abs(to64(out), st.oracle())
    say("verification max err", err)
    assert err <= TOL[torch.float16]


def test_chunks_after_a_shared_prefix():
    need_gpu()
    prefixes = [512, 512, 512, 200, 200]
    chunks = [33, 1, 300, 64, 7]
    say("chunks after shared prefixes")
    st = ChunkStep(kvp, prefixes, chunks, seed=12200, share_groups=[[0, 1, 2], [3, 4]])
    # the forked requests really read the leader's physical prefix blocks
    t = st.table.cpu()
    assert torch.equal(t[0, :32], t[1, :32]) and torch.equal(t[0, :32], t[2, :32])
    out = st.run()
    torch.cuda.synchronize()
    err = max_abs(to64(out), st.oracle())
    say("shared prefix max err", err)
    assert err <= TOL[torch.float16]


def test_one_new_row_matches_decode():
    need_gpu()
    prefixes = [15, 16, 200, 1023, 1500]
    st = ChunkStep(kvp, prefixes, [1] * 5, seed=12300)
    a = st.run()
    b = kvp.paged_decode_attention(st.cache, 0, st.q.cuda(), st.table, st.ctxd)
    torch.cuda.synchronize()
    assert max_abs(to64(a), to64(b)) <= TOL[torch.float16]
    assert max_abs(to64(a), st.oracle()) <= TOL[torch.float16]


def test_prefix_then_chunk_equals_whole_prefill():
    need_gpu()
    # one sequence of 700 tokens: prefill of the whole prompt vs its first 300 cached and the
    # remaining 400 rows as a chunk
    n, split = 700, 300
    whole = ChunkStep(kvp, [0], [n], seed=12400)
    chunk = ChunkStep(kvp, [split], [n - split], seed=12400)
    chunk.q = whole.q[split:].clone()
    a = whole.run()
    b = chunk.run()
    torch.cuda.synchronize()
    assert max_abs(to64(a[split:]), to64(b)) <= TOL[torch.float16]
    assert max_abs(to64(b), chunk.oracle()) <= TOL[torch.float16]


def test_empty_calls_are_no_ops():
    need_gpu()
    st = ChunkStep(kvp, [40], [3], seed=12500)
    out = torch.full_like(st.q.cuda(), 7.0)
    kvp.paged_prefill_attention(st.cache, 0, st.q.cuda(), st.table, st.ctxd, st.cu.cuda(), 0, out=out)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("head_dim", [64, 128])
def test_wide_table_takes_the_narrow_ring_bit_identically(head_dim):
    # a block table wider than the 2-slot ring leaves room for in LDS (its staged ids beside
    # 64 KB of K / V ring, two workgroups per CU) runs the 3-slot ring of single compute
    # tiles: the same compute tiles in the same order, so the outputs are bit-identical
    need_gpu()
    prefixes, chunks = [0, 300, 1000, 2047], [64, 257, 5, 300]
    say("wide block table, head dim", head_dim)
    st = ChunkStep(kvp, prefixes, chunks, seed=12600 + head_dim, head_dim=head_dim)
    a = st.run()
    wide = torch.full((st.B, 4096), -1, dtype=torch.int32, device="cuda")
    wide[:, :st.max_blocks] = st.table
    b = kvp.paged_prefill_attention(st.cache, 0, st.q.cuda(), wide, st.ctxd, st.cu.cuda(), max(st.m))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert max_abs(to64(b), st.oracle()) <= TOL[torch.float16]
