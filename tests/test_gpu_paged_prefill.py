"""Several new query rows per request against the paged cache (paged_prefill_attention) on
the GPU, against the fp64 oracle (oracle.chunk_attention).

The rows of request b are the last m_b of its ctx_b positions and row i attends to
positions 0 .. ctx_b - m_b + i: a chunk of a prompt prefilled into an existing prefix, or
the verification pass over gamma drafted tokens ([CHAP] speculative-decoding section: one
forward pass over gamma positions).  Prefixes may be shared between requests forked from
one prompt ([PAGED] SECTION 3).  Never-written cache rows hold NaN, so a read of one shows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp

HQ, HKV, D, BS = 14, 2, 64, 16


class ChunkStep:
    """Requests with cached prefixes and a chunk of new rows, written through the block
    manager (scattered block ids) into layer 0 of a paged cache; optionally requests fork a
    shared prefix first."""

    def __init__(self, prefixes, chunks, seed, hq=HQ, hkv=HKV, share_groups=None, layers=1):
        self.B = len(prefixes)
        ctx = [p + m for p, m in zip(prefixes, chunks)]
        self.ctx, self.m, self.hq, self.hkv = ctx, list(chunks), hq, hkv
        self.lmax = max(ctx)
        self.max_blocks = math.ceil(self.lmax / BS)
        nblocks = sum(math.ceil(c / BS) for c in ctx) + 64
        self.pool = kvp.BlockPool(nblocks)
        self.pool.set_free_order(W.free_list_permutation(nblocks, seed).tolist())
        self.cache = kvp.PagedKVCache(layers, nblocks, hq, hkv, torch.float16, "cuda")
        self.cache.k_pool.fill_(float("nan"))  # never-written rows show up as NaN
        self.cache.v_pool.fill_(float("nan"))
        # logical K / V of every request, seeded
        self.K = W.randn((self.B, hkv, self.lmax, D), seed + 1)
        self.V = W.randn((self.B, hkv, self.lmax, D), seed + 2)
        if share_groups:
            # requests in one group share the first prefix's tokens (same K/V rows, one set
            # of physical blocks): fork the leader after it is written
            for grp in share_groups:
                lead = grp[0]
                p = prefixes[lead]
                for b in grp[1:]:
                    assert prefixes[b] == p
                    self.K[b, :, :p] = self.K[lead, :, :p]
                    self.V[b, :, :p] = self.V[lead, :, :p]
        self.seqs = [None] * self.B
        grouped = {b for g in (share_groups or []) for b in g}
        for b in range(self.B):
            if b in grouped:
                continue
            s = self.pool.alloc(0)
            self._write(s, b, 0, ctx[b])
            self.seqs[b] = s
        for grp in share_groups or []:
            lead = grp[0]
            p = prefixes[lead]
            base = self.pool.alloc(0)
            self._write(base, lead, 0, p)
            for b in grp:
                s = self.pool.fork(base)
                self._write(s, b, p, ctx[b])
                self.seqs[b] = s
            self.pool.free(base)
        table, ctxt = self.pool.export(self.seqs, self.max_blocks)
        assert ctxt.tolist() == ctx
        self.table, self.ctxd = table.cuda(), ctxt.cuda()
        self.cu = torch.tensor([0] + list(np.cumsum(self.m)), dtype=torch.int32)
        self.q = W.randn((int(self.cu[-1]), hq, D), seed + 3)

    def _write(self, seq, b, lo, hi):
        if hi <= lo:
            return
        slots, cow = self.pool.reserve(seq, hi - lo)
        if cow is not None:  # the chunk starts inside a shared, partly filled prefix block
            kvp.kv_copy_blocks(self.cache, torch.tensor([cow], dtype=torch.int32).cuda())
        k = self.K[b, :, lo:hi].transpose(0, 1).contiguous().cuda()
        v = self.V[b, :, lo:hi].transpose(0, 1).contiguous().cuda()
        kvp.kv_append(self.cache, 0, k, v, slots.cuda())

    def run(self):
        return kvp.paged_prefill_attention(self.cache, 0, self.q.cuda(), self.table, self.ctxd, self.cu.cuda(),
                                           max(self.m))

    def oracle(self):
        return oracle.chunk_attention(to64(self.q), to64(self.K), to64(self.V), np.array(self.ctx, np.int32),
                                      self.cu.numpy())


def test_chunked_prefill_into_prefixes():
    need_gpu()
    prefixes = [0, 17, 300, 511, 1000, 2047]
    chunks = [64, 100, 1, 257, 300, 5]
    say("chunked prefill", list(zip(prefixes, chunks)))
    st = ChunkStep(prefixes, chunks, seed=12000)
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
    st = ChunkStep(prefixes, [5] * 32, seed=12100)
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
    st = ChunkStep(prefixes, chunks, seed=12200, share_groups=[[0, 1, 2], [3, 4]])
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
    st = ChunkStep(prefixes, [1] * 5, seed=12300)
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
    whole = ChunkStep([0], [n], seed=12400)
    chunk = ChunkStep([split], [n - split], seed=12400)
    chunk.q = whole.q[split:].clone()
    a = whole.run()
    b = chunk.run()
    torch.cuda.synchronize()
    assert max_abs(to64(a[split:]), to64(b)) <= TOL[torch.float16]
    assert max_abs(to64(b), chunk.oracle()) <= TOL[torch.float16]


def test_empty_calls_are_no_ops():
    need_gpu()
    st = ChunkStep([40], [3], seed=12500)
    out = torch.full_like(st.q.cuda(), 7.0)
    kvp.paged_prefill_attention(st.cache, 0, st.q.cuda(), st.table, st.ctxd, st.cu.cuda(), 0, out=out)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
