"""Helpers of the GPU tests: device checks and construction of a paged decode step.

Inputs come from `workloads` (seeded), expected values from `oracle`; the HIP library
only ever produces the values under test.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import workloads as W

GPU = torch.cuda.is_available()


def need_gpu():
    if not GPU:
        pytest.skip("no GPU")


def say(*a):
    """Progress line naming the case, flushed before the GPU step runs."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


TOL = {torch.float16: 2e-3, torch.float32: 1e-5}


class ScoreShaper:
    """Inputs whose scores move the kernels' softmax reference during a row.

    The decode and prefill kernels keep a per-row reference maximum and move it only when
    a tile's maximum passes it by more than 2^8; the accumulators are then rescaled by
    2^(old - new), and split partials are merged with the same rescale (chatgpz.de
    "Aufmerksamkeit", FlashAttention post: block softmaxes merged through their maxima).
    N(0,1) inputs never get there, so these shapes force it (values only: no attention
    arithmetic here):
      ramp_up    key dim 0 grows with the position, query dim 0 = 8: the score rises by
                 about 40 log2 units over 2048 positions (moves once per 512 tokens, and
                 split partials whose maxima differ by about 10 units)
      steep      the same ramp four times steeper: a move every second 64-key tile
      ramp_down  the mirrored ramp: the first tile holds the maximum, later partials lie
                 tens of units below it
      late_peak  one key 3 positions before the end of each request (outside any shared
                 prefix) scores about 12 log2 units above the rest
      big_q      queries times 40: scores spread over hundreds of log2 units
    V is halved everywhere (exact in fp16), so outputs stay below 2 in magnitude and their
    single fp16 rounding stays well inside the tolerance."""
    KINDS = ("ramp_up", "steep", "ramp_down", "late_peak", "big_q")
    SPAN = 2048

    def __init__(self, kind):
        assert kind in self.KINDS, kind
        self.kind = kind

    def keys(self, K, V, start=0, peak_at=None):
        """K, V [..., n, d] (positions start .. start + n - 1 along dim -2); peak_at: the
        position to raise (late_peak), or None.  Returns shaped copies in the same dtype."""
        dt = K.dtype
        K = K.to(torch.float32).clone()
        V = (V.to(torch.float32) * 0.5)
        n = K.shape[-2]
        pos = torch.arange(start, start + n, dtype=torch.float32)
        if self.kind in ("ramp_up", "steep"):
            K[..., :, 0] += (28.0 if self.kind == "ramp_up" else 112.0) * pos / self.SPAN
        elif self.kind == "ramp_down":
            K[..., :, 0] += 28.0 * (self.SPAN - pos) / self.SPAN
        elif self.kind == "late_peak" and peak_at is not None and start <= peak_at < start + n:
            K[..., peak_at - start, 0] += 11.0
        return K.to(dt), V.to(dt)

    def query(self, q):
        dt = q.dtype
        q = q.to(torch.float32).clone()
        if self.kind == "big_q":
            q = q * 40.0
        else:
            q[..., 0] = 8.0 if self.kind != "late_peak" else 6.0
        return q.to(dt)


class PagedStep:
    """One decode step of a batch over a paged cache, built through the block manager:
    sharing groups fork a prefix sequence (and truncate to shorter contexts), private
    tokens are reserved after it, then the step appends one token per request (copy-on-
    write where the target block is shared) and writes its K/V in every layer.  With
    take_step=False only the state before the step is built (pool, cache, seqs, logical
    rows of positions below each context)."""

    def __init__(self, kvp, pb: W.PagedBatch, layers, hq, hkv, dtype, seed, device="cuda",
                 extra_blocks=64, poison=True, layers_with_data=None, head_dim=W.HEAD_DIM, take_step=True,
                 shaper=None):
        self.kvp, self.pb, self.layers = kvp, pb, layers
        self.shaper = shaper
        self.hq, self.hkv, self.dtype, self.seed = hq, hkv, dtype, seed
        self.head_dim = head_dim
        # an int8 cache quantizes fp16 rows on append; q, out and the logical rows are fp16
        io = self.io_dtype = torch.float16 if dtype == torch.int8 else dtype
        B = pb.batch
        ctx_after = [c + 1 for c in pb.ctx_before]
        self.lmax = max(ctx_after)
        self.max_blocks = math.ceil(self.lmax / W.BLOCK)
        ngroups = len(set(pb.group))
        need = sum(math.ceil(c / W.BLOCK) for c in ctx_after) + ngroups * math.ceil(pb.prefix / W.BLOCK)
        self.num_blocks = need + extra_blocks
        self.pool = kvp.BlockPool(self.num_blocks)
        self.pool.set_free_order(W.free_list_permutation(self.num_blocks, seed + 17).tolist())
        self.cache = kvp.PagedKVCache(layers, self.num_blocks, hq, hkv, dtype, device, head_dim=head_dim)
        if poison:  # never-written rows hold NaN: any read of them shows up in the output
            if dtype == torch.int8:  # codes cannot be NaN: the scales are
                self.cache.k_pool.fill_(127)
                self.cache.v_pool.fill_(-128)
                self.cache.k_scale.fill_(float("nan"))
                self.cache.v_scale.fill_(float("nan"))
            else:
                self.cache.k_pool.fill_(float("nan"))
                self.cache.v_pool.fill_(float("nan"))
        self.layers_with_data = list(range(layers)) if layers_with_data is None else layers_with_data
        self.logical = {l: W.logical_kv(pb, hkv, self.lmax, seed, io, layer=l, head_dim=head_dim)
                        for l in self.layers_with_data}
        prefix = {l: W.group_prefix_kv(pb, hkv, seed, io, layer=l, head_dim=head_dim)
                  for l in self.layers_with_data}
        if shaper is not None:
            # the same position-dependent shaping of the logical rows and of the group prefixes
            # (the late peak sits past each request's shared prefix)
            for l in self.layers_with_data:
                K, V = self.logical[l]
                Ks, Vs = [], []
                for b in range(B):
                    pk_at = pb.ctx_before[b] - 3
                    assert shaper.kind != "late_peak" or pk_at >= min(pb.ctx_before[b], pb.prefix)
                    kb, vb = shaper.keys(K[b], V[b], 0, pk_at)
                    Ks.append(kb)
                    Vs.append(vb)
                self.logical[l] = (torch.stack(Ks), torch.stack(Vs))
                prefix[l] = {g: shaper.keys(pk, pv, 0, None) for g, (pk, pv) in prefix[l].items()}

        seqs = [None] * B
        for gi in sorted(set(pb.group)):
            members = [i for i in range(B) if pb.group[i] == gi]
            if pb.prefix > 0:
                pre = self.pool.alloc(pb.prefix)
                sl = self.pool.slots(pre, 0, pb.prefix).to(device)
                for l in self.layers_with_data:
                    pk, pv = prefix[l][gi]
                    kvp.kv_append(self.cache, l, pk.transpose(0, 1).contiguous().to(device),
                                  pv.transpose(0, 1).contiguous().to(device), sl)
                for i in members:
                    s = self.pool.fork(pre)
                    L = pb.ctx_before[i]
                    if L < pb.prefix:
                        self.pool.truncate(s, L)
                    elif L > pb.prefix:
                        self._reserve_private(s, i, pb.prefix, L, device)
                    seqs[i] = s
                self.pool.free(pre)
            else:
                for i in members:
                    s = self.pool.alloc(0)
                    self._reserve_private(s, i, 0, pb.ctx_before[i], device)
                    seqs[i] = s
        self.seqs = seqs
        if not take_step:  # the state before the step (a caller drives the steps)
            return
        # the decode step: one new token per request
        pairs, slots = [], []
        for i in range(B):
            slot, cp = self.pool.append_slot(seqs[i])
            slots.append(slot)
            if cp is not None:
                pairs.append(cp)
        self.cow_pairs = pairs
        if pairs:
            kvp.kv_copy_blocks(self.cache, torch.tensor(pairs, dtype=torch.int32, device=device))
        self.new_slots = torch.tensor(slots, dtype=torch.int64, device=device)
        for l in self.layers_with_data:
            K, V = self.logical[l]
            idx = torch.tensor(pb.ctx_before)
            kn = K[torch.arange(B), :, idx].contiguous().to(device)  # [B, hkv, d]
            vn = V[torch.arange(B), :, idx].contiguous().to(device)
            kvp.kv_append(self.cache, l, kn, vn, self.new_slots)
        table, ctx = self.pool.export(seqs, self.max_blocks)
        self.table = table.to(device)
        self.ctx = ctx.to(device)
        self.ctx_host = ctx.tolist()
        assert self.ctx_host == ctx_after

    def _reserve_private(self, s, i, start, end, device):
        n = end - start
        sl, cp = self.pool.reserve(s, n)
        assert cp is None  # private tokens start on a fresh block
        sl = sl.to(device)
        for l in self.layers_with_data:
            K, V = self.logical[l]
            self.kvp.kv_append(self.cache, l, K[i, :, start:end].transpose(0, 1).contiguous().to(device),
                               V[i, :, start:end].transpose(0, 1).contiguous().to(device), sl)

    def q(self, layer):
        q = W.decode_q(self.pb.batch, self.hq, self.seed, self.io_dtype, layer, self.head_dim)
        return q if self.shaper is None else self.shaper.query(q)

    def oracle(self, layer, rows=None):
        """Oracle decode output [B, Hq, d] (float64) for the given requests (all if None)."""
        import oracle
        K, V = self.logical[layer]
        q = self.q(layer)
        rows = list(range(self.pb.batch)) if rows is None else rows
        K64, V64 = to64(K[rows]), to64(V[rows])
        if self.dtype == torch.int8:  # the cache holds the oracle's quantization of the rows
            K64, V64 = self.dequantized(K[rows]), self.dequantized(V[rows])
        out = oracle.decode_gqa(to64(q[rows]), K64, V64, np.array([self.ctx_host[r] for r in rows]))
        return out

    @staticmethod
    def dequantized(x):
        """fp64 reconstruction of the oracle's int8 row quantization of fp16 rows x [..., d]."""
        from oracle import kvquant as KQ
        codes, scales = KQ.absmax_quantize_rows(x.numpy())
        return KQ.dequantize_rows(codes, scales)


class ChunkStep:
    """Requests with cached prefixes and a chunk of new rows, written through the block
    manager (scattered block ids) into layer 0 of a paged cache; optionally requests fork a
    shared prefix first.  Never-written cache rows hold NaN, so a read of one shows."""

    def __init__(self, kvp, prefixes, chunks, seed, hq=14, hkv=2, share_groups=None, layers=1,
                 head_dim=W.HEAD_DIM, shaper=None):
        self.kvp = kvp
        self.B = len(prefixes)
        D = self.head_dim = head_dim
        ctx = [p + m for p, m in zip(prefixes, chunks)]
        self.ctx, self.m, self.hq, self.hkv = ctx, list(chunks), hq, hkv
        self.lmax = max(ctx)
        self.max_blocks = math.ceil(self.lmax / W.BLOCK)
        nblocks = sum(math.ceil(c / W.BLOCK) for c in ctx) + 64
        self.pool = kvp.BlockPool(nblocks)
        self.pool.set_free_order(W.free_list_permutation(nblocks, seed).tolist())
        self.cache = kvp.PagedKVCache(layers, nblocks, hq, hkv, torch.float16, "cuda", head_dim=D)
        self.cache.k_pool.fill_(float("nan"))  # never-written rows show up as NaN
        self.cache.v_pool.fill_(float("nan"))
        # logical K / V of every request, seeded
        self.K = W.randn((self.B, hkv, self.lmax, D), seed + 1)
        self.V = W.randn((self.B, hkv, self.lmax, D), seed + 2)
        if shaper is not None:  # position-dependent shaping; the peak past any shared prefix
            for b in range(self.B):
                assert shaper.kind != "late_peak" or ctx[b] - 3 >= prefixes[b]
                self.K[b], self.V[b] = shaper.keys(self.K[b], self.V[b], 0, ctx[b] - 3)
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
        if shaper is not None:
            self.q = shaper.query(self.q)

    def _write(self, seq, b, lo, hi):
        if hi <= lo:
            return
        slots, cow = self.pool.reserve(seq, hi - lo)
        if cow is not None:  # the chunk starts inside a shared, partly filled prefix block
            self.kvp.kv_copy_blocks(self.cache, torch.tensor([cow], dtype=torch.int32).cuda())
        k = self.K[b, :, lo:hi].transpose(0, 1).contiguous().cuda()
        v = self.V[b, :, lo:hi].transpose(0, 1).contiguous().cuda()
        self.kvp.kv_append(self.cache, 0, k, v, slots.cuda())

    def run(self):
        return self.kvp.paged_prefill_attention(self.cache, 0, self.q.cuda(), self.table, self.ctxd, self.cu.cuda(),
                                           max(self.m))

    def oracle(self):
        import oracle
        return oracle.chunk_attention(to64(self.q), to64(self.K), to64(self.V), np.array(self.ctx, np.int32),
                                      self.cu.numpy())
