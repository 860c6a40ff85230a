"""A serving-loop decode step over the paged cache, as a reusable driver of the C ABI.

One step, for a batch of sequences held by a BlockPool:
  1. the block manager reserves the next slot of every sequence (copy-on-write pairs when
     the target block is shared),
  2. the block table is exported and the host planner turns it into the step's work plan
     (shared prefixes read once per group of members, items placed on XCD queues), padded
     to a fixed item count so that every step launches the same way,
  3. the plan image is uploaded on a copy stream into one of two device buffers, beside
     the previous step's layers, while the copy-on-write block copies run on the compute
     stream,
  4. for every layer one kernel appends the step's K/V row at position context - 1 and
     attends over the whole cache (paged_decode_attention_planned with k_new / v_new),
     replayed as one captured HIP graph per plan buffer.

Pages: neuralialabs "Tornar a inferencia barata" (KV cache and PagedAttention passages:
decode appends one token and attends over the cache through a block table);
gustavoai "La cache de claves y valores" (four-step token recipe: the new k, v go to the
end of the cache before the attention row); chatgpz.de "Aufmerksamkeit", paged-attention
article SECTION 2 / 3 (block pool, block table, copy-on-write of shared prefix blocks).

Only library calls happen here: the block manager and planner are the library's C++
code, the copies and attention its HIP kernels.  q, k_new, v_new and out are the
caller's device tensors [layers, B, ...]; their contents may change between steps (the
graphs read them in place).
"""
import numpy as np
import torch

from . import (BLOCK, BlockPool, PagedKVCache, decode_plan_build, decode_plan_bytes, decode_plan_workspace_bytes,
               kv_copy_blocks, kvp_copy, kvp_decode_plan, paged_decode_attention_planned)

# plans of at most this many (request, KV head) pairs use KVP_PLAN_FILL when fill="auto": a
# lone request's context is then cut into 8-block parts across idle waves (one request of
# 1024 tokens at 14q/2kv: 9.9 against 12.1 us per launch); for batches of 10 or more
# requests the extra parts' partial stores, tickets and merge batches cost more than the
# shorter tile chains save (batch 10: 15.8 against 14.0 us)
FILL_AUTO_PAIRS = 8

# spare items of the fixed launch size: one more round of CU slots per XCD queue (8 XCDs x
# 32 CU slots), so plans of later steps (one token longer each) still fit
SPARE_ITEMS = 8 * 32


class StepRecord:
    """Host copies of what one step ran on: table [B, max_blocks], context lengths [B], the
    copy-on-write pairs, and plan statistics.  split_partials: partial records a layer's
    split pairs exchange (all but one part of each split pair stores one, the merging part
    reads them back)."""

    def __init__(self, table, ctx, cow_pairs, n_items, n_shared, kv_blocks_read, split_partials=0):
        self.table, self.ctx, self.cow_pairs = table, ctx, cow_pairs
        self.n_items, self.n_shared, self.kv_blocks_read = n_items, n_shared, kv_blocks_read
        self.split_partials = split_partials


class DecodeStepRunner:
    """Runs decode steps of the sequences `seqs` of `pool` over `cache`.

    q [L, B, Hq, d], k_new / v_new [L, B, Hkv, d] (io dtype of the cache) and out
    [L, B, Hq, d] are device tensors read and written by every step.  max_blocks is the
    table width, large enough for the longest context of the last step to be run.
    graph=False launches the layers eagerly.  fill: True / False asks for / against
    KVP_PLAN_FILL plans, "auto" uses them for batches of at most FILL_AUTO_PAIRS pairs.
    """

    def __init__(self, cache: PagedKVCache, pool: BlockPool, seqs, max_blocks, q, k_new, v_new, out,
                 share_prefix=True, long_items=False, graph=True, spare_items=SPARE_ITEMS, grow_tokens=64,
                 share_width=1, fill="auto"):
        L, B = q.shape[0], q.shape[1]
        hq, hkv, d = cache.num_q_heads, cache.num_kv_heads, cache.head_dim
        if q.shape != (L, B, hq, d) or out.shape != q.shape:
            raise ValueError("DecodeStepRunner: q / out must be [layers, B, Hq, d]")
        if k_new.shape != (L, B, hkv, d) or v_new.shape != k_new.shape:
            raise ValueError("DecodeStepRunner: k_new / v_new must be [layers, B, Hkv, d]")
        if L > cache.num_layers or len(seqs) != B:
            raise ValueError("DecodeStepRunner: layer count or batch does not match the cache / sequences")
        self.cache, self.pool = cache, pool
        self.L, self.B, self.hq, self.hkv, self.d = L, B, hq, hkv, d
        self.max_blocks = int(max_blocks)
        self.q, self.k_new, self.v_new, self.out = q, k_new, v_new, out
        self.share, self.long_items, self.use_graph = share_prefix, long_items, graph
        if fill not in (True, False, "auto"):
            raise ValueError("DecodeStepRunner: fill is True, False or 'auto'")
        self.share_width = share_width
        self.fill = (B * hkv <= FILL_AUTO_PAIRS) if fill == "auto" else bool(fill)
        self.spare, self.grow = int(spare_items), int(grow_tokens)
        self.ids = torch.tensor([int(s) for s in seqs], dtype=torch.int32)
        self.cows = (kvp_copy * B)()
        self.cows_np = np.frombuffer(self.cows, dtype=np.int32).reshape(B, 2)  # (src, dst) per request
        dev = q.device
        self.dev = dev
        self.stream = torch.cuda.current_stream(dev)
        self.copy_stream = torch.cuda.Stream(device=dev)  # default priority
        self.capture_stream = torch.cuda.Stream(device=dev)  # default priority
        self.pairs_d = torch.empty((B, 2), dtype=torch.int32, device=dev)
        self.steps_run = 0
        self._pending = None
        self.layout = None  # (pad_items, image bytes, launch plan, slot capacity)
        self.graphs = [None, None]

    # ---- layout: fixed item count, plan buffers, workspace and graphs ----
    def _make_layout(self, table, ctx):
        """Size the launch from a plan of the contexts grown by grow_tokens (capped by the
        table width), plus the spare items."""
        plans = []
        # a fill plan's part length follows the batch's blocks: size for the first step too
        for grow in ((self.grow, 0) if self.fill else (self.grow,)):
            c1 = torch.clamp(ctx + 1 + grow, max=self.max_blocks * BLOCK)
            plans.append(decode_plan_build(self.hq, self.hkv, table, c1, self.cache.num_blocks,
                                           share_prefix=self.share, head_dim=self.d, long_items=self.long_items,
                                           kv_dtype=self.cache.dtype, share_width=self.share_width,
                                           fill=self.fill)[0])
        pad = max(p.n_items for p in plans) + self.spare
        img_bytes = decode_plan_bytes(self.hq, self.hkv, self.B, self.max_blocks, pad, head_dim=self.d,
                                      kv_dtype=self.cache.dtype)
        self.host = [dict(table=torch.empty((self.B, self.max_blocks), dtype=torch.int32).pin_memory(),
                          ctx=torch.empty((self.B,), dtype=torch.int32).pin_memory(),
                          slots=torch.empty((self.B,), dtype=torch.int64).pin_memory(),
                          pairs=torch.empty((self.B, 2), dtype=torch.int32).pin_memory(),
                          image=torch.empty((img_bytes,), dtype=torch.uint8).pin_memory(),
                          plan=kvp_decode_plan()) for _ in range(2)]
        for h in self.host:
            h["pairs_np"] = h["pairs"].numpy()  # the same pinned memory
        self.plan_d = [torch.empty((img_bytes,), dtype=torch.uint8, device=self.dev) for _ in range(2)]
        self.uploaded = [torch.cuda.Event(), torch.cuda.Event()]
        self.released = [torch.cuda.Event(), torch.cuda.Event()]
        self.done = [torch.cuda.Event(), torch.cuda.Event()]
        self.in_use = [False, False]
        # partial slots: twice the sizing plans', plus one per pair
        slot_cap = 2 * max(p.n_slots for p in plans) + self.B * self.hkv
        self.layout = dict(pad=pad, img_bytes=img_bytes, slot_cap=slot_cap, launch=None)
        ws_plan = kvp_decode_plan()
        ws_plan.B, ws_plan.num_kv_heads, ws_plan.n_slots, ws_plan.head_dim = self.B, self.hkv, slot_cap, self.d
        ws_plan.group = self.hq // self.hkv
        self.workspace = torch.zeros((max(decode_plan_workspace_bytes(ws_plan), 256),), dtype=torch.uint8,
                                     device=self.dev)
        self.graphs = [None, None]
        self.first_of_layout = True

    def _layers_body(self, pd):
        lp = self.layout["launch"]
        for l in range(self.L):
            paged_decode_attention_planned(self.cache, l, self.q[l], lp, pd, k_new=self.k_new[l], v_new=self.v_new[l],
                                           out=self.out[l], workspace=self.workspace)

    def _capture(self):
        torch.cuda.synchronize(self.dev)
        for i in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.capture_stream):
                self._layers_body(self.plan_d[i])
            self.graphs[i] = g
        torch.cuda.synchronize(self.dev)

    @property
    def launch_plan(self):
        return self.layout["launch"] if self.layout else None

    def plan_buffer(self, k):
        """Device plan buffer used by step k (0-based count of steps run)."""
        return self.plan_d[k % 2]

    def prepare(self, keep=False):
        """Host part of the next step: reserve the slots (copy-on-write pairs), export the
        table and build the plan into pinned memory.  Returns a StepRecord of host copies
        when keep is set, else None.  launch() enqueues the device part."""
        if getattr(self, "_pending", None) is not None:
            raise RuntimeError("DecodeStepRunner: prepare() called twice without launch()")
        k = self.steps_run
        B = self.B
        if self.layout is None:
            tmp_t = torch.empty((B, self.max_blocks), dtype=torch.int32)
            tmp_c = torch.empty((B,), dtype=torch.int32)
            self.pool.export_raw(self.ids.data_ptr(), B, self.max_blocks, tmp_t.data_ptr(), tmp_c.data_ptr())
            self._make_layout(tmp_t, tmp_c)
        h = self.host[k % 2]
        self.done[k % 2].synchronize()  # the copies that last read these pinned buffers are done
        self.pool.append_slots_raw(self.ids.data_ptr(), B, h["slots"].data_ptr(), self.cows)
        # the copy-on-write pairs of the requests that made one, in request order
        sel = np.flatnonzero(self.cows_np[:, 0] >= 0)
        npairs = int(sel.size)
        if npairs:
            h["pairs_np"][:npairs] = self.cows_np[sel]
        self.pool.export_raw(self.ids.data_ptr(), B, self.max_blocks, h["table"].data_ptr(), h["ctx"].data_ptr())
        lay = self.layout
        plan, _ = decode_plan_build(self.hq, self.hkv, h["table"], h["ctx"], self.cache.num_blocks,
                                    share_prefix=self.share, image=h["image"], pad_items=lay["pad"], plan=h["plan"],
                                    head_dim=self.d, long_items=self.long_items, kv_dtype=self.cache.dtype,
                                    share_width=self.share_width, fill=self.fill)
        if lay["launch"] is None:
            # launch arguments shared by every step of this layout: the plan's offsets, the
            # workspace's slot capacity and the whole id area of the buffer
            lp = kvp_decode_plan.from_buffer_copy(plan)
            lp.n_slots = lay["slot_cap"]
            lp.n_ids = (lay["img_bytes"] - plan.off_ids) // 4
            # the widest item any step of this configuration can hold (the kernel build is
            # chosen by it): G / 16 blocks above 16 heads per KV head, else the shared width
            # (at least 2 when a block holds one member), at most 4 (2 at head dim 128)
            G = self.hq // self.hkv
            w = G // 16 if G > 16 else (max(self.share_width, 2 if G > 8 else 1) if self.share else 1)
            lp.col_blocks = max(int(lp.col_blocks), min(w, 4 if self.d == 64 else 2))
            lay["launch"] = lp
        lp = lay["launch"]
        if plan.col_blocks > lp.col_blocks:
            raise RuntimeError("DecodeStepRunner: the step's plan holds wider items than the launch layout")
        if plan.n_slots > lp.n_slots:
            raise RuntimeError(f"DecodeStepRunner: step needs {plan.n_slots} partial slots, the workspace holds "
                               f"{lp.n_slots}")
        if (plan.n_items, plan.off_pair_base, plan.off_req_shared, plan.off_ids) != \
                (lp.n_items, lp.off_pair_base, lp.off_req_shared, lp.off_ids):
            raise RuntimeError("DecodeStepRunner: the step's plan does not fit the launch layout")
        if plan.off_ids + 4 * plan.n_ids > lay["img_bytes"]:
            raise RuntimeError("DecodeStepRunner: plan image larger than its buffer")
        rec = None
        if keep:
            npairs_kv = self.B * self.hkv
            parts = h["image"][plan.off_pair_nparts:plan.off_pair_nparts + 4 * npairs_kv].numpy().view(np.int32)
            rec = StepRecord(h["table"].numpy().copy(), h["ctx"].numpy().copy(),
                             h["pairs"][:npairs].numpy().copy(), int(plan.n_items), int(plan.n_shared),
                             int(plan.kv_blocks_read), int(np.maximum(parts - 1, 0).sum()))
        self._pending = (h, int(plan.bytes), npairs)
        return rec

    def launch(self):
        """Device part of the prepared step, asynchronous on the runner's stream: plan upload
        on the copy stream, copy-on-write block copies, then every layer's fused append +
        decode (a graph replay once captured)."""
        if getattr(self, "_pending", None) is None:
            raise RuntimeError("DecodeStepRunner: launch() without prepare()")
        h, nbytes, npairs = self._pending
        self._pending = None
        i = self.steps_run % 2
        stream = self.stream
        if self.in_use[i]:  # step k - 2 read this buffer
            self.copy_stream.wait_event(self.released[i])
        with torch.cuda.stream(self.copy_stream):
            self.plan_d[i][:nbytes].copy_(h["image"][:nbytes], non_blocking=True)
            self.uploaded[i].record(self.copy_stream)
        with torch.cuda.stream(stream):
            if npairs:
                self.pairs_d[:npairs].copy_(h["pairs"][:npairs], non_blocking=True)
                kv_copy_blocks(self.cache, self.pairs_d[:npairs])
            stream.wait_event(self.uploaded[i])
            if self.graphs[i] is not None:
                self.graphs[i].replay()
            else:
                self._layers_body(self.plan_d[i])
            self.released[i].record(stream)
            self.in_use[i] = True
            self.done[i].record(stream)  # also covers the upload, which the layers waited for
        self.steps_run += 1
        if self.use_graph and self.first_of_layout:
            # the first step ran eagerly (loading the code objects); capture both buffers' graphs
            self.first_of_layout = False
            self._capture()

    def step(self, keep=False):
        """prepare() then launch(): one decode step, asynchronous on the runner's stream.
        Returns the StepRecord of prepare()."""
        rec = self.prepare(keep)
        self.launch()
        return rec

    def replay_layers(self):
        """Enqueue the last step's layers again (same plan buffer; the fused append rewrites
        the same rows, so the outputs do not change).  For timing the layers alone."""
        i = (self.steps_run - 1) % 2
        with torch.cuda.stream(self.stream):
            if self.graphs[i] is not None:
                self.graphs[i].replay()
            else:
                self._layers_body(self.plan_d[i])

    def last_plan_buffer(self):
        return self.plan_d[(self.steps_run - 1) % 2]

    def synchronize(self):
        torch.cuda.synchronize(self.dev)
