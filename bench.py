#!/usr/bin/env python3
"""Benchmark: paged grouped-query decode steps at batch 200 on one MI355X.

Workload (synthetic, seeded): the pages' 24-layer model shape (14 query heads, 2 KV heads,
head_dim 64, fp16), a paged cache of 16-token blocks, 200 requests with context lengths
uniform on 128..2048, groups of 8 consecutive requests sharing a 512-token prefix
(copy-on-write), block ids scattered by a seeded shuffle of the free list.

One step = the host block manager reserves one slot per request (copy-on-write pairs
included), the host planner turns the block table into the step's work plan (shared
prefixes read once per group of members), the plan is uploaded and the copy-on-write block
copies run, then for each of the 24 layers one kernel appends the new token's K/V and runs
the paged decode attention over the whole cache (paged_decode_attention_planned, replayed
as one captured graph).  Contexts grow by one token per step.  The plan upload runs on a
copy stream into one of two device buffers, beside the previous step's layers.

--shape 32q8kv_d128 / 32q32kv_d128 runs the same step at the 7B-class head shapes (32
layers, head dim 128, 8 or 32 KV heads).  --workload prefill / chunked_prefill time the
prefill kernels instead.

Printed: one JSON line with the decode-attention KV throughput (unique bytes), steps/s,
the roofline of the dominant kernel (the paged decode call: split-K partial + merge),
and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# the long-context decode configuration: 32 requests of 32768 cached tokens
LONG_BATCH, LONG_CONTEXT = 32, 32768
HQ, HKV, D, BLOCK = 14, 2, 64, 16
KV_TOKEN_LAYER_BYTES = 2 * HKV * D * 2  # K and V, fp16: 512 B per token per layer

# head shapes of the decode step: (layers, query heads, KV heads, head dim, description)
SHAPES = {
    "14q2kv_d64": (24, 14, 2, 64, "24 layers, 14q/2kv heads d64"),
    # the 7B-class GQA shape (32 layers, 8 KV heads of d = 128) with 32 query heads
    "32q8kv_d128": (32, 32, 8, 128, "32 layers, 32q/8kv heads d128 (7B-class GQA)"),
    # the same model as plain multi-head attention (32 KV heads)
    "32q32kv_d128": (32, 32, 32, 128, "32 layers, 32q/32kv heads d128 (MHA)"),
}
DEFAULT_SHAPE = "14q2kv_d64"


KV_INT8 = False  # the cache holds int8 codes and one fp16 scale per row


def set_shape(name, kv_int8=False):
    global HQ, HKV, D, KV_TOKEN_LAYER_BYTES, KV_INT8
    _, HQ, HKV, D, _ = SHAPES[name]
    KV_INT8 = kv_int8
    # K and V bytes per token and layer: fp16 values, or int8 codes plus a 2-byte scale per row
    KV_TOKEN_LAYER_BYTES = 2 * HKV * (D + 2) if kv_int8 else 2 * HKV * D * 2


# HBM traffic of the decode launch, counted by rocprofv3 (FETCH_SIZE / WRITE_SIZE passes,
# scaled by the same counters on copies of known size) and recorded in the profile summary
# together with a digest of the sources it was measured on; reported only while they match.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_f16_planned_b200.md")
TRAFFIC_SOURCES = ["kv_cache_decode_paged_amd/csrc/" + f for f in
                   ("kvp_decode_f16.hip", "kvp_decode_common.h", "kvp_gfx950.h", "kvp_decode.hip",
                    "kvp_plan.cpp", "kvp_plan_format.h")]


def decode_sources_digest():
    """Digest of the decode sources' code (comments and whitespace removed)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """Bytes per decode launch from the recorded counter passes, or None when the summary is
    missing or was measured on other sources."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)\s+sources:\s*([0-9a-f]+)", text)
    if not m or m.group(2) != decode_sources_digest():
        return None
    return int(m.group(1))


def unique_and_logical_tokens(table, ctx):
    """Distinct cache slots read by one decode call (a block's readers each read a prefix
    of it, so a block contributes the longest prefix read) and the per-request sum."""
    import numpy as np
    blocks, counts = [], []
    for i, c in enumerate(ctx):
        nb = (c + BLOCK - 1) // BLOCK
        if nb <= 0:  # an empty context reads nothing
            continue
        cnt = np.full(nb, BLOCK, dtype=np.int64)
        cnt[-1] = c - BLOCK * (nb - 1)
        blocks.append(table[i, :nb])
        counts.append(cnt)
    if not blocks:
        return 0, 0
    blocks = np.concatenate(blocks)
    counts = np.concatenate(counts)
    order = np.lexsort((counts, blocks))
    b_sorted, c_sorted = blocks[order], counts[order]
    last = np.r_[b_sorted[1:] != b_sorted[:-1], True]
    unique = int(c_sorted[last].sum())
    return unique, sum(int(c) for c in ctx)


def decode_call_bytes(table, ctx, B):
    """Algorithmic bytes of one paged_decode_attention call (one layer): unique K/V bytes,
    q in, out, the block-table entries and the context lengths."""
    uniq, logical = unique_and_logical_tokens(table, ctx)
    # Python integers throughout: a layer of a long batch holds more than 2^31 bytes
    blocks_read = sum((int(c) + BLOCK - 1) // BLOCK for c in ctx)
    qo = 2 * B * HQ * D * 2
    return uniq * KV_TOKEN_LAYER_BYTES + qo + 4 * blocks_read + 4 * B, uniq, logical


def build_state(kvp, torch, W, B, layers, total_steps, seed, long_ctx=None):
    """Block pool, cache (every slot seeded N(0,1)) and the batch's sequences: groups fork
    their prefix, then each member truncates to a shorter context or reserves its private
    tokens.  With long_ctx, B private sequences of long_ctx tokens each (no sharing)."""
    pb = W.paged_batch(B) if long_ctx is None else None
    dev = "cuda"
    ctx_before = pb.ctx_before if pb is not None else [long_ctx] * B
    need = sum(math.ceil((c + total_steps + 1) / BLOCK) for c in ctx_before) + B + 64
    if pb is not None:
        need += len(set(pb.group)) * math.ceil(pb.prefix / BLOCK)
    num_blocks = need
    max_blocks = math.ceil((max(ctx_before) + total_steps + 1) / BLOCK)
    pool = kvp.BlockPool(num_blocks)
    pool.set_free_order(W.free_list_permutation(num_blocks, seed + 1).tolist())
    cache = kvp.PagedKVCache(layers, num_blocks, HQ, HKV, torch.int8 if KV_INT8 else torch.float16, dev, head_dim=D)
    for l in range(layers):  # cache contents: seeded N(0,1) in every slot
        if KV_INT8:  # codes uniform on -127..127, row scales of N(0,1) rows (about 3 / 127)
            g = torch.Generator(device=dev)
            g.manual_seed(seed + 10 + 2 * l)
            for codes in (cache.k_pool[l], cache.v_pool[l]):
                codes.copy_(torch.randint(-127, 128, codes.shape, generator=g, device=dev, dtype=torch.int8))
            for sc in (cache.k_scale[l], cache.v_scale[l]):
                sc.copy_((torch.rand(sc.shape, generator=g, device=dev) * 0.01 + 0.02).to(torch.float16))
            continue
        cache.k_pool[l].copy_(W.randn_device(cache.k_pool[l].shape, seed + 10 + 2 * l, torch.float16, dev))
        cache.v_pool[l].copy_(W.randn_device(cache.v_pool[l].shape, seed + 11 + 2 * l, torch.float16, dev))
    if pb is None:
        return pb, pool, cache, [pool.alloc(long_ctx) for _ in range(B)], max_blocks
    seqs = [None] * B
    for gi in sorted(set(pb.group)):
        pre = pool.alloc(pb.prefix)
        for i in [i for i in range(B) if pb.group[i] == gi]:
            s = pool.fork(pre)
            L = pb.ctx_before[i]
            if L < pb.prefix:
                pool.truncate(s, L)
            elif L > pb.prefix:
                pool.reserve(s, L - pb.prefix)
            seqs[i] = s
        pool.free(pre)
    return pb, pool, cache, seqs, max_blocks


def cpu_baseline(W, layers, seed=42):
    """The fp64 oracle, as it is, on a bounded sample of the same workload, one thread per
    request in flight: every request of 2 layers at the 14q/2kv d64 shape; for the larger
    head shapes one layer of the first requests, sized to about the same oracle work."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    pb = W.paged_batch(200)
    budget = 2 * 200 * 512 // KV_TOKEN_LAYER_BYTES  # request-layers
    n_layers = 2 if budget >= 400 else 1
    n_req = max(8, min(200, budget // n_layers))
    pb = W.PagedBatch(ctx_before=pb.ctx_before[:n_req], group=pb.group[:n_req], prefix=pb.prefix)
    lmax = max(pb.ctx_before) + 1
    threads = min(16, len(os.sched_getaffinity(0)))
    ctx = np.array([c + 1 for c in pb.ctx_before], dtype=np.int32)
    total_bytes = 0
    elapsed = 0.0
    for layer in range(n_layers):
        K, V = W.logical_kv(pb, HKV, lmax, seed, layer=layer, head_dim=D)
        q = W.decode_q(pb.batch, HQ, seed, layer=layer, head_dim=D)
        K64, V64, q64 = K.double().numpy(), V.double().numpy(), q.double().numpy()
        t_q = 0.0
        if KV_INT8:  # the oracle's quantization and reconstruction of the rows, timed too
            from oracle import kvquant as KQ
            t0 = time.perf_counter()
            K64 = KQ.dequantize_rows(*KQ.absmax_quantize_rows(K.numpy()))
            V64 = KQ.dequantize_rows(*KQ.absmax_quantize_rows(V.numpy()))
            t_q = time.perf_counter() - t0

        def one(i):
            n = int(ctx[i])
            return oracle.decode_gqa(q64[i:i + 1], np.ascontiguousarray(K64[i:i + 1, :, :n]),
                                     np.ascontiguousarray(V64[i:i + 1, :, :n]), ctx[i:i + 1])

        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(pb.batch)))
        elapsed += time.perf_counter() - t0 + t_q
        total_bytes += int(ctx.sum()) * KV_TOKEN_LAYER_BYTES
    return {"value": round(total_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_layers} of {layers} layers x {n_req} of the 200 requests of the batch-200 step "
                      f"(logical KV bytes / wall time, fp64 scalar C, {threads} threads"
                      + (", with the numpy quantization and reconstruction of the rows)" if KV_INT8 else ")")}


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak


def prefill_flops(seqlens, hq, d, causal):
    """Algorithmic flops of packed prefill: 2 d for q.k and 2 d for p.v per attended
    (query, key) pair -- the unmasked pairs only when causal."""
    pairs = sum(n * (n + 1) // 2 for n in seqlens) if causal else sum(n * n for n in seqlens)
    return 4 * d * hq * pairs


def prefill_cpu_baseline(W, hq, hkv, causal, n=4096, seed=7):
    """The fp64 oracle on a bounded sample: one of the sequences (n rows, all hq heads)."""
    import oracle
    q, k, v, cu = W.varlen_inputs([n], hq, hkv, seed=seed, head_dim=D)
    args = (q.double().numpy(), k.double().numpy(), v.double().numpy(), cu.numpy())
    t0 = time.perf_counter()
    oracle.varlen_prefill(*args, causal=causal)
    dt = time.perf_counter() - t0
    return {"value": round(prefill_flops([n], hq, D, causal) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"one segment of {n} rows x {hq} query heads ({hkv} KV heads), "
                      f"{'causal' if causal else 'non-causal'}, fp64 scalar C, 1 thread"}


def bench_prefill(args):
    """Packed varlen prefill: 16 sequences of 4096 tokens, 8 query / 2 KV heads of d 64 (or
    the --shape's heads), fp16, causal (the long-prompt prefill shape; MFMA-bound)."""
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    seqlens, causal = [4096] * 16, True
    hq, hkv = (8, 2) if args.shape == DEFAULT_SHAPE else (HQ, HKV)
    q, k, v, cu = W.varlen_inputs(seqlens, hq, hkv, head_dim=D)
    q, k, v, cu = q.cuda(), k.cuda(), v.cuda(), cu.cuda()
    out = torch.empty_like(q)
    for _ in range(args.warmup):
        kvp.varlen_causal_prefill(q, k, v, cu, max(seqlens), causal=causal, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        kvp.varlen_causal_prefill(q, k, v, cu, max(seqlens), causal=causal, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = prefill_flops(seqlens, hq, D, causal)
    tflops = flops / (ms * 1e-3) / 1e12
    # the oracle's sample: one 4096-row segment, or 1536 rows at the wider head shapes
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(W, hq, hkv, causal,
                                                                 n=4096 if hq * D <= 512 else 1536)
    print(f"[bench] prefill {len(seqlens)} x {seqlens[0]} tokens, {hq}q/{hkv}kv heads: {ms * 1e3:.1f} us per call, "
          f"{tflops:.1f} TFLOP/s ({tflops / MFMA_F16_PEAK_TFLOPS * 100:.1f}% of the fp16 MFMA peak)",
          file=sys.stderr, flush=True)
    line = {
        "metric": "packed causal prefill attention TFLOP/s (% of MFMA fp16 peak)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"packed varlen causal prefill, {len(seqlens)} sequences x {seqlens[0]} tokens, "
                               f"{hq}q/{hkv}kv heads d{D} fp16", "sequences": len(seqlens),
                   "seq_len": seqlens[0]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "varlen_causal_prefill (prefill_mfma_f16_kernel)", "flops_per_launch": flops,
                     "avg_launch_us": round(ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def chunk_flops(prefixes, chunks, hq, d):
    """Algorithmic flops of new rows against a cache: row i of a chunk of m after a prefix
    of C attends to C + i + 1 positions, 4 d flops per (row, position) per query head."""
    pairs = sum(m * c + m * (m + 1) // 2 for c, m in zip(prefixes, chunks))
    return 4 * d * hq * pairs


def bench_chunked_prefill(args):
    """Chunked prefill into a shared prefix: 16 requests forked from one 2048-token prompt
    (copy-on-write blocks), each prefilling its own 512-token chunk against the paged cache;
    the model's 14 query / 2 KV heads of d 64 (or the --shape's heads), fp16."""
    import numpy as np
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B, prefix, chunk = 16, 2048, 512
    nblocks = prefix // BLOCK + B * (chunk // BLOCK) + 64
    pool = kvp.BlockPool(nblocks)
    pool.set_free_order(W.free_list_permutation(nblocks, args.seed + 1).tolist())
    cache = kvp.PagedKVCache(1, nblocks, HQ, HKV, torch.float16, "cuda", head_dim=D)
    cache.k_pool.copy_(W.randn_device(cache.k_pool.shape, args.seed + 10, torch.float16, "cuda"))
    cache.v_pool.copy_(W.randn_device(cache.v_pool.shape, args.seed + 11, torch.float16, "cuda"))
    base = pool.alloc(prefix)
    seqs = []
    for _ in range(B):
        s = pool.fork(base)
        pool.reserve(s, chunk)  # the chunk's K/V rows are the pool's seeded contents
        seqs.append(s)
    pool.free(base)
    max_blocks = (prefix + chunk) // BLOCK
    table, ctx = pool.export(seqs, max_blocks)
    table, ctx = table.cuda(), ctx.cuda()
    cu = torch.tensor([0] + [chunk * (b + 1) for b in range(B)], dtype=torch.int32).cuda()
    q = W.randn_device((B * chunk, HQ, D), args.seed + 12, torch.float16, "cuda")
    out = torch.empty_like(q)
    call = lambda: kvp.paged_prefill_attention(cache, 0, q, table, ctx, cu, chunk, out=out)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flops = chunk_flops([prefix] * B, [chunk] * B, HQ, D)
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the oracle on one of the 16 requests (all heads, the whole chunk)
        K = torch.stack([cache.k_pool[0][table[0, j].item()] for j in range(max_blocks)]).permute(1, 0, 2, 3)
        V = torch.stack([cache.v_pool[0][table[0, j].item()] for j in range(max_blocks)]).permute(1, 0, 2, 3)
        K = K.reshape(HKV, -1, D)[None].double().cpu().numpy()
        V = V.reshape(HKV, -1, D)[None].double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.chunk_attention(q[:chunk].double().cpu().numpy(), K, V, np.array([prefix + chunk], np.int32),
                               np.array([0, chunk], np.int32))
        dt = time.perf_counter() - t0
        cpu = {"value": round(chunk_flops([prefix], [chunk], HQ, D) / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": 1, "kind": "oracle",
               "sample": f"one of the {B} requests (its {chunk} rows x {HQ} heads after the {prefix}-token prefix), "
                         "fp64 scalar C, 1 thread"}
    print(f"[bench] chunked prefill {B} x {chunk} rows after a shared {prefix}-token prefix: {ms * 1e3:.1f} us per "
          f"call, {tflops:.1f} TFLOP/s ({tflops / MFMA_F16_PEAK_TFLOPS * 100:.1f}% of the fp16 MFMA peak)",
          file=sys.stderr, flush=True)
    line = {
        "metric": "chunked prefill against the paged cache TFLOP/s (% of MFMA fp16 peak)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{B} requests forked from one {prefix}-token prompt, {chunk}-token chunk each, "
                               f"{HQ}q/{HKV}kv heads d{D} fp16, 16-token blocks", "requests": B,
                   "prefix": prefix, "chunk": chunk},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "paged_prefill_attention (prefill_mfma_f16_kernel, paged keys)",
                     "flops_per_launch": flops, "avg_launch_us": round(ms * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_batching(args):
    """Continuous vs static batching over the block pool (host scheduler, no GPU): 2000
    requests with SECTION 4's response lengths (normal(500, 200) clipped to 200..2048, seeded)
    and 0..255-token prompts on a pool of 8192 blocks of 16 tokens (the naive reservation of
    64 requests of 2048 tokens).  Times the library's scheduler against the oracle's loop."""
    import numpy as np

    import kv_cache_decode_paged_amd as kvp
    from oracle import batching as Bt
    rng = np.random.default_rng(args.seed)
    n, blocks = 2000, 8192
    outs = [int(x) for x in Bt.response_lengths(n, seed=args.seed)]
    prompts = [int(x) for x in rng.integers(0, 256, size=n)]
    runs = {}
    for name, slots, pol, alloc in (("paged continuous 160 places", 160, kvp.SCHED_CONTINUOUS, kvp.ALLOC_PAGED),
                                    ("paged static 160 places", 160, kvp.SCHED_STATIC, kvp.ALLOC_PAGED),
                                    ("naive continuous 64 places", 64, kvp.SCHED_CONTINUOUS, kvp.ALLOC_NAIVE),
                                    ("naive static 64 places", 64, kvp.SCHED_STATIC, kvp.ALLOC_NAIVE)):
        t0 = time.perf_counter()
        res, lat, svc = kvp.sched_simulate(prompts, outs, slots, pol, alloc, 2048 + 256, 16, blocks)
        dt = time.perf_counter() - t0
        runs[name] = (res, dt)
        print(f"[bench] {name}: {res.steps} steps, {res.tokens / res.steps:.1f} tokens/step, mean service "
              f"{res.mean_service:.1f} steps, utilisation {res.mean_utilisation * 100:.1f} %, peak blocks "
              f"{res.peak_blocks}, deferrals {res.deferrals}, stalls {res.stalls}; {dt * 1e3:.1f} ms host",
              file=sys.stderr, flush=True)
    main_res, main_dt = runs["paged continuous 160 places"]
    value = main_res.steps / main_dt
    cpu = None
    if not args.no_cpu_baseline:  # the oracle on the first 500 requests of the same run
        m = 500
        t0 = time.perf_counter()
        w = Bt.simulate(prompts[:m], outs[:m], 160, Bt.CONTINUOUS, Bt.PAGED, 2048 + 256, 16, blocks)
        dt = time.perf_counter() - t0
        cpu = {"value": round(w["steps"] / dt, 2), "unit": "simulated steps/s", "cores": 1, "kind": "oracle",
               "sample": f"the first {m} of the {n} requests, paged continuous, 160 places (pure-Python loop)"}
    st = runs["paged static 160 places"][0]
    nv = runs["naive continuous 64 places"][0]
    line = {
        "metric": "continuous batching over the block pool: simulated decode steps per second (host scheduler)",
        "value": round(value, 2), "unit": "steps/s", "n_gpus": 1, "steps": 1, "warmup": 0,
        "ms_per_step": round(main_dt * 1e3 / max(main_res.steps, 1), 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int64", "data": "synthetic",
        "config": {"workload": f"{n} requests, outputs normal(500, 200) clipped to 200..2048, prompts 0..255, "
                               f"pool of {blocks} blocks x 16 tokens",
                   "requests": n, "blocks": blocks},
        "continuous_vs_static_throughput": round(st.steps / main_res.steps, 3),
        "continuous_vs_static_service": round(st.mean_service / main_res.mean_service, 3),
        "paged_vs_naive_throughput": round(nv.steps / main_res.steps, 3),
        "utilisation_paged_pct": round(main_res.mean_utilisation * 100, 2),
        "utilisation_naive_pct": round(nv.mean_utilisation * 100, 2),
        "roofline": None,
        "roofline_note": "host-only scheduler: no GPU kernel runs in this workload",
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=200)
    ap.add_argument("--layers", type=int, default=None, help="default: the shape's layer count")
    ap.add_argument("--shape", choices=sorted(SHAPES), default=DEFAULT_SHAPE,
                    help="decode head shape (default 14q2kv_d64)")
    ap.add_argument("--kv-dtype", choices=["fp16", "int8"], default="fp16",
                    help="decode cache: fp16, or int8 codes with an fp16 scale per row")
    ap.add_argument("--kernel-reps", type=int, default=4, help="rounds of per-layer decode timing")
    ap.add_argument("--no-graph", action="store_true", help="launch the layers eagerly")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-share", action="store_true", help="plans without shared-prefix items")
    ap.add_argument("--long-items", action="store_true",
                    help="decode workload: plans with long items (KVP_PLAN_LONG_ITEMS, which sizes parts to "
                         "one generation of waves when a batch's private blocks far exceed them and leaves "
                         "smaller batches' plans as they are); always on for long_context")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--workload", choices=["decode", "long_context", "prefill", "chunked_prefill", "batching"],
                    default="decode",
                    help="decode: the batch-200 paged decode step (default); long_context: the same step "
                         "for 32 requests of 32768 cached tokens each (split-K across CUs, 537 MB per "
                         "layer); prefill: packed causal prefill of 16 x 4096 tokens; chunked_prefill: "
                         "16 x 512-token chunks after a shared 2048-token prefix in the paged cache; "
                         "batching: continuous vs static batching over the block pool (host scheduler)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Requests would be sharded across GPUs by whole sharing groups.", flush=True)
        sys.exit(2)
    set_shape(args.shape, args.kv_dtype == "int8")
    if args.kv_dtype == "int8" and args.workload not in ("decode", "long_context"):
        print("--kv-dtype int8 applies to the decode workloads", flush=True)
        sys.exit(2)
    if args.workload == "batching":
        bench_batching(args)
        return
    if args.workload == "prefill":
        bench_prefill(args)
        return
    if args.workload == "chunked_prefill":
        bench_chunked_prefill(args)
        return

    import numpy as np
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda"
    long_ctx = LONG_CONTEXT if args.workload == "long_context" else None
    B = LONG_BATCH if long_ctx is not None else args.batch
    L = args.layers if args.layers is not None else SHAPES[args.shape][0]
    total_steps = args.warmup + args.steps + 1
    t_setup = time.perf_counter()
    pb, pool, cache, seqs, max_blocks = build_state(kvp, torch, W, B, L, total_steps, args.seed, long_ctx)
    print(f"[bench] setup: B={B} layers={L} blocks={cache.num_blocks} max_blocks={max_blocks} "
          f"({time.perf_counter() - t_setup:.1f}s)", file=sys.stderr, flush=True)

    # static per-layer inputs of the step
    q = W.randn_device((L, B, HQ, D), args.seed + 500, torch.float16, dev)
    knew = W.randn_device((L, B, HKV, D), args.seed + 501, torch.float16, dev)
    vnew = W.randn_device((L, B, HKV, D), args.seed + 502, torch.float16, dev)
    out = torch.empty((L, B, HQ, D), dtype=torch.float16, device=dev)
    pairs_d = torch.empty((B, 2), dtype=torch.int32, device=dev)
    ids = torch.tensor(seqs, dtype=torch.int32)

    # the step's work plan (host-built from the block table, shared by the 24 layers): the
    # first plan fixes the item count (with room to grow) so every later plan launches the
    # same way and one captured graph replays all steps
    share = not args.no_share
    t0h = torch.empty((B, max_blocks), dtype=torch.int32)
    c0h = torch.empty((B,), dtype=torch.int32)
    probe_slots = torch.empty((B,), dtype=torch.int64)
    cows = (kvp.kvp_copy * B)()
    pool.export_raw(ids.data_ptr(), B, max_blocks, t0h.data_ptr(), c0h.data_ptr())
    c0h += total_steps + 1  # the longest contexts of this run (plan sizing only)
    long_items = args.long_items or long_ctx is not None  # fewer, longer parts for very large batches
    kv_dtype = torch.int8 if KV_INT8 else torch.float16
    plan0, _ = kvp.decode_plan_build(HQ, HKV, t0h, c0h, cache.num_blocks, share_prefix=share, head_dim=D,
                                     long_items=long_items, kv_dtype=kv_dtype)
    pad_items = plan0.n_items + 8 * 32  # room for one more round of CU slots per XCD queue
    img_bytes = kvp.decode_plan_bytes(HQ, HKV, B, max_blocks, pad_items, head_dim=D)
    hb = [dict(table=torch.empty((B, max_blocks), dtype=torch.int32).pin_memory(),
               ctx=torch.empty((B,), dtype=torch.int32).pin_memory(),
               slots=torch.empty((B,), dtype=torch.int64).pin_memory(),
               pairs=torch.empty((B, 2), dtype=torch.int32).pin_memory(),
               image=torch.empty((img_bytes,), dtype=torch.uint8).pin_memory(),
               plan=kvp.kvp_decode_plan()) for _ in range(2)]
    # two device plan buffers: step k's plan is uploaded on a copy stream into buffer k % 2
    # while step k - 1's layers (reading the other buffer) run; one captured graph per buffer
    plan_d = [torch.empty((img_bytes,), dtype=torch.uint8, device=dev) for _ in range(2)]
    copy_stream = torch.cuda.Stream()  # default priority
    uploaded = [torch.cuda.Event(), torch.cuda.Event()]
    released = [torch.cuda.Event(), torch.cuda.Event()]  # the layers that read buffer i are done
    in_use = [False, False]
    slot_cap = 2 * plan0.n_slots + B * HKV
    ws_plan = kvp.kvp_decode_plan()
    ws_plan.B, ws_plan.num_kv_heads, ws_plan.n_slots, ws_plan.head_dim = B, HKV, slot_cap, D
    ws = torch.zeros((max(kvp.decode_plan_workspace_bytes(ws_plan), 256),), dtype=torch.uint8, device=dev)
    done = [torch.cuda.Event(), torch.cuda.Event()]
    stream = torch.cuda.current_stream()
    launch_plan = [None]

    def layers_body(pd):
        # per layer: the new token's K/V go into the cache and the decode attends over it,
        # in one kernel following the step's plan
        for l in range(L):
            kvp.paged_decode_attention_planned(cache, l, q[l], launch_plan[0], pd, k_new=knew[l], v_new=vnew[l],
                                               out=out[l], workspace=ws)

    graphs = [None, None]
    record = []

    def step(k, keep=False):
        h = hb[k % 2]
        done[k % 2].synchronize()  # the copies that last read these pinned buffers are done
        pool.append_slots_raw(ids.data_ptr(), B, h["slots"].data_ptr(), cows)
        npairs = 0
        for i in range(B):
            if cows[i].src >= 0:
                h["pairs"][npairs, 0] = cows[i].src
                h["pairs"][npairs, 1] = cows[i].dst
                npairs += 1
        pool.export_raw(ids.data_ptr(), B, max_blocks, h["table"].data_ptr(), h["ctx"].data_ptr())
        plan, _ = kvp.decode_plan_build(HQ, HKV, h["table"], h["ctx"], cache.num_blocks, share_prefix=share,
                                        image=h["image"], pad_items=pad_items, plan=h["plan"], head_dim=D,
                                        long_items=long_items, kv_dtype=kv_dtype)
        if launch_plan[0] is None:  # the launch arguments: this layout, slots up to slot_cap, ids
            launch_plan[0] = kvp.kvp_decode_plan.from_buffer_copy(plan)  # up to the buffer's end
            launch_plan[0].n_slots = slot_cap
            launch_plan[0].n_ids = (img_bytes - plan.off_ids) // 4
        lp = launch_plan[0]
        assert plan.n_slots <= slot_cap, "workspace too small for this step's plan"
        assert (plan.n_items, plan.off_pair_base, plan.off_req_shared, plan.off_ids) == \
            (lp.n_items, lp.off_pair_base, lp.off_req_shared, lp.off_ids)
        assert plan.off_ids + 4 * plan.n_ids <= img_bytes
        if keep:
            record.append((h["table"].numpy().copy(), h["ctx"].numpy().copy(), npairs, plan.n_shared,
                           plan.kv_blocks_read))
        i = k % 2
        if in_use[i]:  # step k - 2 read this buffer
            copy_stream.wait_event(released[i])
        with torch.cuda.stream(copy_stream):
            plan_d[i][: plan.bytes].copy_(h["image"][: plan.bytes], non_blocking=True)
            uploaded[i].record(copy_stream)
        if npairs:
            pairs_d[:npairs].copy_(h["pairs"][:npairs], non_blocking=True)
            kvp.kv_copy_blocks(cache, pairs_d[:npairs])
        stream.wait_event(uploaded[i])
        if graphs[i] is not None:
            graphs[i].replay()
        else:
            layers_body(plan_d[i])
        released[i].record(stream)
        in_use[i] = True
        done[i].record(stream)  # also covers the upload, which the layers waited for

    # first step eagerly (loads code objects), then capture the 24-layer body
    step(0)
    torch.cuda.synchronize()
    if not args.no_graph:
        for i in range(2):
            graphs[i] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[i]):
                layers_body(plan_d[i])
        torch.cuda.synchronize()
    k = 1
    for _ in range(args.warmup):
        step(k)
        k += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(k, keep=True)
        k += 1
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # bytes of the timed steps
    uniq_tok = [unique_and_logical_tokens(t, c) for t, c, _, _, _ in record]
    uniq_bytes_step = np.mean([u for u, _ in uniq_tok]) * KV_TOKEN_LAYER_BYTES * L
    logical_bytes_step = np.mean([lg for _, lg in uniq_tok]) * KV_TOKEN_LAYER_BYTES * L
    cow_blocks = sum(r[2] for r in record)
    value = uniq_bytes_step / (ms_per_step * 1e-3) / 1e9
    logical_gbps = logical_bytes_step / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] {ms_per_step:.4f} ms/step, unique {uniq_bytes_step / 1e9:.3f} GB/step -> {value:.1f} GB/s, "
          f"logical {logical_gbps:.1f} GB/s, COW blocks in timed steps {cow_blocks}", file=sys.stderr, flush=True)

    # ---- dominant kernel: the paged decode call, timed per call with HIP events on the
    # stream it runs on; layers are cycled so each call reads cold data (the 24-layer
    # working set is far larger than the on-chip caches) ----
    table_last, ctx_last, _, n_shared_last, blocks_read_last = record[-1]
    call_bytes, call_uniq, call_logical = decode_call_bytes(table_last, ctx_last, B)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.kernel_reps * L)]
    torch.cuda.synchronize()
    i = 0
    for r in range(args.kernel_reps):
        for l in range(L):
            evs[i][0].record(stream)
            kvp.paged_decode_attention_planned(cache, l, q[l], launch_plan[0], plan_d[(k - 1) % 2], k_new=knew[l],
                                               v_new=vnew[l], out=out[l], workspace=ws)
            evs[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b) for a, b in evs]
    avg_ms = float(np.mean(durs[L:])) if len(durs) > L else float(np.mean(durs))  # skip the first round
    achieved = call_bytes / (avg_ms * 1e-3) / 1e9
    print(f"[bench] decode call avg {avg_ms * 1e3:.2f} us over {len(durs) - L} calls, {call_bytes / 1e6:.2f} MB "
          f"-> {achieved:.1f} GB/s ({achieved / HBM_PEAK_GBPS * 100:.1f}% of peak)", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline and long_ctx is None:
        cpu = cpu_baseline(W, L)
        print(f"[bench] cpu oracle {cpu}", file=sys.stderr, flush=True)

    line = {
        "metric": ("decode attention KV GB/s (% of HBM peak) + decode steps/sec at batch 200" if long_ctx is None
                   else "long-context split-K decode attention KV GB/s (% of HBM peak) + decode steps/sec"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if not KV_INT8 else "i8 cache (fp16 scales), f16 arithmetic",
        "data": "synthetic",
        "config": {"workload": f"paged GQA decode step, batch {B}, {L} layers x fused (append + paged decode), "
                               f"{HQ}q/{HKV}kv heads d{D} "
                               + ("int8 cache (absmax codes, fp16 scale per row)" if KV_INT8 else "fp16")
                               + (", 16-token blocks, contexts U{128..2048}, "
                                  "groups of 8 sharing a 512-token prefix (copy-on-write)" if long_ctx is None else
                                  f", 16-token blocks, every context {long_ctx} tokens (+1 per step), no sharing"),
                   "batch": B, "layers": L, "shape": args.shape, "kv_dtype": args.kv_dtype,
                   "graph": graphs[0] is not None},
        "steps_per_sec": round(1e3 / ms_per_step, 2),
        "hbm_pct": round(value / HBM_PEAK_GBPS * 100, 2),
        "logical_GBps": round(logical_gbps, 2),
        "unique_GB_per_step": round(uniq_bytes_step / 1e9, 4),
        "logical_GB_per_step": round(logical_bytes_step / 1e9, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic() if (args.shape == DEFAULT_SHAPE and B == 200
                                                       and long_ctx is None and not KV_INT8) else None,
                     "traffic_unit": "bytes per launch (HBM read + write, counters)",
                     "kernel": "paged_decode_attention_planned (decode_f16_kernel: append + attention + "
                               "split merge)",
                     "bytes_per_launch": int(call_bytes), "avg_launch_us": round(avg_ms * 1e3, 3)},
        "plan": {"items": int(launch_plan[0].n_items), "shared_items": int(n_shared_last),
                 "kv_block_reads": int(blocks_read_last), "share_prefix": share, "long_items": long_items},
        "cpu_baseline": cpu,
    }
    print(f"[bench] decode sources digest {decode_sources_digest()}", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
