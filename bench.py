#!/usr/bin/env python3
"""Benchmark: paged grouped-query decode steps at batch 200 on one MI355X.

Workload (synthetic, seeded): the pages' 24-layer model shape (14 query heads, 2 KV heads,
head_dim 64, fp16), a paged cache of 16-token blocks, 200 requests with context lengths
uniform on 128..2048, groups of 8 consecutive requests sharing a 512-token prefix
(copy-on-write), block ids scattered by a seeded shuffle of the free list.

One step (kv_cache_decode_paged_amd.runner.DecodeStepRunner, the same driver the GPU tests
check against the oracle) = the host block manager reserves one slot per request (copy-on-
write pairs included), the host planner turns the block table into the step's work plan
(shared prefixes read once per group of members), the plan is uploaded on a copy stream
into one of two device buffers and the copy-on-write block copies run, then for each of
the 24 layers one kernel appends the new token's K/V and runs the paged decode attention
over the whole cache (paged_decode_attention_planned, replayed as one captured graph).
Contexts grow by one token per step.

Printed: one JSON line with the decode-attention KV throughput (unique bytes), steps/s,
step-time median / min / max, the roofline of the dominant kernel (per-launch time from
the graph-replayed layers), the achievable read bandwidth of a plain streaming kernel, a
check of the last step's outputs against the fp64 oracle, and the oracle timed on host
cores (all cores and one thread) on a bounded sample of the same data.

Other workloads (--workload): long_context (32 x 32768 tokens, split-K), batch1 (24 layers,
batch 1, contexts 16/64/256/1024), single_head (fp32, 40-token prefill + 48 decode steps,
contiguous cache), varlen (packed prefills (37,120,8,200) x 8 heads and 2 x 256 with 8q/2kv),
prefill (16 x 4096 causal, the MFMA shape), chunked_prefill, batching (host scheduler), and
suite (every configuration above plus batches 10/50/100/200, one JSON line each).
"""
import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
# the long-context decode configuration: 32 requests of 32768 cached tokens
LONG_BATCH, LONG_CONTEXT = 32, 32768
HQ, HKV, D, BLOCK = 14, 2, 64, 16
KV_TOKEN_LAYER_BYTES = 2 * HKV * D * 2  # K and V, fp16: 512 B per token per layer
FLUSH_BYTES = 512 << 20  # written between cold steps: larger than the 256 MB of on-die cache
COLD_LIMIT = 1 << 30     # steps with working sets below this are also timed cold

# head shapes of the decode step: (layers, query heads, KV heads, head dim, description)
SHAPES = {
    "14q2kv_d64": (24, 14, 2, 64, "24 layers, 14q/2kv heads d64"),
    # the 7B-class GQA shape (32 layers, 8 KV heads of d = 128) with 32 query heads
    "32q8kv_d128": (32, 32, 8, 128, "32 layers, 32q/8kv heads d128 (7B-class GQA)"),
    # the same model as plain multi-head attention (32 KV heads)
    "32q32kv_d128": (32, 32, 32, 128, "32 layers, 32q/32kv heads d128 (MHA)"),
    # multi-query attention: every query head on one KV head (the chapter's 14-head model
    # as MQA, and the 7B-class 32 heads)
    "14q1kv_d64": (24, 14, 1, 64, "24 layers, 14q/1kv heads d64 (MQA)"),
    "32q1kv_d128": (32, 32, 1, 128, "32 layers, 32q/1kv heads d128 (MQA)"),
}
DEFAULT_SHAPE = "14q2kv_d64"

KV_INT8 = False  # the cache holds int8 codes and one fp16 scale per row
SCATTER = True   # block ids handed out from a shuffled free list (False: in order)


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
    """(bytes per decode launch, trace mean us) from the recorded profile, or (None, None)
    when the summary is missing or was measured on other sources."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None, None
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)\s+sources:\s*([0-9a-f]+)", text)
    if not m or m.group(2) != decode_sources_digest():
        return None, None
    t = re.search(r"trace_mean_us:\s*([0-9.]+)", text)
    return int(m.group(1)), (float(t.group(1)) if t else None)


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


def step_stats(ms):
    """median / min / max / mean of a list of step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 5), "min_ms": round(float(a.min()), 5),
            "max_ms": round(float(a.max()), 5), "mean_ms": round(float(a.mean()), 5), "n": int(a.size)}


def host_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_units(fn, units, threads):
    """Run fn over units on `threads` host threads (the oracle's C loops release the GIL);
    returns (results, seconds)."""
    t0 = time.perf_counter()
    if threads == 1:
        res = [fn(u) for u in units]
    else:
        with cf.ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(fn, units))
    return res, time.perf_counter() - t0


class Flusher:
    """Writes FLUSH_BYTES of device memory, evicting the on-die caches between cold steps."""

    def __init__(self, torch, dev="cuda"):
        self.buf = torch.empty((FLUSH_BYTES,), dtype=torch.uint8, device=dev)
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(self.k & 0xff)


def event_times(torch, fn, reps, before=None, stream=None):
    """Per-rep device time (ms) of fn() bracketed by events on the current stream; before()
    runs outside the bracket (and is synchronised when given)."""
    stream = stream or torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        if before is not None:
            before()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        out.append(a.elapsed_time(b))
    return out


def read_probe(torch, kvp, layer_bytes, layers=24):
    """Achievable read bandwidth of a plain streaming kernel (kvp_read_bandwidth_probe): a
    cold 1 GiB read, and launches that each read one window the size of a decode launch's
    bytes, `layers` windows in a row captured in one graph and replayed like the decode
    layers (each window is evicted before it is read again: the windows cover 1 GiB)."""
    import numpy as np
    n = 1 << 30
    buf = torch.ones((n // 4,), dtype=torch.int32, device="cuda")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    flat = buf.view(torch.uint8)
    kvp.read_bandwidth_probe(flat, sink=sink)  # warm-up (code load)
    torch.cuda.synchronize()
    full = event_times(torch, lambda: kvp.read_bandwidth_probe(flat, sink=sink), 5)
    wb = max(16, int(layer_bytes) // 4096 * 4096)
    nwin = max(1, n // wb)
    wins = [flat[i * wb:(i + 1) * wb] for i in range(nwin)]
    res = {"GBps_1GiB": round(n / (float(np.median(full)) * 1e-3) / 1e9, 1), "launch_sized_bytes": wb,
           "kernel": "kvp_read_bandwidth_probe (16-byte loads, 8 in flight per lane)"}
    best = None
    for wpc in (8, 16):  # waves per CU
        waves = wpc * 256
        graphs = []
        for g0 in range(2):  # two graphs over disjoint windows, replayed alternately
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for l in range(layers):
                    kvp.read_bandwidth_probe(wins[(g0 * layers + l) % nwin], waves=waves, sink=sink)
            graphs.append(g)
        torch.cuda.synchronize()
        k = [0]

        def rep():
            graphs[k[0] % 2].replay()
            k[0] += 1
        us = float(np.median(event_times(torch, rep, 10))) * 1e3 / layers
        res[f"us_per_launch_{wpc}w"] = round(us, 3)
        if best is None or us < best:
            best = us
        del graphs
    res["us_launch_sized"] = round(best, 3)
    res["GBps_launch_sized"] = round(wb / (best * 1e-6) / 1e9, 1)
    res["launch_sized_from"] = f"graph replay of {layers} launches / {layers}, median of 10, best of 8 / 16 waves per CU"
    del buf, wins, flat
    return res


# ---------------------------------------------------------------------------------------
# decode state
# ---------------------------------------------------------------------------------------
def build_state(kvp, torch, W, ctx_before, group, prefix, layers, total_steps, seed):
    """Block pool, cache (every slot seeded N(0,1)) and the batch's sequences: groups fork
    their prefix, then each member truncates to a shorter context or reserves its private
    tokens; a request alone in its group (or prefix 0) gets a private sequence."""
    dev = "cuda"
    B = len(ctx_before)
    ngroups = len(set(group))
    need = sum(math.ceil((c + total_steps + 1) / BLOCK) for c in ctx_before) + B + 64
    need += ngroups * math.ceil(prefix / BLOCK)
    num_blocks = need
    max_blocks = math.ceil((max(ctx_before) + total_steps + 1) / BLOCK)
    pool = kvp.BlockPool(num_blocks)
    if SCATTER:  # block ids from a seeded shuffle of the free list: scattered tables
        pool.set_free_order(W.free_list_permutation(num_blocks, seed + 1).tolist())
    cache = kvp.PagedKVCache(layers, num_blocks, HQ, HKV, torch.int8 if KV_INT8 else torch.float16, dev,
                             head_dim=D)
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
    seqs = [None] * B
    for gi in sorted(set(group)):
        members = [i for i in range(B) if group[i] == gi]
        if prefix > 0 and len(members) > 1:
            pre = pool.alloc(prefix)
            for i in members:
                s = pool.fork(pre)
                L = ctx_before[i]
                if L < prefix:
                    pool.truncate(s, L)
                elif L > prefix:
                    pool.reserve(s, L - prefix)
                seqs[i] = s
            pool.free(pre)
        else:
            for i in members:
                seqs[i] = pool.alloc(ctx_before[i])
    return pool, cache, seqs, max_blocks


def snapshot_state(torch, pool, cache, seqs, max_blocks, layers):
    """Host copies of the cache layers `layers` and of the tables before the first step:
    the oracle's inputs are read from these and from the appended rows, never from what
    the kernels later wrote into the cache."""
    import numpy as np
    B = len(seqs)
    table = torch.empty((B, max_blocks), dtype=torch.int32)
    ctx = torch.empty((B,), dtype=torch.int32)
    ids = torch.tensor(seqs, dtype=torch.int32)
    pool.export_raw(ids.data_ptr(), B, max_blocks, table.data_ptr(), ctx.data_ptr())
    snap = {"table": table.numpy().copy(), "ctx": ctx.numpy().copy(), "layers": {}}
    for l in layers:
        ent = {"k": cache.k_pool[l].cpu().numpy(), "v": cache.v_pool[l].cpu().numpy()}
        if KV_INT8:
            ent["ks"] = cache.k_scale[l].cpu().numpy()
            ent["vs"] = cache.v_scale[l].cpu().numpy()
        snap["layers"][l] = ent
    return snap


def logical_rows(snap, l, b, ctx_final, knew_h, vnew_h):
    """fp64 K, V [Hkv, ctx_final, d] of request b in layer l after the run: positions below
    its context before the first step come from the snapshot through the first table; every
    later position holds the step's appended row (the same knew / vnew each step)."""
    import numpy as np
    from oracle import kvquant as KQ
    c0 = int(snap["ctx"][b])
    ent = snap["layers"][l]
    j = np.arange(c0)
    blk = snap["table"][b, j // BLOCK]
    row = j % BLOCK
    K = np.empty((HKV, ctx_final, D), dtype=np.float64)
    V = np.empty_like(K)
    if KV_INT8:
        K[:, :c0] = (ent["k"][blk, :, row, :].astype(np.float64) *
                     ent["ks"][blk, :, row].astype(np.float64)[..., None]).transpose(1, 0, 2)
        V[:, :c0] = (ent["v"][blk, :, :, row].astype(np.float64) *
                     ent["vs"][blk, :, row].astype(np.float64)[..., None]).transpose(1, 0, 2)
        kn = KQ.dequantize_rows(*KQ.absmax_quantize_rows(knew_h[l, b]))
        vn = KQ.dequantize_rows(*KQ.absmax_quantize_rows(vnew_h[l, b]))
    else:
        K[:, :c0] = ent["k"][blk, :, row, :].astype(np.float64).transpose(1, 0, 2)
        V[:, :c0] = ent["v"][blk, :, row, :].astype(np.float64).transpose(1, 0, 2)
        kn = knew_h[l, b].astype(np.float64)
        vn = vnew_h[l, b].astype(np.float64)
    K[:, c0:] = kn[:, None, :]
    V[:, c0:] = vn[:, None, :]
    return K, V


def decode_check_and_baseline(torch, snap, rec, q, knew, vnew, out, layers, one_thread_layers, total_layers):
    """The oracle on the bench's own data after the last step: every request of `layers`
    on all host threads (timed: cpu_baseline), and every request of the first
    `one_thread_layers` of them again on one thread (timed); the outputs of the last step are
    compared with it.  The inputs of one layer are assembled (untimed) before that layer's
    oracle runs.  Rates use the GPU line's unit: the step's unique K/V bytes per layer times
    the layers computed, over the oracle's wall time."""
    import numpy as np

    import oracle
    B = q.shape[1]
    ctx = rec.ctx
    knew_h, vnew_h = knew.cpu().numpy(), vnew.cpu().numpy()
    q_h = q.cpu().numpy()
    out_h = out.cpu().numpy()
    threads = host_threads()
    secs = secs1 = 0.0
    err = 0.0
    n1 = min(len(layers), one_thread_layers)
    for li, l in enumerate(layers):
        inputs = []
        for b in range(B):
            K, V = logical_rows(snap, l, b, int(ctx[b]), knew_h, vnew_h)
            inputs.append((q_h[l, b:b + 1].astype(np.float64), K[None], V[None]))

        def one(b):
            qq, K, V = inputs[b]
            return oracle.decode_gqa(qq, K, V, np.array([K.shape[2]], dtype=np.int32))
        res, dt = run_units(one, list(range(B)), threads)
        secs += dt
        for b, want in enumerate(res):
            err = max(err, float(np.abs(out_h[l, b].astype(np.float64) - want[0]).max()))
        if li < n1:
            _, dt1 = run_units(one, list(range(B)), 1)
            secs1 += dt1
        del inputs
    _, uniq, logical = decode_call_bytes(rec.table, ctx, B)
    uniq_b, logical_b = uniq * KV_TOKEN_LAYER_BYTES, logical * KV_TOKEN_LAYER_BYTES
    tol = 2e-3
    check = {"layers": list(layers), "requests": B, "max_abs_err": err, "tol": tol, "ok": bool(err <= tol),
             "reference": "fp64 oracle on the initial cache snapshot + the appended rows"}
    what = (f"all {total_layers} layers" if len(layers) == total_layers else
            f"{len(layers)} of {total_layers} layers")
    cpu = {"value": round(uniq_b * len(layers) / secs / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{what} x all {B} requests of the last timed step, fp64 scalar C on {threads} host threads "
                     f"(unique K/V bytes of the layers computed / wall time, as the GPU value)",
           "seconds": round(secs, 3),
           "logical_GBps": round(logical_b * len(layers) / secs / 1e9, 4),
           "one_thread": {"value": round(uniq_b * n1 / secs1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "sample": f"{n1} layer(s) x all {B} requests, 1 thread",
                          "seconds": round(secs1, 3)},
           "step_seconds": {"all_cores": round(secs / len(layers) * total_layers, 3),
                            "one_thread": round(secs1 / n1 * total_layers, 3),
                            "note": f"all {B} requests x {total_layers} layers"
                                    + ("" if len(layers) == total_layers else " (scaled from the sample)")}}
    return check, cpu


def decode_line(args, metric, B, L, ctx_before, group, prefix, long_items, share, workload_desc, extra_cfg,
                check_layers, one_thread_layers):
    """Build the state, run the steps through DecodeStepRunner and return the JSON line."""
    import numpy as np
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W
    from kv_cache_decode_paged_amd.runner import DecodeStepRunner
    dev = "cuda"
    total_steps = 1 + args.warmup + args.steps + args.cold_steps
    t_setup = time.perf_counter()
    pool, cache, seqs, max_blocks = build_state(kvp, torch, W, ctx_before, group, prefix, L, total_steps, args.seed)
    print(f"[bench] {workload_desc}: setup B={B} layers={L} blocks={cache.num_blocks} max_blocks={max_blocks} "
          f"({time.perf_counter() - t_setup:.1f}s)", file=sys.stderr, flush=True)
    q = W.randn_device((L, B, HQ, D), args.seed + 500, torch.float16, dev)
    knew = W.randn_device((L, B, HKV, D), args.seed + 501, torch.float16, dev)
    vnew = W.randn_device((L, B, HKV, D), args.seed + 502, torch.float16, dev)
    out = torch.empty((L, B, HQ, D), dtype=torch.float16, device=dev)
    want_cpu = not args.no_cpu_baseline
    snap = snapshot_state(torch, pool, cache, seqs, max_blocks, check_layers) if want_cpu else None
    runner = DecodeStepRunner(cache, pool, seqs, max_blocks, q, knew, vnew, out, share_prefix=share,
                              long_items=long_items, graph=not args.no_graph, grow_tokens=total_steps + 1,
                              spare_items=8 * 32 if B >= 8 else 8, share_width=args.share_width,
                              fill={"auto": "auto", "on": True, "off": False}[args.fill])
    stream = runner.stream
    runner.step()  # first step: eager launches (code objects load), the first copy-on-write; graphs captured
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        runner.step()
    torch.cuda.synchronize()
    # warm: steps back to back, the host planning of step k + 1 beside the device work of k
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    records = []
    host = np.zeros((args.steps, 2))  # host seconds of prepare() and launch() per step
    t0 = time.perf_counter()
    for s in range(args.steps):
        ta = time.perf_counter()
        rec = runner.prepare(keep=True)
        tb = time.perf_counter()
        evs[s][0].record(stream)
        runner.launch()
        evs[s][1].record(stream)
        host[s] = (tb - ta, time.perf_counter() - tb)
        records.append(rec)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    warm = step_stats([a.elapsed_time(b) for a, b in evs])
    uniq_tok = [unique_and_logical_tokens(r.table, r.ctx) for r in records]
    uniq_bytes_step = float(np.mean([u for u, _ in uniq_tok])) * KV_TOKEN_LAYER_BYTES * L
    logical_bytes_step = float(np.mean([lg for _, lg in uniq_tok])) * KV_TOKEN_LAYER_BYTES * L
    cow_blocks = sum(len(r.cow_pairs) for r in records)
    value = uniq_bytes_step / (ms_per_step * 1e-3) / 1e9
    logical_gbps = logical_bytes_step / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] {ms_per_step:.4f} ms/step (events: median {warm['median_ms']:.4f}, min {warm['min_ms']:.4f}, "
          f"max {warm['max_ms']:.4f}), unique {uniq_bytes_step / 1e9:.3f} GB/step -> {value:.1f} GB/s, logical "
          f"{logical_gbps:.1f} GB/s, COW blocks in timed steps {cow_blocks}", file=sys.stderr, flush=True)
    host_us = {"prepare_median": round(float(np.median(host[:, 0])) * 1e6, 1),
               "launch_median": round(float(np.median(host[:, 1])) * 1e6, 1),
               "first_step": round(float(host[0].sum()) * 1e6, 1)}
    print(f"[bench] host per step: prepare {host_us['prepare_median']} us, launch {host_us['launch_median']} us "
          f"(medians; the first step's {host_us['first_step']} us run before any device work)", file=sys.stderr,
          flush=True)
    # cold: each step alone after a 512 MB write, when the step's bytes could sit in the
    # on-die caches
    cold = None
    if args.cold_steps > 0 and uniq_bytes_step < COLD_LIMIT:
        flush = Flusher(torch)
        cms = []
        for _ in range(args.cold_steps):
            records.append(runner.prepare(keep=True))
            flush()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            runner.launch()
            b.record(stream)
            b.synchronize()
            cms.append(a.elapsed_time(b))
        cold = step_stats(cms)
        cold["GBps_unique_median"] = round(uniq_bytes_step / (cold["median_ms"] * 1e-3) / 1e9, 2)
        del flush
        print(f"[bench] cold steps: median {cold['median_ms']:.4f} ms ({cold['GBps_unique_median']:.1f} GB/s)",
              file=sys.stderr, flush=True)

    # ---- dominant kernel: the layers' launches alone, replayed from the last step's graph
    # (no host work between them); per launch = replay time / layers ----
    torch.cuda.synchronize()
    reps = max(3, args.kernel_reps)
    rep_ms = event_times(torch, runner.replay_layers, reps, stream=stream)
    launch_ms = float(np.median(rep_ms)) / L
    last = records[-1]
    call_bytes, call_uniq, call_logical = decode_call_bytes(last.table, last.ctx, B)
    achieved = call_bytes / (launch_ms * 1e-3) / 1e9
    print(f"[bench] decode launch {launch_ms * 1e3:.2f} us (graph replay of {L} layers, median of {reps}), "
          f"{call_bytes / 1e6:.2f} MB -> {achieved:.1f} GB/s ({achieved / HBM_PEAK_GBPS * 100:.1f}% of peak)",
          file=sys.stderr, flush=True)
    traffic, trace_us = (None, None)
    if args.shape == DEFAULT_SHAPE and B == 200 and not long_items and not KV_INT8 and share:
        traffic, trace_us = measured_traffic()
    probe = None if args.no_probe else read_probe(torch, kvp, call_bytes, L)
    if probe:
        print(f"[bench] read probe {probe}", file=sys.stderr, flush=True)
    check = cpu = None
    if want_cpu:
        check, cpu = decode_check_and_baseline(torch, snap, last, q, knew, vnew, out, check_layers,
                                                one_thread_layers, L)
        print(f"[bench] check {check}\n[bench] cpu oracle {cpu}", file=sys.stderr, flush=True)
    part_rec = (HQ // HKV) * (D + 4) * 4  # one partial record: G rows of (o[d], m, l, 2 pad) fp32
    line = {
        "metric": metric,
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
        "config": dict({"workload": workload_desc, "batch": B, "layers": L, "shape": args.shape,
                        "kv_dtype": "int8" if KV_INT8 else "fp16", "graph": runner.graphs[0] is not None,
                        "scattered_blocks": SCATTER},
                       **extra_cfg),
        "steps_per_sec": round(1e3 / ms_per_step, 2),
        "hbm_pct": round(value / HBM_PEAK_GBPS * 100, 2),
        "logical_GBps": round(logical_gbps, 2),
        "unique_GB_per_step": round(uniq_bytes_step / 1e9, 4),
        "logical_GB_per_step": round(logical_bytes_step / 1e9, 4),
        "step_time_warm": warm,
        "host_us": host_us,
        "step_time_cold": cold,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM read + write, counters)",
                     "traffic_ratio": round(traffic / call_bytes, 4) if traffic else None,
                     "trace_mean_us": trace_us,
                     "kernel": "paged_decode_attention_planned (decode_f16_kernel: append + attention + "
                               "split merge)",
                     "bytes_per_launch": int(call_bytes), "avg_launch_us": round(launch_ms * 1e3, 3),
                     "avg_launch_from": f"graph replay of the {L} layers / {L}, median of {reps}"},
        "hbm_read_probe": probe,
        "split_overhead": {"partials_per_launch": int(last.split_partials),
                           "record_bytes": part_rec,
                           "bytes_per_launch": 2 * int(last.split_partials) * part_rec,
                           "note": "fp32 (m, l, o) partials of split pairs, stored and read back once each; "
                                   "implementation overhead, not in bytes_per_launch"},
        "plan": {"items": int(last.n_items), "shared_items": int(last.n_shared),
                 "kv_block_reads": int(last.kv_blocks_read), "share_prefix": share, "long_items": long_items,
                 "fill": bool(runner.fill),
                 "share_width": args.share_width},
        "check": check,
        "cpu_baseline": cpu,
    }
    print(f"[bench] decode sources digest {decode_sources_digest()}", file=sys.stderr, flush=True)
    del runner, cache, pool, q, knew, vnew, out
    torch.cuda.empty_cache()
    return line


def bench_decode(args, B=None):
    """The batch decode step (C4 shapes; head shapes and int8 by flag)."""
    import workloads as W
    B = args.batch if B is None else B
    L = args.layers if args.layers is not None else SHAPES[args.shape][0]
    pb = W.paged_batch(B)
    share = not args.no_share
    desc = (f"paged GQA decode step, batch {B}, {L} layers x fused (append + paged decode), {HQ}q/{HKV}kv heads "
            f"d{D} " + ("int8 cache (absmax codes, fp16 scale per row)" if KV_INT8 else "fp16") +
            ", 16-token blocks, contexts U{128..2048}, groups of 8 sharing a 512-token prefix (copy-on-write)")
    metric = ("decode attention KV GB/s (% of HBM peak) + decode steps/sec at batch 200" if B == 200 else
              f"decode attention KV GB/s (% of HBM peak) + decode steps/sec at batch {B}")
    return decode_line(args, metric, B, L, pb.ctx_before, pb.group, pb.prefix, args.long_items, share, desc, {},
                       check_layers=list(range(L)) if args.shape == DEFAULT_SHAPE else list(range(min(L, 4))),
                       one_thread_layers=2)


def bench_long_context(args):
    """32 requests of 32768 cached tokens, no sharing, split-K across CUs (long items)."""
    L = args.layers if args.layers is not None else SHAPES[args.shape][0]
    B = LONG_BATCH
    desc = (f"long-context split-K decode step, batch {B}, {L} layers x fused (append + paged decode), "
            f"{HQ}q/{HKV}kv heads d{D} " + ("int8 cache" if KV_INT8 else "fp16") +
            f", 16-token blocks, every context {LONG_CONTEXT} tokens (+1 per step), no sharing")
    return decode_line(args, "long-context split-K decode attention KV GB/s (% of HBM peak) + decode steps/sec", B,
                       L, [LONG_CONTEXT] * B, list(range(B)), 0, True, False, desc, {"context": LONG_CONTEXT},
                       check_layers=[0, 1], one_thread_layers=1)


def bench_batch1(args, contexts=(16, 64, 256, 1024)):
    """Batch 1, 24 layers, contexts C (cached before the step): a latency regime (the
    chapter's decode-step timing at 16..1024 cached tokens)."""
    lines = []
    L = args.layers if args.layers is not None else SHAPES[args.shape][0]
    for C in contexts:
        desc = (f"batch-1 decode step, {L} layers x fused (append + paged decode), {HQ}q/{HKV}kv heads d{D} fp16, "
                f"context {C} cached tokens (+1 per step)")
        line = decode_line(args, "batch-1 decode step latency (us per step) and KV GB/s", 1, L, [C], [0], 0, False,
                           False, desc, {"context": C}, check_layers=list(range(min(L, 24))), one_thread_layers=24)
        # the latency regime: the headline figure is the step time
        line["latency_regime"] = True
        line["value_GBps"] = line["value"]
        line["value"] = round(line["ms_per_step"] * 1e3, 3)
        line["unit"] = "us/step"
        line["higher_is_better"] = False
        lines.append(line)
    return lines


# ---------------------------------------------------------------------------------------
# single head fp32 (contiguous cache): 40-token prefill, then 48 decode steps
# ---------------------------------------------------------------------------------------
def bench_single_head(args):
    import numpy as np
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W
    dev = "cuda"
    q, k, v = W.single_head_sequence(args.seed)
    n = q.shape[0]
    P = W.SINGLE_PROMPT
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kc = torch.zeros((1, 1, n, 64), dtype=torch.float32, device=dev)
    vc = torch.zeros_like(kc)
    outs = torch.zeros((n, 1, 64), dtype=torch.float32, device=dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    ctxs = torch.arange(1, n + 1, dtype=torch.int32, device=dev)
    cu = torch.tensor([0, P], dtype=torch.int32, device=dev)
    ws = kvp.make_workspace(1, 1, torch.float32, 1, n)

    def prefill():
        # the prompt's K/V rows into the cache, then its causal prefill
        kc[0, 0, :P].copy_(kd[:P, 0])
        vc[0, 0, :P].copy_(vd[:P, 0])
        kvp.varlen_causal_prefill(qd[:P], kd[:P], vd[:P], cu, P, causal=True, out=outs[:P])

    def dstep(t):
        kvp.contiguous_kv_append(kc, vc, kd[t:t + 1], vd[t:t + 1], pos[t:t + 1])
        kvp.contiguous_decode_attention(qd[t:t + 1], kc, vc, ctxs[t:t + 1], out=outs[t:t + 1], workspace=ws)

    prefill()
    for t in range(P, n):
        dstep(t)
    torch.cuda.synchronize()
    reps = max(1, args.steps // 4)
    warm_pre, warm_dec = [], []
    for _ in range(reps):
        warm_pre += event_times(torch, prefill, 1)
        for t in range(P, n):
            warm_dec += event_times(torch, lambda: dstep(t), 1)
    flush = Flusher(torch)
    cold_pre = event_times(torch, prefill, 3, before=flush)
    cold_dec = []
    for t in range(P, n):
        cold_dec += event_times(torch, lambda: dstep(t), 1, before=flush)
    del flush
    got = outs.double().cpu().numpy()
    import oracle
    t0 = time.perf_counter()
    full = oracle.full_causal(q.double().numpy(), k.double().numpy(), v.double().numpy())
    secs = time.perf_counter() - t0
    err = float(np.abs(got[:, 0] - full[:, 0]).max())
    wd = step_stats(warm_dec)
    line = {
        "metric": "single-head fp32 decode step latency (us per step: append + attention)",
        "value": round(wd["median_ms"] * 1e3, 3), "unit": "us/step", "n_gpus": 1, "steps": len(warm_dec),
        "warmup": 1, "ms_per_step": wd["median_ms"], "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"1 head d64 fp32, contiguous cache [1,1,{n},64]: {P}-token causal prefill, then "
                               f"{n - P} decode steps (contiguous_kv_append + contiguous_decode_attention)",
                   "prompt": P, "decode_steps": n - P},
        "latency_regime": True,
        "step_time_warm": wd, "step_time_cold": step_stats(cold_dec),
        "prefill_us_warm": step_stats([x * 1e3 for x in warm_pre]),
        "prefill_us_cold": step_stats([x * 1e3 for x in cold_pre]),
        "roofline": None,
        "roofline_note": "launch-latency regime (22-45 KB per step): no roofline claim",
        "check": {"max_abs_err": err, "tol": 1e-5, "ok": bool(err <= 1e-5),
                  "reference": "fp64 oracle full causal recompute (every prompt and decode row)"},
        "cpu_baseline": {"value": round(secs * 1e6 / n, 3), "unit": "us per row (full recompute, all rows)",
                         "cores": 1, "kind": "oracle",
                         "sample": f"the whole {n}-row recompute (n x n scores, masked), fp64 scalar C, 1 thread"},
    }
    return line


# ---------------------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------------------
def prefill_flops(seqlens, hq, d, causal):
    """Algorithmic flops of packed prefill: 2 d for q.k and 2 d for p.v per attended
    (query, key) pair -- the unmasked pairs only when causal."""
    pairs = sum(n * (n + 1) // 2 for n in seqlens) if causal else sum(n * n for n in seqlens)
    return 4 * d * hq * pairs


def prefill_oracle(q, k, v, cu, causal, threads):
    """The oracle's packed prefill, one unit per query head on `threads` host threads;
    returns (out [T, Hq, d], seconds)."""
    import numpy as np

    import oracle
    hq, hkv = q.shape[1], k.shape[1]
    grp = hq // hkv
    q64, k64, v64, cu_n = q.double().numpy(), k.double().numpy(), v.double().numpy(), cu.cpu().numpy()

    def one(h):
        g = h // grp
        return oracle.varlen_prefill(np.ascontiguousarray(q64[:, h:h + 1]), np.ascontiguousarray(k64[:, g:g + 1]),
                                     np.ascontiguousarray(v64[:, g:g + 1]), cu_n, causal=causal)
    res, secs = run_units(one, list(range(hq)), threads)
    return np.concatenate(res, axis=1), secs


def varlen_line(args, name, seqlens, hq, hkv, causal, desc):
    import numpy as np
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W
    q, k, v, cu = W.varlen_inputs(seqlens, hq, hkv, head_dim=64)
    qd, kd, vd, cud = q.cuda(), k.cuda(), v.cuda(), cu.cuda()
    out = torch.empty_like(qd)
    call = lambda: kvp.varlen_causal_prefill(qd, kd, vd, cud, max(seqlens), causal=causal, out=out)
    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    warm = step_stats(event_times(torch, call, max(5, args.steps)))
    flush = Flusher(torch)
    cold = step_stats(event_times(torch, call, max(5, args.steps // 2), before=flush))
    del flush
    flops = prefill_flops(seqlens, hq, 64, causal)
    tf = flops / (warm["median_ms"] * 1e-3) / 1e12
    want, secs = prefill_oracle(q, k, v, cu, causal, host_threads())
    _, secs1 = prefill_oracle(q, k, v, cu, causal, 1)
    err = float(np.abs(out.double().cpu().numpy() - want).max())
    return {
        "metric": f"packed varlen prefill TFLOP/s (% of MFMA fp16 peak): {name}",
        "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": warm["n"], "warmup": max(1, args.warmup),
        "ms_per_step": warm["median_ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": desc, "seqlens": list(seqlens), "q_heads": hq, "kv_heads": hkv, "causal": causal},
        "latency_regime": True,
        "step_time_warm": warm, "step_time_cold": cold,
        "cold_TFLOPs": round(flops / (cold["median_ms"] * 1e-3) / 1e12, 3),
        "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 6), "traffic": None,
                     "kernel": "varlen_causal_prefill (prefill_mfma_f16_kernel)", "flops_per_launch": flops,
                     "avg_launch_us": round(warm["median_ms"] * 1e3, 3),
                     "note": "launch-bound at this size: a few microseconds of work per call"},
        "check": {"max_abs_err": err, "tol": 2e-3, "ok": bool(err <= 2e-3), "reference": "fp64 oracle, every row"},
        "cpu_baseline": {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": host_threads(),
                         "kind": "oracle", "sample": "the whole call (every row and head), fp64 scalar C",
                         "seconds": round(secs, 4),
                         "one_thread": {"value": round(flops / secs1 / 1e12, 6), "seconds": round(secs1, 4)}},
    }


def bench_varlen(args):
    """The pages' packed prefills at their own sizes: seqlens (37, 120, 8, 200) with 8 heads
    (causal, and the block-diagonal non-causal form of the demo), and B = 2 x M = 256 with
    8 query / 2 KV heads (the GQA demo, non-causal, and causal)."""
    out = []
    for causal in (True, False):
        out.append(varlen_line(args, f"seqlens (37,120,8,200) x 8 heads {'causal' if causal else 'non-causal'}",
                               (37, 120, 8, 200), 8, 8, causal,
                               "packed varlen prefill, seqlens (37, 120, 8, 200), 8 heads d64 fp16, "
                               + ("causal" if causal else "block-diagonal (non-causal)")))
    for causal in (False, True):
        out.append(varlen_line(args, f"2 x 256, 8q/2kv {'causal' if causal else 'non-causal'}", (256, 256), 8, 2,
                               causal, "GQA prefill, B = 2 x M = 256, 8 query / 2 KV heads d64 fp16, "
                               + ("causal" if causal else "non-causal")))
    return out


def bench_prefill(args):
    """Packed varlen prefill: 16 sequences of 4096 tokens, 8 query / 2 KV heads of d 64 (or
    the --shape's heads), fp16, causal (the long-prompt prefill shape; MFMA-bound)."""
    import numpy as np
    import torch

    import kv_cache_decode_paged_amd as kvp
    import workloads as W
    seqlens, causal = [4096] * 16, True
    hq, hkv = (8, 2) if args.shape == DEFAULT_SHAPE else (HQ, HKV)
    q, k, v, cu = W.varlen_inputs(seqlens, hq, hkv, head_dim=D)
    q, k, v, cu = q.cuda(), k.cuda(), v.cuda(), cu.cuda()
    out = torch.empty_like(q)
    call = lambda: kvp.varlen_causal_prefill(q, k, v, cu, max(seqlens), causal=causal, out=out)
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
    per = step_stats(event_times(torch, call, args.steps))
    flops = prefill_flops(seqlens, hq, D, causal)
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = check = None
    if not args.no_cpu_baseline:
        # the oracle on one sequence of the call (all heads on all host threads, then one
        # head on one thread); its rows also check the call's output for that sequence
        n = 4096 if hq * D <= 512 else 1536
        q0, k0, v0 = q[:n].cpu(), k[:n].cpu(), v[:n].cpu()
        cu0 = torch.tensor([0, n], dtype=torch.int32)
        want, secs = prefill_oracle(q0, k0, v0, cu0, causal, host_threads())
        _, secs1 = prefill_oracle(q0[:, :1], k0[:, :1], v0[:, :1], cu0, causal, 1)
        f1 = prefill_flops([n], hq, D, causal)
        if n == 4096:
            err = float(np.abs(out[:n].double().cpu().numpy() - want).max())
            check = {"rows": f"sequence 0 ({n} rows, every head)", "max_abs_err": err, "tol": 2e-3,
                     "ok": bool(err <= 2e-3)}
        cpu = {"value": round(f1 / secs / 1e12, 6), "unit": "TFLOP/s", "cores": host_threads(), "kind": "oracle",
               "sample": f"one segment of {n} rows x {hq} query heads ({hkv} KV heads), causal, fp64 scalar C, "
                         f"heads across {host_threads()} threads", "seconds": round(secs, 3),
               "one_thread": {"value": round(f1 / hq / secs1 / 1e12, 6), "sample": f"one head of the segment",
                              "seconds": round(secs1, 3)}}
    print(f"[bench] prefill {len(seqlens)} x {seqlens[0]} tokens, {hq}q/{hkv}kv heads: {ms * 1e3:.1f} us per call, "
          f"{tflops:.1f} TFLOP/s ({tflops / MFMA_F16_PEAK_TFLOPS * 100:.1f}% of the fp16 MFMA peak)",
          file=sys.stderr, flush=True)
    return {
        "metric": "packed causal prefill attention TFLOP/s (% of MFMA fp16 peak)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"packed varlen causal prefill, {len(seqlens)} sequences x {seqlens[0]} tokens, "
                               f"{hq}q/{hkv}kv heads d{D} fp16", "sequences": len(seqlens),
                   "seq_len": seqlens[0]},
        "step_time_warm": per,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "varlen_causal_prefill (prefill_mfma_f16_kernel)", "flops_per_launch": flops,
                     "avg_launch_us": round(ms * 1e3, 3)},
        "check": check,
        "cpu_baseline": cpu,
    }


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
    per = step_stats(event_times(torch, call, args.steps))
    flops = chunk_flops([prefix] * B, [chunk] * B, HQ, D)
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = check = None
    if not args.no_cpu_baseline:
        import oracle
        # the oracle on one of the 16 requests (all heads, the whole chunk); its rows also
        # check the call's output for that request
        K = torch.stack([cache.k_pool[0][table[0, j].item()] for j in range(max_blocks)]).permute(1, 0, 2, 3)
        V = torch.stack([cache.v_pool[0][table[0, j].item()] for j in range(max_blocks)]).permute(1, 0, 2, 3)
        K = K.reshape(HKV, -1, D)[None].double().cpu().numpy()
        V = V.reshape(HKV, -1, D)[None].double().cpu().numpy()
        t0 = time.perf_counter()
        want = oracle.chunk_attention(q[:chunk].double().cpu().numpy(), K, V, np.array([prefix + chunk], np.int32),
                                      np.array([0, chunk], np.int32))
        dt = time.perf_counter() - t0
        err = float(np.abs(out[:chunk].double().cpu().numpy() - want).max())
        check = {"rows": f"request 0 ({chunk} rows, every head)", "max_abs_err": err, "tol": 2e-3,
                 "ok": bool(err <= 2e-3)}
        cpu = {"value": round(chunk_flops([prefix], [chunk], HQ, D) / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": 1, "kind": "oracle",
               "sample": f"one of the {B} requests (its {chunk} rows x {HQ} heads after the {prefix}-token prefix), "
                         "fp64 scalar C, 1 thread"}
    print(f"[bench] chunked prefill {B} x {chunk} rows after a shared {prefix}-token prefix: {ms * 1e3:.1f} us per "
          f"call, {tflops:.1f} TFLOP/s ({tflops / MFMA_F16_PEAK_TFLOPS * 100:.1f}% of the fp16 MFMA peak)",
          file=sys.stderr, flush=True)
    return {
        "metric": "chunked prefill against the paged cache TFLOP/s (% of MFMA fp16 peak)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{B} requests forked from one {prefix}-token prompt, {chunk}-token chunk each, "
                               f"{HQ}q/{HKV}kv heads d{D} fp16, 16-token blocks", "requests": B,
                   "prefix": prefix, "chunk": chunk},
        "step_time_warm": per,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "paged_prefill_attention (prefill_mfma_f16_kernel, paged keys)",
                     "flops_per_launch": flops, "avg_launch_us": round(ms * 1e3, 3)},
        "check": check,
        "cpu_baseline": cpu,
    }


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
    return {
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


def emit(line):
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed alone after a 512 MB cache flush, where a step's bytes are under 1 GB")
    ap.add_argument("--batch", type=int, default=200)
    ap.add_argument("--layers", type=int, default=None, help="default: the shape's layer count")
    ap.add_argument("--shape", choices=sorted(SHAPES), default=DEFAULT_SHAPE,
                    help="decode head shape (default 14q2kv_d64)")
    ap.add_argument("--kv-dtype", choices=["fp16", "int8"], default="fp16",
                    help="decode cache: fp16, or int8 codes with an fp16 scale per row")
    ap.add_argument("--kernel-reps", type=int, default=10, help="graph replays of the layers for the launch time")
    ap.add_argument("--no-graph", action="store_true", help="launch the layers eagerly")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (and the output check)")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    ap.add_argument("--no-share", action="store_true", help="plans without shared-prefix items")
    ap.add_argument("--share-width", type=int, choices=[1, 2, 4], default=1,
                    help="shared items span this many blocks of 16 query columns (KVP_PLAN_SHARE_WIDE2 / 4)")
    ap.add_argument("--long-items", action="store_true",
                    help="decode workload: plans with long items (KVP_PLAN_LONG_ITEMS, which sizes parts to "
                         "one generation of waves when a batch's private blocks far exceed them and leaves "
                         "smaller batches' plans as they are); always on for long_context")
    ap.add_argument("--fill", choices=["auto", "on", "off"], default="auto",
                    help="plans with KVP_PLAN_FILL (parts shorter than 32 blocks while the batch leaves resident "
                         "waves idle): on, off, or auto (batches of at most 8 request x KV-head pairs)")
    ap.add_argument("--no-scatter", action="store_true", help="hand out block ids in order (no free-list shuffle)")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "long_context", "batch1", "single_head", "varlen", "prefill",
                             "chunked_prefill", "batching", "suite"],
                    help="decode: the batch paged decode step (default batch 200); long_context: 32 requests "
                         "of 32768 cached tokens (split-K); batch1: 24 layers at batch 1, contexts 16..1024; "
                         "single_head: fp32 40-token prefill + 48 decode steps; varlen: the pages' packed "
                         "prefills at their sizes; prefill: 16 x 4096 causal; chunked_prefill: 16 x 512-token "
                         "chunks after a shared 2048-token prefix; batching: host scheduler; suite: all of them "
                         "(and batches 10, 50, 100, 200), one JSON line each")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Requests would be sharded across GPUs by whole sharing groups.", flush=True)
        sys.exit(2)
    set_shape(args.shape, args.kv_dtype == "int8")
    global SCATTER
    SCATTER = not args.no_scatter
    if args.kv_dtype == "int8" and args.workload not in ("decode", "long_context"):
        print("--kv-dtype int8 applies to the decode workloads", flush=True)
        sys.exit(2)
    if args.workload == "batching":
        emit(bench_batching(args))
        return
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = args.workload
    if w == "decode":
        emit(bench_decode(args))
    elif w == "long_context":
        emit(bench_long_context(args))
    elif w == "batch1":
        for line in bench_batch1(args):
            emit(line)
    elif w == "single_head":
        emit(bench_single_head(args))
    elif w == "varlen":
        for line in bench_varlen(args):
            emit(line)
    elif w == "prefill":
        emit(bench_prefill(args))
    elif w == "chunked_prefill":
        emit(bench_chunked_prefill(args))
    elif w == "suite":
        emit(bench_single_head(args))
        for line in bench_batch1(args):
            emit(line)
        for line in bench_varlen(args):
            emit(line)
        for B in (10, 50, 100, 200):
            emit(bench_decode(args, B))
        emit(bench_long_context(args))
        emit(bench_prefill(args))
        emit(bench_chunked_prefill(args))
        emit(bench_batching(args))


if __name__ == "__main__":
    main()
