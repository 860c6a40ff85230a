"""The decode step exactly as the benchmark times it (kv_cache_decode_paged_amd.runner):
batch 200, 24-layer pool, groups of 8 forked from a 512-token prefix (copy-on-write on the
first step), a padded plan whose launch carries the workspace's slot capacity and the plan
buffer's whole id area, the fused append, two device plan buffers uploaded on a copy
stream, and captured graphs replayed step after step.

Every step's outputs of layers 0 and 23, all 200 requests, are checked against the fp64
oracle on the logical rows (the seeded cache contents plus each step's appended row), and
the appended rows must sit in the cache bit for bit.  Pages: neuralialabs "Tornar a
inferencia barata" (decode appends one token and attends over the cache; PagedAttention);
gustavoai "La cache de claves y valores" (the new k, v join the cache before the attention
row); chatgpz.de "Aufmerksamkeit", paged-attention article SECTION 3 (copy-on-write
prefix sharing)."""
import concurrent.futures as cf
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, PagedStep, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp
    from kv_cache_decode_paged_amd.runner import DecodeStepRunner


def oracle_decode_rows(q64, K64, V64, ctx):
    """orc_decode_gqa request by request on the host threads (q64 [B, Hq, d], K64 / V64
    [B, Hkv, Lmax, d], ctx [B])."""
    B = q64.shape[0]

    def one(b):
        n = int(ctx[b])
        return oracle.decode_gqa(q64[b:b + 1], np.ascontiguousarray(K64[b:b + 1, :, :n]),
                                 np.ascontiguousarray(V64[b:b + 1, :, :n]), np.array([n], dtype=np.int32))[0]
    with cf.ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        return np.stack(list(ex.map(one, range(B))))


def _run_steps(B, n_steps, seed, check_layers, layers=24, graph=True, dtype=torch.float16, pb=None):
    pb = W.paged_batch(B) if pb is None else pb
    say("step runner: batch", B, "layers", layers, "steps", n_steps, "graph", graph, "dtype", dtype)
    st = PagedStep(kvp, pb, layers=layers, hq=14, hkv=2, dtype=dtype, seed=seed, layers_with_data=check_layers,
                   take_step=False, extra_blocks=2 * B + 64)
    io = st.io_dtype
    max_blocks = math.ceil((max(pb.ctx_before) + n_steps + 1) / W.BLOCK)
    dev = "cuda"
    q = torch.empty((layers, B, 14, 64), dtype=io, device=dev)
    for l in range(layers):
        q[l].copy_(W.decode_q(B, 14, seed, io, l))
    knew = torch.empty((layers, B, 2, 64), dtype=io, device=dev)
    vnew = torch.empty_like(knew)
    out = torch.empty_like(q)
    runner = DecodeStepRunner(st.cache, st.pool, st.seqs, max_blocks, q, knew, vnew, out, graph=graph,
                              grow_tokens=n_steps + 1, spare_items=256 if B >= 8 else 8)
    say("step runner: fill plans", runner.fill)
    # the logical rows of the checked layers, extended by every step's appended row
    Lmax = max(pb.ctx_before) + n_steps
    logical = {}
    for l in check_layers:
        K, V = st.logical[l]
        K2 = torch.zeros((B, 2, Lmax, 64), dtype=io)
        V2 = torch.zeros_like(K2)
        for b in range(B):
            c = pb.ctx_before[b]
            K2[b, :, :c] = K[b, :, :c]
            V2[b, :, :c] = V[b, :, :c]
        logical[l] = (K2, V2)
    appended = []
    worst = 0.0
    for t in range(n_steps):
        kn = W.randn((layers, B, 2, 64), seed + 100 + 2 * t, io)
        vn = W.randn((layers, B, 2, 64), seed + 101 + 2 * t, io)
        knew.copy_(kn.to(dev))
        vnew.copy_(vn.to(dev))
        appended.append((kn, vn))
        rec = runner.step(keep=True)
        torch.cuda.synchronize()
        if t == 0:
            cows = len(rec.cow_pairs)
            say("step 0: copy-on-write pairs", cows, "plan items", rec.n_items, "shared", rec.n_shared)
            # members shorter than the prefix append into a shared block: it is copied first
            # (at most one copy per such member)
            if pb.prefix > 0:
                assert 0 < cows <= sum(1 for c in pb.ctx_before if c < pb.prefix and c % W.BLOCK != 0)
            else:
                assert cows == 0
        ctx = rec.ctx
        assert list(ctx) == [c + t + 1 for c in pb.ctx_before]
        for l in check_layers:
            K2, V2 = logical[l]
            for b in range(B):
                K2[b, :, pb.ctx_before[b] + t] = kn[l, b]
                V2[b, :, pb.ctx_before[b] + t] = vn[l, b]
            K64, V64 = to64(K2), to64(V2)
            if dtype == torch.int8:  # the cache holds the oracle's quantization of each row
                K64, V64 = PagedStep.dequantized(K2), PagedStep.dequantized(V2)
            want = oracle_decode_rows(to64(q[l]), K64, V64, ctx)
            got = to64(out[l])
            err = float(np.abs(got - want).max())
            worst = max(worst, err)
            say("step", t, "layer", l, "max err", err, "graph replay" if runner.graphs[t % 2] is not None and t > 0
                else "eager")
            assert err <= TOL[torch.float16], f"step {t} layer {l}: {err}"
    if graph:
        assert runner.graphs[0] is not None and runner.graphs[1] is not None
    return st, runner, rec, appended, worst


def test_runner_batch200_steps_match_oracle():
    """Four steps (the eager first step with its copy-on-write, then replays of both plan
    buffers' graphs); all 200 requests of layers 0 and 23 at every step."""
    need_gpu()
    B, n_steps = 200, 4
    st, runner, rec, appended, worst = _run_steps(B, n_steps, 9900, [0, 23])
    say("runner b200 worst err", worst)
    # every appended row sits in its slot bit for bit (torch indexing of the pool)
    table = torch.from_numpy(rec.table).long()
    pb = st.pb
    for l in (0, 23):
        for t, (kn, vn) in enumerate(appended):
            pos = torch.tensor([c + t for c in pb.ctx_before])
            blk = table[torch.arange(B), pos // W.BLOCK].cuda()
            row = (pos % W.BLOCK).cuda()
            kc = st.cache.k_pool[l][blk, :, row, :].cpu()
            vc = st.cache.v_pool[l][blk, :, row, :].cpu()
            assert torch.equal(kc.view(torch.int16), kn[l].view(torch.int16)), f"K rows of step {t}, layer {l}"
            assert torch.equal(vc.view(torch.int16), vn[l].view(torch.int16)), f"V rows of step {t}, layer {l}"
    # the launch is the padded, capacity-carrying layout the benchmark replays
    lp = runner.launch_plan
    assert lp.n_items == rec.n_items and lp.n_slots >= 1
    assert lp.n_ids == (runner.layout["img_bytes"] - lp.off_ids) // 4


def test_runner_batch100_eager_matches_oracle():
    need_gpu()
    _, _, _, _, worst = _run_steps(100, 2, 9950, [0, 5], layers=6, graph=False)
    say("runner b100 eager worst err", worst)


def test_runner_int8_cache_batch200():
    need_gpu()
    _, _, _, _, worst = _run_steps(200, 3, 9970, [0, 3], layers=4, dtype=torch.int8)
    say("runner b200 int8 worst err", worst)


def test_runner_lone_request_fill_plans():
    """One request of 1500 tokens: the runner's automatic fill plans cut its context into
    8-block parts (12 per KV head, merged by the rescale); three graph-replayed steps."""
    need_gpu()
    _, runner, _, _, worst = _run_steps(1, 3, 9990, [0, 5], layers=6, pb=W.uniform_batch(1, 1500))
    assert runner.fill
    say("runner lone request worst err", worst)
