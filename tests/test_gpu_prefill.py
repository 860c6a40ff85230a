"""Packed varlen prefill on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32)


def _run(seqlens, hq, hkv, causal, dtype=torch.float16, seed=42):
    q, k, v, cu = W.varlen_inputs(seqlens, hq, hkv, seed=seed, dtype=dtype)
    out = kvp.varlen_causal_prefill(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(seqlens), causal=causal)
    torch.cuda.synchronize()
    want = oracle.varlen_prefill(to64(q), to64(k), to64(v), cu.numpy(), causal=causal)
    return out, want, (q, k, v, cu)


@pytest.mark.parametrize("causal", [True, False])
def test_packed_varlen_8_heads(causal):
    need_gpu()
    say("varlen (37,120,8,200) causal", causal)
    out, want, _ = _run(W.VARLEN_SEQLENS, 8, 8, causal)
    err = max_abs(to64(out), want)
    say("max err", err)
    assert err <= TOL[torch.float16]


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_two_sequences_256(causal):
    need_gpu()
    say("gqa B=2 M=256 8q/2kv causal", causal)
    out, want, _ = _run((256, 256), 8, 2, causal)
    err = max_abs(to64(out), want)
    say("max err", err)
    assert err <= TOL[torch.float16]
    # (B, M, G, Hq/G, K) view of the packed output
    assert out.reshape(2, 256, 2, 4, 64).shape == (2, 256, 2, 4, 64)


def test_single_head_fp32_prompt_matches_full_recompute():
    need_gpu()
    q, k, v = W.single_head_sequence()
    n = W.SINGLE_PROMPT
    cu = torch.tensor([0, n], dtype=torch.int32)
    out = kvp.varlen_causal_prefill(q[:n].cuda(), k[:n].cuda(), v[:n].cuda(), cu.cuda(), n, causal=True)
    torch.cuda.synchronize()
    full = oracle.full_causal(to64(q[:n]), to64(k[:n]), to64(v[:n]))
    assert max_abs(to64(out), full) <= TOL[torch.float32]


@pytest.mark.parametrize("seqlens", [(1,), (1, 1, 1), (63, 64, 65), (129, 7, 300, 1, 64), (1000,)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_ragged_segments(seqlens, dtype):
    need_gpu()
    say("ragged prefill", seqlens, dtype)
    for causal in (True, False):
        out, want, _ = _run(seqlens, 4, 2, causal, dtype=dtype, seed=sum(seqlens))
        assert max_abs(to64(out), want) <= TOL[dtype], causal


def test_block_diagonal_isolation():
    need_gpu()
    seqlens = W.VARLEN_SEQLENS
    q, k, v, cu = W.varlen_inputs(seqlens, 8, 2)
    base = kvp.varlen_causal_prefill(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), 200, causal=False)
    k2, v2 = k.clone(), v.clone()
    a, e = int(cu[1]), int(cu[2])
    k2[a:e] = -k2[a:e]
    v2[a:e] = float("nan")
    pert = kvp.varlen_causal_prefill(q.cuda(), k2.cuda(), v2.cuda(), cu.cuda(), 200, causal=False)
    torch.cuda.synchronize()
    keep = torch.cat([torch.arange(0, a), torch.arange(e, int(cu[-1]))])
    assert torch.equal(_bits(base.cpu()[keep]), _bits(pert.cpu()[keep]))


def test_causal_future_rows_never_read():
    need_gpu()
    q, k, v, cu = W.varlen_inputs((300,), 4, 2)
    base = kvp.varlen_causal_prefill(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), 300, causal=True)
    k2, v2 = k.clone(), v.clone()
    # finite perturbation: a masked key inside a needed tile still meets a zero weight
    k2[150:] = -3 * k2[150:]
    v2[150:] = 5 - v2[150:]
    pert = kvp.varlen_causal_prefill(q.cuda(), k2.cuda(), v2.cuda(), cu.cuda(), 300, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(base.cpu()[:150]), _bits(pert.cpu()[:150]))
