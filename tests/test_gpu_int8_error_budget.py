"""Error budget of the int8 cache against the fp16 cache.

The int8 cache stores each (token, KV head) row of K and of V as absmax codes with one fp16
scale (neuralialabs "Tornar a inferencia barata", quantization section: symmetric absmax
quantization, finer granularity for a smaller error; applied here to cache rows).  The
parity tests compare the int8 kernel with the oracle run on the reconstructed rows; this
file bounds what the quantization itself costs, against the oracle on the original fp16
rows, at the batch-200 workload and at 32 requests of 32,768 tokens.

For one query row (request b, query head h) with scores s_j = scale q.k_j, weights p_j and
output o = sum_j p_j v_j, quantization replaces k_j, v_j by k'_j, v'_j.  With
    D = max_j |scale q.(k'_j - k_j)|     (the largest score change),
each weight ratio p'_j / p_j lies in [e^-2D, e^2D], so sum_j |p'_j - p_j| <= e^2D - 1, and
since sum_j (p'_j - p_j) = 0, for every output dimension c
    |o'_c - o_c| <= max_j |v'_jc - v_jc| + (e^2D - 1) (max_j v_jc - min_j v_jc) / 2.
The kernel's own error against the oracle on the reconstructed rows is within the fp16
tolerance (2e-3), so the int8 output must lie within that bound plus 2e-3 of the fp16
oracle, element by element.  The test computes the bound exactly (fp64) from the oracle's
quantization of the same rows."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import GPU, TOL, PagedStep, need_gpu, say, to64
from oracle import kvquant as KQ

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp


def _budget(q64, K, V, ctx, scale):
    """Per (request, head, dim) bound of |o_int8 - o_fp16| and the fp16 oracle output; K, V:
    fp16 host tensors [B, Hkv, Lmax, d]."""
    B, hq, d = q64.shape
    hkv = K.shape[1]
    grp = hq // hkv
    threads = max(1, min(16, len(os.sched_getaffinity(0))))

    def one(b):
        n = int(ctx[b])
        k = K[b, :, :n].numpy()
        v = V[b, :, :n].numpy()
        k64, v64 = k.astype(np.float64), v.astype(np.float64)
        kq = KQ.dequantize_rows(*KQ.absmax_quantize_rows(k))
        vq = KQ.dequantize_rows(*KQ.absmax_quantize_rows(v))
        want = oracle.decode_gqa(q64[b:b + 1], k64[None], v64[None], np.array([n], dtype=np.int32))[0]
        bound = np.empty((hq, d))
        for h in range(hq):
            g = h // grp
            ds = np.abs((kq[g] - k64[g]) @ q64[b, h]) * scale
            D = ds.max()
            dv = np.abs(vq[g] - v64[g]).max(axis=0)
            rng = v64[g].max(axis=0) - v64[g].min(axis=0)
            bound[h] = dv + np.expm1(2 * D) * rng / 2
        return want, bound
    with cf.ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, range(B)))
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def _check(step, label):
    q = step.q(0)
    out = kvp.paged_decode_attention(step.cache, 0, q.cuda(), step.table, step.ctx)
    torch.cuda.synchronize()
    K, V = step.logical[0]
    want, bound = _budget(to64(q), K, V, step.ctx_host, 1.0 / 8.0)
    err = np.abs(to64(out) - want)
    ratio = float((err / (bound + TOL[torch.float16])).max())
    say(f"int8 budget {label}: max |o_int8 - o_fp16| {err.max():.3e}, max bound {bound.max():.3e}, "
        f"median bound {np.median(bound):.3e}, max err / (bound + 2e-3) {ratio:.3f}")
    assert (err <= bound + TOL[torch.float16]).all(), label
    return float(err.max()), float(bound.max())


def test_int8_error_budget_batch200():
    need_gpu()
    step = PagedStep(kvp, W.paged_batch(200), layers=1, hq=14, hkv=2, dtype=torch.int8, seed=12300)
    _check(step, "batch 200, contexts 128..2048")


def test_int8_error_budget_long_context():
    need_gpu()
    step = PagedStep(kvp, W.uniform_batch(32, 32768), layers=1, hq=14, hkv=2, dtype=torch.int8, seed=12400,
                     poison=False)
    _check(step, "32 x 32768")
