"""The allocation-free decode entry point (paged_decode_attention_noalloc), called through
the C ABI: its outputs must equal paged_decode_attention's bit for bit (same kernels, same
splits; only the split state lives in the library's static scratch instead of a caller
workspace) and the fp64 oracle within the fp16 tolerance, over consecutive calls that
share the scratch -- a large call, a smaller one, then a large one again (the counters a
call leaves behind must be zero for the next).  Pages: neuralialabs "Tornar a inferencia
barata" (decode over a paged cache); chatgpz.de "Aufmerksamkeit", FlashAttention post
(split partials merged by rescaling)."""
import ctypes

import pytest
import torch

import workloads as W
from gpu_support import GPU, TOL, PagedStep, max_abs, need_gpu, say, to64

pytestmark = pytest.mark.gpu

if GPU:
    import kv_cache_decode_paged_amd as kvp


def _bits(t):
    return t.contiguous().view(torch.int16)


def _noalloc_raw(step, layer, q, out):
    """The entry point through the raw ctypes handle of libkvp.so."""
    lib = kvp.lib()
    st = lib.paged_decode_attention_noalloc(ctypes.byref(step.cache.desc), layer, ctypes.c_void_p(out.data_ptr()),
                                            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(step.table.data_ptr()),
                                            step.table.shape[1], ctypes.c_void_p(step.ctx.data_ptr()), q.shape[0],
                                            ctypes.c_float(0.0),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvp.KVP_OK, kvp.last_error()
    return out


def test_noalloc_matches_workspace_call_over_consecutive_calls():
    need_gpu()
    cases = [(W.paged_batch(50), 9800), (W.paged_batch(10), 9810), (W.paged_batch(60, lo=1500, hi=3000), 9820)]
    for i, (pb, seed) in enumerate(cases):
        say("noalloc call", i, "batch", pb.batch, "max ctx", max(pb.ctx_before))
        step = PagedStep(kvp, pb, layers=2, hq=14, hkv=2, dtype=torch.float16, seed=seed)
        for layer in (0, 1):
            q = step.q(layer).cuda()
            want_bits = kvp.paged_decode_attention(step.cache, layer, q, step.table, step.ctx)
            got = _noalloc_raw(step, layer, q, torch.empty_like(q))
            torch.cuda.synchronize()
            assert torch.equal(_bits(got.cpu()), _bits(want_bits.cpu())), f"call {i} layer {layer}"
            err = max_abs(to64(got), step.oracle(layer))
            say("noalloc call", i, "layer", layer, "max err", err)
            assert err <= TOL[torch.float16]


def test_noalloc_rejects_sizes_beyond_the_scratch():
    need_gpu()
    pb = W.paged_batch(4)
    step = PagedStep(kvp, pb, layers=1, hq=14, hkv=2, dtype=torch.float16, seed=9830)
    q = step.q(0).cuda()
    # a table of 2^20 tokens per request: its split partials exceed the static scratch
    wide = torch.full((pb.batch, 65536), -1, dtype=torch.int32, device="cuda")
    wide[:, : step.table.shape[1]] = step.table
    with pytest.raises(kvp.KvpError) as e:
        kvp.paged_decode_attention_noalloc(step.cache, 0, q, wide, step.ctx)
    assert e.value.status == kvp.KVP_ERR_INVALID and "static scratch" in str(e.value)
    # the rejected call left the scratch usable
    got = kvp.paged_decode_attention_noalloc(step.cache, 0, q, step.table, step.ctx)
    want = kvp.paged_decode_attention(step.cache, 0, q, step.table, step.ctx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got.cpu()), _bits(want.cpu()))
