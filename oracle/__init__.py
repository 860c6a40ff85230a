"""fp64 CPU oracle for attention against a key-value cache -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product library never does, and the oracle imports nothing from it.

Contents
  * libkvp_oracle.so (kvp_oracle.c): plain scalar fp64 loops -- attention row, GQA decode,
    several new rows per request against a cache (chunked prefill / draft verification),
    full causal recompute, packed varlen prefill, block partial + merge, KV bytes/token.
  * brute.py   : an independent pure-Python brute force (math.fsum) for tiny shapes.
  * pagepool.py: the block pool / block table / copy-on-write model.
  * opcount.py : the multiply-accumulate cost model of cached vs uncached generation.
  * kvquant.py : symmetric absmax quantization of cache rows (int8 codes, fp16 scale per
                 row) and its exact reconstruction.
  * batching.py: static vs continuous batching over a page pool (step-by-step schedule,
                 latencies, pages, utilisation) and the naive vs paged utilisation formulas.

Parity status: every function here is pinned by a CPU test (see tests/test_oracle_*.py);
none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("KVP_ORACLE_LIB") or os.path.join(_HERE, "libkvp_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_attention_row.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, ctypes.c_long, _dp,
                                      ctypes.c_long, ctypes.c_double, _dp, _dp]
    lib.orc_attention_row.restype = None
    lib.orc_kv_head.argtypes = [ctypes.c_int] * 3
    lib.orc_kv_head.restype = ctypes.c_int
    lib.orc_decode_gqa.argtypes = [ctypes.c_int] * 5 + [_ip, _dp, _dp, _dp, ctypes.c_double, _dp]
    lib.orc_decode_gqa.restype = None
    lib.orc_full_causal.argtypes = [ctypes.c_int] * 4 + [_dp, _dp, _dp, ctypes.c_double, _dp]
    lib.orc_full_causal.restype = None
    lib.orc_varlen_prefill.argtypes = [ctypes.c_int] * 4 + [_dp, _dp, _dp, _ip, ctypes.c_int,
                                                            ctypes.c_int, ctypes.c_double, _dp]
    lib.orc_varlen_prefill.restype = None
    lib.orc_chunk_attention.argtypes = [ctypes.c_int] * 5 + [_ip, _ip, _dp, _dp, _dp, ctypes.c_double, _dp]
    lib.orc_chunk_attention.restype = None
    lib.orc_partial.argtypes = [ctypes.c_int] * 3 + [_dp, _dp, ctypes.c_long, _dp, ctypes.c_long,
                                                     ctypes.c_double, _dp, _dp, _dp]
    lib.orc_partial.restype = None
    lib.orc_merge.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp]
    lib.orc_merge.restype = None
    lib.orc_kv_bytes_per_token.argtypes = [ctypes.c_int] * 4
    lib.orc_kv_bytes_per_token.restype = ctypes.c_longlong
    _lib = lib
    return lib


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _i(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_ip)


def default_scale(d):
    """1/sqrt(d): the score divisor of the TraditionalAttention module (linear-attention post)."""
    return 1.0 / np.sqrt(d)


def attention_row(q, K, V, scale=None, return_p=False):
    """q [d], K [n, d], V [n, d] -> out [d] (and p [n])."""
    lib = _load()
    q, qp = _d(q)
    K, Kp = _d(K)
    V, Vp = _d(V)
    n, d = K.shape
    scale = default_scale(d) if scale is None else scale
    out, op = _d(np.zeros(d))
    p, pp = _d(np.zeros(n))
    lib.orc_attention_row(d, n, qp, Kp, d, Vp, d, scale, op, pp)
    return (out, p) if return_p else out


def kv_head(h, Hq, Hkv):
    return _load().orc_kv_head(h, Hq, Hkv)


def decode_gqa(q, K, V, ctx, scale=None):
    """q [B, Hq, d]; K, V [B, Hkv, Lmax, d] (logical, contiguous); ctx [B] (includes the
    token appended this step) -> out [B, Hq, d]."""
    lib = _load()
    q, qp = _d(q)
    K, Kp = _d(K)
    V, Vp = _d(V)
    ctx, cp = _i(ctx)
    B, Hq, d = q.shape
    _, Hkv, Lmax, _ = K.shape
    assert (ctx >= 1).all() and (ctx <= Lmax).all()
    scale = default_scale(d) if scale is None else scale
    out, op = _d(np.zeros((B, Hq, d)))
    lib.orc_decode_gqa(B, Hq, Hkv, d, Lmax, cp, qp, Kp, Vp, scale, op)
    return out


def full_causal(q, k, v, scale=None):
    """q [n, Hq, d]; k, v [n, Hkv, d] -> out [n, Hq, d] (n x n scores, masked afterwards)."""
    lib = _load()
    q, qp = _d(q)
    k, kp = _d(k)
    v, vp = _d(v)
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = default_scale(d) if scale is None else scale
    out, op = _d(np.zeros((n, Hq, d)))
    lib.orc_full_causal(n, Hq, Hkv, d, qp, kp, vp, scale, op)
    return out


def chunk_attention(q, K, V, ctx, cu_q, scale=None):
    """Several new rows per request against its cache: q [T, Hq, d] packed by cu_q [B+1];
    K, V [B, Hkv, Lmax, d]; the rows of request b are positions ctx[b] - m_b .. ctx[b] - 1
    and row i attends to positions 0 .. ctx[b] - m_b + i.  -> out [T, Hq, d]."""
    lib = _load()
    q, qp = _d(q)
    K, Kp = _d(K)
    V, Vp = _d(V)
    ctx, cp = _i(ctx)
    cu, cup = _i(cu_q)
    T, Hq, d = q.shape
    B, Hkv, Lmax, _ = K.shape
    m = np.diff(cu)
    assert len(cu) == B + 1 and cu[0] == 0 and cu[-1] == T and (m >= 0).all()
    assert (ctx >= m).all() and (ctx <= Lmax).all()
    scale = default_scale(d) if scale is None else scale
    out, op = _d(np.zeros((T, Hq, d)))
    lib.orc_chunk_attention(B, Hq, Hkv, d, Lmax, cp, cup, qp, Kp, Vp, scale, op)
    return out


def varlen_prefill(q, k, v, cu_seqlens, causal=True, scale=None):
    """q [T, Hq, d]; k, v [T, Hkv, d]; cu_seqlens [nseg+1] -> out [T, Hq, d]."""
    lib = _load()
    q, qp = _d(q)
    k, kp = _d(k)
    v, vp = _d(v)
    cu, cup = _i(cu_seqlens)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = default_scale(d) if scale is None else scale
    out, op = _d(np.zeros((T, Hq, d)))
    lib.orc_varlen_prefill(T, Hq, Hkv, d, qp, kp, vp, cup, len(cu) - 1, int(bool(causal)),
                           scale, op)
    return out


def partial(q, K, V, j0, j1, scale=None):
    """Unnormalised block softmax over keys [j0, j1): returns (m, l, o[d])."""
    lib = _load()
    q, qp = _d(q)
    K, Kp = _d(K)
    V, Vp = _d(V)
    d = K.shape[1]
    scale = default_scale(d) if scale is None else scale
    m = ctypes.c_double()
    l = ctypes.c_double()
    o, op = _d(np.zeros(d))
    lib.orc_partial(d, j0, j1, qp, Kp, d, Vp, d, scale, ctypes.byref(m), ctypes.byref(l), op)
    return m.value, l.value, o


def merge(ms, ls, os_):
    """Merge block partials in index order -> normalised out [d]."""
    lib = _load()
    ms, mp = _d(ms)
    ls, lp = _d(ls)
    os_, op_ = _d(os_)
    nparts, d = os_.shape
    out, outp = _d(np.zeros(d))
    lib.orc_merge(d, nparts, mp, lp, op_, outp)
    return out


def kv_bytes_per_token(L, Hkv, d, elem_bytes):
    return int(_load().orc_kv_bytes_per_token(L, Hkv, d, elem_bytes))
