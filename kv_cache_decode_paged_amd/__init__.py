"""Python binding of the MI355X paged KV-cache attention library (libkvp.so).

Argument marshalling only: every computation runs in the library's HIP kernels (device
work) or its C++ block manager (host bookkeeping).  PyTorch tensors supply device memory
and the current HIP stream.  There is no fallback: if libkvp.so is missing, importing the
module raises.

The C functions keep their names; see include/kvp.h for layouts and error behaviour.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_decode_paged_amd._build` "
                      "(or __graft_entry__.build()) before using the library")

_lib = ctypes.CDLL(LIB_PATH)

KVP_OK = 0
KVP_ERR_INVALID = -1
KVP_ERR_OOM = -2
KVP_ERR_NOT_FOUND = -3
KVP_ERR_HIP = -4
KVP_ERR_UNSUPPORTED = -5
_STATUS = {KVP_ERR_INVALID: "INVALID", KVP_ERR_OOM: "OOM", KVP_ERR_NOT_FOUND: "NOT_FOUND",
           KVP_ERR_HIP: "HIP", KVP_ERR_UNSUPPORTED: "UNSUPPORTED"}
KVP_F16 = 0
KVP_F32 = 1
KVP_I8 = 2
BLOCK = 16
HEAD_DIM = 64


class KvpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"kvp status {status} ({_STATUS.get(status, '?')}): {msg}")
        self.status = status


class KvpOOM(KvpError):
    pass


class kvp_dims(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class kvp_cache_desc(ctypes.Structure):
    _fields_ = [("dims", kvp_dims), ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class kvp_copy(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("dst", ctypes.c_int32)]


class kvp_pool_stats(ctypes.Structure):
    _fields_ = [("total_blocks", ctypes.c_int32), ("used_blocks", ctypes.c_int32),
                ("free_blocks", ctypes.c_int32), ("shared_blocks", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("utilisation_pct", ctypes.c_double)]


class kvp_decode_plan(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("group", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("n_items", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("col_blocks", ctypes.c_int32), ("n_slots", ctypes.c_int64), ("bytes", ctypes.c_int64), ("off_pair_base", ctypes.c_int64),
                ("off_pair_nparts", ctypes.c_int64), ("off_req_shared", ctypes.c_int64),
                ("kv_blocks_read", ctypes.c_int64), ("off_ids", ctypes.c_int64), ("n_ids", ctypes.c_int64)]


PLAN_SHARE_PREFIX = 1
PLAN_LONG_ITEMS = 2
PLAN_SHARE_WIDE2 = 4
PLAN_SHARE_WIDE4 = 8
PLAN_FILL = 16

SCHED_STATIC, SCHED_CONTINUOUS = 0, 1
ALLOC_PAGED, ALLOC_NAIVE = 0, 1


class kvp_sched_config(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_int32), ("policy", ctypes.c_int32), ("alloc", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32)]


class kvp_sched_result(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("steps", "tokens", "busy_slot_steps", "padding_slot_steps",
                                              "peak_blocks", "deferrals", "stalls", "max_latency")] + \
               [(f, ctypes.c_double) for f in ("mean_latency", "mean_service", "mean_utilisation")]

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_lib.kvp_last_error.restype = ctypes.c_char_p
_lib.kvp_version.restype = ctypes.c_char_p
_sig("block_pool_create", _i32, [_i32, _i32, ctypes.POINTER(_p)])
_sig("block_pool_destroy", None, [_p])
_sig("block_pool_set_free_order", _i32, [_p, _pi32, _i32])
_sig("block_table_alloc", _i32, [_p, _i32, _pi32])
_sig("block_table_append_slot", _i32, [_p, _i32, _pi64, ctypes.POINTER(kvp_copy)])
_sig("block_table_append_slots", _i32, [_p, _pi32, _i32, _pi64, ctypes.POINTER(kvp_copy)])
_sig("block_table_reserve", _i32, [_p, _i32, _i32, _pi64, ctypes.POINTER(kvp_copy)])
_sig("block_table_fork", _i32, [_p, _i32, _pi32])
_sig("block_table_cow", _i32, [_p, _i32, _i32, _pi32, _pi32])
_sig("block_table_free", _i32, [_p, _i32])
_sig("block_table_truncate", _i32, [_p, _i32, _i32])
_sig("block_table_export", _i32, [_p, _pi32, _i32, _i32, _pi32, _pi32])
_sig("block_table_slots", _i32, [_p, _i32, _i32, _i32, _pi64])
_sig("block_table_get", _i32, [_p, _i32, _pi32, _pi32, _pi32, _i32])
_sig("block_pool_stats", _i32, [_p, ctypes.POINTER(kvp_pool_stats)])
_sig("block_pool_refcount", _i32, [_p, _i32, _pi32])
_sig("kv_bytes_per_token", _i64, [_i32, _i32, _i32, _i32])
_sig("kv_copy_blocks", _i32, [ctypes.POINTER(kvp_cache_desc), _p, _i32, _p])
_sig("kv_append", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _p, _p, _i32, _p])
_sig("contiguous_kv_append", _i32, [ctypes.POINTER(kvp_dims), _p, _p, _i32, _p, _p, _p, _i32, _p])
_sig("decode_workspace_bytes", _sz, [ctypes.POINTER(kvp_dims), _i32, _i32])
_sig("paged_decode_attention", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _p, _p, _i32, _p,
                                      _i32, _f32, _p, _sz, _p])
_sig("paged_decode_append_attention", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _p, _p, _p, _p, _i32,
                                             _p, _i32, _f32, _p, _sz, _p])
_sig("paged_decode_attention_noalloc", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _p, _p, _i32, _p, _i32,
                                              _f32, _p])
_sig("decode_plan_bytes", _sz, [ctypes.POINTER(kvp_dims), _i32, _i32, _i32])
_sig("decode_plan_build", _i32, [ctypes.POINTER(kvp_dims), _p, _i32, _p, _i32, _i32, ctypes.c_uint32, _i32, _p, _sz,
                                 ctypes.POINTER(kvp_decode_plan)])
_sig("sched_simulate", _i32, [ctypes.POINTER(kvp_sched_config), _p, _p, _i32, _p, _p, ctypes.POINTER(kvp_sched_result)])
_sig("decode_plan_workspace_bytes", _sz, [ctypes.POINTER(kvp_decode_plan)])
_sig("paged_decode_attention_planned", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _p, _p, _p,
                                              ctypes.POINTER(kvp_decode_plan), _p, _f32, _p, _sz, _p])
_sig("contiguous_decode_attention", _i32, [ctypes.POINTER(kvp_dims), _p, _p, _p, _p, _i32, _p, _i32,
                                           _f32, _p, _sz, _p])
_sig("varlen_causal_prefill", _i32, [ctypes.POINTER(kvp_dims), _p, _p, _p, _p, _p, _i32, _i32, _i32,
                                     _f32, _p])
_sig("kvp_decode_merge_polls", _i32, [_i32])
_sig("paged_prefill_attention", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _p, _p, _i32, _p, _p, _i32,
                                       _i32, _f32, _p])
_sig("kvp_read_bandwidth_probe", _i32, [_p, _sz, _i32, _p, _p])
_sig("kv_gather", _i32, [ctypes.POINTER(kvp_cache_desc), _i32, _p, _i32, _p, _i32, _i32, _p, _p, _p])


def last_error():
    return _lib.kvp_last_error().decode()


def version():
    return _lib.kvp_version().decode()


def _check(st):
    if st != KVP_OK:
        cls = KvpOOM if st == KVP_ERR_OOM else KvpError
        raise cls(st, last_error())


def lib():
    """The raw ctypes handle (for tests of the C ABI itself)."""
    return _lib


# ---------------------------------------------------------------------------------------
# tensors and streams
# ---------------------------------------------------------------------------------------
_DT = {torch.float16: KVP_F16, torch.float32: KVP_F32, torch.int8: KVP_I8}


def _dtype_code(dt):
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt} (float16, float32 or int8)")
    return _DT[dt]


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def dims(num_layers, num_q_heads, num_kv_heads, dtype, head_dim=HEAD_DIM):
    return kvp_dims(num_layers, num_q_heads, num_kv_heads, head_dim, _dtype_code(dtype))


class PagedKVCache:
    """K and V pools of shape [num_layers][num_blocks][H_kv][16][head_dim] in device memory
    (owned by the torch tensors held here); head_dim 64 or 128.  dtype torch.int8 holds
    quantized rows: int8 code pools (V dim-major within a block: [..][H_kv][head_dim][16])
    plus fp16 scale pools k_scale / v_scale of shape [num_layers][num_blocks][H_kv][16]; q,
    out and appended rows are then fp16 (`io_dtype`)."""

    def __init__(self, num_layers, num_blocks, num_q_heads, num_kv_heads, dtype=torch.float16,
                 device="cuda", k_pool=None, v_pool=None, head_dim=HEAD_DIM):
        shape = (num_layers, num_blocks, num_kv_heads, BLOCK, head_dim)
        # int8: V codes dim-major within a block
        vshape = shape[:3] + (head_dim, BLOCK) if dtype == torch.int8 else shape
        self.k_pool = torch.empty(shape, dtype=dtype, device=device) if k_pool is None else k_pool
        self.v_pool = torch.empty(vshape, dtype=dtype, device=device) if v_pool is None else v_pool
        for t, n, shp in ((self.k_pool, "k_pool", shape), (self.v_pool, "v_pool", vshape)):
            if tuple(t.shape) != shp:
                raise ValueError(f"{n} must have shape {shp}")
            _dev(t, n, dtype)
        self.k_scale = self.v_scale = None
        if dtype == torch.int8:
            self.k_scale = torch.empty(shape[:-1], dtype=torch.float16, device=device)
            self.v_scale = torch.empty(shape[:-1], dtype=torch.float16, device=device)
        self.num_layers, self.num_blocks = num_layers, num_blocks
        self.num_q_heads, self.num_kv_heads, self.dtype = num_q_heads, num_kv_heads, dtype
        self.io_dtype = torch.float16 if dtype == torch.int8 else dtype
        self.head_dim = head_dim
        self.desc = kvp_cache_desc(dims(num_layers, num_q_heads, num_kv_heads, dtype, head_dim), BLOCK,
                                   num_blocks, self.k_pool.data_ptr(), self.v_pool.data_ptr(),
                                   self.k_scale.data_ptr() if self.k_scale is not None else None,
                                   self.v_scale.data_ptr() if self.v_scale is not None else None)

    @property
    def dims(self):
        return self.desc.dims


# ---------------------------------------------------------------------------------------
# host block manager
# ---------------------------------------------------------------------------------------
class BlockPool:
    """Wrapper of the C++ block manager (pool, block tables, fork, copy-on-write)."""

    def __init__(self, num_blocks, block_size=BLOCK):
        h = _p()
        _check(_lib.block_pool_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self):
        if self._h:
            _lib.block_pool_destroy(self._h)
            self._h = _p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_free_order(self, perm):
        arr = (ctypes.c_int32 * len(perm))(*[int(x) for x in perm])
        _check(_lib.block_pool_set_free_order(self._h, arr, len(perm)))

    def alloc(self, n_tokens):
        sid = ctypes.c_int32()
        _check(_lib.block_table_alloc(self._h, int(n_tokens), ctypes.byref(sid)))
        return sid.value

    def append_slot(self, seq):
        """-> (slot, (src, dst) or None)"""
        slot = ctypes.c_int64()
        cp = kvp_copy()
        _check(_lib.block_table_append_slot(self._h, int(seq), ctypes.byref(slot), ctypes.byref(cp)))
        return slot.value, (None if cp.src < 0 else (cp.src, cp.dst))

    def append_slots(self, seqs):
        """One step for a batch: -> (slots int64 [n] host tensor, [(src, dst) or None] * n)."""
        n = len(seqs)
        ids = torch.tensor([int(x) for x in seqs] or [0], dtype=torch.int32)
        slots = torch.empty((max(n, 1),), dtype=torch.int64)
        cows = (kvp_copy * max(n, 1))()
        _check(_lib.block_table_append_slots(self._h, ctypes.cast(ids.data_ptr(), _pi32), n,
                                             ctypes.cast(slots.data_ptr(), _pi64), cows))
        return slots[:n], [None if cows[i].src < 0 else (cows[i].src, cows[i].dst) for i in range(n)]

    def append_slots_raw(self, ids_ptr, n, slots_ptr, cows):
        """Zero-copy variant for hot loops: caller-owned int32 ids / int64 slots buffers
        (addresses) and a (kvp_copy * n) array."""
        _check(_lib.block_table_append_slots(self._h, ctypes.cast(ids_ptr, _pi32), int(n),
                                             ctypes.cast(slots_ptr, _pi64), cows))

    def export_raw(self, ids_ptr, n, max_blocks, table_ptr, ctx_ptr):
        _check(_lib.block_table_export(self._h, ctypes.cast(ids_ptr, _pi32), int(n), int(max_blocks),
                                       ctypes.cast(table_ptr, _pi32), ctypes.cast(ctx_ptr, _pi32)))

    def reserve(self, seq, n):
        """-> (slots int64 [n] on the host, (src, dst) or None)"""
        out = torch.empty((max(int(n), 1),), dtype=torch.int64)
        cp = kvp_copy()
        _check(_lib.block_table_reserve(self._h, int(seq), int(n), ctypes.cast(out.data_ptr(), _pi64),
                                        ctypes.byref(cp)))
        return out[:int(n)], (None if cp.src < 0 else (cp.src, cp.dst))

    def fork(self, parent):
        c = ctypes.c_int32()
        _check(_lib.block_table_fork(self._h, int(parent), ctypes.byref(c)))
        return c.value

    def cow(self, seq, logical_block):
        s, d = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.block_table_cow(self._h, int(seq), int(logical_block), ctypes.byref(s), ctypes.byref(d)))
        return s.value, d.value

    def free(self, seq):
        _check(_lib.block_table_free(self._h, int(seq)))

    def truncate(self, seq, n_tokens):
        _check(_lib.block_table_truncate(self._h, int(seq), int(n_tokens)))

    def export(self, seqs, max_blocks):
        """-> (table int32 [n, max_blocks] (pad -1), context_lens int32 [n]) on the host."""
        n = len(seqs)
        table = torch.empty((n, max_blocks), dtype=torch.int32)
        ctx = torch.empty((n,), dtype=torch.int32)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(s) for s in seqs])
        _check(_lib.block_table_export(self._h, arr, n, int(max_blocks),
                                       ctypes.cast(table.data_ptr(), _pi32), ctypes.cast(ctx.data_ptr(), _pi32)))
        return table, ctx

    def slots(self, seq, start, n):
        out = torch.empty((n,), dtype=torch.int64)
        _check(_lib.block_table_slots(self._h, int(seq), int(start), int(n), ctypes.cast(out.data_ptr(), _pi64)))
        return out

    def table(self, seq):
        nt, nb = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.block_table_get(self._h, int(seq), ctypes.byref(nt), ctypes.byref(nb), None, 0))
        buf = (ctypes.c_int32 * max(nb.value, 1))()
        _check(_lib.block_table_get(self._h, int(seq), ctypes.byref(nt), ctypes.byref(nb), buf, nb.value))
        return list(buf)[:nb.value]

    def tokens(self, seq):
        nt, nb = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.block_table_get(self._h, int(seq), ctypes.byref(nt), ctypes.byref(nb), None, 0))
        return nt.value

    def stats(self):
        st = kvp_pool_stats()
        _check(_lib.block_pool_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in kvp_pool_stats._fields_}

    def refcount(self, block):
        r = ctypes.c_int32()
        _check(_lib.block_pool_refcount(self._h, int(block), ctypes.byref(r)))
        return r.value


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes):
    return int(_lib.kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes))


# ---------------------------------------------------------------------------------------
# device operations
# ---------------------------------------------------------------------------------------
def kv_copy_blocks(cache: PagedKVCache, pairs, stream=None):
    """pairs: device int32 [n, 2] (src, dst)."""
    n = pairs.shape[0] if pairs.numel() else 0
    if n == 0:
        return
    _check(_lib.kv_copy_blocks(ctypes.byref(cache.desc), _dev(pairs, "pairs", torch.int32), n,
                               _stream(stream)))


def kv_append(cache: PagedKVCache, layer, k, v, slots, stream=None):
    """k, v: device [n, H_kv, head_dim] in the cache dtype (fp16 for an int8 cache, which
    stores each row's codes and scale); slots: device int64 [n]."""
    n = k.shape[0]
    if v.shape != k.shape or k.shape[1:] != (cache.num_kv_heads, cache.head_dim) or slots.shape != (n,):
        raise ValueError("kv_append: shape mismatch")
    _check(_lib.kv_append(ctypes.byref(cache.desc), int(layer), _dev(k, "k", cache.io_dtype),
                          _dev(v, "v", cache.io_dtype), _dev(slots, "slots", torch.int64), n,
                          _stream(stream)))


def contiguous_kv_append(k_cache, v_cache, k, v, pos, num_q_heads=None, stream=None):
    """k_cache, v_cache: [B, H_kv, Lmax, d]; k, v: [B, H_kv, d]; pos: device int32 [B]."""
    B, hkv, lmax, d = k_cache.shape
    if v_cache.shape != k_cache.shape or k.shape != (B, hkv, d) or v.shape != k.shape or pos.shape != (B,):
        raise ValueError("contiguous_kv_append: shape mismatch")
    dm = dims(1, num_q_heads or hkv, hkv, k_cache.dtype, d)
    _check(_lib.contiguous_kv_append(ctypes.byref(dm), _dev(k_cache, "k_cache", k.dtype),
                                     _dev(v_cache, "v_cache", k.dtype), lmax, _dev(k, "k"), _dev(v, "v"),
                                     _dev(pos, "pos", torch.int32), B, _stream(stream)))


def decode_workspace_bytes(num_q_heads, num_kv_heads, dtype, B, max_context, head_dim=HEAD_DIM):
    dm = dims(1, num_q_heads, num_kv_heads, dtype, head_dim)
    return int(_lib.decode_workspace_bytes(ctypes.byref(dm), int(B), int(max_context)))


def make_workspace(num_q_heads, num_kv_heads, dtype, B, max_context, device="cuda", head_dim=HEAD_DIM):
    """Decode workspace, zero-filled as the C ABI requires before first use (torch's
    allocator returns 256-byte aligned blocks)."""
    n = decode_workspace_bytes(num_q_heads, num_kv_heads, dtype, B, max_context, head_dim)
    return torch.zeros((max(n, 256),), dtype=torch.uint8, device=device)


def paged_decode_attention(cache: PagedKVCache, layer, q, block_table, context_lens, out=None,
                           scale=0.0, workspace=None, stream=None):
    """q: device [B, H_q, d] (d = cache.head_dim); block_table: device int32 [B, max_blocks];
    context_lens: device int32 [B].  Returns out [B, H_q, d]."""
    B, hq, d = q.shape
    if hq != cache.num_q_heads or d != cache.head_dim:
        raise ValueError("paged_decode_attention: q shape does not match the cache")
    max_blocks = block_table.shape[1]
    if block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("paged_decode_attention: table / context_lens shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_workspace(hq, cache.num_kv_heads, cache.dtype, B, max_blocks * BLOCK, q.device, d)
    _check(_lib.paged_decode_attention(ctypes.byref(cache.desc), int(layer), _dev(out, "out", cache.io_dtype),
                                       _dev(q, "q", cache.io_dtype), _dev(block_table, "block_table", torch.int32),
                                       max_blocks, _dev(context_lens, "context_lens", torch.int32), B,
                                       float(scale), _dev(workspace, "workspace"), workspace.numel(),
                                       _stream(stream)))
    return out


def paged_decode_attention_noalloc(cache: PagedKVCache, layer, q, block_table, context_lens, out=None, scale=0.0,
                                   stream=None):
    """paged_decode_attention without a workspace (the library's static scratch holds the
    split state; for callers that cannot allocate).  Same arguments and result."""
    B, hq, d = q.shape
    if hq != cache.num_q_heads or d != cache.head_dim:
        raise ValueError("paged_decode_attention_noalloc: q shape does not match the cache")
    max_blocks = block_table.shape[1]
    if block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("paged_decode_attention_noalloc: table / context_lens shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.paged_decode_attention_noalloc(ctypes.byref(cache.desc), int(layer), _dev(out, "out", cache.io_dtype),
                                               _dev(q, "q", cache.io_dtype),
                                               _dev(block_table, "block_table", torch.int32), max_blocks,
                                               _dev(context_lens, "context_lens", torch.int32), B, float(scale),
                                               _stream(stream)))
    return out


def paged_decode_append_attention(cache: PagedKVCache, layer, q, k_new, v_new, block_table, context_lens,
                                  out=None, scale=0.0, workspace=None, stream=None):
    """Fused step: k_new / v_new [B, H_kv, d] go to position context_lens[b] - 1 of each
    request (through block_table) and the decode of q attends over them in the same call."""
    B, hq, d = q.shape
    if hq != cache.num_q_heads or d != cache.head_dim:
        raise ValueError("paged_decode_append_attention: q shape does not match the cache")
    if k_new.shape != (B, cache.num_kv_heads, d) or v_new.shape != k_new.shape:
        raise ValueError("paged_decode_append_attention: k_new / v_new shape mismatch")
    max_blocks = block_table.shape[1]
    if block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("paged_decode_append_attention: table / context_lens shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_workspace(hq, cache.num_kv_heads, cache.dtype, B, max_blocks * BLOCK, q.device, d)
    _check(_lib.paged_decode_append_attention(ctypes.byref(cache.desc), int(layer), _dev(out, "out", cache.io_dtype),
                                              _dev(q, "q", cache.io_dtype), _dev(k_new, "k_new", cache.io_dtype),
                                              _dev(v_new, "v_new", cache.io_dtype),
                                              _dev(block_table, "block_table", torch.int32), max_blocks,
                                              _dev(context_lens, "context_lens", torch.int32), B, float(scale),
                                              _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))
    return out


def decode_plan_bytes(num_q_heads, num_kv_heads, B, max_blocks, pad_items=0, head_dim=HEAD_DIM,
                      kv_dtype=torch.float16):
    """Bytes of a plan image for B requests and tables of max_blocks entries.  kv_dtype is
    the cache's (torch.float16 or torch.int8): the int8 cache at head dim 64 splits into
    shorter parts, so its plans can hold more items."""
    dm = dims(1, num_q_heads, num_kv_heads, kv_dtype, head_dim)
    return int(_lib.decode_plan_bytes(ctypes.byref(dm), int(B), int(max_blocks), int(pad_items)))


def _host_i32(t, name):
    if t.device.type != "cpu" or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous host int32 tensor")
    return ctypes.c_void_p(t.data_ptr())


def decode_plan_build(num_q_heads, num_kv_heads, block_table, context_lens, num_blocks, share_prefix=True,
                      image=None, pin=False, pad_items=0, plan=None, head_dim=HEAD_DIM, long_items=False,
                      kv_dtype=torch.float16, share_width=1, fill=False):
    """Build a decode plan on the host from the HOST block table [B, max_blocks] and context
    lengths [B] (int32 CPU tensors).  Returns (plan, image): plan is a kvp_decode_plan, image
    a uint8 CPU tensor whose first plan.bytes bytes are to be copied to the device.
    pad_items > 0 fixes the item count (see decode_plan_build in kvp.h); long_items asks for
    KVP_PLAN_LONG_ITEMS (fewer, longer parts for batches of long contexts), sized for the
    waves the kernel of kv_dtype's cache keeps resident; share_width (1, 2 or 4 blocks of 16
    query columns) is the width of shared items (KVP_PLAN_SHARE_WIDE2 / 4); fill asks for
    KVP_PLAN_FILL (shorter parts when the batch leaves resident waves idle).  kv_dtype (torch.float16 or
    torch.int8, the cache's) also sets the split size: an int8 cache at head dim 64 is cut
    into 16-block parts, as the unplanned call does, so pass it for int8 caches."""
    B, max_blocks = block_table.shape
    if context_lens.shape != (B,):
        raise ValueError("decode_plan_build: context_lens shape mismatch")
    if share_width not in (1, 2, 4):
        raise ValueError("decode_plan_build: share_width is 1, 2 or 4 column blocks")
    need = decode_plan_bytes(num_q_heads, num_kv_heads, B, max_blocks, pad_items, head_dim, kv_dtype)
    if image is None:
        image = torch.empty((max(need, 16),), dtype=torch.uint8, pin_memory=pin)
    if image.device.type != "cpu" or image.dtype != torch.uint8:
        raise ValueError("decode_plan_build: image must be a uint8 host tensor")
    dm = dims(1, num_q_heads, num_kv_heads, kv_dtype, head_dim)
    plan = kvp_decode_plan() if plan is None else plan
    _check(_lib.decode_plan_build(ctypes.byref(dm), _host_i32(block_table, "block_table"), int(max_blocks),
                                  _host_i32(context_lens, "context_lens"), int(B), int(num_blocks),
                                  (PLAN_SHARE_PREFIX if share_prefix else 0) |
                                  (PLAN_LONG_ITEMS if long_items else 0) | (PLAN_FILL if fill else 0) |
                                  {1: 0, 2: PLAN_SHARE_WIDE2, 4: PLAN_SHARE_WIDE4}[share_width], int(pad_items),
                                  ctypes.c_void_p(image.data_ptr()), image.numel(), ctypes.byref(plan)))
    return plan, image


def decode_plan_workspace_bytes(plan):
    return int(_lib.decode_plan_workspace_bytes(ctypes.byref(plan)))


def upload_plan(plan, image, device="cuda"):
    """Device copy of a plan image (16-byte aligned torch allocation)."""
    return image[: max(int(plan.bytes), 16)].to(device)


def make_plan_workspace(plan, device="cuda"):
    """Zero-filled workspace for paged_decode_attention_planned with this plan."""
    return torch.zeros((max(decode_plan_workspace_bytes(plan), 256),), dtype=torch.uint8, device=device)


def paged_decode_attention_planned(cache: PagedKVCache, layer, q, plan, d_plan, k_new=None, v_new=None,
                                   out=None, scale=0.0, workspace=None, stream=None):
    """Decode following a plan (decode_plan_build + upload_plan).  With k_new / v_new
    ([B, H_kv, d]) the step's token is appended in the same kernel."""
    B, hq, d = q.shape
    if hq != cache.num_q_heads or d != cache.head_dim or B != plan.B:
        raise ValueError("paged_decode_attention_planned: q shape does not match the cache / plan")
    if (k_new is None) != (v_new is None):
        raise ValueError("paged_decode_attention_planned: give both k_new and v_new or neither")
    if k_new is not None and (k_new.shape != (B, cache.num_kv_heads, d) or v_new.shape != k_new.shape):
        raise ValueError("paged_decode_attention_planned: k_new / v_new shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_plan_workspace(plan, q.device)
    kn = _dev(k_new, "k_new", cache.io_dtype) if k_new is not None else None
    vn = _dev(v_new, "v_new", cache.io_dtype) if v_new is not None else None
    _check(_lib.paged_decode_attention_planned(ctypes.byref(cache.desc), int(layer), _dev(out, "out", cache.io_dtype),
                                               _dev(q, "q", cache.io_dtype), kn, vn, ctypes.byref(plan),
                                               _dev(d_plan, "plan"), float(scale), _dev(workspace, "workspace"),
                                               workspace.numel(), _stream(stream)))
    return out


def paged_prefill_attention(cache: PagedKVCache, layer, q, block_table, context_lens, cu_q, max_q, out=None,
                            scale=0.0, stream=None):
    """Several new rows per request against the paged cache (chunked prefill, draft
    verification).  q: [T, H_q, d] fp16 packed by cu_q (device int32 [B+1]); the rows of
    request b are the last cu_q[b+1]-cu_q[b] of its context_lens[b] positions, already
    appended to the cache; row i attends to positions 0 .. ctx - m + i."""
    T, hq, d = q.shape
    if hq != cache.num_q_heads or d != cache.head_dim:
        raise ValueError("paged_prefill_attention: q shape does not match the cache")
    B = cu_q.numel() - 1
    if block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("paged_prefill_attention: table / context_lens / cu_q shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.paged_prefill_attention(ctypes.byref(cache.desc), int(layer), _dev(out, "out", cache.io_dtype),
                                        _dev(q, "q", cache.io_dtype),
                                        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]),
                                        _dev(context_lens, "context_lens", torch.int32),
                                        _dev(cu_q, "cu_q", torch.int32), B, int(max_q), float(scale),
                                        _stream(stream)))
    return out


def sched_simulate(prompt_lens, output_lens, slots, policy=SCHED_CONTINUOUS, alloc=ALLOC_PAGED, max_seq_len=2048,
                   block_size=BLOCK, num_blocks=1 << 20):
    """Static or continuous batching of the requests over a block pool (sched_simulate in
    kvp.h).  Returns (kvp_sched_result, latency int32 [n], service int32 [n]) on the host."""
    p = torch.as_tensor(prompt_lens, dtype=torch.int32).contiguous()
    o = torch.as_tensor(output_lens, dtype=torch.int32).contiguous()
    n = int(o.numel())
    if p.numel() != n:
        raise ValueError("sched_simulate: prompt_lens and output_lens differ in length")
    lat = torch.zeros(max(n, 1), dtype=torch.int32)
    svc = torch.zeros(max(n, 1), dtype=torch.int32)
    cfg = kvp_sched_config(int(slots), int(policy), int(alloc), int(max_seq_len), int(block_size), int(num_blocks))
    res = kvp_sched_result()
    _check(_lib.sched_simulate(ctypes.byref(cfg), ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(o.data_ptr()), n,
                               ctypes.c_void_p(lat.data_ptr()), ctypes.c_void_p(svc.data_ptr()), ctypes.byref(res)))
    return res, lat[:n], svc[:n]


def decode_merge_polls(polls=-1):
    """Wait bound of the fp16 split merge (kvp_decode_merge_polls): polls of a pair's
    counter by its merging item before the counted merge takes over; 0 always takes the
    counted merge.  Returns the previous bound; a negative value only queries it."""
    return int(_lib.kvp_decode_merge_polls(int(polls)))


def contiguous_decode_attention(q, k_cache, v_cache, context_lens, out=None, scale=0.0,
                                workspace=None, stream=None):
    """q: [B, H_q, d]; k_cache, v_cache: [B, H_kv, Lmax, d]; context_lens: int32 [B]."""
    B, hq, d = q.shape
    Bk, hkv, lmax, dk = k_cache.shape
    if Bk != B or dk != d or v_cache.shape != k_cache.shape or context_lens.shape != (B,):
        raise ValueError("contiguous_decode_attention: shape mismatch")
    dm = dims(1, hq, hkv, q.dtype, d)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_workspace(hq, hkv, q.dtype, B, lmax, q.device, d)
    _check(_lib.contiguous_decode_attention(ctypes.byref(dm), _dev(out, "out", q.dtype), _dev(q, "q"),
                                            _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
                                            lmax, _dev(context_lens, "context_lens", torch.int32), B,
                                            float(scale), _dev(workspace, "workspace"), workspace.numel(),
                                            _stream(stream)))
    return out


def varlen_causal_prefill(q, k, v, cu_seqlens, max_seqlen, causal=True, out=None, scale=0.0,
                          stream=None):
    """q: [T, H_q, d]; k, v: [T, H_kv, d]; cu_seqlens: device int32 [nseg+1];
    max_seqlen: host int >= every segment length."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, d) or v.shape != k.shape:
        raise ValueError("varlen_causal_prefill: shape mismatch")
    dm = dims(1, hq, hkv, q.dtype, d)
    if out is None:
        out = torch.empty_like(q)
    nseg = cu_seqlens.numel() - 1
    _check(_lib.varlen_causal_prefill(ctypes.byref(dm), _dev(out, "out", q.dtype), _dev(q, "q"),
                                      _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                                      _dev(cu_seqlens, "cu_seqlens", torch.int32), nseg, int(max_seqlen),
                                      int(bool(causal)), float(scale), _stream(stream)))
    return out


def kv_gather(cache: PagedKVCache, layer, block_table, context_lens, lmax, k_out=None, v_out=None,
              stream=None):
    B, max_blocks = block_table.shape
    shape = (B, cache.num_kv_heads, lmax, cache.head_dim)
    if k_out is None:
        k_out = torch.zeros(shape, dtype=cache.dtype, device=block_table.device)
    if v_out is None:
        v_out = torch.zeros(shape, dtype=cache.dtype, device=block_table.device)
    _check(_lib.kv_gather(ctypes.byref(cache.desc), int(layer), _dev(block_table, "block_table", torch.int32),
                          max_blocks, _dev(context_lens, "context_lens", torch.int32), B, int(lmax),
                          _dev(k_out, "k_out", cache.dtype), _dev(v_out, "v_out", cache.dtype),
                          _stream(stream)))
    return k_out, v_out


def read_bandwidth_probe(buf, waves=0, sink=None, stream=None):
    """Stream-read every byte of the device tensor `buf` once (kvp_read_bandwidth_probe);
    time it with events on the stream.  sink: device int32 [1] (allocated if None)."""
    if sink is None:
        sink = torch.zeros((1,), dtype=torch.int32, device=buf.device)
    _check(_lib.kvp_read_bandwidth_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(), int(waves),
                                         _dev(sink, "sink", torch.int32), _stream(stream)))
    return sink
