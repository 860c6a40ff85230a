"""The C ABI library: it loads without a GPU, exports every symbol kvp.h declares, and its
host-side calls validate arguments (CPU only; no device work is launched here)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    names = set()
    for m in re.finditer(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text):
        name = m.group(1)
        prefix = text[max(0, m.start() - 80):m.start()]
        # declarations: return type precedes the name on the same statement
        if name in {"if", "for", "while", "sizeof", "defined"}:
            continue
        if re.search(r"(kvp_status|void|size_t|int32_t|int64_t|const char\s*\*)\s*\**\s*$", prefix):
            names.add(name)
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ["kv_append", "paged_decode_attention", "varlen_causal_prefill", "block_table_alloc",
                 "block_table_fork", "block_table_cow", "block_table_free", "block_table_append_slot",
                 "kv_copy_blocks", "contiguous_decode_attention", "kv_gather", "decode_workspace_bytes",
                 "kv_bytes_per_token", "kvp_last_error", "decode_plan_build", "decode_plan_bytes",
                 "decode_plan_workspace_bytes", "paged_decode_attention_planned"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    import kv_cache_decode_paged_amd as kvp
    lib = kvp.lib()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in kvp.h but not exported: {missing}"


def test_version_and_error_text():
    import kv_cache_decode_paged_amd as kvp
    assert "gfx950" in kvp.version()
    lib = kvp.lib()
    out = ctypes.c_void_p()
    assert lib.block_pool_create(0, 16, ctypes.byref(out)) == kvp.KVP_ERR_INVALID
    assert "num_blocks" in kvp.last_error()


def test_kv_bytes_per_token_matches_pages():
    import kv_cache_decode_paged_amd as kvp
    assert kvp.kv_bytes_per_token(24, 2, 64, 2) == 12288
    assert kvp.kv_bytes_per_token(24, 14, 64, 2) == 86016


def test_device_calls_reject_bad_arguments_before_launch():
    import kv_cache_decode_paged_amd as kvp
    lib = kvp.lib()
    d = kvp.kvp_dims(1, 14, 4, 64, kvp.KVP_F16)  # 14 % 4 != 0
    assert lib.decode_workspace_bytes(ctypes.byref(d), 1, 100) == 0
    st = lib.contiguous_decode_attention(ctypes.byref(d), None, None, None, None, 16, None, 1, 0.0,
                                         None, 0, None)
    assert st == kvp.KVP_ERR_INVALID
    for hd, dt in ((96, kvp.KVP_F16), (128, kvp.KVP_F32), (256, kvp.KVP_F16)):  # not built
        d = kvp.kvp_dims(1, 14, 2, hd, dt)
        st = lib.varlen_causal_prefill(ctypes.byref(d), None, None, None, None, None, 1, 8, 1, 0.0, None)
        assert st == kvp.KVP_ERR_UNSUPPORTED
        assert lib.decode_workspace_bytes(ctypes.byref(d), 1, 100) == 0
        st = lib.contiguous_decode_attention(ctypes.byref(d), None, None, None, None, 16, None, 1, 0.0,
                                             None, 0, None)
        assert st == kvp.KVP_ERR_UNSUPPORTED
    desc = kvp.kvp_cache_desc(kvp.kvp_dims(2, 14, 2, 96, kvp.KVP_F16), 16, 8, 16, 16)
    assert lib.kv_copy_blocks(ctypes.byref(desc), None, 1, None) == kvp.KVP_ERR_UNSUPPORTED
    desc = kvp.kvp_cache_desc(kvp.kvp_dims(2, 14, 2, 64, kvp.KVP_F16), 16, 8, None, None)
    st = lib.kv_append(ctypes.byref(desc), 0, None, None, None, 1, None)
    assert st == kvp.KVP_ERR_INVALID  # NULL pools
    st = lib.paged_decode_attention(ctypes.byref(desc), 5, None, None, None, 4, None, 1, 0.0, None, 0, None)
    assert st == kvp.KVP_ERR_INVALID  # layer out of range
    # zero-sized work is a valid no-op and launches nothing
    desc2 = kvp.kvp_cache_desc(kvp.kvp_dims(2, 14, 2, 64, kvp.KVP_F16), 16, 8, 16, 16)
    assert lib.kv_copy_blocks(ctypes.byref(desc2), None, 0, None) == kvp.KVP_OK


def test_workspace_size():
    import kv_cache_decode_paged_amd as kvp
    # fp16: a pair longer than 32 blocks is cut into ceil(blocks / 32) parts, one partial per
    # part (one 68-float record per query head of the group: 7 here) + one ticket per pair;
    # 32768 tokens = 2048 blocks -> 64
    ws = kvp.decode_workspace_bytes(14, 2, torch.float16, 32, 32768)
    assert ws == 32 * 2 * 64 * 7 * 68 * 4 + 256
    # contexts of at most 512 tokens are never split: no workspace
    assert kvp.decode_workspace_bytes(14, 2, torch.float16, 200, 512) == 0
    assert kvp.decode_workspace_bytes(14, 2, torch.float16, 200, 513) == 1792 + 200 * 2 * 2 * 7 * 68 * 4
    # head_dim 128: 132-float partial records (group 4)
    assert kvp.decode_workspace_bytes(32, 8, torch.float16, 4, 4096, head_dim=128) == 256 + 4 * 8 * 8 * 4 * 132 * 4
    # multi-query: 14 and 32 query heads on one KV head
    assert kvp.decode_workspace_bytes(14, 1, torch.float16, 2, 1024) == 256 + 2 * 1 * 2 * 14 * 68 * 4
    assert kvp.decode_workspace_bytes(32, 1, torch.float16, 2, 1024, head_dim=128) == 256 + 2 * 1 * 2 * 32 * 132 * 4
    # groups above 16 that are not a multiple of 16 are refused (no workspace)
    assert kvp.decode_workspace_bytes(20, 1, torch.float16, 2, 1024) == 0
    # fp32 single head, short context: one split, no workspace needed
    assert kvp.decode_workspace_bytes(1, 1, torch.float32, 1, 88) == 0
    # 5000 tokens: at most 16 splits (256-token splits up to 4096 tokens, 512 beyond)
    assert kvp.decode_workspace_bytes(1, 1, torch.float32, 4, 5000) == 256 + 4 * 1 * 16 * 66 * 4
