"""Host planner of the fp16 decode (decode_plan_build), checked on the CPU against what a
plan must guarantee, read independently from the image:

* every (request, KV head) pair attends over every token j < context length exactly once,
  each token through the block its own table names (a shared item reads the leading
  member's block, which must be the same physical block);
* a pair split into several parts has slots pbase .. pbase+nparts-1, each written once,
  in token order (the merge order), and single-part pairs are written directly;
* shared items hold at most 16 / G members per block of 16 query columns (1, 2 or 4 blocks)
  and a prefix's items run on one XCD;
* each XCD's items are spread over its 32 CUs (queue indices 32 apart share a CU) so that
  no CU carries more than its share of the work plus one item;
* without prefix sharing the plan is exactly the per-pair split (one item up to 32 blocks,
  else ceil(blocks/32) parts, the last ceil(tiles/parts) long, the others sharing the rest) that
  paged_decode_attention uses (so the two are bit-identical on the GPU).

Prefix sharing follows the pages: requests forked from one prefix share its physical
blocks until copy-on-write ([PAGED] paged-attention article, SECTION 3).
"""
import math
import random

import numpy as np
import pytest
import torch

import kv_cache_decode_paged_amd as kvp
import workloads as W

REC, BPI, R_ENT, XCDS = 48, 32, 16, 8
F_SHARED, F_EMPTY, F_LONG = 1, 2, 4
LONG_BPI = 192
BS = 16


def parse(plan, image, B, hkv):
    raw = image[: plan.bytes].numpy().view(np.int32)
    items = raw[: plan.n_items * REC].reshape(plan.n_items, REC)
    pb = raw[plan.off_pair_base // 4: plan.off_pair_base // 4 + B * hkv]
    npt = raw[plan.off_pair_nparts // 4: plan.off_pair_nparts // 4 + B * hkv]
    rs = raw[plan.off_req_shared // 4: plan.off_req_shared // 4 + B]
    ids = raw[plan.off_ids // 4: plan.off_ids // 4 + plan.n_ids]
    assert plan.off_ids // 4 + plan.n_ids <= raw.size
    return items, pb, npt, rs, ids


def check_plan(plan, image, table, ctx, num_blocks, hq, hkv, shared_expected=None):
    B, mb = table.shape
    G = hq // hkv
    items, pbase, nparts, req_shared, long_ids = parse(plan, image, B, hkv)
    assert plan.n_items % XCDS == 0
    ctx = np.clip(ctx, 0, mb * BS)

    def ent(b, j):
        e = int(table[b, j])
        return e if 0 <= e < num_blocks else -1

    # sharing runs: maximal runs of consecutive requests with the same usable first block
    run_of, run = [], -1
    for b in range(B):
        cont = b > 0 and ctx[b] > 0 and ctx[b - 1] > 0 and ent(b, 0) >= 0 and ent(b, 0) == ent(b - 1, 0)
        run += 0 if cont else 1
        run_of.append(run)

    cover = {}   # (b, g) -> token coverage count array
    writes = {}  # (b, g) -> list of (slot or 'direct', first token)
    bundles = {}
    for p, r in enumerate(items):
        fl = int(r[0])
        if fl == F_EMPTY:
            continue
        b, g, nmem, blk0, nblk, end, slot, np_, pb_ = (int(x) for x in r[1:10])
        longi = bool(fl & F_LONG)
        fl &= ~F_LONG
        assert 0 <= g < hkv and nmem >= 1 and b + nmem <= B and blk0 >= 0
        assert 0 <= nblk <= (LONG_BPI if longi else BPI)
        if longi:  # a private item whose ids sit in the id area
            assert fl == 0 and nblk > BPI
            off = int(r[R_ENT])
            assert 0 <= off and off + nblk <= long_ids.size
            assert [int(e) for e in long_ids[off: off + nblk]] == [ent(b, blk0 + j) for j in range(nblk)], p
            assert (r[R_ENT + 1: R_ENT + BPI] == -1).all()
        else:
            for j in range(BPI):
                want = ent(b, blk0 + j) if j < nblk else -1
                assert int(r[R_ENT + j]) == want, (p, j)
        if fl == F_SHARED:
            # a shared item serves at most 16 / G members per block of 16 query columns, 4
            # blocks at head dim 64 (2 at 128); groups above 16 have no shared items
            assert G <= 16 and nmem <= min(16, (16 // G) * (4 if plan.head_dim == 64 else 2)) and slot >= 0
            key = (run_of[b], g)  # one sharing run and KV head
            xs, n = bundles.get(key, (set(), 0))
            bundles[key] = (xs | {p % XCDS}, n + 1)
            for m in range(b, b + nmem):
                E = int(req_shared[m])
                if E <= BS * blk0:  # the member's shared extent ends before this item
                    continue
                assert E % BS == 0 and E < ctx[m]
                lo, hi = BS * blk0, min(BS * (blk0 + nblk), E)
                for j in range(lo // BS, (hi + BS - 1) // BS):
                    assert ent(m, j) == ent(b, j) and ent(m, j) >= 0, "shared block differs"
                c = cover.setdefault((m, g), np.zeros(mb * BS + 1, np.int32))
                c[lo:hi] += 1
                pair = m * hkv + g
                writes.setdefault((m, g), []).append((int(pbase[pair]) + slot, lo))
        else:
            assert fl == 0 and nmem == 1 and end == ctx[b]
            pair = b * hkv + g
            assert np_ == nparts[pair] and pb_ == pbase[pair]
            lo, hi = BS * blk0, min(BS * (blk0 + nblk), end)
            c = cover.setdefault((b, g), np.zeros(mb * BS + 1, np.int32))
            c[lo:max(lo, hi)] += 1
            writes.setdefault((b, g), []).append(("direct" if np_ == 1 else slot, lo))
    for b in range(B):
        for g in range(hkv):
            c = cover.get((b, g))
            assert c is not None, f"pair {(b, g)} has no item"
            assert (c[: ctx[b]] == 1).all() and (c[ctx[b]:] == 0).all(), f"coverage of {(b, g)}"
            w = writes[(b, g)]
            pair = b * hkv + g
            if nparts[pair] == 1:
                assert w == [("direct", 0)] or (ctx[b] == 0 and w[0][0] == "direct")
            else:
                slots = [s for s, _ in sorted(w, key=lambda x: x[1])]
                assert slots == list(range(int(pbase[pair]), int(pbase[pair]) + int(nparts[pair])))
    # per CU: position p runs on XCD p % 8 at queue index p // 8, and queue indices 32 apart
    # share a CU; the planner spreads each XCD's work over its 32 CUs longest first, so no
    # CU carries more than its share plus one item
    # Each CU slot takes its items longest first (the k-th item of slot s sits at queue index
    # 32 k + s) and at most ceil(items of the XCD / 32) of them.
    for x in range(XCDS):
        loads, costs = np.zeros(32), []
        per_slot = [[] for _ in range(32)]
        for qi in range(plan.n_items // XCDS):
            r = items[qi * XCDS + x]
            if int(r[0]) != F_EMPTY:
                cst = int(r[5]) + 2
                loads[qi % 32] += cst
                costs.append(cst)
                per_slot[qi % 32].append(cst)
        if costs:
            assert loads.max() <= loads.sum() / 32 + max(costs), (x, loads.max(), loads.sum() / 32)
            k_max = -(-len(costs) // 32)
            for sl in per_slot:
                assert len(sl) <= k_max, (x, len(sl), k_max)
                assert all(a >= b for a, b in zip(sl, sl[1:])), (x, sl)
    for key, (xs, n) in bundles.items():
        if n <= 8:  # a run's shared items of one head (at most one bundle) share an XCD
            assert len(xs) == 1, f"shared items of run {key} spread over XCDs {xs}"
    if shared_expected is not None:
        assert (plan.n_shared > 0) == shared_expected
    return items, pbase, nparts, req_shared


def build(table, ctx, num_blocks, hq=14, hkv=2, share=True, long_items=False, share_width=1, fill=False,
          kv_dtype=torch.float16):
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32))
    c = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32))
    return kvp.decode_plan_build(hq, hkv, t, c, num_blocks, share_prefix=share, long_items=long_items,
                                 share_width=share_width, fill=fill, kv_dtype=kv_dtype)


def c4_tables(B, steps_done=1, seed=42):
    """Host block tables of the batch-B shared-prefix workload after one reserved step."""
    pb = W.paged_batch(B)
    need = sum(math.ceil((c + 8) / BS) for c in pb.ctx_before) + 64 * B
    pool = kvp.BlockPool(need)
    pool.set_free_order(W.free_list_permutation(need, seed + 1).tolist())
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
    for _ in range(steps_done):
        pool.append_slots(seqs)
    max_blocks = max(math.ceil(pool.tokens(s) / BS) for s in seqs)
    table, ctx = pool.export(seqs, max_blocks)
    return table.numpy(), ctx.numpy(), need, pool, seqs


@pytest.mark.parametrize("B", [10, 50, 200])
def test_plan_shared_prefix_workload(B):
    table, ctx, nb, _, _ = c4_tables(B)
    plan, image = build(table, ctx, nb)
    check_plan(plan, image, table, ctx, nb, 14, 2, shared_expected=True)
    for w in (2, 4):  # wider shared items read each prefix through fewer block reads
        wide, image_w = build(table, ctx, nb, share_width=w)
        check_plan(wide, image_w, table, ctx, nb, 14, 2, shared_expected=True)
        assert wide.kv_blocks_read < plan.kv_blocks_read
    # reading each shared prefix through fewer items than requests
    plain, image0 = build(table, ctx, nb, share=False)
    check_plan(plain, image0, table, ctx, nb, 14, 2, shared_expected=False)
    assert plan.kv_blocks_read < plain.kv_blocks_read


def test_plan_without_sharing_is_the_plain_split():
    table, ctx, nb, _, _ = c4_tables(50)
    plan, image = build(table, ctx, nb, share=False)
    items, pbase, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    got = sorted((int(r[1]), int(r[2]), int(r[4]), int(r[5])) for r in items if r[0] != F_EMPTY)
    want = []
    for b in range(len(ctx)):
        nbt = math.ceil(ctx[b] / BS)
        n, T = (1 if nbt <= BPI else math.ceil(nbt / BPI)), math.ceil(nbt / 4)
        # the last part (it holds the final blocks) takes ceil(T / n) tiles, the others share
        # the rest evenly
        last = -(-T // n)
        rest = T - last
        starts = [0] + [k * rest // (n - 1) for k in range(1, n - 1)] + ([rest] if n > 1 else []) + [T]
        for g in range(2):
            for k in range(n):
                b0, b1 = min(nbt, 4 * starts[k]), min(nbt, 4 * starts[k + 1])
                want.append((b, g, b0, b1 - b0))
    assert got == sorted(want)


def test_plan_members_without_shared_blocks():
    # consecutive requests with the same first block but a short leader whose later blocks
    # were made private; a member whose context ends inside the first block
    table = np.array([[5, 6, 7, 8], [5, 6, 9, 10], [5, 11, -1, -1], [5, 6, 7, 12]], np.int32)
    ctx = np.array([64, 60, 20, 10], np.int32)
    plan, image = build(table, ctx, 16, hq=4, hkv=1)  # group 4: four members per shared item
    items, pbase, nparts, rs = check_plan(plan, image, table, ctx, 16, 4, 1)
    assert list(rs) == [32, 32, 16, 0]  # last member: its only block holds its last token
    assert list(nparts) == [2, 2, 2, 1]  # one shared part (if any) + one private part
    plan, image = build(table, ctx, 16, hq=8, hkv=1)  # group 8: one column block, pairs of members
    items, pbase, nparts, rs = check_plan(plan, image, table, ctx, 16, 8, 1)
    assert list(rs) == [32, 32, 0, 0]  # requests 2 and 3 share no whole block
    for w in (2, 4):  # wider shared items: all four requests in one item again
        plan, image = build(table, ctx, 16, hq=8, hkv=1, share_width=w)
        items, pbase, nparts, rs = check_plan(plan, image, table, ctx, 16, 8, 1)
        assert list(rs) == [32, 32, 16, 0]
    plan, image = build(table, ctx, 16, hq=32, hkv=1)  # group 32: two blocks per member, no sharing
    items, pbase, nparts, rs = check_plan(plan, image, table, ctx, 16, 32, 1)
    assert list(rs) == [0, 0, 0, 0] and plan.n_shared == 0


def test_plan_empty_and_unusable_entries():
    table = np.array([[3, -1, 99, 4], [3, -1, 99, 4], [0, 1, 2, 3]], np.int32)
    ctx = np.array([64, 0, 50], np.int32)
    plan, image = build(table, ctx, 10, hq=4, hkv=2)
    check_plan(plan, image, table, ctx, 10, 4, 2)


@pytest.mark.parametrize("G", [1, 2, 7, 8])
def test_plan_random_forks(G):
    rng = random.Random(1000 + G)
    for trial in range(20):
        hkv = rng.choice([1, 2])
        hq = G * hkv
        B = rng.randint(1, 40)
        mb = rng.randint(1, 80)
        nb = B * mb + 8
        free = list(range(nb))
        rng.shuffle(free)
        table = np.full((B, mb), -1, np.int32)
        ctx = np.zeros(B, np.int32)
        b = 0
        while b < B:
            run = min(B - b, rng.randint(1, 20))
            pre = rng.randint(0, mb)
            pre_blocks = [free.pop() for _ in range(pre)]
            for m in range(b, b + run):
                c = rng.randint(0, mb * BS)
                nbt = math.ceil(c / BS)
                keep = min(rng.randint(0, pre), nbt)
                row = pre_blocks[:keep] + [free.pop() for _ in range(nbt - keep)]
                table[m, :nbt] = row
                ctx[m] = c
            b += run
        if rng.random() < 0.3:  # unusable entries
            i, j = rng.randrange(B), rng.randrange(mb)
            table[i, j] = rng.choice([-7, nb + 3])
        plan, image = build(table, ctx, nb, hq=hq, hkv=hkv)
        check_plan(plan, image, table, ctx, nb, hq, hkv)
        need = kvp.decode_plan_bytes(hq, hkv, B, mb)
        assert plan.bytes <= need


def test_plan_validation():
    table = torch.zeros((2, 4), dtype=torch.int32)
    ctx = torch.tensor([5, 6], dtype=torch.int32)
    with pytest.raises(kvp.KvpError) as e:
        kvp.decode_plan_build(14, 2, table, ctx, 0)
    assert e.value.status == kvp.KVP_ERR_INVALID
    with pytest.raises(kvp.KvpError) as e:
        kvp.decode_plan_build(40, 2, table, ctx, 8)  # group 20: above 16 and not a multiple of 16
    assert e.value.status == kvp.KVP_ERR_UNSUPPORTED
    with pytest.raises(kvp.KvpError) as e:
        kvp.decode_plan_build(96, 1, table, ctx, 8, head_dim=128)  # group 96: more than 2 blocks at d128
    assert e.value.status == kvp.KVP_ERR_UNSUPPORTED
    for hq, hkv in ((18, 2), (14, 1), (32, 1), (64, 1)):  # groups 9, 14, 32 and 64 are served
        plan, _ = kvp.decode_plan_build(hq, hkv, table, ctx, 8)
        assert plan.group == hq // hkv
    small = torch.empty((64,), dtype=torch.uint8)
    with pytest.raises(kvp.KvpError) as e:
        kvp.decode_plan_build(14, 2, table, ctx, 8, image=small)
    assert e.value.status == kvp.KVP_ERR_INVALID
    plan, _ = kvp.decode_plan_build(14, 2, table, ctx, 8)
    assert plan.B == 2 and plan.group == 7 and plan.n_items % XCDS == 0


def test_plan_padding_fixes_the_launch():
    # successive steps of the same batch, padded to one item count: same item count and
    # offsets, so a graph captured with the first plan replays the later ones
    table, ctx, nb, pool, seqs = c4_tables(50)
    plan, _ = build(table, ctx, nb)
    pad = plan.n_items + 40
    got = []
    for step in range(3):
        t = torch.from_numpy(np.ascontiguousarray(table))
        c = torch.from_numpy(np.ascontiguousarray(ctx))
        p, image = kvp.decode_plan_build(14, 2, t, c, nb, pad_items=pad)
        check_plan(p, image, table, ctx, nb, 14, 2)
        got.append((p.n_items, p.bytes, p.off_pair_base, p.off_pair_nparts, p.off_req_shared))
        pool.append_slots(seqs)
        table, ctx = (x.numpy() for x in pool.export(seqs, table.shape[1] + 1))
    assert got[0][0] == ((pad + 7) // 8) * 8
    assert len(set(got)) == 1
    t = torch.from_numpy(np.ascontiguousarray(table))
    c = torch.from_numpy(np.ascontiguousarray(ctx))
    with pytest.raises(kvp.KvpError) as e:
        kvp.decode_plan_build(14, 2, t, c, nb, pad_items=8)
    assert e.value.status == kvp.KVP_ERR_INVALID


def long_tables(B, ctx_len, seed=3, num_blocks=None):
    """B private contexts of ctx_len tokens on a shuffled pool (the long-context batch)."""
    nbt = (ctx_len + BS - 1) // BS
    nb = num_blocks or B * nbt + 16
    ids = np.random.default_rng(seed).permutation(nb)[: B * nbt].astype(np.int32)
    return ids.reshape(B, nbt), np.full(B, ctx_len, np.int32), nb


def test_long_items_fill_one_generation():
    # 32 requests x 32790 tokens, 2 KV heads: 131200 private blocks over 1024 waves -> parts
    # of 132 blocks (whole tiles), 16 per pair, 1024 items, ids in the id area
    table, ctx, nb = long_tables(32, 32790)
    plan, image = build(table, ctx, nb, share=False, long_items=True)
    items, pbase, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    live = items[items[:, 0] != F_EMPTY]
    assert len(live) == 1024 and (live[:, 0] == F_LONG).all()
    assert live[:, 5].max() <= 132 and (nparts == 16).all()
    assert plan.n_ids == live[:, 5].sum() == 32 * 2 * 2050
    assert plan.bytes >= plan.off_ids + 4 * plan.n_ids
    # without the flag: the 32-block splits, no id area
    plain, image0 = build(table, ctx, nb, share=False)
    items0, _, nparts0, _ = check_plan(plain, image0, table, ctx, nb, 14, 2)
    assert plain.n_ids == 0 and ((items0[:, 0] & F_LONG) == 0).all() and (nparts0 == 65).all()


@pytest.mark.parametrize("B,ctx_len", [(1, 40000), (4, 70000), (200, 3000)])
def test_long_items_only_when_the_batch_is_long(B, ctx_len):
    # long items appear only when the private blocks exceed 1024 waves x 32 blocks: a small
    # total keeps the 32-block splits, a larger one (many short contexts too) gets parts of
    # up to 192 blocks
    table, ctx, nb = long_tables(B, ctx_len, seed=B)
    plan, image = build(table, ctx, nb, share=False, long_items=True)
    items, _, _, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    live = items[items[:, 0] != F_EMPTY]
    priv_blocks = 2 * B * ((ctx_len + BS - 1) // BS)
    if priv_blocks <= 1024 * BPI:
        assert plan.n_ids == 0 and live[:, 5].max() <= BPI
    else:
        assert live[:, 5].max() <= LONG_BPI and plan.n_ids > 0


def test_long_items_with_shared_prefixes_and_padding():
    # shared-prefix items keep their 32-block records; private ranges after the prefix become
    # long items; a padded plan keeps its offsets when the id area grows
    B, pre, tail = 16, 8192, 40000
    nbp, nbt = pre // BS, (pre + tail) // BS
    rng = np.random.default_rng(9)
    nb = nbp + B * (nbt - nbp) + 8
    ids = rng.permutation(nb).astype(np.int32)
    table = np.empty((B, nbt), np.int32)
    table[:, :nbp] = ids[:nbp]
    table[:, nbp:] = ids[nbp: nbp + B * (nbt - nbp)].reshape(B, nbt - nbp)
    ctx = np.full(B, pre + tail, np.int32)
    plan, image = build(table, ctx, nb, share=True, long_items=True)
    items, _, _, _ = check_plan(plan, image, table, ctx, nb, 14, 2, shared_expected=True)
    sh = items[(items[:, 0] & F_SHARED) != 0]
    assert len(sh) > 0 and sh[:, 5].max() <= BPI
    assert ((items[:, 0] & F_LONG) != 0).any()
    t = torch.from_numpy(table)
    c = torch.from_numpy(ctx)
    p1, im1 = kvp.decode_plan_build(14, 2, t, c, nb, long_items=True, pad_items=plan.n_items + 64)
    check_plan(p1, im1, table, ctx, nb, 14, 2)
    c2 = torch.from_numpy(ctx + 1)
    p2, im2 = kvp.decode_plan_build(14, 2, t, c2, nb, long_items=True, pad_items=plan.n_items + 64)
    assert (p1.n_items, p1.off_pair_base, p1.off_req_shared, p1.off_ids) == \
        (p2.n_items, p2.off_pair_base, p2.off_req_shared, p2.off_ids)


def test_long_items_sized_for_the_int8_kernel():
    # the int8 kernel keeps 2048 waves resident (18 KB of LDS each): the same batch gets
    # parts of about half the length (131200 / 2048 blocks, whole tiles: 68), 31 per pair,
    # 1984 items in one generation
    table, ctx, nb = long_tables(32, 32790)
    t = torch.from_numpy(table)
    c = torch.from_numpy(ctx)
    plan, image = kvp.decode_plan_build(14, 2, t, c, nb, share_prefix=False, long_items=True, kv_dtype=torch.int8)
    items, _, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    live = items[items[:, 0] != F_EMPTY]
    assert len(live) == 1984 and live[:, 5].max() <= 68 and (nparts == 31).all()


def test_int8_plans_split_at_16_blocks():
    # an int8 cache's plan (kv_dtype=int8): without sharing, one item up to 16 blocks, else
    # ceil(blocks / 16) parts -- the unplanned int8 call's own splits
    rng = np.random.default_rng(21)
    B = 12
    ctx = rng.integers(1, 900, size=B).astype(np.int32)
    nbt = (ctx + BS - 1) // BS
    nb = int(nbt.sum()) + 4
    ids = rng.permutation(nb).astype(np.int32)
    table = np.full((B, int(nbt.max())), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, : nbt[b]] = ids[o: o + nbt[b]]
        o += nbt[b]
    t, c = torch.from_numpy(table), torch.from_numpy(ctx)
    plan, image = kvp.decode_plan_build(14, 2, t, c, nb, share_prefix=False, kv_dtype=torch.int8)
    items, _, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    for b in range(B):
        want = 1 if nbt[b] <= 16 else -(-int(nbt[b]) // 16)
        assert int(nparts[2 * b]) == want == int(nparts[2 * b + 1]), b
    live = items[items[:, 0] != F_EMPTY]
    assert live[:, 5].max() <= 16


# ---- KVP_PLAN_FILL: shorter parts while the batch leaves resident waves idle ----

def test_fill_cuts_a_lone_request_into_short_parts():
    # one request of 1024 tokens, 2 KV heads: 64 blocks per pair; the default split is 2
    # parts of 32 blocks, fill takes 8 parts of 8 blocks (16 items for 1024 waves)
    table, ctx, nb = long_tables(1, 1024)
    plain, image0 = build(table, ctx, nb, share=False)
    items0, _, nparts0, _ = check_plan(plain, image0, table, ctx, nb, 14, 2)
    assert (nparts0 == 2).all()
    plan, image = build(table, ctx, nb, share=False, fill=True)
    items, _, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    live = items[items[:, 0] != F_EMPTY]
    assert len(live) == 16 and (live[:, 5] == 8).all() and (nparts == 8).all()
    # a short context: one 2-tile part per 8 blocks, the last part shorter
    table, ctx, nb = long_tables(1, 200)
    plan, image = build(table, ctx, nb, share=False, fill=True)
    items, _, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
    assert (nparts == 2).all()


@pytest.mark.parametrize("B", [10, 50, 100, 200])
def test_fill_on_the_shared_prefix_workload(B):
    table, ctx, nb, _, _ = c4_tables(B)
    plain, image0 = build(table, ctx, nb)
    items0, _, _, _ = check_plan(plain, image0, table, ctx, nb, 14, 2, shared_expected=True)
    plan, image = build(table, ctx, nb, fill=True)
    items, _, nparts, _ = check_plan(plan, image, table, ctx, nb, 14, 2, shared_expected=True)
    live = items[items[:, 0] != F_EMPTY]
    priv = live[live[:, 0] == 0]
    if priv[:, 5].max() < BPI:
        # shorter parts only while every item fits the 1024 waves at once
        assert len(live) <= 1024 and priv[:, 5].max() >= 8
        assert len(live) > len(items0[items0[:, 0] != F_EMPTY])
    else:
        # a batch whose 32-block parts fill the waves keeps its plan
        assert plan.n_items == plain.n_items and plan.bytes == plain.bytes
        assert torch.equal(image[: plan.bytes], image0[: plain.bytes])
    if B <= 50:
        assert priv[:, 5].max() == 8


def test_fill_counts_the_int8_kernels_waves():
    # 24 requests of 4096 tokens, 2 KV heads: 12288 private blocks.  fp16 (1024 waves) keeps
    # 16-block parts or longer; the int8 kernel (2048 waves, 16-block default parts) takes
    # 8-block parts only if they fit its waves
    table, ctx, nb = long_tables(24, 4096)
    for dt, waves in ((torch.float16, 1024), (torch.int8, 2048)):
        plan, image = build(table, ctx, nb, share=False, fill=True, kv_dtype=dt)
        items, _, _, _ = check_plan(plan, image, table, ctx, nb, 14, 2)
        live = items[items[:, 0] != F_EMPTY]
        default = 32 if dt == torch.float16 else 16
        if live[:, 5].max() < default:
            assert len(live) <= waves


def test_fill_leaves_long_items_alone():
    # the long-context batch: long items decide the parts, fill adds nothing
    table, ctx, nb = long_tables(32, 32790)
    a, ia = build(table, ctx, nb, share=False, long_items=True)
    b, ib = build(table, ctx, nb, share=False, long_items=True, fill=True)
    assert a.n_items == b.n_items and torch.equal(ia[: a.bytes], ib[: b.bytes])
