"""The block pool model against the paged-attention article's printed examples (CPU)."""
import math

import pytest

from conftest import golden_kv
from oracle.pagepool import PagePoolModel, PoolError, PoolOOM


def test_section2_allocation_example():
    g = golden_kv("paged_allocation.txt")
    pool = PagePoolModel(int(g["pool_pages"][0]), int(g["page_size"][0]))
    seqs = []
    for n in map(int, g["tokens"]):
        sid = pool.alloc_seq(0)
        for _ in range(n):
            pool.append_slot(sid)
        seqs.append(sid)
    assert [len(pool.table(s)) for s in seqs] == list(map(int, g["pages"]))
    ps = pool.page_size
    waste = [(ps - pool.tokens(s) % ps) % ps for s in seqs]
    assert waste == list(map(int, g["waste"]))
    assert f"{pool.utilisation:.1f}" == g["utilisation_1dp"][0]
    # pages are handed out front-first from 0..N-1: tables are consecutive runs
    assert pool.table(seqs[0]) == list(range(20))
    assert pool.table(seqs[1]) == [20, 21, 22]
    pool.free_seq(seqs[1])
    assert pool.used == int(g["used_after_free_req1"][0])
    # released pages go to the back of the free list
    assert list(pool.free)[-3:] == [20, 21, 22]


def test_section3_copy_on_write_example():
    g = golden_kv("cow_prefix.txt")
    pool = PagePoolModel(int(g["pool_pages"][0]), int(g["page_size"][0]))
    sys_seq = pool.alloc_seq(int(g["system_tokens"][0]))
    assert len(pool.table(sys_seq)) == int(g["system_pages"][0])
    assert pool.table(sys_seq) == list(map(int, g["system_page_ids"]))
    users = [pool.fork(sys_seq) for _ in range(int(g["users"][0]))]
    assert all(pool.refcount(p) == int(g["refcount_after_share"][0]) for p in pool.table(sys_seq))
    assert len(users) * len(pool.table(sys_seq)) == int(g["naive_pages"][0])
    assert pool.used == int(g["system_pages"][0])
    mb_per_token = 524288 / 1024 / 1024
    saved = (int(g["naive_pages"][0]) - int(g["system_pages"][0])) * 16 * mb_per_token
    assert saved == float(g["saved_mb"][0])
    # req-3 writes its first private token: 200 % 16 = 8, so the last page is shared
    slot, copy = pool.append_slot(users[3])
    assert copy == (int(g["cow_old"][0]), int(g["cow_new"][0]))
    assert pool.refcount(int(g["cow_old"][0])) == int(g["refcount_old_after_cow"][0])
    assert pool.table(users[3])[-1] == int(g["cow_new"][0])
    assert slot == int(g["cow_new"][0]) * 16 + 8
    # every other user still maps page 12
    assert all(pool.table(u)[-1] == 12 for i, u in enumerate(users) if i != 3)


def test_append_in_place_when_not_shared():
    pool = PagePoolModel(8, 16)
    s = pool.alloc_seq(3)
    slot, copy = pool.append_slot(s)
    assert copy is None and slot == 3


def test_oom_leaves_state_unchanged():
    pool = PagePoolModel(4, 16)
    a = pool.alloc_seq(40)  # 3 pages
    before = (list(pool.free), dict(pool.ref), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()})
    with pytest.raises(PoolOOM):
        pool.alloc_seq(33)  # needs 3, 1 free
    after = (list(pool.free), dict(pool.ref), {k: (list(v[0]), v[1]) for k, v in pool.seqs.items()})
    assert before == after
    b = pool.fork(a)
    pool.alloc_seq(16)  # takes the last page
    with pytest.raises(PoolOOM):
        pool.append_slot(b)  # 40 % 16 = 8 -> shared last page needs a copy, none free
    assert pool.tokens(b) == 40 and pool.table(b) == pool.table(a)


def test_double_release_is_an_error():
    pool = PagePoolModel(4, 16)
    pid = pool.allocate()
    pool.release(pid)
    with pytest.raises(PoolError):
        pool.release(pid)


def test_fork_then_free_returns_pages_only_at_zero():
    pool = PagePoolModel(16, 16)
    a = pool.alloc_seq(50)
    b = pool.fork(a)
    pool.free_seq(a)
    assert pool.used == math.ceil(50 / 16)
    pool.free_seq(b)
    assert pool.used == 0


def test_cow_noop_when_private():
    pool = PagePoolModel(8, 16)
    a = pool.alloc_seq(20)
    assert pool.cow(a, 1) == (1, 1)
