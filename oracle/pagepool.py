"""Block pool / block table / copy-on-write model -- TEST INFRASTRUCTURE ONLY.

The semantics follow the paged-attention article of the chatgpz.de "Aufmerksamkeit" feed
("SECTION 2 -- Paged Attention: Pages + Block Table" and "SECTION 3 -- Copy-on-Write:
Shared System Prompts"), restated here in my own code:

  * the pool is a flat array of equal pages; the free list starts as 0..N-1, allocation
    takes the page at the FRONT of the list, a released page goes to the BACK;
  * every allocated page carries a reference count; sharing a page adds one; releasing
    subtracts one and the page returns to the free list when the count reaches zero;
  * copy-on-write takes a new page and releases the old one;
  * utilisation is the allocated fraction of the pool, in percent;
  * a request holds a block table (logical block -> physical page) and a token count; a
    new page is taken whenever the token count sits on a page boundary.

Readings where the article is silent (each is listed with its reason in the design notes):
  * fork: the child copies the parent's table and token count and shares every page;
  * appending into a page whose count is above one copies it first (private only when
    needed); with a count of one the write goes in place;
  * running out of pages raises PoolOOM and leaves every table, count and the free-list
    order exactly as before (capacity is checked before anything is taken);
  * releasing a page that is not allocated raises PoolError (a double free);
  * truncating a sequence releases the pages past its new length; a kept shared page
    stays shared (a later append into it is copied first).
"""
import math
from collections import deque


class PoolError(Exception):
    pass


class PoolOOM(PoolError):
    pass


class PagePoolModel:
    def __init__(self, num_pages, page_size=16):
        if num_pages <= 0 or page_size <= 0:
            raise PoolError("bad pool geometry")
        self.total = num_pages
        self.page_size = page_size
        self.free = deque(range(num_pages))
        self.ref = {}
        self.seqs = {}          # seq id -> [table(list), tokens(int)]
        self._next_seq = 0

    # -- pages ---------------------------------------------------------------------------
    def allocate(self):
        if not self.free:
            raise PoolOOM("no free pages")
        pid = self.free.popleft()
        self.ref[pid] = 1
        return pid

    def release(self, pid):
        if pid not in self.ref:
            raise PoolError(f"page {pid} is not allocated")
        self.ref[pid] -= 1
        if self.ref[pid] == 0:
            del self.ref[pid]
            self.free.append(pid)

    def share(self, pid):
        if pid not in self.ref:
            raise PoolError(f"page {pid} is not allocated")
        self.ref[pid] += 1

    def cow_copy(self, pid):
        new = self.allocate()
        self.release(pid)
        return new

    @property
    def used(self):
        return self.total - len(self.free)

    @property
    def utilisation(self):
        return self.used / self.total * 100.0

    @property
    def shared(self):
        return sum(1 for c in self.ref.values() if c > 1)

    # -- sequences -----------------------------------------------------------------------
    def alloc_seq(self, n_tokens):
        if n_tokens < 0:
            raise PoolError("negative token count")
        need = math.ceil(n_tokens / self.page_size)
        if need > len(self.free):
            raise PoolOOM("no free pages")
        table = [self.allocate() for _ in range(need)]
        sid = self._next_seq
        self._next_seq += 1
        self.seqs[sid] = [table, n_tokens]
        return sid

    def fork(self, parent):
        if parent not in self.seqs:
            raise KeyError(parent)
        table, tokens = self.seqs[parent]
        for pid in table:
            self.share(pid)
        sid = self._next_seq
        self._next_seq += 1
        self.seqs[sid] = [list(table), tokens]
        return sid

    def cow(self, sid, logical_block):
        """Make logical block private to `sid`; returns (src, dst) (equal when no copy)."""
        table, _ = self.seqs[sid]
        if not 0 <= logical_block < len(table):
            raise PoolError("logical block out of range")
        old = table[logical_block]
        if self.ref[old] == 1:
            return old, old
        new = self.cow_copy(old)
        table[logical_block] = new
        return old, new

    def append_slot(self, sid):
        """Reserve the position of the next token.  Returns (slot, (src, dst) or None)."""
        table, tokens = self.seqs[sid]
        ps = self.page_size
        copy = None
        if tokens % ps == 0:
            table.append(self.allocate())
        else:
            lb = tokens // ps
            if self.ref[table[lb]] > 1:
                src, dst = self.cow(sid, lb)
                copy = (src, dst)
        slot = table[tokens // ps] * ps + tokens % ps
        self.seqs[sid][1] = tokens + 1
        return slot, copy

    def append_batch(self, sids):
        """append_slot for each id in order; all or nothing (state restored on OOM)."""
        import copy as _copy
        if len(set(sids)) != len(sids):
            raise PoolError("repeated sequence in batch")
        saved = (_copy.deepcopy(self.free), dict(self.ref),
                 {k: [list(v[0]), v[1]] for k, v in self.seqs.items()})
        try:
            return [self.append_slot(s) for s in sids]
        except PoolOOM:
            self.free, self.ref, self.seqs = saved
            raise

    def reserve(self, sid, n):
        """n appends in one call, all or nothing: returns (slots, (src, dst) or None)."""
        table, tokens = self.seqs[sid]
        ps = self.page_size
        need = math.ceil((tokens + n) / ps) - len(table)
        copy_needed = n > 0 and tokens % ps != 0 and self.ref[table[tokens // ps]] > 1
        if need + int(copy_needed) > len(self.free):
            raise PoolOOM("no free pages")
        slots, copy = [], None
        for _ in range(n):
            slot, c = self.append_slot(sid)
            slots.append(slot)
            if c is not None:
                copy = c
        return slots, copy

    def truncate(self, sid, n_tokens):
        """Shorten to n_tokens: pages past ceil(n/page_size) are released (in table
        order); kept pages keep their sharing, so a later append copies a shared one."""
        table, tokens = self.seqs[sid]
        if not 0 <= n_tokens <= tokens:
            raise PoolError("bad truncate length")
        keep = math.ceil(n_tokens / self.page_size)
        for pid in table[keep:]:
            self.release(pid)
        del table[keep:]
        self.seqs[sid][1] = n_tokens

    def free_seq(self, sid):
        table, _ = self.seqs.pop(sid)
        for pid in table:
            self.release(pid)

    def table(self, sid):
        return list(self.seqs[sid][0])

    def tokens(self, sid):
        return self.seqs[sid][1]

    def slots(self, sid, start, n):
        table, tokens = self.seqs[sid]
        ps = self.page_size
        assert 0 <= start and start + n <= tokens
        return [table[j // ps] * ps + j % ps for j in range(start, start + n)]

    def refcount(self, pid):
        return self.ref.get(pid, 0)
