"""Reference model of the KV page manager (qd_blocks_* in include/qd.h).

TEST INFRASTRUCTURE ONLY: the tests compare the library's C++ manager with
it operation by operation; the library never uses it.  It shares no code
with the library.  Plain Python lists and dicts.

It follows the rkmt page ("从零构建 Qwen3-8B 推理引擎"): section 4.3.1 (fixed
pages, a free pool reused in O(1), one page list per sequence) and section
4.4.4 (an automatic prefix cache keyed by token content, longest match
first).  The pages leave the policies open; the readings taken:

* pages hold 16 tokens; a sequence's pages cover positions [0, length);
* the free pool is a stack: the first page taken is 0, a released page is
  the next one taken;
* a page is shared only while full: a fork shares the full pages and gives
  the new sequence a fresh page for the partly filled one (the caller copies
  it);
* the prefix cache registers full pages under (key of the previous page,
  16 tokens); registered pages stay cached when their sequences end and
  are evicted, least recently released first, only when the free stack is
  empty; a sequence releases its pages from the last to the first;
* a cache key is a fresh serial number per registration, so evicting a
  page orphans every key built on it.
"""
from __future__ import annotations

PAGE = 16
OK, EINVAL, EUNSUPPORTED, ENOMEM = 0, -1, -2, -5


class PageModel:
    def __init__(self, num_pages: int, max_pages: int):
        self.num_pages, self.max_pages = num_pages, max_pages
        self.free = list(range(num_pages - 1, -1, -1))  # stack: take from the end
        self.lru = []          # cached pages nobody references: [0] evicted first
        self.refs = [0] * num_pages
        self.key_of = {}       # cached page -> its key
        self.serial = {}       # cached page -> serial number
        self.table = {}        # key -> cached page
        self.next_serial = 1
        self.seqs = {}         # id -> [pages, length]

    def available(self) -> int:
        return len(self.free) + len(self.lru)

    def _take(self) -> int:
        if self.free:
            p = self.free.pop()
        else:
            p = self.lru.pop(0)
            del self.table[self.key_of.pop(p)]
            del self.serial[p]
        self.refs[p] = 1
        return p

    def _add_ref(self, p: int) -> None:
        if self.refs[p] == 0 and p in self.key_of:
            self.lru.remove(p)
        self.refs[p] += 1

    def _drop_ref(self, p: int) -> None:
        self.refs[p] -= 1
        if self.refs[p] == 0:
            (self.lru if p in self.key_of else self.free).append(p)

    def add(self, seq: int) -> int:
        if seq in self.seqs:
            return EINVAL
        self.seqs[seq] = [[], 0]
        return OK

    def reserve(self, seq: int, n: int) -> int:
        if seq not in self.seqs or n < 0:
            return EINVAL
        if n > self.max_pages * PAGE:
            return EUNSUPPORTED
        pages, length = self.seqs[seq]
        more = -(-n // PAGE) - len(pages)
        if more > self.available():
            return ENOMEM
        for _ in range(more):
            pages.append(self._take())
        self.seqs[seq][1] = max(length, n)
        return OK

    def release(self, seq: int) -> int:
        if seq not in self.seqs:
            return EINVAL
        for p in reversed(self.seqs.pop(seq)[0]):
            self._drop_ref(p)
        return OK

    def fork(self, src: int, dst: int):
        """(return code, copy_src, copy_dst)"""
        if src not in self.seqs or dst in self.seqs:
            return EINVAL, -1, -1
        pages, length = self.seqs[src]
        full = length // PAGE
        partial = len(pages) > full
        if partial and self.available() < 1:
            return ENOMEM, -1, -1
        new = []
        for p in pages[:full]:
            self._add_ref(p)
            new.append(p)
        cs = cd = -1
        if partial:
            cd = self._take()
            cs = pages[full]
            new.append(cd)
        self.seqs[dst] = [new, length]
        return (1 if partial else 0), cs, cd

    def tables(self, seqs, pad: int):
        rows = []
        for s in seqs:
            if s not in self.seqs:
                return EINVAL, None
            pages = self.seqs[s][0]
            rows.append([pages[j] if j < len(pages) else pad for j in range(self.max_pages)])
        return OK, rows

    def length(self, seq: int) -> int:
        return self.seqs[seq][1] if seq in self.seqs else EINVAL

    def publish(self, seq: int, tokens) -> int:
        if seq not in self.seqs or len(tokens) > self.seqs[seq][1]:
            return EINVAL
        pages = self.seqs[seq][0]
        parent, added = 0, 0
        for i in range(len(tokens) // PAGE):
            key = (parent, tuple(int(t) for t in tokens[i * PAGE:(i + 1) * PAGE]))
            if key in self.table:
                parent = self.serial[self.table[key]]
                continue
            p = pages[i]
            if p in self.key_of:
                break
            self.table[key] = p
            self.key_of[p] = key
            self.serial[p] = self.next_serial
            parent = self.next_serial
            self.next_serial += 1
            added += 1
        return added

    def match(self, seq: int, tokens) -> int:
        if seq not in self.seqs or self.seqs[seq][0]:
            return EINVAL
        pages = self.seqs[seq][0]
        parent, i = 0, 0
        while i < len(tokens) // PAGE and i < self.max_pages:
            key = (parent, tuple(int(t) for t in tokens[i * PAGE:(i + 1) * PAGE]))
            if key not in self.table:
                break
            p = self.table[key]
            self._add_ref(p)
            pages.append(p)
            parent = self.serial[p]
            i += 1
        self.seqs[seq][1] = i * PAGE
        return i * PAGE

    def check_invariants(self) -> None:
        """Every page is in exactly one state and its count of holders is its
        reference count; cached pages are exactly the table's values."""
        held = [0] * self.num_pages
        for pages, length in self.seqs.values():
            assert len(pages) == -(-length // PAGE) or len(pages) * PAGE >= length
            for p in pages:
                held[p] += 1
        assert held == self.refs
        free, lru = set(self.free), set(self.lru)
        assert len(free) == len(self.free) and len(lru) == len(self.lru)
        for p in range(self.num_pages):
            states = (p in free) + (p in lru) + (self.refs[p] > 0)
            assert states == 1, p
            assert (p in lru) <= (p in self.key_of)
        assert sorted(self.table.values()) == sorted(self.key_of)
