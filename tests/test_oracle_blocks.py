"""Pins of the page-manager model (oracle/blocks.py) against hand-worked
cases and invariants.

* Pages are taken 0, 1, 2, ...; a released sequence's pages go back last
  page first, so its first page is the next one taken.
* reserve covers ceil(n / 16) pages; running out changes nothing; more than
  max_pages_per_seq pages is refused.
* A fork shares the full pages (their reference counts rise) and gives the
  new sequence a fresh page for the partly filled one, with the copy to make.
* The prefix cache returns the longest run of full pages whose tokens match
  from the start, only whole pages, and nothing once the first differs.
* Cached pages are evicted least recently released first, a chain from its
  last page, so that what remains of a chain still matches from its start.
* Random operation sequences keep every page in exactly one state, with a
  reference count equal to the number of sequences that hold it.
"""
import numpy as np

from oracle.blocks import EINVAL, ENOMEM, EUNSUPPORTED, OK, PAGE, PageModel


def test_take_order_and_release_stack():
    m = PageModel(8, 4)
    assert m.add(1) == OK and m.reserve(1, 20) == OK
    assert m.seqs[1][0] == [0, 1]
    assert m.add(2) == OK and m.reserve(2, 1) == OK
    assert m.seqs[2][0] == [2]
    assert m.release(1) == OK          # pushes page 1, then page 0
    assert m.reserve(2, 17) == OK      # takes page 0 first
    assert m.seqs[2][0] == [2, 0]
    assert m.reserve(2, 33) == OK
    assert m.seqs[2][0] == [2, 0, 1]
    assert m.available() == 5
    m.check_invariants()


def test_reserve_limits():
    m = PageModel(3, 8)
    m.add(1)
    assert m.reserve(1, 3 * PAGE + 1) == ENOMEM
    assert m.seqs[1] == [[], 0] and m.available() == 3
    assert m.reserve(1, 3 * PAGE) == OK and m.available() == 0
    assert m.reserve(1, 2 * PAGE) == OK and len(m.seqs[1][0]) == 3  # never shrinks
    m2 = PageModel(100, 2)
    m2.add(5)
    assert m2.reserve(5, 2 * PAGE + 1) == EUNSUPPORTED
    assert m2.reserve(7, 1) == EINVAL and m2.add(5) == EINVAL
    m.check_invariants()


def test_fork_shares_full_pages():
    m = PageModel(10, 4)
    m.add(1)
    m.reserve(1, 40)                   # pages 0, 1 full; 2 partly filled
    rc, cs, cd = m.fork(1, 2)
    assert (rc, cs, cd) == (1, 2, 3)
    assert m.seqs[2] == [[0, 1, 3], 40]
    assert m.refs[:4] == [2, 2, 1, 1]
    m.add(3)
    m.reserve(3, 32)                   # pages 4, 5, both full
    assert m.fork(3, 4) == (0, -1, -1)
    assert m.seqs[4] == [[4, 5], 32]
    assert m.fork(9, 10)[0] == EINVAL and m.fork(1, 2)[0] == EINVAL
    m.check_invariants()


def test_prefix_cache_longest_match():
    m = PageModel(20, 8)
    a = np.arange(48)
    m.add(1)
    m.reserve(1, 48)
    assert m.publish(1, a) == 3
    assert m.publish(1, a) == 0        # already registered
    m.add(2)
    b = a.copy()
    b[40] = 999                        # third page differs
    assert m.match(2, b) == 32
    assert m.seqs[2][0] == m.seqs[1][0][:2]
    m.add(3)
    c = a.copy()
    c[0] = -1                          # first page differs: nothing
    assert m.match(3, c) == 0
    m.add(4)
    assert m.match(4, a[:47]) == 32    # only whole pages
    m.add(5)
    assert m.match(5, a) == 48
    assert m.refs[m.seqs[1][0][0]] == 4
    assert m.match(5, a) == EINVAL     # not empty any more
    m.check_invariants()


def test_eviction_order_and_orphaned_keys():
    m = PageModel(4, 4)
    toks = np.arange(64)
    m.add(1)
    m.reserve(1, 48)                   # pages 0, 1, 2
    m.publish(1, toks[:48])
    m.release(1)                       # cached, released 2, 1, 0: page 2 is evicted first
    assert m.lru == [2, 1, 0]
    m.add(2)
    m.reserve(2, 32)                   # free page 3, then evicts page 2
    assert m.seqs[2][0] == [3, 2]
    m.add(3)
    assert m.match(3, toks) == 32      # pages 0 and 1 still match
    m.release(3)
    m.release(2)
    assert m.lru == [1, 0]
    m.add(4)
    m.reserve(4, 64)                   # free pages 3, 2 (sequence 2 gave back 2, then 3),
    assert m.seqs[4][0] == [3, 2, 1, 0]  # then the cached 1 and 0 are evicted
    m.release(4)
    m.add(5)
    assert m.match(5, toks) == 0
    # a chain that lost its last page still matches up to it
    m2 = PageModel(3, 4)
    m2.add(1)
    m2.reserve(1, 32)
    m2.publish(1, toks[:32])
    m2.release(1)                      # lru [1, 0]
    m2.add(2)
    m2.reserve(2, 16)                  # free page 2
    m2.add(3)
    m2.reserve(3, 16)                  # evicts page 1 (the chain's end)
    m2.release(2)
    m2.release(3)
    m2.add(4)
    assert m2.match(4, toks) == 16     # page 0 remains
    m.check_invariants()
    m2.check_invariants()


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(7)
    for trial in range(20):
        m = PageModel(int(rng.integers(4, 40)), int(rng.integers(1, 8)))
        prompts = [rng.integers(0, 5, size=int(rng.integers(0, 130))) for _ in range(6)]
        for step in range(300):
            op = rng.integers(0, 6)
            s = int(rng.integers(0, 8))
            if op == 0:
                m.add(s)
            elif op == 1:
                m.reserve(s, int(rng.integers(0, 140)))
            elif op == 2:
                m.release(s)
            elif op == 3:
                m.fork(s, int(rng.integers(0, 8)))
            elif op == 4 and s in m.seqs:
                p = prompts[int(rng.integers(0, 6))]
                m.publish(s, p[:m.seqs[s][1]])
            elif op == 5:
                m.match(s, prompts[int(rng.integers(0, 6))])
            m.check_invariants()
