"""The oracle's paged pool and tree (page size p > 1) against what the page
reading fixes, worked out by hand, and against invariants that hold for any
workload.  At p = 1 the paged code is the token-granular code: every other
oracle test runs it that way."""

import numpy as np
import pytest

from oracle.radix_tree import NaivePool, NaiveRadixTree, OracleInvalid
from oracle.runner import run_workload
from synth import workloads


def test_pool_pages_fifo_and_first_appearance_free():
    pool = NaivePool(32, page_size=4)               # pages 0..7: slots 4j+1 .. 4j+4
    assert pool.available() == 32
    assert pool.alloc(8) == [1, 2, 3, 4, 5, 6, 7, 8]
    with pytest.raises(OracleInvalid):
        pool.alloc(3)                               # not a whole page
    pool.release([7, 6, 2])                         # pages 1, 0 in order of first appearance
    assert list(pool.free_pages) == [2, 3, 4, 5, 6, 7, 1, 0]
    assert pool.free[:4] == [9, 10, 11, 12] and pool.free[-8:] == [5, 6, 7, 8, 1, 2, 3, 4]


def test_paged_walkthrough_by_hand():
    """p = 4, 32 slots.  A (10 prompt tokens, 3 generated), then B sharing
    A's first 6 tokens: matches, splits and slots on page boundaries."""
    pool = NaivePool(32, page_size=4)
    tree = NaiveRadixTree(pool)
    A = list(range(1, 11))
    # A: nothing cached; positions 0..9 start pages at 0, 4, 8
    slots, node_a = tree.match_prefix(A)
    assert slots == [] and node_a == 0
    loc, _ = tree.alloc_positions([([], 0, 10)])
    assert loc == [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]   # page 2's slots 11, 12 stay with A
    # decode positions 10, 11 continue page 2; 12 starts page 3
    a_slots = list(loc)
    for pos, want in ((10, 11), (11, 12), (12, 13)):
        s, _ = tree.alloc_positions([(a_slots, pos, 1)])
        assert s == [want]
        a_slots += s
    assert list(pool.free_pages) == [4, 5, 6, 7]
    # finish A: 13 positions, the aligned 12 are inserted; page 3 (slot 13) is freed
    gen = [50, 51, 52]
    full = A + gen
    assert tree.insert(full[:12], a_slots[:12]) == 0
    pool.release(a_slots[12:13])
    assert list(pool.free_pages) == [4, 5, 6, 7, 3]
    # B = A[0:6] + six new tokens: only the first page matches; the edge is
    # split after 4 tokens, not 6
    Bt = A[:6] + [100, 101, 102, 103, 104, 105]
    slots, node_b = tree.match_prefix(Bt)
    assert slots == [1, 2, 3, 4]
    loc, _ = tree.alloc_positions([(slots, 4, 8)])
    assert loc == [17, 18, 19, 20, 21, 22, 23, 24]  # pages 4 and 5
    assert tree.insert(Bt, slots + loc) == 4
    dump = tree.dump().splitlines()
    assert len(dump) == 4                            # root, [A0..A3], [A4..A11 gen..], [B4..B11]
    assert dump[1].endswith("k=1,2,3,4 v=1,2,3,4")
    # children of the split node in first-page order: A's page (5,6,7,8) < B's (5,6,100,101)
    assert dump[2].endswith("k=5,6,7,8,9,10,50,51 v=5,6,7,8,9,10,11,12")
    assert dump[3].endswith("k=5,6,100,101,102,103,104,105 v=17,18,19,20,21,22,23,24")
    # a partial trailing page never matches: 11 tokens of B match 8, not 11
    slots, _ = tree.match_prefix(Bt[:11])
    assert slots == [1, 2, 3, 4, 17, 18, 19, 20]
    # eviction frees whole leaves, whole pages, least recently used first:
    # A's leaf (stamped by B's first match) before B's leaf
    freed_n, freed = tree.evict(1)
    assert freed == [5, 6, 7, 8, 9, 10, 11, 12] and freed_n == 8
    assert list(pool.free_pages)[-2:] == [1, 2]


def test_insert_of_partial_page_is_rejected():
    tree = NaiveRadixTree(NaivePool(16, page_size=4))
    with pytest.raises(OracleInvalid):
        tree.insert([1, 2, 3], [1, 2, 3])


def _check_paged_invariants(tr, wl):
    p = wl.page_size
    free = tr.free_list
    assert len(free) % p == 0
    pages = [free[i:i + p] for i in range(0, len(free), p)]
    assert all(pg == list(range(pg[0], pg[0] + p)) and (pg[0] - 1) % p == 0 for pg in pages)
    # every node of the final tree holds whole pages of consecutive slots
    for line in tr.final_dump.splitlines()[1:]:
        v = [int(x) for x in line.split(" v=")[1].split(",")]
        assert len(v) % p == 0
        for i in range(0, len(v), p):
            assert (v[i] - 1) % p == 0 and v[i:i + p] == list(range(v[i], v[i] + p))
    # conservation at the end (nothing running): free + cached = pool
    cached = sum(len(line.split(" v=")[1].split(",")) for line in tr.final_dump.splitlines()[1:])
    assert len(free) + cached == wl.num_slots
    # every request's slots follow the page rule
    for slots in tr.request_slots.values():
        for x in range(1, len(slots)):
            if x % p:
                assert slots[x] == slots[x - 1] + 1
            else:
                assert (slots[x] - 1) % p == 0


@pytest.mark.parametrize("page_size", [2, 4, 16])
def test_paged_chat_invariants(page_size):
    wl = workloads.paged(workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6),
                         page_size)
    tr = run_workload(wl, attention=False, max_running=4, max_extend_tokens=128)
    _check_paged_invariants(tr, wl)
    assert any(it["extend_freed"] or it["decode_freed"] for it in tr.iterations)
    # cached lengths are whole pages
    for it in tr.iterations:
        for _, p_len, _ in it["admitted"]:
            assert p_len % page_size == 0


def test_paged_few_shot_hit_rate():
    """64-token shared prefix, 8 requests of 64 + 24 tokens, pages of 16: the
    prefix's 4 pages are reused; the suffixes' partial pages are not."""
    wl = workloads.paged(workloads.few_shot(batch=8, prefix_len=64, suffix_len=24, decode_steps=3,
                                            num_slots=4096), 16)
    tr = run_workload(wl, attention=False)
    # the warm-up request caches the prefix; each batch request matches its 4 pages
    admitted = [a for it in tr.iterations for a in it["admitted"]]
    assert [a[1] for a in admitted] == [0] + [64] * 8
    _check_paged_invariants(tr, wl)


def test_page_size_one_is_the_token_granular_tree():
    wl = workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6)
    a = run_workload(wl, attention=False, max_running=4, max_extend_tokens=128)
    b = run_workload(workloads.paged(wl, 1), attention=False, max_running=4, max_extend_tokens=128)
    assert a.final_dump == b.final_dump and a.free_list == b.free_list and a.iterations == b.iterations
