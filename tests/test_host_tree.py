"""The C++ radix tree and pool (through the C ABI) against the naive oracle:
identical dumps, slot lists, freed-slot order, sizes and free lists on the
page's walkthrough and on random operation sequences.  CPU only."""

import json
import os
import random
import re

import numpy as np
import pytest

from oracle.radix_tree import NaivePool, NaiveRadixTree, OracleInvalid, OracleOOM
from prefix_shared_kv_rt_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "radixrt.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    names = set(re.findall(r"\b(?:int|void|int32_t|int64_t|const char\*)\s+\**\s*([a-z_][a-z0-9_]*)\s*\(", header))
    assert {"rt_match_prefix", "kv_store", "radix_extend_attention", "radix_decode_attention"} <= names
    lib = B.lib()
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(B.EXPORTS) == names


class Pair:
    """The library tree and the oracle tree driven in lockstep."""

    def __init__(self, num_slots, page_size=1):
        self.num_slots = num_slots
        self.page = page_size
        self.cpool = B.rt_pool_create(num_slots, page_size)
        self.ctree = B.rt_tree_create(self.cpool)
        self.opool = NaivePool(num_slots, page_size)
        self.otree = NaiveRadixTree(self.opool)

    def close(self):
        B.rt_tree_destroy(self.ctree)
        B.rt_pool_destroy(self.cpool)

    def same(self):
        assert B.rt_tree_dump(self.ctree) == self.otree.dump()
        assert B.rt_evictable_size(self.ctree) == self.otree.evictable_size()
        assert B.rt_protected_size(self.ctree) == self.otree.protected_size()
        assert list(B.rt_pool_free_list(self.cpool)) == list(self.opool.free)

    def match(self, toks):
        cs, cn = B.rt_match_prefix(self.ctree, toks)
        os_, on = self.otree.match_prefix(toks)
        assert list(cs) == os_ and cn == on
        return os_, on

    def insert(self, toks, slots):
        a = B.rt_insert(self.ctree, toks, slots)
        b = self.otree.insert(toks, slots)
        assert a == b
        return a

    def lock(self, node):
        B.rt_lock(self.ctree, node)
        self.otree.lock(node)

    def unlock(self, node):
        err_c = err_o = None
        try:
            B.rt_unlock(self.ctree, node)
        except B.RadixRTError as e:
            err_c = e
        try:
            self.otree.unlock(node)
        except OracleInvalid as e:
            err_o = e
        assert (err_c is None) == (err_o is None)
        return err_c is None

    def alloc(self, n):
        err_c = err_o = None
        try:
            cs, _ = B.rt_alloc_with_evict(self.ctree, n)
        except B.OOMError as e:
            err_c, cs = e, None
        try:
            os_, _ = self.otree.alloc_with_evict(n)
        except OracleOOM as e:
            err_o, os_ = e, None
        assert (err_c is None) == (err_o is None)
        if cs is not None:
            assert list(cs) == os_
        return os_

    def evict(self, n):
        ce, cf = B.rt_evict_lru_leaves(self.ctree, n)
        oe, of = self.otree.evict(n)
        assert ce == oe and list(cf) == of
        return of

    def free(self, slots):
        B.rt_pool_free(self.cpool, slots)
        self.opool.release(slots)


def test_walkthrough_fixture_on_library():
    fx = json.load(open(os.path.join(ROOT, "tests", "golden", "walkthrough_t1.json")))
    segs = fx["segments"]
    pr = Pair(fx["pool_slots"])
    running = {}
    for step in fx["steps"]:
        if "request" in step:
            toks = segs["S"] + segs[step["request"]]
            slots, node = pr.match(toks)
            assert len(slots) == step["match_len"]
            pr.lock(node)
            new = pr.alloc(len(toks) - len(slots))
            assert new == list(range(step["alloc"][0], step["alloc"][1] + 1))
            pr.insert(toks, slots + new)
            _, leaf = pr.match(toks)
            pr.lock(leaf)
            pr.unlock(node)
            running[step["request"]] = leaf
            if step["request"] == "A":
                pr.unlock(running.pop("A"))
        else:
            freed = pr.evict(step["evict_tokens"])
            if step["freed"]:
                assert freed == list(range(step["freed"][0], step["freed"][1] + 1))
        pr.same()
    pr.close()


def _prompt(rng):
    p = []
    for d in range(rng.randint(1, 4)):
        c = rng.randrange(3)
        p += [(d * 31 + c * 7 + j) % 40 for j in range(rng.randint(1, 7))]
    return p


@pytest.mark.parametrize("seed", range(25))
def test_random_operations_match_oracle(seed):
    rng = random.Random(seed)
    pr = Pair(rng.choice([40, 80, 200]))
    running = []
    for _ in range(200):
        op = rng.random()
        if op < 0.45:
            p = _prompt(rng)
            slots, node = pr.match(p)
            pr.lock(node)
            new = pr.alloc(len(p) - len(slots))
            if new is None:
                pr.unlock(node)
            else:
                running.append((p, node, slots + new, len(slots)))
        elif op < 0.8 and running:
            p, node, slots, plen = running.pop(rng.randrange(len(running)))
            present = pr.insert(p, slots)
            if present > plen:
                pr.free(slots[plen:present])
            pr.unlock(node)
        elif op < 0.9:
            pr.evict(rng.randint(0, 25))
        elif op < 0.95 and running:
            # lock / unlock pairs on a running request's node, and an underflow attempt
            p, node, slots, plen = running[rng.randrange(len(running))]
            pr.lock(node)
            assert pr.unlock(node)
        else:
            # unlock of a path that may hold no lock: an error on both sides
            # unless a running request holds it; then restore that lock
            _, node = pr.match(_prompt(rng))
            if pr.unlock(node) and node != 0:
                pr.lock(node)
        pr.same()
    pr.close()


def test_errors_match_and_leave_state_unchanged():
    pr = Pair(8)
    toks = [1, 2, 3]
    s = pr.alloc(3)
    pr.insert(toks, s)
    _, node = pr.match(toks)
    assert not pr.unlock(node)
    pr.lock(node)
    assert pr.alloc(6) is None     # 5 free, nothing evictable while locked
    pr.same()
    with pytest.raises(B.RadixRTError):
        B.rt_pool_free(pr.cpool, [0])    # slot 0 is reserved
    with pytest.raises(B.RadixRTError):
        B.rt_pool_free(pr.cpool, [9])    # out of range
    with pytest.raises(B.RadixRTError):
        B.rt_lock(pr.ctree, 12345)        # unknown handle
    pr.same()
    pr.close()


def test_allocation_beyond_free_plus_evictable_evicts_nothing_on_library():
    """The library and the oracle agree: free + evictable < n fails before
    any eviction; a fitting allocation evicts the deficit."""
    pr = Pair(10)
    for toks in ([1, 2, 3], [4, 5, 6]):
        s = pr.alloc(3)
        pr.insert(toks, s)
    _, node = pr.match([4, 5, 6])
    pr.lock(node)
    assert pr.alloc(8) is None
    pr.same()
    assert B.rt_evictable_size(pr.ctree) == 3 and B.rt_pool_available(pr.cpool) == 4
    assert pr.alloc(7) is not None
    pr.same()
    pr.close()


def test_batch_helpers_refuse_rows_outside_the_table():
    """Every batch helper checks its rows against the table's row count
    before it writes the table or allocates: the call fails and the tree,
    the pool and the table are as they were."""
    pr = Pair(64)
    r2t = np.zeros((4, 16), dtype=np.int32)
    toks = np.array([1, 2, 3, 4, 5], dtype=np.int32)
    off = np.array([0, 5], dtype=np.int64)
    pl, el, nodes, loc = B.rt_admit_batch(pr.ctree, toks, off, r2t, np.array([1], dtype=np.int32))
    before = r2t.copy()
    free_before = B.rt_pool_available(pr.cpool)
    for bad in (4, 5, -1, 1 << 20):
        rows = np.array([bad], dtype=np.int32)
        with pytest.raises(B.RadixRTError):
            B.rt_admit_batch(pr.ctree, toks, off, r2t, rows)
        with pytest.raises(B.RadixRTError):
            B.rt_decode_slots_batch(pr.ctree, rows, np.array([5], dtype=np.int32), r2t)
        with pytest.raises(B.RadixRTError):
            B.rt_alloc_positions(pr.ctree, rows, np.array([5], dtype=np.int32), np.array([2], dtype=np.int32), r2t)
        with pytest.raises(B.RadixRTError):
            B.rt_finish_batch(pr.ctree, toks, off, r2t, rows, pl, nodes)
    # a bad row after good ones: nothing is written for the good ones either
    with pytest.raises(B.RadixRTError):
        B.rt_decode_slots_batch(pr.ctree, np.array([0, 4], dtype=np.int32), np.array([0, 0], dtype=np.int32), r2t)
    assert np.array_equal(r2t, before)
    assert B.rt_pool_available(pr.cpool) == free_before
    # the host table must be one writable int32 block
    with pytest.raises(ValueError):
        B.rt_decode_slots_batch(pr.ctree, np.array([0], dtype=np.int32), np.array([5], dtype=np.int32),
                                r2t.astype(np.int64))
    with pytest.raises(ValueError):
        B.rt_decode_slots_batch(pr.ctree, np.array([0], dtype=np.int32), np.array([5], dtype=np.int32), r2t[:, ::2])
    B.rt_finish_batch(pr.ctree, toks, off, r2t, np.array([1], dtype=np.int32), pl, nodes)
    pr.close()


@pytest.mark.parametrize("seed", range(6))
def test_batch_helpers_equal_the_primitive_sequence(seed):
    rng = random.Random(seed)
    num_slots = 300
    pr = Pair(num_slots)
    stride = 64
    r2t = np.zeros((8, stride), dtype=np.int32)
    for _round in range(12):
        reqs = [_prompt(rng) + [rng.randrange(40) for _ in range(rng.randint(0, 5))] for _ in range(rng.randint(1, 5))]
        toks = np.concatenate([np.array(r, dtype=np.int32) for r in reqs])
        off = np.cumsum([0] + [len(r) for r in reqs]).astype(np.int64)
        rows = np.arange(len(reqs), dtype=np.int32)
        # library: one call
        try:
            pl, el, nodes, loc = B.rt_admit_batch(pr.ctree, toks, off, r2t, rows)
            c_ok = True
        except B.OOMError:
            c_ok = False
        # oracle: the documented composition
        onodes, oslots = [], []
        for r in reqs:
            s, n = pr.otree.match_prefix(r)
            pr.otree.lock(n)
            onodes.append(n)
            oslots.append(s)
        need = sum(len(r) - len(s) for r, s in zip(reqs, oslots))
        try:
            oloc, _ = pr.otree.alloc_with_evict(need)
            o_ok = True
        except OracleOOM:
            o_ok = False
            for n in reversed(onodes):
                pr.otree.unlock(n)
        assert c_ok == o_ok
        pr.same()
        if not c_ok:
            continue
        assert list(nodes) == onodes and list(loc) == oloc
        assert list(pl) == [len(s) for s in oslots]
        off_new = 0
        for i, r in enumerate(reqs):
            e = len(r) - len(oslots[i])
            assert list(r2t[i, :len(r)]) == oslots[i] + oloc[off_new:off_new + e]
            off_new += e
        # one decode slot per request
        pos = np.array([len(r) for r in reqs], dtype=np.int32)
        if (pos < stride).all():
            dl = B.rt_decode_slots_batch(pr.ctree, rows, pos, r2t)
            odl, _ = pr.otree.alloc_with_evict(len(reqs))
            assert list(dl) == odl
            full = [r + [rng.randrange(40)] for r in reqs]
            for i in range(len(reqs)):
                assert r2t[i, pos[i]] == odl[i]
        else:
            full = reqs
        pr.same()
        # finish
        ftoks = np.concatenate([np.array(r, dtype=np.int32) for r in full])
        foff = np.cumsum([0] + [len(r) for r in full]).astype(np.int64)
        B.rt_finish_batch(pr.ctree, ftoks, foff, r2t, rows, pl, nodes)
        for i, r in enumerate(full):
            row = [int(x) for x in r2t[i, :len(r)]]
            present = pr.otree.insert(r, row)
            if present > pl[i]:
                pr.opool.release(row[pl[i]:present])
            pr.otree.unlock(onodes[i])
        pr.same()
    pr.close()


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("page", [2, 4])
def test_random_paged_operations_match_oracle(seed, page):
    """Pages: page-aligned matches and inserts, slots by the page rule
    (fresh pages at page starts, the next slot otherwise), finishes that free
    the tree's duplicates and the trailing partial page, evictions of whole
    pages; library and oracle in lockstep."""
    rng = random.Random(1000 * page + seed)
    pr = Pair(page * rng.choice([20, 40, 100]), page)
    assert B.rt_pool_page_size(pr.cpool) == page
    stride = 64
    r2t = np.zeros((1, stride), dtype=np.int32)
    running = []
    for _ in range(200):
        op = rng.random()
        if op < 0.45:
            p = _prompt(rng) + [rng.randrange(40) for _ in range(rng.randint(0, 6))]
            slots, node = pr.match(p)
            assert len(slots) % page == 0
            pr.lock(node)
            # positions len(slots) .. len(p)-1 by the page rule, both sides
            r2t[0, :len(slots)] = slots
            err_c = err_o = None
            try:
                cs, _ = B.rt_alloc_positions(pr.ctree, [0], [len(slots)], [len(p) - len(slots)], r2t)
            except B.OOMError as e:
                err_c, cs = e, None
            try:
                os_, _ = pr.otree.alloc_positions([(slots, len(slots), len(p) - len(slots))])
            except OracleOOM as e:
                err_o, os_ = e, None
            assert (err_c is None) == (err_o is None)
            if os_ is None:
                pr.unlock(node)
            else:
                assert list(cs) == os_ and list(r2t[0, :len(p)]) == slots + os_
                running.append((p, node, slots + os_, len(slots)))
        elif op < 0.8 and running:
            p, node, slots, plen = running.pop(rng.randrange(len(running)))
            aligned = len(p) - len(p) % page
            present = pr.insert(p[:aligned], slots[:aligned])
            rel = (slots[plen:present] if present > plen else []) + slots[aligned:]
            if rel:
                pr.free(rel)
            pr.unlock(node)
        elif op < 0.9:
            pr.evict(rng.randint(0, 25))
        else:
            _, node = pr.match(_prompt(rng))
            if pr.unlock(node) and node != 0:
                pr.lock(node)
        pr.same()
    with pytest.raises(B.RadixRTError):
        B.rt_insert(pr.ctree, [1] * (page + 1), [1] * (page + 1))   # not whole pages
    with pytest.raises(B.RadixRTError):
        B.rt_alloc_with_evict(pr.ctree, page + 1)
    pr.close()
