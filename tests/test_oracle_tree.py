"""Pins for the naive radix tree and pool (oracle side, CPU only)."""

import json
import os
import random

import pytest

from oracle.radix_tree import NaivePool, NaiveRadixTree, OracleInvalid, OracleOOM
from oracle.hit_rate import distinct_prefix_tokens, hit_rate, optimal_hit_rate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_dump(text):
    nodes = {}
    for line in text.splitlines():
        head, k, v = line.split(" k=")[0], line.split(" k=")[1].split(" v=")[0], line.split(" v=")[1]
        nid, parent, lock, last = (int(x) for x in head.split())
        key = [int(t) for t in k.split(",")] if k else []
        val = [int(s) for s in v.split(",")] if v else []
        nodes[nid] = dict(parent=parent, lock=lock, last=last, key=key, value=val)
    return nodes


def _shape(tree, segs):
    """Tree as {label: (parent label, [first slot, last slot])} with labels
    resolved from the fixture's token segments."""
    nodes = _parse_dump(tree.dump())
    by_tokens = {}
    for name, toks in segs.items():
        by_tokens[tuple(toks)] = name
    for a in segs:
        for b in segs:
            by_tokens.setdefault(tuple(segs[a] + segs[b]), a + "+" + b)
    label = {0: None}
    out = {}
    for nid in sorted(nodes):
        if nid == 0:
            continue
        n = nodes[nid]
        label[nid] = by_tokens[tuple(n["key"])]
    for nid, n in nodes.items():
        if nid == 0:
            continue
        out[label[nid]] = (label[n["parent"]], [n["value"][0], n["value"][-1]],
                           n["value"] == list(range(n["value"][0], n["value"][-1] + 1)))
    return out


def test_walkthrough_matches_page_figure():
    fx = json.load(open(os.path.join(GOLDEN, "walkthrough_t1.json")))
    segs = fx["segments"]
    pool = NaivePool(fx["pool_slots"])
    tree = NaiveRadixTree(pool)
    cached = prefill = 0
    running = {}
    for step in fx["steps"]:
        if "request" in step:
            name = step["request"]
            toks = segs["S"] + segs[name]
            slots, node = tree.match_prefix(toks)
            assert len(slots) == step["match_len"]
            if "match_slots" in step:
                lo, hi = step["match_slots"]
                assert slots == list(range(lo, hi + 1))
            tree.lock(node)
            new, _ = tree.alloc_with_evict(len(toks) - len(slots))
            lo, hi = step["alloc"]
            assert new == list(range(lo, hi + 1))
            cached += len(slots)
            prefill += len(toks)
            present = tree.insert(toks, slots + new)
            assert present == len(slots)
            # the request keeps running: protect its full path, drop the admission lock
            _, leaf = tree.match_prefix(toks)
            tree.lock(leaf)
            tree.unlock(node)
            running[name] = leaf
            # A finished before B arrived (page step 1 -> 2)
            if name == "A":
                tree.unlock(running.pop("A"))
        else:
            evicted, freed = tree.evict(step["evict_tokens"])
            if step["freed"] is None:
                assert freed == []
            else:
                lo, hi = step["freed"]
                assert freed == list(range(lo, hi + 1))
            if "protected" in step:
                assert tree.protected_size() == step["protected"]
                assert tree.evictable_size() == step["evictable"]
        shape = _shape(tree, segs)
        want = {lab: (par, rng, True) for lab, par, rng in step["tree"]}
        assert shape == want, (step, shape)
    assert (cached, prefill) == tuple(fx["hit_rate"])
    assert hit_rate(cached, prefill) == hit_rate(*fx["hit_rate"])


def _random_prompts(rng, n, depth=3, fan=3, seg=(1, 6)):
    """Prompts drawn from a random token tree so that they share prefixes."""
    prompts = []
    for _ in range(n):
        p = []
        for d in range(rng.randint(1, depth)):
            choice = rng.randrange(fan)
            p += [d * 10 + choice] * 0 + [(d * 97 + choice * 13 + j) % 50 for j in range(rng.randint(*seg))]
        prompts.append(p)
    return prompts


def _serve_one_at_a_time(prompts, usable_slots):
    pool = NaivePool(usable_slots)
    tree = NaiveRadixTree(pool)
    cached = prefill = 0
    for p in prompts:
        slots, node = tree.match_prefix(p)
        tree.lock(node)
        new, _ = tree.alloc_with_evict(len(p) - len(slots))
        present = tree.insert(p, slots + new)
        pool.release((slots + new)[len(slots):present])
        tree.unlock(node)
        cached += len(slots)
        prefill += len(p)
    return cached, prefill, tree


@pytest.mark.parametrize("seed", range(12))
def test_theorem_3_1_dfs_order_reaches_optimum(seed):
    """Theorem 3.1: with cache >= the longest request, depth-first order
    computes exactly sum_e |e| tokens, i.e. reaches H_opt."""
    rng = random.Random(seed)
    prompts = _random_prompts(rng, 25)
    dfs = sorted(prompts)  # lexicographic order visits the prefix tree depth first
    cached, prefill, _ = _serve_one_at_a_time(dfs, max(len(p) for p in prompts))
    assert prefill - cached == distinct_prefix_tokens(prompts)
    assert hit_rate(cached, prefill) == optimal_hit_rate(prompts)


@pytest.mark.parametrize("seed", range(6))
def test_unbounded_pool_any_order_reaches_optimum(seed):
    rng = random.Random(100 + seed)
    prompts = _random_prompts(rng, 30)
    rng.shuffle(prompts)
    total = sum(len(p) for p in prompts)
    cached, prefill, tree = _serve_one_at_a_time(prompts, total)
    assert hit_rate(cached, prefill) == optimal_hit_rate(prompts)
    # sum over edges of the final radix tree equals the distinct-prefix count
    assert tree.total_size() == distinct_prefix_tokens(prompts)


def test_interleaving_with_small_cache_is_worse_than_dfs():
    """The explainer's A1,B1,A2,B2 example: switching between prefixes with a
    cache that holds one of them recomputes; grouping them does not."""
    a, b = list(range(0, 20)), list(range(100, 120))
    a1, a2, b1, b2 = a + [1], a + [2], b + [1], b + [2]
    c_bad, p_bad, _ = _serve_one_at_a_time([a1, b1, a2, b2], 21)
    c_good, p_good, _ = _serve_one_at_a_time([a1, a2, b1, b2], 21)
    assert c_bad == 0 and c_good == 40
    assert hit_rate(c_good, p_good) == optimal_hit_rate([a1, a2, b1, b2])


@pytest.mark.parametrize("seed", range(8))
def test_match_is_longest_common_prefix_with_what_was_inserted(seed):
    """Brute force: with nothing evicted, the matched length is the longest
    common prefix with any inserted sequence, and the slots are those of the
    first sequence that inserted each token."""
    rng = random.Random(seed)
    pool = NaivePool(10000)
    tree = NaiveRadixTree(pool)
    owner = {}  # prefix tuple -> slot of its last token
    seqs = _random_prompts(rng, 20)
    for s in seqs:
        slots = pool.alloc(len(s))
        tree.insert(s, slots)
        for i in range(len(s)):
            owner.setdefault(tuple(s[:i + 1]), slots[i])
    for q in _random_prompts(rng, 30) + seqs:
        best = max((i for i in range(len(q) + 1) if i == 0 or tuple(q[:i]) in owner))
        got, _ = tree.match_prefix(q)
        assert len(got) == best
        assert got == [owner[tuple(q[:i + 1])] for i in range(best)]


def _check_invariants(tree, pool, private):
    nodes = _parse_dump(tree.dump())
    tree_tokens = sum(len(n["key"]) for n in nodes.values())
    assert pool.available() + tree_tokens + len(private) == pool.num_slots
    assert tree.evictable_size() + tree.protected_size() == tree_tokens
    every = list(pool.free) + [s for n in nodes.values() for s in n["value"]] + list(private)
    assert sorted(every) == list(range(1, pool.num_slots + 1))
    children = {}
    for nid, n in nodes.items():
        if n["parent"] >= 0:
            children.setdefault(n["parent"], []).append(n["key"][0])
            if n["parent"] != 0:
                assert nodes[n["parent"]]["lock"] >= n["lock"]
            assert len(n["key"]) == len(n["value"]) > 0
    for firsts in children.values():
        assert len(firsts) == len(set(firsts))


@pytest.mark.parametrize("seed", range(10))
def test_random_operations_keep_invariants(seed):
    rng = random.Random(seed)
    pool = NaivePool(120)
    tree = NaiveRadixTree(pool)
    running = []  # (prompt, node, slots, prefix_len)
    private = []
    for _ in range(150):
        op = rng.random()
        if op < 0.5:
            p = _random_prompts(rng, 1, depth=4, seg=(2, 8))[0]
            slots, node = tree.match_prefix(p)
            tree.lock(node)
            try:
                new, _ = tree.alloc_with_evict(len(p) - len(slots))
            except OracleOOM:
                tree.unlock(node)
                continue
            running.append((p, node, slots + new, len(slots)))
            private += new
        elif op < 0.85 and running:
            p, node, slots, plen = running.pop(rng.randrange(len(running)))
            present = tree.insert(p, slots)
            dups = slots[plen:present]
            pool.release(dups)
            for s in slots[plen:]:
                private.remove(s)
            tree.unlock(node)
        else:
            evicted, freed = tree.evict(rng.randint(1, 30))
            assert evicted == len(freed)
        _check_invariants(tree, pool, private)


def test_unlock_underflow_and_oom_are_errors():
    pool = NaivePool(8)
    tree = NaiveRadixTree(pool)
    tree.insert([1, 2, 3], pool.alloc(3))
    _, node = tree.match_prefix([1, 2, 3])
    with pytest.raises(OracleInvalid):
        tree.unlock(node)
    tree.lock(node)
    before = pool.available()
    with pytest.raises(OracleOOM):
        tree.alloc_with_evict(6)  # 5 free, nothing evictable while locked
    assert pool.available() == before


def test_allocation_beyond_free_plus_evictable_evicts_nothing():
    """free + evictable < n: OOM before any eviction, so the cache keeps
    every unlocked prefix (and an allocation that fits after evicting still
    evicts only the deficit)."""
    pool = NaivePool(10)
    tree = NaiveRadixTree(pool)
    tree.insert([1, 2, 3], pool.alloc(3))
    tree.insert([4, 5, 6], pool.alloc(3))
    _, node = tree.match_prefix([4, 5, 6])
    tree.lock(node)                      # 4 free, [1, 2, 3] evictable, [4, 5, 6] locked
    assert pool.available() == 4 and tree.evictable_size() == 3
    with pytest.raises(OracleOOM):
        tree.alloc_with_evict(8)         # 4 + 3 < 8
    assert pool.available() == 4 and tree.evictable_size() == 3
    assert tree.match_prefix([1, 2, 3])[0] != []
    slots, freed = tree.alloc_with_evict(7)   # 4 + 3 = 7: evicts [1, 2, 3]
    assert len(slots) == 7 and len(freed) == 3 and tree.evictable_size() == 0


def test_eviction_takes_least_recent_leaf_and_spares_locked_paths():
    pool = NaivePool(100)
    tree = NaiveRadixTree(pool)
    seqs = [[1, 2, 3, 4], [1, 2, 5, 6], [7, 8], [9]]
    for s in seqs:
        tree.insert(s, pool.alloc(len(s)))
    tree.match_prefix([7, 8])          # refresh [7, 8]
    _, locked = tree.match_prefix([9])
    tree.lock(locked)                   # [9] is in use
    order = []
    while True:
        n, freed = tree.evict(1)
        if n == 0:
            break
        order.append(freed)
    # [3,4] and [5,6] (stamped by the second insert / split) go first, then the
    # now-childless [1,2], then [7,8]; [9] is locked and survives.
    remaining = _parse_dump(tree.dump())
    assert [n["key"] for n in remaining.values() if n["key"]] == [[9]]
    assert order == [[3, 4], [7, 8], [1, 2], [9, 10]]  # slots 1-4, 5-8 (5, 6 were duplicates), 9-10, 11
