"""Naive radix tree and token-slot pool (oracle).

Sources (SGLang paper summary, section 3 "RadixAttention" / "Cache
management"; SGLang explainer, section 04, the tree walkthrough figure, the
lifetime figure, and the two source excerpts on prefix match and eviction):

* a node holds a run of tokens (its key) and the KV slot index of each of
  those tokens (its value); children are found by their first token; the
  path from the root spells a cached prefix;
* match walks edge by edge; a fully matched edge contributes its slots and
  the walk descends; a partially matched edge is split so that the matched
  part becomes its own node, and the walk stops there;  every visited child
  gets the walk's access time;
* insert splits a diverging edge so the shared part becomes an ancestor and
  the new suffix a sibling leaf;
* nodes on the path of a running request carry a reference count and are
  never evicted;
* eviction repeatedly frees the least-recently-used unlocked leaf, returns
  its slots to the pool, deletes it, and lets a parent that has become an
  unlocked leaf compete too.

Readings where the pages are silent (kept identical in the library):
slot 0 is reserved and slots 1..N start in a FIFO free list; allocation
takes from the head and frees append at the tail in the given order; an
allocation short of free slots first evicts the deficit; the LRU clock is a
logical counter advanced once per match or insert call; ties break on the
node creation id; a split's upper node gets a fresh id, the walk's stamp
and a copy of the child's lock count; evicted leaves are not re-merged.

Everything here is written for obviousness, not speed: children are a list
scanned linearly, sizes are recomputed by full traversal, and the eviction
candidate is found by scanning every node.
"""

from collections import deque


class OracleOOM(Exception):
    pass


class OracleInvalid(Exception):
    pass


class NaivePool:
    """FIFO free list of KV slots 1..num_slots (slot 0 reserved)."""

    def __init__(self, num_slots):
        self.num_slots = num_slots
        self.free = deque(range(1, num_slots + 1))

    def available(self):
        return len(self.free)

    def alloc(self, n):
        if n < 0:
            raise OracleInvalid("negative allocation")
        if n > len(self.free):
            raise OracleOOM(f"need {n}, have {len(self.free)}")
        return [self.free.popleft() for _ in range(n)]

    def release(self, slots):
        for s in slots:
            self.free.append(int(s))


class _Node:
    def __init__(self, node_id, key, value, parent, stamp):
        self.id = node_id
        self.key = list(key)
        self.value = list(value)
        self.children = []  # plain list, scanned linearly
        self.parent = parent
        self.lock_ref = 0
        self.last_access = stamp


class NaiveRadixTree:
    def __init__(self, pool):
        self.pool = pool
        self.clock = 0
        self.next_id = 1
        self.root = _Node(0, [], [], None, 0)

    # -- helpers ---------------------------------------------------------
    def _new_node(self, key, value, parent, stamp):
        n = _Node(self.next_id, key, value, parent, stamp)
        self.next_id += 1
        return n

    def _all_nodes(self):
        out, stack = [], [self.root]
        while stack:
            n = stack.pop()
            out.append(n)
            stack.extend(n.children)
        return out

    def _find(self, node_id):
        for n in self._all_nodes():
            if n.id == node_id:
                return n
        raise OracleInvalid(f"no node {node_id}")

    @staticmethod
    def _child_starting_with(node, token):
        for c in node.children:
            if c.key[0] == token:
                return c
        return None

    @staticmethod
    def _common_len(a, b):
        k = 0
        while k < len(a) and k < len(b) and a[k] == b[k]:
            k += 1
        return k

    def _split(self, child, k, stamp):
        """Cut child's edge after k tokens; the upper part becomes a new node."""
        parent = child.parent
        upper = self._new_node(child.key[:k], child.value[:k], parent, stamp)
        upper.lock_ref = child.lock_ref
        upper.last_access = child.last_access
        parent.children[parent.children.index(child)] = upper
        upper.children = [child]
        child.parent = upper
        child.key = child.key[k:]
        child.value = child.value[k:]
        return upper

    # -- API -------------------------------------------------------------
    def match_prefix(self, tokens):
        """Returns (slots of the longest cached prefix, id of its last node)."""
        self.clock += 1
        stamp = self.clock
        node, key, slots = self.root, list(tokens), []
        while key:
            child = self._child_starting_with(node, key[0])
            if child is None:
                break
            child.last_access = stamp
            k = self._common_len(child.key, key)
            if k < len(child.key):
                upper = self._split(child, k, stamp)
                slots += upper.value
                node = upper
                break
            slots += child.value
            node = child
            key = key[k:]
        return slots, node.id

    def insert(self, tokens, slots):
        """Insert tokens with their slots; returns the length already present.
        Where the tree already holds a token, the tree's slot is kept."""
        if len(tokens) != len(slots):
            raise OracleInvalid("tokens/slots length mismatch")
        self.clock += 1
        stamp = self.clock
        node, key, val, present = self.root, list(tokens), list(slots), 0
        while key:
            child = self._child_starting_with(node, key[0])
            if child is None:
                break
            child.last_access = stamp
            k = self._common_len(child.key, key)
            if k < len(child.key):
                child = self._split(child, k, stamp)
            present += k
            node = child
            key, val = key[k:], val[k:]
        if key:
            leaf = self._new_node(key, val, node, stamp)
            node.children.append(leaf)
        return present

    def lock(self, node_id):
        n = self._find(node_id)
        while n is not self.root:
            n.lock_ref += 1
            n = n.parent

    def unlock(self, node_id):
        n = self._find(node_id)
        path = []
        while n is not self.root:
            path.append(n)
            n = n.parent
        if any(p.lock_ref == 0 for p in path):
            raise OracleInvalid("unlock below zero")
        for p in path:
            p.lock_ref -= 1

    def evictable_size(self):
        return sum(len(n.key) for n in self._all_nodes() if n is not self.root and n.lock_ref == 0)

    def protected_size(self):
        return sum(len(n.key) for n in self._all_nodes() if n is not self.root and n.lock_ref > 0)

    def total_size(self):
        return sum(len(n.key) for n in self._all_nodes())

    def evict(self, num_tokens):
        """Free whole unlocked leaves, least recently used first, until at
        least num_tokens tokens are freed or none is left.  Returns
        (tokens freed, slots freed in order)."""
        evicted, freed = 0, []
        while evicted < num_tokens:
            best = None
            for n in self._all_nodes():
                if n is self.root or n.children or n.lock_ref != 0:
                    continue
                if best is None or (n.last_access, n.id) < (best.last_access, best.id):
                    best = n
            if best is None:
                break
            self.pool.release(best.value)
            freed += best.value
            evicted += len(best.value)
            best.parent.children.remove(best)
        return evicted, freed

    def alloc_with_evict(self, n):
        """Allocate n slots, evicting the deficit first if the pool is short.
        Raises OracleOOM (allocating nothing) if still short."""
        short = n - self.pool.available()
        freed = []
        if short > 0:
            _, freed = self.evict(short)
        return self.pool.alloc(n), freed

    def dump(self):
        """Canonical text: pre-order, children by first token ascending; one
        line per node: id parent lock_ref last_access k=<tokens> v=<slots>."""
        lines = []

        def visit(n, parent_id):
            lines.append("%d %d %d %d k=%s v=%s\n" % (
                n.id, parent_id, n.lock_ref, n.last_access,
                ",".join(str(t) for t in n.key), ",".join(str(s) for s in n.value)))
            for c in sorted(n.children, key=lambda c: c.key[0]):
                visit(c, n.id)

        visit(self.root, -1)
        return "".join(lines)
