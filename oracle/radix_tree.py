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

Pages (page_size p > 1; the explainer's source excerpt compares a child's
key with the remaining key under the tree's page size, and the engine makes
the page size configurable).  Readings taken, all reducing to the above at
p = 1:

* the pool hands out whole pages: page j holds slots 1 + j*p .. (j+1)*p,
  the free list is a FIFO of pages (ascending at start), an allocation of n
  slots takes n / p pages, and a free returns the distinct pages of the
  given slots in order of first appearance;
* keys are compared page by page: a child is found by its first page, a
  common length counts whole pages only, so matches and splits fall on page
  boundaries; a trailing partial page of a key never matches; inserts carry
  whole pages only;
* positions get slots by the page rule (``alloc_positions``): a position
  that starts a page takes a fresh page and its first slot, any other
  position takes the slot after the previous position's.

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
    """FIFO free list of pages of KV slots 1..num_slots (slot 0 reserved);
    page j holds slots 1 + j*p .. (j+1)*p."""

    def __init__(self, num_slots, page_size=1):
        if page_size < 1 or num_slots % page_size:
            raise OracleInvalid("num_slots must be a positive multiple of page_size")
        self.num_slots = num_slots
        self.page_size = page_size
        self.free_pages = deque(range(num_slots // page_size))

    def page_slots(self, j):
        return [1 + j * self.page_size + i for i in range(self.page_size)]

    @property
    def free(self):
        """Free slots in free-list order (each free page's slots in order)."""
        return [s for j in self.free_pages for s in self.page_slots(j)]

    def available(self):
        return len(self.free_pages) * self.page_size

    def alloc(self, n):
        if n < 0 or n % self.page_size:
            raise OracleInvalid("allocation must be a non-negative multiple of the page size")
        if n > self.available():
            raise OracleOOM(f"need {n}, have {self.available()}")
        out = []
        for _ in range(n // self.page_size):
            out += self.page_slots(self.free_pages.popleft())
        return out

    def release(self, slots):
        """Frees the distinct pages of the given slots, in order of first
        appearance."""
        seen = set()
        for s in slots:
            j = (int(s) - 1) // self.page_size
            if j not in seen:
                seen.add(j)
                self.free_pages.append(j)


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
        self.page_size = pool.page_size
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

    def _child_starting_with(self, node, page):
        """The child whose key begins with this page (its first p tokens)."""
        for c in node.children:
            if c.key[:self.page_size] == list(page):
                return c
        return None

    def _common_len(self, a, b):
        """Common prefix length of a and b in whole pages."""
        k = 0
        while k < len(a) and k < len(b) and a[k] == b[k]:
            k += 1
        return k - k % self.page_size

    def _aligned(self, tokens):
        return list(tokens)[:len(tokens) - len(tokens) % self.page_size]

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
        node, key, slots = self.root, self._aligned(tokens), []
        while key:
            child = self._child_starting_with(node, key[:self.page_size])
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
        Where the tree already holds a token, the tree's slot is kept.  The
        length must be a whole number of pages."""
        if len(tokens) != len(slots):
            raise OracleInvalid("tokens/slots length mismatch")
        if len(tokens) % self.page_size:
            raise OracleInvalid("insert of a partial page")
        self.clock += 1
        stamp = self.clock
        node, key, val, present = self.root, list(tokens), list(slots), 0
        while key:
            child = self._child_starting_with(node, key[:self.page_size])
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
        """Allocate n slots (whole pages), evicting the deficit first if the
        pool is short.  An allocation that cannot succeed even after every
        unlocked node is evicted (free + evictable < n, the quantity the
        scheduler's admission test uses) raises OracleOOM before anything is
        evicted or allocated."""
        if n > self.pool.available() + self.evictable_size():
            raise OracleOOM(f"need {n}, have {self.pool.available()} free + {self.evictable_size()} evictable")
        short = n - self.pool.available()
        freed = []
        if short > 0:
            _, freed = self.evict(short)
        return self.pool.alloc(n), freed

    def alloc_positions(self, runs):
        """Slots for runs of positions by the page rule.  runs: list of
        (slots of the request's positions 0 .. first-1, first, count), in
        order.  Pages for every position that starts a page are allocated
        together (evicting first if short), taken in run order.  Returns
        (slots of every run's positions, concatenated; slots freed by
        eviction)."""
        p = self.page_size
        starts = sum(1 for _, first, cnt in runs for x in range(first, first + cnt) if x % p == 0)
        fresh, freed = self.alloc_with_evict(starts * p)
        out, nxt = [], 0
        for prev, first, cnt in runs:
            mine = list(prev)
            for x in range(first, first + cnt):
                if x % p == 0:
                    s = fresh[nxt * p]
                    nxt += 1
                else:
                    s = mine[x - 1] + 1
                mine.append(s)
                out.append(s)
        return out, freed

    def dump(self):
        """Canonical text: pre-order, children by first page ascending
        (lexicographic); one line per node: id parent lock_ref last_access
        k=<tokens> v=<slots>."""
        lines = []

        def visit(n, parent_id):
            lines.append("%d %d %d %d k=%s v=%s\n" % (
                n.id, parent_id, n.lock_ref, n.last_access,
                ",".join(str(t) for t in n.key), ",".join(str(s) for s in n.value)))
            for c in sorted(n.children, key=lambda c: c.key[:self.page_size]):
                visit(c, n.id)

        visit(self.root, -1)
        return "".join(lines)
