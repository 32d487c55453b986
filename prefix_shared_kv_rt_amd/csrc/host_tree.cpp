// Host-side radix tree and token-slot pool behind the C ABI.
//
// Behaviour follows the SGLang explainer, section 04 (RadixAttention): the
// walkthrough figure (insert, split on a shared prefix, evict an idle LRU
// leaf while running paths stay protected), and the two source excerpts
// (prefix match that stamps each visited child and splits a partially
// matched edge; eviction from a heap of unlocked leaves that re-pushes a
// parent once it is an unlocked leaf).  Locks and the shared pool follow the
// SGLang paper summary, section 3 ("Cache management").
//
// Pages: the pool may hand out slots in pages of p (the explainer's match
// excerpt compares keys under a configurable page size); keys are then
// compared in whole pages, children are keyed by their first page, and new
// positions take slots by the page rule (a fresh page at a page start, the
// next slot otherwise).  With p = 1 everything is token-granular.
//
// Data layout: nodes own their key and slot runs in std::vector; children are
// keyed by a hash of their first page (checked against the page itself), in
// a short array while a node has few of them and in a hash multimap beyond
// that; nodes are found by id through a vector (ids are
// handed out in order and never reused) and their storage is recycled after
// eviction; the unlocked leaves sit in an array with back-indices so that
// eviction heapifies only the candidates; evictable and protected token
// counts are kept incrementally.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <memory>
#include <queue>
#include <string>
#include <unordered_map>
#include <vector>

#include "radixrt.h"
#include "rt_internal.h"

namespace rt {
// memcpy of n int32 values; n == 0 copies nothing (and lets either pointer
// be null, which memcpy itself does not allow).
inline void copy_i32(int32_t* dst, const int32_t* src, int64_t n) {
  if (n > 0) std::memcpy(dst, src, sizeof(int32_t) * size_t(n));
}
}  // namespace rt

namespace rt {

// ------------------------------------------------------------------ pool --
// Slots 1..capacity in pages of `page` slots: page j holds slots
// 1 + j*page .. (j+1)*page.  The free list is a FIFO ring of pages, each held
// as its first slot (with one-slot pages that is the slot itself).  An
// allocation takes whole pages from the head; a free appends the distinct
// pages of the given slots at the tail, in order of first appearance.
struct Pool {
  int32_t capacity = 0;       // slots
  int32_t page = 1;           // slots per page
  int32_t pages = 0;          // capacity / page
  std::vector<int32_t> ring;  // first slot of each free page, FIFO
  int64_t head = 0;           // index of the first free page in ring
  int32_t count = 0;          // number of free pages
  std::vector<uint32_t> mark; // per page: call number of its last free (page > 1)
  uint32_t epoch = 0;

  Pool(int32_t n, int32_t page_size) : capacity(n), page(page_size), pages(n / page_size), ring(n / page_size) {
    for (int32_t j = 0; j < pages; ++j) ring[j] = 1 + j * page;
    count = pages;
    if (page > 1) mark.assign(size_t(pages), 0u);
  }
  int64_t free_slots() const { return int64_t(count) * page; }
  int alloc(int32_t n, int32_t* out) {
    if (n < 0 || n % page) return fail(RT_ERR_INVALID, "pool: allocation must be a whole number of pages");
    const int32_t k = n / page;
    if (k > count) return fail(RT_ERR_OOM, "pool: need " + std::to_string(n) + ", free " +
                                               std::to_string(free_slots()));
    if (page == 1) {  // runs of slots move with at most two block copies
      const int64_t first = std::min<int64_t>(k, pages - head);
      copy_i32(out, ring.data() + head, first);
      copy_i32(out + first, ring.data(), k - first);
    } else {
      for (int32_t i = 0; i < k; ++i) {
        const int32_t f = ring[(head + i) % pages];
        for (int32_t t = 0; t < page; ++t) out[int64_t(i) * page + t] = f + t;
      }
    }
    head += k;
    if (head >= pages) head -= pages;
    count -= k;
    return RT_OK;
  }
  int release(const int32_t* slots, int64_t n) {
    if (n < 0) return fail(RT_ERR_INVALID, "negative free");
    for (int64_t i = 0; i < n; ++i)
      if (slots[i] < 1 || slots[i] > capacity)
        return fail(RT_ERR_INVALID, "pool: slot " + std::to_string(slots[i]) + " out of range");
    int64_t tail = head + count;
    if (tail >= pages) tail -= pages;
    if (page == 1) {
      if (int64_t(count) + n > pages) return fail(RT_ERR_INVALID, "pool: free list overflow (double free?)");
      const int64_t first = std::min<int64_t>(n, pages - tail);
      copy_i32(ring.data() + tail, slots, first);
      copy_i32(ring.data(), slots + first, n - first);
      count += int32_t(n);
      return RT_OK;
    }
    // distinct pages in order of first appearance
    if (++epoch == 0) {
      std::fill(mark.begin(), mark.end(), 0u);
      epoch = 1;
    }
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i) {
      const int32_t j = (slots[i] - 1) / page;
      if (mark[j] != epoch) {
        mark[j] = epoch;
        ++k;
      }
    }
    if (int64_t(count) + k > pages) return fail(RT_ERR_INVALID, "pool: free list overflow (double free?)");
    ++epoch;  // second pass appends each page at its first appearance
    if (epoch == 0) {
      std::fill(mark.begin(), mark.end(), 0u);
      epoch = 1;
    }
    for (int64_t i = 0; i < n; ++i) {
      const int32_t j = (slots[i] - 1) / page;
      if (mark[j] != epoch) {
        mark[j] = epoch;
        ring[tail] = 1 + j * page;
        if (++tail == pages) tail = 0;
      }
    }
    count += int32_t(k);
    return RT_OK;
  }
};

// ------------------------------------------------------------------ tree --
struct Node;

// Hash of a key's first page (one-token pages hash to the token itself).
inline uint64_t page_hash(const int32_t* t, int32_t p) {
  if (p == 1) return uint32_t(t[0]);
  uint64_t h = 1469598103934665603ull;
  for (int32_t i = 0; i < p; ++i) h = (h ^ uint32_t(t[i])) * 1099511628211ull;
  return h;
}

// Children by their first page: a short array up to kSmall entries, then a
// hash multimap; every lookup confirms the page itself.
class ChildMap {
 public:
  static constexpr size_t kSmall = 8;
  Node* find(uint64_t h, const int32_t* page, int32_t p) const;
  // Puts n (whose key starts with the page hashed to h) in place of the child
  // with the same first page, or adds it.
  void set(uint64_t h, Node* n, int32_t p);
  void erase(uint64_t h, const int32_t* page, int32_t p);
  bool empty() const { return small_.empty() && big_.empty(); }
  void clear() {
    small_.clear();
    big_.clear();
  }
  template <typename F>
  void for_each(F f) const {
    for (const auto& kv : small_) f(kv.second);
    for (const auto& kv : big_) f(kv.second);
  }

 private:
  std::vector<std::pair<uint64_t, Node*>> small_;
  std::unordered_multimap<uint64_t, Node*> big_;
};

struct Node {
  int64_t id = 0;
  std::vector<int32_t> key;
  std::vector<int32_t> value;
  ChildMap children;
  Node* parent = nullptr;
  int32_t lock_ref = 0;
  uint64_t last_access = 0;
  int64_t leaf_pos = -1;  // index in Tree::leaves while an eviction candidate
};

inline bool same_page(const Node* n, const int32_t* page, int32_t p) {
  return p == 1 ? n->key[0] == page[0] : std::memcmp(n->key.data(), page, sizeof(int32_t) * p) == 0;
}

inline Node* ChildMap::find(uint64_t h, const int32_t* page, int32_t p) const {
  if (!big_.empty()) {
    auto range = big_.equal_range(h);
    for (auto it = range.first; it != range.second; ++it)
      if (same_page(it->second, page, p)) return it->second;
    return nullptr;
  }
  for (const auto& kv : small_)
    if (kv.first == h && same_page(kv.second, page, p)) return kv.second;
  return nullptr;
}

inline void ChildMap::set(uint64_t h, Node* n, int32_t p) {
  const int32_t* page = n->key.data();
  if (!big_.empty()) {
    auto range = big_.equal_range(h);
    for (auto it = range.first; it != range.second; ++it)
      if (same_page(it->second, page, p)) {
        it->second = n;
        return;
      }
    big_.emplace(h, n);
    return;
  }
  for (auto& kv : small_)
    if (kv.first == h && same_page(kv.second, page, p)) {
      kv.second = n;
      return;
    }
  if (small_.size() < kSmall) {
    small_.emplace_back(h, n);
    return;
  }
  big_.reserve(2 * kSmall);
  for (const auto& kv : small_) big_.emplace(kv.first, kv.second);
  big_.emplace(h, n);
  small_.clear();
}

inline void ChildMap::erase(uint64_t h, const int32_t* page, int32_t p) {
  if (!big_.empty()) {
    auto range = big_.equal_range(h);
    for (auto it = range.first; it != range.second; ++it)
      if (same_page(it->second, page, p)) {
        big_.erase(it);
        return;
      }
    return;
  }
  for (size_t i = 0; i < small_.size(); ++i)
    if (small_[i].first == h && same_page(small_[i].second, page, p)) {
      small_[i] = small_.back();
      small_.pop_back();
      return;
    }
}

struct Tree {
  Pool* pool;
  int32_t P;                                   // slots per page (the pool's)
  std::vector<int32_t> fresh_;                 // scratch of alloc_positions: the fresh pages' slots
  uint64_t clock = 0;
  int64_t next_id = 1;
  std::unique_ptr<Node> root_owner;
  Node* root;
  std::vector<Node*> by_id;                    // by_id[id - 1]: live node or null
  std::vector<std::unique_ptr<Node>> storage;  // every node object ever made
  std::vector<Node*> spare;                    // evicted node objects, reused
  int64_t live = 0;                            // non-root nodes in the tree
  std::vector<Node*> leaves;                   // unlocked, childless, non-root
  // (last_access, id) of leaves[i], kept beside it so that building the
  // eviction heap reads one contiguous array instead of every leaf node.
  std::vector<std::pair<uint64_t, int64_t>> leaf_keys;
  int64_t evictable = 0;
  int64_t protected_ = 0;

  explicit Tree(Pool* p) : pool(p), P(p->page), root_owner(new Node()) {
    root = root_owner.get();
    root->id = 0;
  }

  bool is_candidate(const Node* n) const {
    return n != root && n->children.empty() && n->lock_ref == 0;
  }
  void leaf_add(Node* n) {
    if (n->leaf_pos >= 0) return;
    n->leaf_pos = int64_t(leaves.size());
    leaves.push_back(n);
    leaf_keys.push_back({n->last_access, n->id});
  }
  void leaf_remove(Node* n) {
    if (n->leaf_pos < 0) return;
    Node* last = leaves.back();
    leaves[n->leaf_pos] = last;
    leaf_keys[n->leaf_pos] = leaf_keys.back();
    last->leaf_pos = n->leaf_pos;
    leaves.pop_back();
    leaf_keys.pop_back();
    n->leaf_pos = -1;
  }
  void stamp(Node* n, uint64_t t) {
    n->last_access = t;
    if (n->leaf_pos >= 0) leaf_keys[n->leaf_pos].first = t;
  }
  void refresh(Node* n) {
    if (n == root) return;
    if (is_candidate(n))
      leaf_add(n);
    else
      leaf_remove(n);
  }

  Node* make_node(Node* parent, const int32_t* key, const int32_t* val, int64_t len, uint64_t stamp) {
    Node* n;
    if (!spare.empty()) {
      n = spare.back();
      spare.pop_back();
    } else {
      storage.push_back(std::make_unique<Node>());
      n = storage.back().get();
    }
    n->id = next_id++;
    n->key.assign(key, key + len);
    n->value.assign(val, val + len);
    n->children.clear();
    n->parent = parent;
    n->lock_ref = 0;
    n->last_access = stamp;
    n->leaf_pos = -1;
    by_id.push_back(n);  // by_id[id - 1]
    ++live;
    return n;
  }
  void drop_node(Node* n) {
    by_id[size_t(n->id - 1)] = nullptr;
    n->parent = nullptr;
    --live;
    spare.push_back(n);
  }

  Node* find(int64_t id) {
    if (id == 0) return root;
    if (id < 0 || id > int64_t(by_id.size())) return nullptr;
    return by_id[size_t(id - 1)];
  }

  // Cut child's edge after k tokens (0 < k < len); the upper part becomes a
  // new node with a fresh id, the child's stamp and lock count.
  Node* split(Node* child, int64_t k) {
    Node* parent = child->parent;
    Node* upper = make_node(parent, child->key.data(), child->value.data(), k, child->last_access);
    upper->lock_ref = child->lock_ref;
    parent->children.set(page_hash(upper->key.data(), P), upper, P);
    child->key.erase(child->key.begin(), child->key.begin() + k);
    child->value.erase(child->value.begin(), child->value.begin() + k);
    child->parent = upper;
    upper->children.set(page_hash(child->key.data(), P), child, P);
    // token counts are unchanged (same lock count on both parts)
    refresh(upper);
    return upper;
  }

  // Length of the common prefix of an edge key and a token run; long runs
  // are compared 64 tokens at a time with memcmp.
  static int64_t common_len(const std::vector<int32_t>& a, const int32_t* b, int64_t nb) {
    const int64_t m = std::min<int64_t>(int64_t(a.size()), nb);
    const int32_t* pa = a.data();
    int64_t k = 0;
    while (k + 64 <= m && std::memcmp(pa + k, b + k, 64 * sizeof(int32_t)) == 0) k += 64;
    while (k < m && pa[k] == b[k]) ++k;
    return k;
  }

  // Returns the last matched node; appends matched slots to out (if given).
  // Keys are compared in whole pages: a trailing partial page never matches.
  Node* match(const int32_t* tokens, int64_t n, int32_t* out, int64_t* out_len) {
    uint64_t stamp = ++clock;
    Node* node = root;
    int64_t pos = 0, len = 0;
    n -= n % P;
    while (pos < n) {
      Node* child = node->children.find(page_hash(tokens + pos, P), tokens + pos, P);
      if (!child) break;
      this->stamp(child, stamp);
      int64_t k = common_len(child->key, tokens + pos, n - pos);
      k -= k % P;  // at least one page: the first page matched
      if (k < int64_t(child->key.size())) {
        Node* upper = split(child, k);
        if (out) copy_i32(out + len, upper->value.data(), k);
        len += k;
        node = upper;
        break;
      }
      if (out) copy_i32(out + len, child->value.data(), k);
      len += k;
      pos += k;
      node = child;
    }
    *out_len = len;
    return node;
  }

  // n must be a whole number of pages (checked by the callers).
  int64_t insert(const int32_t* tokens, const int32_t* slots, int64_t n) {
    uint64_t stamp = ++clock;
    Node* node = root;
    int64_t pos = 0;
    while (pos < n) {
      Node* child = node->children.find(page_hash(tokens + pos, P), tokens + pos, P);
      if (!child) break;
      this->stamp(child, stamp);
      int64_t k = common_len(child->key, tokens + pos, n - pos);
      k -= k % P;
      if (k < int64_t(child->key.size())) child = split(child, k);
      pos += k;
      node = child;
    }
    if (pos < n) {
      Node* leaf = make_node(node, tokens + pos, slots + pos, n - pos, stamp);
      node->children.set(page_hash(leaf->key.data(), P), leaf, P);
      evictable += n - pos;
      refresh(node);
      refresh(leaf);
    }
    return pos;
  }

  void lock(Node* n) {
    for (; n != root; n = n->parent) {
      if (n->lock_ref++ == 0) {
        evictable -= int64_t(n->key.size());
        protected_ += int64_t(n->key.size());
        refresh(n);
      }
    }
  }

  bool unlock(Node* n) {
    for (Node* p = n; p != root; p = p->parent)
      if (p->lock_ref == 0) return false;
    for (; n != root; n = n->parent) {
      if (--n->lock_ref == 0) {
        protected_ -= int64_t(n->key.size());
        evictable += int64_t(n->key.size());
        refresh(n);
      }
    }
    return true;
  }

  // Evicts leaves; appends freed slots to `freed` (if given).
  int64_t evict(int64_t num_tokens, std::vector<int32_t>* freed) {
    int64_t evicted = 0;
    // Frees leaf x; a parent that becomes an unlocked leaf joins the
    // candidates (and the heap, once there is one).
    auto evict_one = [&](Node* x) -> Node* {
      int64_t len = int64_t(x->value.size());
      pool->release(x->value.data(), len);  // cannot fail: the slots came from this pool
      if (freed) freed->insert(freed->end(), x->value.begin(), x->value.end());
      evicted += len;
      evictable -= len;
      Node* parent = x->parent;
      parent->children.erase(page_hash(x->key.data(), P), x->key.data(), P);
      leaf_remove(x);
      drop_node(x);
      if (is_candidate(parent)) {
        leaf_add(parent);
        return parent;
      }
      return nullptr;
    };
    // The first few victims: a scan of the contiguous candidate keys for the
    // least recently used (ties by id) -- cheaper than a heap when only a
    // few leaves go, as in a decode step's allocation.
    for (int k = 0; k < 8 && evicted < num_tokens && !leaves.empty(); ++k) {
      size_t best = 0;
      for (size_t i = 1; i < leaf_keys.size(); ++i)
        if (leaf_keys[i] < leaf_keys[best]) best = i;
      evict_one(leaves[best]);
    }
    if (evicted >= num_tokens || leaves.empty()) return evicted;
    // Many victims: a min-heap of all candidates.
    using Key = std::pair<std::pair<uint64_t, int64_t>, Node*>;
    auto cmp = [](const Key& a, const Key& b) { return a.first > b.first; };  // min-heap
    std::vector<Key> init;
    init.reserve(leaves.size());
    for (size_t i = 0; i < leaves.size(); ++i) init.push_back({leaf_keys[i], leaves[i]});
    std::priority_queue<Key, std::vector<Key>, decltype(cmp)> heap(cmp, std::move(init));
    while (evicted < num_tokens && !heap.empty()) {
      Node* x = heap.top().second;
      heap.pop();
      if (Node* parent = evict_one(x)) heap.push({{parent->last_access, parent->id}, parent});
    }
    return evicted;
  }

  // n slots (whole pages); the deficit is evicted first.
  int alloc_with_evict(int32_t n, int32_t* out, int32_t* out_evicted) {
    if (n < 0 || n % P) return fail(RT_ERR_INVALID, "allocation must be a whole number of pages");
    if (out_evicted) *out_evicted = 0;
    // An allocation that would fail even after evicting every unlocked node
    // fails before evicting anything (free + evictable is what the
    // scheduler's admission test counts as available).
    if (int64_t(n) > pool->free_slots() + evictable)
      return fail(RT_ERR_OOM, "need " + std::to_string(n) + " slots, " + std::to_string(pool->free_slots()) +
                                  " free + " + std::to_string(evictable) + " evictable");
    int64_t ev = 0;
    if (n > pool->free_slots()) ev = evict(int64_t(n) - pool->free_slots(), nullptr);
    if (out_evicted) *out_evicted = int32_t(ev);
    if (n > pool->free_slots())
      return fail(RT_ERR_OOM, "need " + std::to_string(n) + " slots, " + std::to_string(pool->free_slots()) +
                                  " free after evicting " + std::to_string(ev));
    return pool->alloc(n, out);
  }

  // Slots of runs of positions by the page rule: a position that starts a
  // page takes a fresh page (allocated for all runs at once, evicting first
  // if short, taken in run order) and its first slot; any other position
  // takes the slot after the previous position's, read from that request's
  // row.  Writes every slot into its row and into out (concatenated).
  int alloc_positions(int32_t n_runs, const int32_t* rows, const int32_t* first, const int32_t* counts,
                      int32_t* req_to_token, int64_t stride, int32_t num_rows, int32_t* out, int64_t out_cap,
                      int32_t* out_evicted) {
    int64_t starts = 0, total = 0;
    for (int32_t i = 0; i < n_runs; ++i) {
      if (rows[i] < 0 || rows[i] >= num_rows || first[i] < 0 || counts[i] < 0 ||
          int64_t(first[i]) + counts[i] > stride)
        return fail(RT_ERR_INVALID, "alloc_positions: bad run " + std::to_string(i));
      // multiples of P in [first, first + count)
      starts += (int64_t(first[i]) + counts[i] + P - 1) / P - (int64_t(first[i]) + P - 1) / P;
      total += counts[i];
    }
    if (total > out_cap || (total > 0 && !out)) return fail(RT_ERR_INVALID, "alloc_positions: out too small");
    if (starts * P > INT32_MAX) return fail(RT_ERR_INVALID, "alloc_positions: too many pages");
    fresh_.resize(size_t(starts * P));
    int rc = alloc_with_evict(int32_t(starts * P), fresh_.data(), out_evicted);
    if (rc != RT_OK) return rc;
    const int32_t* fresh = fresh_.data();
    int64_t next = 0, o = 0;
    for (int32_t i = 0; i < n_runs; ++i) {
      int32_t* row = req_to_token + int64_t(rows[i]) * stride;
      const int64_t x0 = first[i], cnt = counts[i];
      if (P == 1) {  // every position starts a page: the fresh slots in order
        copy_i32(row + x0, fresh + next, cnt);
        copy_i32(out + o, fresh + next, cnt);
        next += cnt;
        o += cnt;
        continue;
      }
      int64_t r = x0 % P;  // offset of position x within its page
      for (int64_t x = x0; x < x0 + cnt; ++x) {
        const int32_t sl = r == 0 ? fresh[next++ * P] : row[x - 1] + 1;
        row[x] = sl;
        out[o++] = sl;
        if (++r == P) r = 0;
      }
    }
    return RT_OK;
  }

  void dump_node(const Node* n, int64_t parent_id, std::string& s) const {
    s += std::to_string(n->id);
    s += ' ';
    s += std::to_string(parent_id);
    s += ' ';
    s += std::to_string(n->lock_ref);
    s += ' ';
    s += std::to_string(n->last_access);
    s += " k=";
    for (size_t i = 0; i < n->key.size(); ++i) {
      if (i) s += ',';
      s += std::to_string(n->key[i]);
    }
    s += " v=";
    for (size_t i = 0; i < n->value.size(); ++i) {
      if (i) s += ',';
      s += std::to_string(n->value[i]);
    }
    s += '\n';
    // children by first page, lexicographic
    std::vector<const Node*> kids;
    n->children.for_each([&](const Node* c) { kids.push_back(c); });
    const int32_t p = P;
    std::sort(kids.begin(), kids.end(), [p](const Node* a, const Node* b) {
      return std::lexicographical_compare(a->key.begin(), a->key.begin() + p, b->key.begin(), b->key.begin() + p);
    });
    for (const Node* c : kids) dump_node(c, n->id, s);
  }
};

}  // namespace rt

// ===================================================================== ABI ==
using rt::fail;

struct rt_pool {
  rt::Pool impl;
  rt_pool(int32_t n, int32_t page) : impl(n, page) {}
};
struct rt_tree {
  rt::Tree impl;
  explicit rt_tree(rt_pool* p) : impl(&p->impl) {}
};

#define RT_GUARD_BEGIN try {
#define RT_GUARD_END                                        \
  }                                                         \
  catch (const std::bad_alloc&) {                           \
    return fail(RT_ERR_OOM, "host allocation failed");      \
  }                                                         \
  catch (const std::exception& e) {                         \
    return fail(RT_ERR_INVALID, e.what());                  \
  }

extern "C" {

int rt_pool_create_paged(int32_t num_slots, int32_t page_size, rt_pool** out) {
  if (!out || num_slots < 1 || page_size < 1 || num_slots % page_size)
    return fail(RT_ERR_INVALID, "rt_pool_create_paged: num_slots a positive multiple of page_size, out required");
  RT_GUARD_BEGIN
  *out = new rt_pool(num_slots, page_size);
  return RT_OK;
  RT_GUARD_END
}

int rt_pool_create(int32_t num_slots, rt_pool** out) { return rt_pool_create_paged(num_slots, 1, out); }

int32_t rt_pool_page_size(const rt_pool* pool) { return pool ? pool->impl.page : 0; }

void rt_pool_destroy(rt_pool* pool) { delete pool; }

int rt_pool_alloc(rt_pool* pool, int32_t n, int32_t* out_slots) {
  if (!pool || (n > 0 && !out_slots)) return fail(RT_ERR_INVALID, "rt_pool_alloc: null argument");
  return pool->impl.alloc(n, out_slots);
}

int rt_pool_free(rt_pool* pool, const int32_t* slots, int32_t n) {
  if (!pool || (n > 0 && !slots)) return fail(RT_ERR_INVALID, "rt_pool_free: null argument");
  return pool->impl.release(slots, n);
}

int32_t rt_pool_available(const rt_pool* pool) { return pool ? int32_t(pool->impl.free_slots()) : 0; }
int32_t rt_pool_capacity(const rt_pool* pool) { return pool ? pool->impl.capacity : 0; }

int rt_pool_free_list(const rt_pool* pool, int32_t* out, int32_t cap, int32_t* out_len) {
  if (!pool || !out_len) return fail(RT_ERR_INVALID, "rt_pool_free_list: null argument");
  const rt::Pool& p = pool->impl;
  const int32_t n = int32_t(p.free_slots());
  *out_len = n;
  if (cap < n || (n > 0 && !out)) return fail(RT_ERR_INVALID, "rt_pool_free_list: buffer too small");
  for (int32_t i = 0; i < p.count; ++i)
    for (int32_t t = 0; t < p.page; ++t) out[int64_t(i) * p.page + t] = p.ring[(p.head + i) % p.pages] + t;
  return RT_OK;
}

int rt_tree_create(rt_pool* pool, rt_tree** out) {
  if (!pool || !out) return fail(RT_ERR_INVALID, "rt_tree_create: null argument");
  RT_GUARD_BEGIN
  *out = new rt_tree(pool);
  return RT_OK;
  RT_GUARD_END
}

void rt_tree_destroy(rt_tree* tree) { delete tree; }

int rt_match_prefix(rt_tree* tree, const int32_t* tokens, int32_t n, int32_t* out_slots,
                    int32_t out_cap, int32_t* out_len, rt_node* out_last) {
  if (!tree || n < 0 || (n > 0 && (!tokens || !out_slots)) || !out_len || !out_last)
    return fail(RT_ERR_INVALID, "rt_match_prefix: bad argument");
  if (out_cap < n) return fail(RT_ERR_INVALID, "rt_match_prefix: out_cap < n");
  RT_GUARD_BEGIN
  int64_t len = 0;
  rt::Node* last = tree->impl.match(tokens, n, out_slots, &len);
  *out_len = int32_t(len);
  *out_last = last->id;
  return RT_OK;
  RT_GUARD_END
}

int rt_insert(rt_tree* tree, const int32_t* tokens, const int32_t* slots, int32_t n,
              int32_t* out_present_len) {
  if (!tree || n < 0 || (n > 0 && (!tokens || !slots))) return fail(RT_ERR_INVALID, "rt_insert: bad argument");
  if (n % tree->impl.P) return fail(RT_ERR_INVALID, "rt_insert: length is not a whole number of pages");
  RT_GUARD_BEGIN
  int64_t present = tree->impl.insert(tokens, slots, n);
  if (out_present_len) *out_present_len = int32_t(present);
  return RT_OK;
  RT_GUARD_END
}

int rt_lock(rt_tree* tree, rt_node node) {
  if (!tree) return fail(RT_ERR_INVALID, "rt_lock: null tree");
  rt::Node* n = tree->impl.find(node);
  if (!n) return fail(RT_ERR_INVALID, "rt_lock: unknown node " + std::to_string(node));
  tree->impl.lock(n);
  return RT_OK;
}

int rt_unlock(rt_tree* tree, rt_node node) {
  if (!tree) return fail(RT_ERR_INVALID, "rt_unlock: null tree");
  rt::Node* n = tree->impl.find(node);
  if (!n) return fail(RT_ERR_INVALID, "rt_unlock: unknown node " + std::to_string(node));
  if (!tree->impl.unlock(n)) return fail(RT_ERR_INVALID, "rt_unlock: lock count would go below zero");
  return RT_OK;
}

int rt_evict_lru_leaves(rt_tree* tree, int32_t num_tokens, int32_t* out_evicted,
                        int32_t* out_freed_slots, int32_t freed_cap) {
  if (!tree || num_tokens < 0) return fail(RT_ERR_INVALID, "rt_evict_lru_leaves: bad argument");
  RT_GUARD_BEGIN
  std::vector<int32_t> freed;
  int64_t ev = tree->impl.evict(num_tokens, out_freed_slots ? &freed : nullptr);
  if (out_evicted) *out_evicted = int32_t(ev);
  if (out_freed_slots) {
    int64_t m = std::min<int64_t>(int64_t(freed.size()), std::max(freed_cap, 0));
    rt::copy_i32(out_freed_slots, freed.data(), m);
  }
  return RT_OK;
  RT_GUARD_END
}

int rt_alloc_positions(rt_tree* tree, int32_t n_runs, const int32_t* rows, const int32_t* first_positions,
                       const int32_t* counts, int32_t* req_to_token, int64_t stride, int32_t num_rows,
                       int32_t* out_slots, int64_t out_cap, int32_t* out_evicted) {
  if (!tree || n_runs < 0 || (n_runs > 0 && (!rows || !first_positions || !counts || !req_to_token)) ||
      stride < 1 || num_rows < 0)
    return fail(RT_ERR_INVALID, "rt_alloc_positions: bad argument");
  RT_GUARD_BEGIN
  return tree->impl.alloc_positions(n_runs, rows, first_positions, counts, req_to_token, stride, num_rows, out_slots,
                                    out_cap, out_evicted);
  RT_GUARD_END
}

int rt_alloc_with_evict(rt_tree* tree, int32_t n, int32_t* out_slots, int32_t* out_evicted) {
  if (!tree || (n > 0 && !out_slots)) return fail(RT_ERR_INVALID, "rt_alloc_with_evict: bad argument");
  RT_GUARD_BEGIN
  return tree->impl.alloc_with_evict(n, out_slots, out_evicted);
  RT_GUARD_END
}

int64_t rt_evictable_size(const rt_tree* tree) { return tree ? tree->impl.evictable : 0; }
int64_t rt_protected_size(const rt_tree* tree) { return tree ? tree->impl.protected_ : 0; }
int64_t rt_tree_num_nodes(const rt_tree* tree) { return tree ? tree->impl.live + 1 : 0; }

int rt_tree_dump(const rt_tree* tree, char* buf, int64_t cap, int64_t* out_len) {
  if (!tree || !out_len) return fail(RT_ERR_INVALID, "rt_tree_dump: null argument");
  RT_GUARD_BEGIN
  std::string s;
  tree->impl.dump_node(tree->impl.root, -1, s);
  *out_len = int64_t(s.size());
  if (!buf || cap < int64_t(s.size())) return fail(RT_ERR_INVALID, "rt_tree_dump: buffer too small");
  std::memcpy(buf, s.data(), s.size());
  if (cap > int64_t(s.size())) buf[s.size()] = '\0';
  return RT_OK;
  RT_GUARD_END
}

int rt_admit_batch(rt_tree* tree, const int32_t* tokens, const int64_t* token_offsets, int32_t n,
                   int32_t* req_to_token, int64_t stride, int32_t num_rows, const int32_t* rows,
                   int32_t* prefix_lens, int32_t* extend_lens, rt_node* nodes, int32_t* out_cache_loc,
                   int64_t out_cache_cap, int64_t* out_num_new) {
  if (!tree || n < 0 || !token_offsets || (n > 0 && (!tokens || !req_to_token || !rows || !prefix_lens ||
                                                      !extend_lens || !nodes)) ||
      stride < 1 || num_rows < 0 || !out_num_new)
    return fail(RT_ERR_INVALID, "rt_admit_batch: bad argument");
  RT_GUARD_BEGIN
  rt::Tree& t = tree->impl;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t len = token_offsets[i + 1] - token_offsets[i];
    if (len < 0 || len > stride) return fail(RT_ERR_INVALID, "rt_admit_batch: request longer than stride");
    if (rows[i] < 0 || rows[i] >= num_rows) return fail(RT_ERR_INVALID, "rt_admit_batch: row out of range");
    total += len;
  }
  int64_t new_total = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t* tk = tokens + token_offsets[i];
    int64_t len = token_offsets[i + 1] - token_offsets[i];
    int32_t* row = req_to_token + int64_t(rows[i]) * stride;
    int64_t plen = 0;
    rt::Node* last = t.match(tk, len, row, &plen);
    t.lock(last);
    nodes[i] = last->id;
    prefix_lens[i] = int32_t(plen);
    extend_lens[i] = int32_t(len - plen);
    new_total += len - plen;
  }
  *out_num_new = new_total;
  auto unlock_all = [&]() {
    for (int32_t i = n - 1; i >= 0; --i) t.unlock(t.find(nodes[i]));
  };
  if (new_total > out_cache_cap || (new_total > 0 && !out_cache_loc)) {
    unlock_all();
    return fail(RT_ERR_INVALID, "rt_admit_batch: out_cache_loc too small");
  }
  if (new_total > INT32_MAX) {
    unlock_all();
    return fail(RT_ERR_INVALID, "rt_admit_batch: too many new tokens");
  }
  // slots of positions [prefix, prefix + extend) of every request, by the
  // page rule, written into the rows and into out_cache_loc
  int rc = t.alloc_positions(n, rows, prefix_lens, extend_lens, req_to_token, stride, num_rows, out_cache_loc,
                             out_cache_cap, nullptr);
  if (rc != RT_OK) {
    unlock_all();
    return rc;
  }
  (void)total;
  return RT_OK;
  RT_GUARD_END
}

int rt_decode_slots_batch(rt_tree* tree, int32_t n, const int32_t* rows, const int32_t* positions,
                          int32_t* req_to_token, int64_t stride, int32_t num_rows, int32_t* out_cache_loc) {
  if (!tree || n < 0 || (n > 0 && (!rows || !positions || !req_to_token || !out_cache_loc)) || stride < 1 ||
      num_rows < 0)
    return fail(RT_ERR_INVALID, "rt_decode_slots_batch: bad argument");
  for (int32_t i = 0; i < n; ++i)
    if (rows[i] < 0 || rows[i] >= num_rows || positions[i] < 0 || positions[i] >= stride)
      return fail(RT_ERR_INVALID, "rt_decode_slots_batch: row or position out of range");
  RT_GUARD_BEGIN
  std::vector<int32_t> ones(size_t(n), 1);
  return tree->impl.alloc_positions(n, rows, positions, ones.data(), req_to_token, stride, num_rows, out_cache_loc,
                                    n, nullptr);
  RT_GUARD_END
}

int rt_finish_batch(rt_tree* tree, const int32_t* tokens, const int64_t* token_offsets, int32_t n,
                    const int32_t* req_to_token, int64_t stride, int32_t num_rows, const int32_t* rows,
                    const int32_t* prefix_lens, const rt_node* nodes, int64_t* out_freed) {
  if (!tree || n < 0 || !token_offsets ||
      (n > 0 && (!tokens || !req_to_token || !rows || !prefix_lens || !nodes)) || stride < 1 || num_rows < 0)
    return fail(RT_ERR_INVALID, "rt_finish_batch: bad argument");
  RT_GUARD_BEGIN
  rt::Tree& t = tree->impl;
  for (int32_t i = 0; i < n; ++i) {
    int64_t len = token_offsets[i + 1] - token_offsets[i];
    if (len < 0 || len > stride || rows[i] < 0 || rows[i] >= num_rows || prefix_lens[i] < 0 ||
        prefix_lens[i] > len)
      return fail(RT_ERR_INVALID, "rt_finish_batch: bad request " + std::to_string(i));
    if (!t.find(nodes[i])) return fail(RT_ERR_INVALID, "rt_finish_batch: unknown node");
  }
  int64_t freed = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t* tk = tokens + token_offsets[i];
    int64_t len = token_offsets[i + 1] - token_offsets[i];
    const int32_t* row = req_to_token + int64_t(rows[i]) * stride;
    // the whole pages go into the tree; pages the tree already held and the
    // trailing partial page go back to the pool, in one free
    const int64_t aligned = len - len % t.P;
    const int64_t present = t.insert(tk, row, aligned);
    std::vector<int32_t> rel;
    if (present > prefix_lens[i]) rel.assign(row + prefix_lens[i], row + present);
    rel.insert(rel.end(), row + aligned, row + len);
    if (!rel.empty()) {
      int rc = t.pool->release(rel.data(), int64_t(rel.size()));
      if (rc != RT_OK) return rc;
      freed += int64_t(rel.size());
    }
    rt::Node* node = t.find(nodes[i]);
    if (!node || !t.unlock(node)) return fail(RT_ERR_INVALID, "rt_finish_batch: unlock failed");
  }
  if (out_freed) *out_freed = freed;
  return RT_OK;
  RT_GUARD_END
}

}  // extern "C"
