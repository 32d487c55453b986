/*
 * radixrt -- the RadixAttention hot path for AMD Instinct MI355X (gfx950).
 *
 * A host-side radix tree over a token-granular KV pool finds each request's
 * cached prefix; HIP kernels scatter new K/V rows into the pool and run
 * attention over pool rows gathered through a per-request slot table
 * (req_to_token).  Sources (the four pages the project is built from):
 *
 *  [P1] SGLang paper summary (paperlayer.ai, arXiv 2312.07104v2), section 3
 *       "Efficient KV Cache Reuse with RadixAttention": the tree maps token
 *       sequences to KV tensors, LRU eviction of leaves, reference counters
 *       protect nodes of running requests, cache and running requests share
 *       one dynamically allocated pool.
 *  [P2] SGLang explainer (yaopepe.com/papers/sglang), section 04
 *       "RadixAttention": longest-prefix match from the root, edge split on a
 *       partial match, the walkthrough figure (insert S+A, split on S+B,
 *       evict leaf A while S and B are protected, C reuses S), the
 *       token-weighted hit-rate formula, and the source excerpts on prefix
 *       match (stamp access time, split, accumulate slots) and eviction (heap
 *       of evictable leaves, free the leaf's slots, re-push a parent that
 *       became an unlocked leaf).
 *  [P4] SGLang v0.2 handbook chapter (anrans.github.io), sections "CUDA
 *       Graph" and "new_token_ratio and retract": runtime metadata
 *       req_pool_indices / seq_lens / out_cache_loc, padded entries writing
 *       slot 0, and the admission estimate free + evictable - reservations.
 *
 * Conventions for every call:
 *  - Status: RT_OK (0) or a negative RT_ERR_*; no exception crosses the ABI.
 *    rt_last_error() returns a message for the calling thread's last error.
 *  - Slots: the pool has usable slots 1..num_slots; slot 0 is reserved as the
 *    harmless target of padded writes [P4] and is never handed out.
 *  - Host pointers are marked (host); device pointers (device).  The caller
 *    owns every buffer; the library never keeps a caller pointer after a call
 *    returns.  Device calls allocate nothing, launch asynchronously on
 *    `stream` (a hipStream_t; NULL is the default stream) and do not
 *    synchronise.  A device call must follow, on the same stream, the
 *    kv_store that wrote the slots it reads.
 *  - The tree and pool are single-threaded objects: calls on one tree (or
 *    its pool) must not overlap.
 */
#ifndef RADIXRT_H
#define RADIXRT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum rt_status {
  RT_OK = 0,
  RT_ERR_INVALID = -1, /* bad argument, shape, length or handle */
  RT_ERR_OOM = -2,     /* not enough free + evictable slots; nothing allocated */
  RT_ERR_LOCKED = -3,  /* reserved: operation refused on a locked node */
  RT_ERR_HIP = -4      /* a HIP launch or runtime call failed */
};

enum rt_dtype { RT_F32 = 0, RT_BF16 = 1 };

typedef struct rt_pool rt_pool;
typedef struct rt_tree rt_tree;
/* Node handle: the node's creation id.  Valid until that node is evicted;
 * a split keeps the handle on the lower part of the edge.  0 is the root. */
typedef int64_t rt_node;

/* Message of the calling thread's last failed call ("" if none). */
const char* rt_last_error(void);
/* ABI version of this header (incremented on incompatible changes). */
int rt_abi_version(void);

/* ---------------------------------------------------------------- pool --
 * Token-slot allocator [P1 cache management: cached and running requests share one pool; P2 freeing a leaf's slots].
 * Slots come in pages of page_size (1 unless created paged): page j holds
 * slots 1 + j*page_size .. (j+1)*page_size [P2 prefix-match excerpt: the
 * engine compares keys under a configurable page size].  Free pages form a
 * FIFO list that starts ascending; allocation takes whole pages from the
 * head, a free appends the distinct pages of the given slots at the tail in
 * order of first appearance.  With one-slot pages: a FIFO of slots, frees
 * appended in the order given. */

/* num_slots >= 1.  *out receives the pool (free with rt_pool_destroy). */
int rt_pool_create(int32_t num_slots, rt_pool** out);
/* A pool of pages: num_slots a positive multiple of page_size >= 1. */
int rt_pool_create_paged(int32_t num_slots, int32_t page_size, rt_pool** out);
void rt_pool_destroy(rt_pool* pool);
int32_t rt_pool_page_size(const rt_pool* pool);
/* Take n slots (host out_slots[n]): n / page_size whole pages, each page's
 * slots in order.  RT_ERR_INVALID if n is not a whole number of pages;
 * RT_ERR_OOM if fewer are free (nothing taken).  Never evicts: see
 * rt_alloc_with_evict. */
int rt_pool_alloc(rt_pool* pool, int32_t n, int32_t* out_slots);
/* Return the pages of n slots (host).  Each must be in 1..num_slots;
 * RT_ERR_INVALID if a slot is out of range or the free list would exceed
 * the pool (nothing is freed then). */
int rt_pool_free(rt_pool* pool, const int32_t* slots, int32_t n);
/* Free slots (whole free pages times page_size) and all usable slots. */
int32_t rt_pool_available(const rt_pool* pool);
int32_t rt_pool_capacity(const rt_pool* pool);
/* Copy the free list as slots, head page first, each page's slots in
 * order, into host out[cap]; *out_len = its length (RT_ERR_INVALID, nothing
 * copied, if cap < length). */
int rt_pool_free_list(const rt_pool* pool, int32_t* out, int32_t cap, int32_t* out_len);

/* ---------------------------------------------------------------- tree --
 * Radix tree of cached prefixes bound to a pool [P1, P2].  A node holds a
 * run of tokens and the KV slot of each; children are keyed by their first
 * page of tokens (their first token with one-slot pages).  Keys are compared
 * in whole pages of the pool's page size: matches, splits and inserts fall
 * on page boundaries and a trailing partial page never matches.  An LRU
 * clock advances by one per rt_match_prefix / rt_insert call; every node
 * such a call walks through or creates is stamped with it.  Eviction order
 * is (last access, node id) ascending. */

int rt_tree_create(rt_pool* pool, rt_tree** out);
/* Destroys the tree; its slots are NOT returned to the pool. */
void rt_tree_destroy(rt_tree* tree);

/* Longest cached prefix of tokens[n] (host) [P2 prefix-match excerpt].
 * Writes its slots to host out_slots (out_cap >= n required), its length to
 * *out_len and the handle of its last node to *out_last (0 = root when
 * nothing matches).  If the match ends inside an edge, the edge is split so
 * that the matched part becomes its own node, which is returned; the new
 * upper node copies the lower node's lock count. */
int rt_match_prefix(rt_tree* tree, const int32_t* tokens, int32_t n, int32_t* out_slots,
                    int32_t out_cap, int32_t* out_len, rt_node* out_last);

/* Insert tokens[n] with their slots[n] (host) [P2 walkthrough step 2]; n
 * must be a whole number of pages (RT_ERR_INVALID otherwise).
 * Diverging edges are split; the unmatched rest becomes a new leaf.  Where
 * the tree already holds a token its slot is kept; *out_present_len (may be
 * NULL) receives how many leading tokens were already present, and the
 * caller owns (and must free) its own slots in that range that it
 * allocated. */
int rt_insert(rt_tree* tree, const int32_t* tokens, const int32_t* slots, int32_t n,
              int32_t* out_present_len);

/* Reference counts on every non-root node from `node` up to the root
 * [P1 cache management: counts that keep running requests' nodes from eviction; P2 lifetime figure].  Locked nodes are never
 * evicted.  rt_unlock on a path with a zero count fails with
 * RT_ERR_INVALID and changes nothing.  Locking the root is a no-op. */
int rt_lock(rt_tree* tree, rt_node node);
int rt_unlock(rt_tree* tree, rt_node node);

/* Evict whole unlocked leaves, least recently used first, until at least
 * num_tokens tokens are freed or no candidate is left [P2 eviction
 * excerpt]; a parent that becomes an unlocked leaf joins the candidates.
 * Freed slots go to the pool's tail in node order.  *out_evicted (may be
 * NULL) receives the number of tokens freed; the first min(that, freed_cap)
 * freed slots are copied to host out_freed_slots (may be NULL). */
int rt_evict_lru_leaves(rt_tree* tree, int32_t num_tokens, int32_t* out_evicted,
                        int32_t* out_freed_slots, int32_t freed_cap);

/* Allocate n slots (whole pages), first evicting the deficit (n - free) if
 * the pool is short.  RT_ERR_OOM if still short: nothing is allocated, but
 * evictions already made stand.  *out_evicted (may be NULL) = tokens
 * evicted. */
int rt_alloc_with_evict(rt_tree* tree, int32_t n, int32_t* out_slots, int32_t* out_evicted);

/* Slots for runs of positions of requests, by the page rule: run i is
 * positions first_positions[i] .. + counts[i] - 1 of slot-table row rows[i]
 * (host table req_to_token, row stride `stride`).  A position that starts a
 * page (position % page_size == 0) takes a fresh page and its first slot;
 * the fresh pages for all runs are allocated at once (evicting first if
 * short, as rt_alloc_with_evict) and taken in run order.  Any other position
 * takes the slot after the previous position's, read from its row (which
 * must hold that request's slot).  Every slot is written into its row and,
 * concatenated in run order, into host out_slots (out_cap entries).
 * *out_evicted (may be NULL) = tokens evicted.  With one-slot pages this is
 * rt_alloc_with_evict of all positions, in order.  The table has num_rows
 * rows: a row outside [0, num_rows) or a run past the stride is
 * RT_ERR_INVALID before anything is allocated. */
int rt_alloc_positions(rt_tree* tree, int32_t n_runs, const int32_t* rows, const int32_t* first_positions,
                       const int32_t* counts, int32_t* req_to_token, int64_t stride, int32_t num_rows,
                       int32_t* out_slots, int64_t out_cap, int32_t* out_evicted);

/* Tokens held by unlocked nodes / by locked nodes (root excluded). */
int64_t rt_evictable_size(const rt_tree* tree);
int64_t rt_protected_size(const rt_tree* tree);
int64_t rt_tree_num_nodes(const rt_tree* tree);

/* Canonical text dump into host buf[cap]: pre-order from the root, children
 * by first page ascending (lexicographic), one line per node
 *   "<id> <parent id> <lock count> <last access> k=<t,t,...> v=<s,s,...>\n"
 * with the root as "0 -1 0 0 k= v=".  *out_len = bytes needed (without a
 * terminating NUL, which is written when it fits); RT_ERR_INVALID if cap is
 * too small (then only *out_len is set). */
int rt_tree_dump(const rt_tree* tree, char* buf, int64_t cap, int64_t* out_len);

/* ------------------------------------------------------ batch helpers --
 * Compositions of the calls above for a whole batch, so that a batch costs
 * one crossing of the ABI.  Request i's tokens are
 * tokens[token_offsets[i] .. token_offsets[i+1]) (host).  Row r of the slot
 * table is req_to_token[r * stride .. r * stride + stride) (host), for r in
 * [0, num_rows); every call checks each rows[i] against num_rows before it
 * touches the table (RT_ERR_INVALID). */

/* For i in order: rt_match_prefix, rt_lock; then one rt_alloc_positions of
 * positions prefix_len_i .. len_i - 1 of every request (with one-slot
 * pages: sum_i (len_i - prefix_len_i) slots split among the requests in
 * order).  Row rows[i] of req_to_token receives the matched slots followed
 * by the new ones.  Outputs (host, n entries): prefix_lens, extend_lens, nodes;
 * out_cache_loc receives the new slots (cap out_cache_cap), *out_num_new
 * their count.  On RT_ERR_OOM every lock taken here is released (the
 * matches' splits and stamps remain).  RT_ERR_INVALID if a request is
 * longer than stride. */
int rt_admit_batch(rt_tree* tree, const int32_t* tokens, const int64_t* token_offsets,
                   int32_t n, int32_t* req_to_token, int64_t stride, int32_t num_rows, const int32_t* rows,
                   int32_t* prefix_lens, int32_t* extend_lens, rt_node* nodes,
                   int32_t* out_cache_loc, int64_t out_cache_cap, int64_t* out_num_new);

/* One decode step's slots: rt_alloc_positions of one position
 * positions[i] per row rows[i], which sets
 * req_to_token[rows[i] * stride + positions[i]] = slot i (host).
 * out_cache_loc (host, n) receives the slots. */
int rt_decode_slots_batch(rt_tree* tree, int32_t n, const int32_t* rows, const int32_t* positions,
                          int32_t* req_to_token, int64_t stride, int32_t num_rows, int32_t* out_cache_loc);

/* Finish requests: for i in order, rt_insert of the whole pages of tokens_i
 * (the first len_i - len_i % page_size) with row rows[i] of req_to_token,
 * then one rt_pool_free of the row's slots in [prefix_lens[i],
 * present_len) (the duplicates the tree already held) followed by those in
 * [aligned len, len_i) (the trailing partial page), then
 * rt_unlock(nodes[i]).  *out_freed (may be NULL) = total slots passed to
 * those frees. */
int rt_finish_batch(rt_tree* tree, const int32_t* tokens, const int64_t* token_offsets,
                    int32_t n, const int32_t* req_to_token, int64_t stride, int32_t num_rows, const int32_t* rows,
                    const int32_t* prefix_lens, const rt_node* nodes, int64_t* out_freed);

/* -------------------------------------------------------------- device --
 * Pools k_pool / v_pool: (device) [num_slots + 1, num_kv_heads, head_dim],
 * contiguous, element type `dtype` (RT_F32 or RT_BF16), the same as q / o.
 * head_dim is 64 or 128; num_q_heads is a positive multiple of num_kv_heads;
 * query head h reads KV head h / (num_q_heads / num_kv_heads).
 * req_to_token: (device) int32 [rows, req_to_token_stride]; request b uses
 * row req_pool_indices[b] (or row b when req_pool_indices is NULL), whose
 * first prefix_lens[b] + extend_lens[b] entries are pool slots.  Slot
 * contents are not range-checked on the device; the host checks shapes and
 * host-side scalars and returns RT_ERR_INVALID before launching anything. */

/* Scatter new rows into the pool [P4 out_cache_loc]:
 * k_pool[out_cache_loc[t]] = k_new[t], v_pool[...] = v_new[t] for
 * t < n_tokens; k_new / v_new (device) [n_tokens, num_kv_heads, head_dim].
 * Bit-exact copy.  Repeated slots (e.g. padding to slot 0) race: each
 * 16-byte piece of such a slot ends up holding that piece of one of the rows
 * written to it. */
int kv_store(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
             const int32_t* out_cache_loc, int32_t n_tokens, int32_t num_kv_heads,
             int32_t head_dim, int dtype, void* stream);

/* Per-step update of the device slot table [P4 req_to_token written from
 * out_cache_loc]: req_to_token[rows[i] * stride + positions[i]] = slots[i]
 * for i < n.  rows, positions, slots: (device) int32 [n].  Positions must
 * be < stride and rows inside the table (not checked on the device). */
int req_to_token_scatter(int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* rows,
                         const int32_t* positions, const int32_t* slots, int32_t n, void* stream);

/* Staging of a step's slot-table rows and metadata [P4 "CUDA Graph": the
 * runtime writes req_pool_indices, seq_lens and out_cache_loc into fixed
 * device buffers before each step]: copies bytes from pinned host memory
 * src to device memory dst with a kernel on `stream`, so that the copy
 * stays on the compute queue beside the step's kernels.  src must lie
 * inside one pinned (hipHostMalloc) allocation, checked on the host through
 * the allocation's recorded range; pageable memory is refused with RT_ERR_INVALID before
 * anything is launched.  bytes a multiple of 4, both pointers 4-byte
 * aligned (16-byte alignment takes the faster path).  dst must be device
 * memory, with [dst, dst + bytes) inside its allocation (checked on the
 * host; the allocation may be a larger pool block than the caller's
 * buffer).  The host must not change src until the copy has run (as for an
 * asynchronous copy). */
int rt_copy_from_host(void* dst, const void* src, int64_t bytes, void* stream);

/* rt_copy_from_host over height rows of width bytes: row r goes from
 * src + r * src_pitch (pinned host) to dst + r * dst_pitch (device), so a
 * step can move only the columns of its slot-table rows that changed.
 * width and the pitches multiples of 4, pitches >= width when height > 1;
 * the whole source span must lie in one pinned allocation and the whole
 * destination span in one device allocation (checked as above). */
int rt_copy_from_host_2d(void* dst, int64_t dst_pitch, const void* src, int64_t src_pitch, int64_t width,
                         int64_t height, void* stream);

/* The host-side checks of rt_copy_from_host_2d alone, launching nothing:
 * RT_OK when the copy would be accepted, else RT_ERR_INVALID with the
 * reason in rt_last_error().  The source range must lie inside one pinned
 * host allocation as the HIP runtime records it (hipMemGetAddressRange),
 * the destination range inside one device allocation. */
int rt_copy_from_host_check(void* dst, int64_t dst_pitch, const void* src, int64_t src_pitch, int64_t width,
                            int64_t height);

/* One decode step's writes in a single launch: req_to_token_scatter of
 * (rows, positions, slots) and kv_store of (k_new, v_new) at slots, for i < n
 * [P4 the decode step writes its new token's slot into req_to_token and its
 * K/V into the pool before attention].  rows, positions, slots: (device)
 * int32 [n]; k_new, v_new: (device) [n, num_kv_heads, head_dim].  Same
 * results as the two calls; same unchecked device contents.  Repeated
 * slots (padding to slot 0) race: each 16-byte piece of such a slot ends up
 * holding that piece of one of the rows written to it. */
int decode_append(int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* rows,
                  const int32_t* positions, const int32_t* slots, int32_t n, void* k_pool, void* v_pool,
                  const void* k_new, const void* v_new, int32_t num_kv_heads, int32_t head_dim, int dtype,
                  void* stream);

/* The extend batch's scatter with its targets read from the slot table [P4
 * out_cache_loc; the new slots are the entries req_to_token[row_b][prefix_lens[b]
 * .. prefix_lens[b] + extend_lens[b]) that the host already wrote]: for request
 * b and j < extend_lens[b], row qo_indptr[b] + j of k_new / v_new goes to slot
 * req_to_token[row_b][prefix_lens[b] + j], row_b = req_pool_indices[b] (or b
 * when req_pool_indices is NULL).  The metadata arguments mean what they mean
 * for radix_extend_attention, so one set of device arrays drives both calls;
 * qo_indptr[b] only locates request b's first row (rows between requests are
 * not read).  k_new, v_new: (device) [rows, num_kv_heads, head_dim] in the
 * pool's dtype (RT_F32 or RT_BF16).  Same results as kv_store with
 * out_cache_loc = those table entries in request order; the same race on
 * repeated slots; table entries and lengths are not checked on the device.
 * batch <= 65535; max_extend_len (host) bounds every extend_lens[b]. */
int kv_store_extend(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                    const int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* req_pool_indices,
                    const int32_t* prefix_lens, const int32_t* extend_lens, const int32_t* qo_indptr,
                    int32_t batch, int32_t max_extend_len, int32_t num_kv_heads, int32_t head_dim, int dtype,
                    void* stream);

/* Extend (prefill of the uncached suffix) attention [P2 section 04: after the
 * longest-prefix match only the tokens past the cached prefix are computed,
 * attending to the cached K/V].
 * For request b, extend row j < extend_lens[b] and query head h:
 *   o[qo_indptr[b] + j][h] = sum_i softmax_i(sm_scale * q.k_i) v_i over keys
 *   i = 0 .. prefix_lens[b] + j, k_i / v_i = pool rows at slot
 *   req_to_token[row_b][i] of KV head h / (Hq / Hkv).
 * q, o: (device) [total extend rows, num_q_heads, head_dim]; request b's
 * rows start at row qo_indptr[b] (device, int32 [batch + 1]), normally the
 * exclusive prefix sum of extend_lens.  Only qo_indptr[0 .. batch - 1] is
 * read, so rows between requests may be left out (they are neither read
 * nor written).  prefix_lens, extend_lens (device, int32
 * [batch]).  max_extend_len (host) bounds every extend_lens[b] and sizes the
 * grid.  extend_lens[b] = 0 is allowed (no rows).  fp32 accumulation; o has
 * the input dtype. */
int radix_extend_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                           const int32_t* req_to_token, int32_t req_to_token_stride,
                           const int32_t* req_pool_indices, const int32_t* prefix_lens,
                           const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                           int32_t max_extend_len, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, float sm_scale, int dtype, void* stream);

/* One launch for a mixed batch [P4, the #800 entry of the release timeline:
 * chunked prefill runs prompt chunks beside the running requests' decode
 * steps]: requests 0 .. num_extend - 1 are extend requests with
 * extend_lens[b] <= max_extend_len, requests num_extend .. batch - 1 are
 * short ones with extend_lens[b] <= max_tail_len; a decode row is a short
 * request with prefix_lens[b] = its position and extend_lens[b] = 1 (its new
 * K/V already stored at req_to_token[row_b][prefix_lens[b]]).  The result is
 * radix_extend_attention's over the whole batch; the grid sizes the extend
 * requests by max_extend_len and the short ones by max_tail_len, so many
 * decode rows beside a long chunk do not each pay for the chunk's length.
 * 0 <= num_extend <= batch (both host). */
int radix_mixed_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                          const int32_t* req_to_token, int32_t req_to_token_stride,
                          const int32_t* req_pool_indices, const int32_t* prefix_lens,
                          const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                          int32_t num_extend, int32_t max_extend_len, int32_t max_tail_len,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                          int dtype, void* stream);

/* Bytes of device workspace radix_decode_attention needs for these sizes
 * (split-K partial maxima, sums and accumulators, fp32).  Negative on bad
 * arguments. */
int64_t radix_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_kv_len);

/* Batched decode attention: one query row per request, at sequence position
 * prefix_lens[b] (its K/V already stored at req_to_token[row_b][prefix_lens[b]]):
 *   o[b][h] = softmax-weighted sum over keys 0 .. prefix_lens[b] of KV head
 *   h / (Hq / Hkv), gathered through req_to_token.
 * q, o: (device) [batch, num_q_heads, head_dim].  extend_lens (device) may
 * be NULL; if given every entry must be 1 (not checked on the device).
 * max_kv_len (host) >= every prefix_lens[b] + 1.  The context is split into
 * chunks processed in parallel and merged exactly by their (max, sum)
 * statistics.  workspace (device) of workspace_bytes >=
 * radix_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
 * max_kv_len). */
int radix_decode_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                           const int32_t* req_to_token, int32_t req_to_token_stride,
                           const int32_t* req_pool_indices, const int32_t* prefix_lens,
                           const int32_t* extend_lens, int32_t batch, int32_t max_kv_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           float sm_scale, int dtype, void* workspace, int64_t workspace_bytes,
                           void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * radix_decode_attention with the same arguments minus the workspace.  Its
 * split-K partials go to a device array the library owns, of
 * RT_NOALLOC_MAX_WORKSPACE_BYTES (32 MiB) per GPU, held until the process
 * ends; nothing is allocated or freed by the call.
 * Sizes whose radix_decode_workspace_bytes() exceeds that maximum are
 * refused with RT_ERR_INVALID before any launch.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (concurrent
 * streams, or host threads) race and must be ordered by the caller.  The
 * array's device address is looked up on a device's first call
 * (RT_ERR_HIP if that fails). */
#define RT_NOALLOC_MAX_WORKSPACE_BYTES ((int64_t)32 << 20)
int radix_decode_attention_noalloc(const void* q, void* o, const void* k_pool, const void* v_pool,
                                   const int32_t* req_to_token, int32_t req_to_token_stride,
                                   const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                   const int32_t* extend_lens, int32_t batch, int32_t max_kv_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                   int dtype, void* stream);

/* Decode for batches whose requests share cached prefixes.  The radix tree
 * hands requests that matched the same path the same slots for that path
 * [P2 section 04: requests that match a common prefix reference one copy of
 * its K/V]; this call reads such a shared part once per group instead of
 * once per request.  The result is radix_decode_attention's (same q, o,
 * pools, req_to_token, req_pool_indices, prefix_lens = positions), computed
 * in two passes whose split-K partials one combine merges exactly:
 *  - shared pass: for each group, the queries of all its members (x all
 *    heads of a KV head) against the group's shared keys, as MFMA tiles
 *    (the extend kernel, without a causal mask);
 *  - private pass: each request's keys shared_lens[b] .. prefix_lens[b]
 *    (the split-K decode).
 * Groups: requests group_start[g] .. group_start[g+1] - 1 (device, int32
 * [n_groups + 1]; group_start[0] = 0, increasing, group_start[n_groups] =
 * batch), so the groups are consecutive runs of the batch.  shared_lens
 * (device, int32 [batch]): every member of a group has the same value S_g,
 * and the members' req_to_token rows hold the same slots at 0 .. S_g - 1;
 * 0 <= S_g <= prefix_lens[b] + 1 (a group of one with S_g = 0 is a plain
 * decode row).  None of this is checked on the device.  Host bounds:
 * max_group_size >= every group's size, max_shared_len >= every S_g,
 * max_private_len >= every prefix_lens[b] + 1 - shared_lens[b] (>= 1);
 * req_to_token_stride >= max_shared_len + max_private_len.  bf16 q / o and
 * pools; at most 16 query heads per KV head.  workspace (device) of at least
 * radix_decode_shared_workspace_bytes(...) bytes.  Rounding differs from
 * radix_decode_attention's (other chunking and operand order); both are
 * fp32-accumulated. */
int64_t radix_decode_shared_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t n_groups, int32_t max_group_size,
                                            int32_t max_shared_len, int32_t max_private_len);
int radix_decode_attention_shared(const void* q, void* o, const void* k_pool, const void* v_pool,
                                  const int32_t* req_to_token, int32_t req_to_token_stride,
                                  const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                  const int32_t* shared_lens, const int32_t* group_start, int32_t batch,
                                  int32_t n_groups, int32_t max_group_size, int32_t max_shared_len,
                                  int32_t max_private_len, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float sm_scale, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/* FP8 K/V pool [P4 the v0.2 release was measured in FP8 as well as bf16;
 * the pool format is OCP 8-bit floating point E4M3: sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinity, S.1111.111 NaN, largest finite
 * 448].  Pools are uint8 [N+1, num_kv_heads, head_dim]; a stored code c
 * stands for E4M3(c) * scale, with one k_scale for the K pool and one
 * v_scale for the V pool (both > 0).
 *
 * kv_store_fp8: k_new, v_new (device) bf16 [n_tokens, num_kv_heads,
 * head_dim]; row t is written at slot out_cache_loc[t] as
 * E4M3(x * fl32(1 / scale)) with x * fl32(1 / scale) rounded in fp32, then
 * to the nearest E4M3 value with ties to the even mantissa; magnitudes of
 * 448 and above saturate to 448, NaN stays NaN.  Otherwise as kv_store. */
int kv_store_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                 const int32_t* out_cache_loc, int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                 float k_scale, float v_scale, void* stream);

/* decode_append for FP8 pools: req_to_token_scatter of (rows, positions,
 * slots) and kv_store_fp8 of (k_new, v_new) at slots, in one launch, with the
 * encoding and scales of kv_store_fp8.  k_new, v_new: (device) bf16 [n,
 * num_kv_heads, head_dim].  Repeated slots (padding to slot 0) race: each
 * 8-byte piece of such a slot ends up holding that piece of one of the rows
 * written to it. */
int decode_append_fp8(int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* rows,
                      const int32_t* positions, const int32_t* slots, int32_t n, void* k_pool, void* v_pool,
                      const void* k_new, const void* v_new, int32_t num_kv_heads, int32_t head_dim,
                      float k_scale, float v_scale, void* stream);

/* kv_store_extend into FP8 pools: the rows and slots of kv_store_extend, the
 * encoding and scales of kv_store_fp8.  k_new, v_new: (device) bf16. */
int kv_store_extend_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                        const int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* req_pool_indices,
                        const int32_t* prefix_lens, const int32_t* extend_lens, const int32_t* qo_indptr,
                        int32_t batch, int32_t max_extend_len, int32_t num_kv_heads, int32_t head_dim,
                        float k_scale, float v_scale, void* stream);

/* radix_extend_attention over FP8 pools: q, o bf16; keys and values read as
 * E4M3(code) * k_scale and E4M3(code) * v_scale.  Same arguments and checks
 * otherwise. */
int radix_extend_attention_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                 const int32_t* req_to_token, int32_t req_to_token_stride,
                                 const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                 const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                 int32_t max_extend_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float sm_scale, float k_scale, float v_scale, void* stream);

/* radix_decode_attention_shared over FP8 pools (q, o bf16; pools and scales
 * as in radix_decode_attention_fp8kv). */
int radix_decode_attention_shared_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                        const int32_t* req_to_token, int32_t req_to_token_stride,
                                        const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                        const int32_t* shared_lens, const int32_t* group_start, int32_t batch,
                                        int32_t n_groups, int32_t max_group_size, int32_t max_shared_len,
                                        int32_t max_private_len, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                        void* workspace, int64_t workspace_bytes, void* stream);

/* radix_mixed_attention over FP8 pools (q, o bf16; pools and scales as in
 * radix_extend_attention_fp8kv). */
int radix_mixed_attention_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                const int32_t* req_to_token, int32_t req_to_token_stride,
                                const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                int32_t num_extend, int32_t max_extend_len, int32_t max_tail_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                float k_scale, float v_scale, void* stream);

/* radix_decode_attention over FP8 pools: q, o bf16; keys and values read as
 * E4M3(code) * k_scale and E4M3(code) * v_scale.  Same arguments, workspace
 * (radix_decode_workspace_bytes) and checks otherwise. */
int radix_decode_attention_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                 const int32_t* req_to_token, int32_t req_to_token_stride,
                                 const int32_t* req_pool_indices, const int32_t* prefix_lens, int32_t batch,
                                 int32_t max_kv_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 float sm_scale, float k_scale, float v_scale, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Decode with the step's append folded in [P4 "CUDA Graph": a decode
 * forward receives out_cache_loc, the slot of each request's new token, and
 * writes that token's K/V there before attending over the context]: the
 * result of decode_append (bf16 pools) or decode_append_fp8 (FP8 pools, same
 * encoding and scales) of (rows = req_pool_indices or 0 .. batch - 1,
 * positions = prefix_lens, slots = new_slots, k_new, v_new) followed by the
 * named decode call on the same arguments, in the launches of the decode
 * call alone: the work item whose chunk holds key prefix_lens[b] writes the
 * new token's K/V row of its KV head at new_slots[b] and, once per request,
 * req_to_token[row_b][prefix_lens[b]] = new_slots[b], then reads that key
 * back; the key's slot comes from new_slots, so the table entry need not be
 * written beforehand.  Pools and req_to_token are written, hence not const.
 * k_new, v_new: (device) bf16 [batch, num_kv_heads, head_dim]; new_slots:
 * (device) int32 [batch], not read by any other request of the call; a slot
 * repeated by padded entries (slot 0) races as in decode_append and only
 * those entries' outputs are affected.  The _shared forms need the new token outside every shared run
 * (shared_lens[b] <= prefix_lens[b]; not checked on the device).  bf16 q / o;
 * other arguments, workspace and checks as in the decode call named. */
int radix_decode_attention_append(const void* q, void* o, void* k_pool, void* v_pool, int32_t* req_to_token,
                                  int32_t req_to_token_stride, const int32_t* req_pool_indices,
                                  const int32_t* prefix_lens, int32_t batch, int32_t max_kv_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, float sm_scale, const void* k_new,
                                  const void* v_new, const int32_t* new_slots, void* workspace,
                                  int64_t workspace_bytes, void* stream);
int radix_decode_attention_append_fp8kv(const void* q, void* o, void* k_pool, void* v_pool, int32_t* req_to_token,
                                        int32_t req_to_token_stride, const int32_t* req_pool_indices,
                                        const int32_t* prefix_lens, int32_t batch, int32_t max_kv_len,
                                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                        float k_scale, float v_scale, const void* k_new, const void* v_new,
                                        const int32_t* new_slots, void* workspace, int64_t workspace_bytes,
                                        void* stream);
int radix_decode_attention_shared_append(const void* q, void* o, void* k_pool, void* v_pool, int32_t* req_to_token,
                                         int32_t req_to_token_stride, const int32_t* req_pool_indices,
                                         const int32_t* prefix_lens, const int32_t* shared_lens,
                                         const int32_t* group_start, int32_t batch, int32_t n_groups,
                                         int32_t max_group_size, int32_t max_shared_len, int32_t max_private_len,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                         const void* k_new, const void* v_new, const int32_t* new_slots,
                                         void* workspace, int64_t workspace_bytes, void* stream);
int radix_decode_attention_shared_append_fp8kv(const void* q, void* o, void* k_pool, void* v_pool,
                                               int32_t* req_to_token, int32_t req_to_token_stride,
                                               const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                               const int32_t* shared_lens, const int32_t* group_start, int32_t batch,
                                               int32_t n_groups, int32_t max_group_size, int32_t max_shared_len,
                                               int32_t max_private_len, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                               const void* k_new, const void* v_new, const int32_t* new_slots,
                                               void* workspace, int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RADIXRT_H */
