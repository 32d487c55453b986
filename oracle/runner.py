"""Batch scheduler over the naive tree (oracle).

The request path follows the SGLang explainer, section 04 ("from request
arrival to cache reclamation" figure): waiting queue, tree match, admit
within memory while protecting the matched path, evict reclaimable leaves
when memory is short, run, then insert the new path.  The admission test
follows the v0.2 handbook chapter ("new_token_ratio and retract" section):
available = free slots + evictable tokens - sum over running requests of
their remaining new tokens times a ratio; the ratio is fixed at 1.0 here
because every request's output length is known in advance.

Readings where the pages are silent: first come first served by arrival
and request id, stop at the first request that does not fit; at most 256
running requests and 16384 extend tokens per iteration (the first admitted
request is exempt from the token cap); a request extended in iteration k
decodes from iteration k+1; a request is inserted into the tree only when
it finishes (prompt plus the tokens it fed), duplicate slots that the tree
already holds are freed, then the admission lock is released.

Policy "lspf" (longest shared prefix first; SGLang paper summary, section
3 "Cache-aware scheduling" and appendix A.3; SGLang explainer, section 04,
cache-aware scheduling): at each iteration every waiting request is matched
against the tree in arrival order (each match stamps the LRU clock and may
split an edge, as any match does), and admission walks the waiting requests
by matched length, longest first, ties in arrival order, still stopping at
the first that does not fit.

Chunked prefill (``chunk_size``; v0.2 handbook, the #800 entry of the
release timeline: long prompts are cut into chunks of a fixed size that run
beside decode, and admission changes with it).  Reading taken: each
iteration extends at most chunk_size prompt tokens, first the next chunks of
requests still being prefilled (in admission order), then the first chunks
of newly admitted requests; admission stops once the budget is spent or a
request does not fit.  A request's whole remaining prompt and output are
reserved at admission; its slots are allocated chunk by chunk.  It decodes
from the iteration after its last chunk.

Pages (``wl.page_size`` p; see ``radix_tree``): matches and inserts are
page-aligned, every position's slot follows the page rule, and a request's
need counts whole pages: a request holding x of its L = prompt + generated
positions still needs ceil(L / p) - ceil(x / p) pages, p slots each (at
admission x is its page-aligned matched length).  On finish only the
page-aligned part ceil-down(L / p) * p is inserted; the request's pages that
the tree already held and the page of its trailing partial page are freed.
At p = 1 all of this is the token-granular behaviour above.

Attention outputs come from ``recompute_rows`` (full recompute, float64).
"""

from dataclasses import dataclass, field

import numpy as np

from .attention import recompute_rows
from .radix_tree import NaivePool, NaiveRadixTree


@dataclass
class _Running:
    req: object
    prefix_len: int
    node: int
    slots: list       # slot of every position computed so far
    admit_iter: int   # the iteration that completed the prompt
    generated: int = 0
    n_chunks: int = 0


@dataclass
class OracleTrace:
    iterations: list = field(default_factory=list)
    cached_tokens: int = 0
    prefill_tokens: int = 0
    request_slots: dict = field(default_factory=dict)
    dumps: list = field(default_factory=list)
    outputs: dict = field(default_factory=dict)
    free_list: list = field(default_factory=list)


def run_workload(wl, num_slots=None, max_running=256, max_extend_tokens=16384,
                 attention=True, want=None, keep_dumps=False, max_iterations=100000, policy="fcfs",
                 chunk_size=None, kv_fp8_scales=None):
    """Drive workload ``wl`` through the naive tree.  ``want(kind, rid, step)``
    (kind 'ext' or 'dec') selects which attention outputs are recomputed;
    by default all of them when ``attention`` is true."""
    page = getattr(wl, "page_size", 1)
    pool = NaivePool(num_slots if num_slots is not None else wl.num_slots, page)
    tree = NaiveRadixTree(pool)

    def pages_left(total_len, held):
        """Slots still to be allocated for a request of total_len positions
        that holds held of them: whole pages."""
        return (-(-total_len // page) - (-(-held // page))) * page
    tr = OracleTrace()
    pending = list(wl.requests)
    finished = set()
    waiting, running, prefilling = [], [], []

    def arrive():
        nonlocal pending
        still = []
        for r in pending:
            if all(a in finished for a in r.after):
                waiting.append(r)
            else:
                still.append(r)
        pending = still

    def finish(run, it_rec):
        full = list(run.req.prompt) + list(run.req.gen)
        aligned = len(full) - len(full) % page
        present = tree.insert(full[:aligned], run.slots[:aligned])
        dups = run.slots[run.prefix_len:present] if present > run.prefix_len else []
        dups = list(dups) + list(run.slots[aligned:len(full)])  # and the trailing partial page
        pool.release(dups)
        tree.unlock(run.node)
        tr.request_slots[run.req.rid] = list(run.slots[:len(full)])
        it_rec["finished"].append((run.req.rid, present, list(dups)))
        finished.add(run.req.rid)

    def selected(kind, rid, step):
        if not attention:
            return False
        return True if want is None else want(kind, rid, step)

    arrive()
    it = 0
    while waiting or running or pending or prefilling:
        if it >= max_iterations:
            raise RuntimeError("workload did not drain")
        rec = {"admitted": [], "extend_loc": [], "extend_freed": [], "decode": [],
               "decode_freed": [], "finished": []}
        # 1. admission in policy order
        if policy == "fcfs":
            order = list(waiting)
        elif policy == "lspf":
            matched = [len(tree.match_prefix(r.prompt)[0]) for r in waiting]
            order = [waiting[i] for i in sorted(range(len(waiting)), key=lambda i: (-matched[i], i))]
        else:
            raise ValueError(f"unknown policy {policy!r}")
        if chunk_size is not None:
            _chunked_admit_and_extend(wl, tree, pool, tr, rec, it, order, waiting, running, prefilling,
                                      max_running, chunk_size, selected, finish, kv_fp8_scales)
        else:
            reserved = sum(pages_left(len(r.req.prompt) + len(r.req.gen), len(r.slots)) for r in running)
            budget = max_extend_tokens
            admitted = []
            for req in order:
                if len(running) + len(admitted) >= max_running:
                    break
                slots, node = tree.match_prefix(req.prompt)
                tree.lock(node)
                p = len(slots)
                e = len(req.prompt) - p
                need = pages_left(len(req.prompt) + len(req.gen), p)
                avail = pool.available() + tree.evictable_size() - reserved
                if need > avail or (admitted and e > budget):
                    tree.unlock(node)
                    break
                waiting.remove(req)
                admitted.append(_Running(req, p, node, list(slots), it))
                reserved += need
                budget -= e
            # 2. extend the admitted batch
            if admitted:
                runs = [(r.slots, r.prefix_len, len(r.req.prompt) - r.prefix_len) for r in admitted]
                loc, freed = tree.alloc_positions(runs)
                rec["extend_loc"], rec["extend_freed"] = list(loc), list(freed)
                off = 0
                for r in admitted:
                    e = len(r.req.prompt) - r.prefix_len
                    r.slots += loc[off:off + e]
                    off += e
                    rec["admitted"].append((r.req.rid, r.prefix_len, e))
                    tr.cached_tokens += r.prefix_len
                    tr.prefill_tokens += len(r.req.prompt)
                    if e > 0 and not wl.skip_extend_attention and selected("ext", r.req.rid, 0):
                        pos = np.arange(r.prefix_len, len(r.req.prompt))
                        tr.outputs[("ext", r.req.rid, 0)] = recompute_rows(
                            r.req.prompt, pos, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                            wl.seed, wl.sm_scale, kv_fp8_scales)
                for r in admitted:
                    if len(r.req.gen) == 0:
                        finish(r, rec)
                    else:
                        running.append(r)
        # 3. one decode step for requests admitted in earlier iterations
        dec = [r for r in running if r.admit_iter < it]
        if dec:
            loc, freed = tree.alloc_positions([(r.slots, len(r.slots), 1) for r in dec])
            rec["decode_freed"] = list(freed)
            for r, s in zip(dec, loc):
                pos = len(r.req.prompt) + r.generated
                r.slots.append(s)
                rec["decode"].append((r.req.rid, pos, s))
                if selected("dec", r.req.rid, r.generated):
                    seq = list(r.req.prompt) + list(r.req.gen[:r.generated + 1])
                    tr.outputs[("dec", r.req.rid, r.generated)] = recompute_rows(
                        seq, [pos], wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                        wl.seed, wl.sm_scale, kv_fp8_scales)
                r.generated += 1
            done = [r for r in dec if r.generated == len(r.req.gen)]
            for r in done:
                running.remove(r)
                finish(r, rec)
        tr.iterations.append(rec)
        if keep_dumps:
            tr.dumps.append(tree.dump())
        arrive()
        it += 1
    tr.free_list = list(pool.free)
    tr.final_dump = tree.dump()
    return tr


def _chunked_admit_and_extend(wl, tree, pool, tr, rec, it, order, waiting, running, prefilling,
                              max_running, chunk_size, selected, finish, kv_fp8_scales=None):
    """One iteration's admission and extend under chunked prefill."""
    page = tree.page_size
    pages_left = lambda total_len, held: (-(-total_len // page) - (-(-held // page))) * page
    budget = chunk_size
    plan = []  # (request, first position, token count), in launch order
    for r in prefilling:
        if budget <= 0:
            break
        cnt = min(len(r.req.prompt) - len(r.slots), budget)
        plan.append((r, len(r.slots), cnt))
        budget -= cnt
    reserved = sum(pages_left(len(r.req.prompt) + len(r.req.gen), len(r.slots)) for r in running + prefilling)
    admitted = []
    for req in order:
        if len(running) + len(prefilling) + len(admitted) >= max_running or budget <= 0:
            break
        slots, node = tree.match_prefix(req.prompt)
        tree.lock(node)
        p = len(slots)
        e = len(req.prompt) - p
        need = pages_left(len(req.prompt) + len(req.gen), p)
        if need > pool.available() + tree.evictable_size() - reserved:
            tree.unlock(node)
            break
        waiting.remove(req)
        run = _Running(req, p, node, list(slots), it)
        admitted.append(run)
        reserved += need
        rec["admitted"].append((req.rid, p, e))
        tr.cached_tokens += p
        tr.prefill_tokens += len(req.prompt)
        cnt = min(e, budget)
        if cnt > 0:
            plan.append((run, p, cnt))
            budget -= cnt
    loc, freed = tree.alloc_positions([(r.slots, first, cnt) for r, first, cnt in plan])
    rec["extend_loc"], rec["extend_freed"] = list(loc), list(freed)
    rec["chunks"] = [(r.req.rid, first, cnt) for r, first, cnt in plan]
    off = 0
    for r, first, cnt in plan:
        r.slots += loc[off:off + cnt]
        off += cnt
        if not wl.skip_extend_attention and selected("ext", r.req.rid, r.n_chunks):
            tr.outputs[("ext", r.req.rid, r.n_chunks)] = recompute_rows(
                r.req.prompt, np.arange(first, first + cnt), wl.num_q_heads, wl.num_kv_heads,
                wl.head_dim, wl.seed, wl.sm_scale, kv_fp8_scales)
        r.n_chunks += 1
    continuing = [r for r, _, _ in plan if all(r is not a for a in admitted)]
    for r in continuing + admitted:
        complete = len(r.slots) == len(r.req.prompt)
        is_new = any(r is a for a in admitted)
        if not complete:
            if is_new:
                prefilling.append(r)
            continue
        if not is_new:
            prefilling[:] = [x for x in prefilling if x is not r]
        r.admit_iter = it
        if len(r.req.gen) == 0:
            finish(r, rec)
        else:
            running.append(r)
