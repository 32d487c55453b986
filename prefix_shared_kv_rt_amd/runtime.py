"""Host driver of the RadixAttention hot path.

``RadixRuntime`` owns one tree + pool (C++, through the C ABI), the device
K/V pools, the request-to-slot table and the decode workspace, and runs the
device steps (scatter, extend attention, decode attention) on one stream.

``Scheduler`` drives a list of requests through it, batch by batch.  The
request path follows the SGLang explainer, section 04 (figure "from request
arrival to cache reclamation"): waiting queue, tree match, admission within
memory while the matched path is protected, eviction when memory is short,
execution, then insertion of the finished sequence.  Admission uses the v0.2
handbook's estimate (section "new_token_ratio and retract"): free slots +
evictable tokens - remaining new tokens of running requests, with the ratio
fixed at 1 since output lengths are known in advance.  Where the pages are
silent the policy is: first come first served, stop at the first request
that does not fit, at most ``max_running`` requests and
``max_extend_tokens`` extend tokens per iteration (the first admitted
request is exempt from the token cap), a request extended in iteration k
decodes from iteration k+1, and a request enters the tree only when it
finishes (its duplicate slots are freed, then its admission lock released).

``chunk_size=C`` is chunked prefill (v0.2 handbook, the #800 entry of the
release timeline: long prompts no longer take a whole step, they are cut
into chunks of a fixed size that run beside decode, and admission changes
with it).  Each iteration extends at most C prompt tokens: first the next
chunks of requests still being prefilled, in admission order, then the
first chunks of newly admitted requests; admission stops when the budget is
spent.  Admission reserves a request's whole remaining prompt and output,
and slots are allocated chunk by chunk.  A request decodes from the
iteration after its last chunk.

``policy="lspf"`` is the paper's cache-aware order (SGLang paper summary,
section 3 "Cache-aware scheduling", appendix A.3): each iteration matches
every waiting request against the tree in arrival order, then admits by
matched length, longest first, ties in arrival order.

Q/K/V of new tokens come from a caller-supplied ``qkv_source(rid, tokens,
positions)`` returning device tensors; the runtime itself computes no
attention values on the host.
"""

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B


class RadixRuntime:
    """device=None runs the host half only (tree, pool, slot table): the
    device steps are skipped and return None.  Used to check host decisions
    on machines without a GPU.  ``kv_fp8_scales=(k_scale, v_scale)`` keeps the
    K/V pools in FP8 (E4M3 codes, uint8) under bf16 queries and outputs."""

    def __init__(self, num_slots, num_q_heads, num_kv_heads, head_dim, dtype, max_reqs, max_ctx,
                 device="cuda", stream=None, kv_fp8_scales=None, page_size=1):
        self.num_slots = int(num_slots)
        self.page_size = int(page_size)
        self.hq, self.hkv, self.d = int(num_q_heads), int(num_kv_heads), int(head_dim)
        self.dtype = dtype
        if kv_fp8_scales is not None and dtype not in (None, torch.bfloat16):
            raise ValueError("FP8 pools run under bf16 queries")
        self.kv_fp8_scales = None if kv_fp8_scales is None else (float(kv_fp8_scales[0]), float(kv_fp8_scales[1]))
        self.max_reqs, self.max_ctx = int(max_reqs), int(max_ctx)
        self.pool = B.rt_pool_create(self.num_slots, self.page_size)
        self.tree = B.rt_tree_create(self.pool)
        self.free_rows = list(range(self.max_reqs))
        self.sm_scale = 1.0 / float(np.sqrt(self.d))
        self.device = None if device is None else torch.device(device)
        if self.device is None:
            self.stream = None
            self.r2t_host = np.zeros((self.max_reqs, self.max_ctx), dtype=np.int32)
            return
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        # Slot 0 stays zero: padded writes land there and it is never read as data.
        pool_dtype = torch.uint8 if self.kv_fp8_scales else dtype
        self.k_pool = torch.zeros((self.num_slots + 1, self.hkv, self.d), dtype=pool_dtype, device=self.device)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.r2t_host_t = torch.zeros((self.max_reqs, self.max_ctx), dtype=torch.int32, pin_memory=True)
        self.r2t_host = self.r2t_host_t.numpy()
        self.r2t_dev = torch.zeros((self.max_reqs, self.max_ctx), dtype=torch.int32, device=self.device)
        self._ws = torch.empty(0, dtype=torch.uint8, device=self.device)
        # When a list, every device step appends (kind, start event, end event,
        # info) for the kernels it launches; kind is 'kv_store', 'extend',
        # 'decode' (the attention launch alone; the step's slot-table and K/V
        # append runs just before it) or 'mixed'.
        self.events = None

    def _event(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def close(self):
        if self.tree is not None:
            B.rt_tree_destroy(self.tree)
            B.rt_pool_destroy(self.pool)
            self.tree = self.pool = None

    # ----------------------------------------------------------- helpers --
    def _to_dev(self, arr, dtype=torch.int32):
        t = torch.from_numpy(np.ascontiguousarray(arr)).to(dtype)
        return t.pin_memory().to(self.device, non_blocking=True)

    def workspace(self, batch, max_kv_len):
        need = B.radix_decode_workspace_bytes(batch, self.hq, self.hkv, self.d, max_kv_len)
        if self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def _store(self, k_new, v_new, loc):
        """Write new K/V rows at pool slots, in the pool's format."""
        if self.kv_fp8_scales:
            B.kv_store_fp8(self.k_pool, self.v_pool, k_new, v_new, loc, *self.kv_fp8_scales, stream=self.stream)
        else:
            B.kv_store(self.k_pool, self.v_pool, k_new, v_new, loc, stream=self.stream)

    def upload_rows(self, rows, lens):
        """Copy the first lens[i] entries of host rows rows[i] to the device table."""
        if self.device is None:
            return
        with torch.cuda.stream(self.stream):
            for r, n in zip(rows, lens):
                if n > 0:
                    self.r2t_dev[r, :n].copy_(self.r2t_host_t[r, :n], non_blocking=True)

    # ------------------------------------------------------ device steps --
    def run_extend(self, rows, prefix_lens, extend_lens, q, k_new, v_new, out_cache_loc, attention=True):
        """kv_store of the new rows, then extend attention.  Returns o (or None)."""
        if self.device is None:
            return None
        n = len(rows)
        with torch.cuda.stream(self.stream):
            loc = self._to_dev(out_cache_loc)
            if loc.numel() > 0:
                e0 = self._event() if self.events is not None else None
                self._store(k_new, v_new, loc)
                if e0 is not None:
                    self.events.append(("kv_store", e0, self._event(), {"rows": int(loc.numel())}))
            if not attention or loc.numel() == 0:
                return None
            qo = np.zeros(n + 1, dtype=np.int32)
            qo[1:] = np.cumsum(extend_lens)
            o = torch.empty_like(q)
            args = (self._to_dev(rows), self._to_dev(prefix_lens), self._to_dev(extend_lens), self._to_dev(qo))
            e0 = self._event() if self.events is not None else None
            if self.kv_fp8_scales:
                B.radix_extend_attention_fp8kv(q, o, self.k_pool, self.v_pool, self.r2t_dev, *args,
                                               int(max(extend_lens)), self.sm_scale, *self.kv_fp8_scales,
                                               stream=self.stream)
            else:
                B.radix_extend_attention(q, o, self.k_pool, self.v_pool, self.r2t_dev, *args,
                                         int(max(extend_lens)), self.sm_scale, stream=self.stream)
            if e0 is not None:
                pl = np.asarray(prefix_lens, dtype=np.float64)
                el = np.asarray(extend_lens, dtype=np.float64)
                flops = 4.0 * self.d * self.hq * float(np.sum(el * pl + el * (el + 1) / 2))
                self.events.append(("extend", e0, self._event(), {"tokens": int(el.sum()), "flops": flops}))
            return o

    def run_decode(self, rows, positions, slots, q, k_new, v_new, shared_len=0):
        """Write the new slots into the table, store the new rows, decode.
        bf16 and FP8 pools do all three in the decode's own launches (the
        _append decode calls); fp32 pools run decode_append first.
        shared_len > 0: every row's first shared_len slots are the same (the
        caller checked), so the batch decodes as one group through
        radix_decode_attention_shared, reading those K/V once."""
        if self.device is None:
            return None
        n = len(rows)
        with torch.cuda.stream(self.stream):
            rows_d, pos_d, slots_d = self._to_dev(rows), self._to_dev(positions), self._to_dev(slots)
            o = torch.empty_like(q)
            max_kv = int(max(positions)) + 1
            fused = self.kv_fp8_scales is not None or self.dtype == torch.bfloat16
            sc = tuple(self.kv_fp8_scales or ())
            if not fused:
                B.decode_append(self.r2t_dev, rows_d, pos_d, slots_d, self.k_pool, self.v_pool, k_new, v_new,
                                stream=self.stream)
            if shared_len > 0:
                sl = self._to_dev(np.full(n, shared_len, dtype=np.int32))
                gs = self._to_dev(np.array([0, n], dtype=np.int32))
                priv = max_kv - shared_len
                need = B.radix_decode_shared_workspace_bytes(n, self.hq, self.hkv, self.d, 1, n, shared_len, priv)
                if self._ws.numel() < need:
                    self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
                # the timing events bracket the decode launches alone (their
                # inputs and workspace are ready before the first event)
                e0 = self._event() if self.events is not None else None
                args = (q, o, self.k_pool, self.v_pool, self.r2t_dev, rows_d, pos_d, sl, gs, n, shared_len, priv,
                        self.sm_scale)
                if self.kv_fp8_scales:
                    B.radix_decode_attention_shared_append_fp8kv(*args, k_new, v_new, slots_d, self._ws, *sc,
                                                                 stream=self.stream)
                elif fused:
                    B.radix_decode_attention_shared_append(*args, k_new, v_new, slots_d, self._ws,
                                                           stream=self.stream)
                else:
                    B.radix_decode_attention_shared(*args, self._ws, stream=self.stream)
            else:
                ws = self.workspace(n, max_kv)
                e0 = self._event() if self.events is not None else None
                args = (q, o, self.k_pool, self.v_pool, self.r2t_dev, rows_d, pos_d, max_kv, self.sm_scale)
                if self.kv_fp8_scales:
                    B.radix_decode_attention_append_fp8kv(*args, k_new, v_new, slots_d, ws, *sc, stream=self.stream)
                elif fused:
                    B.radix_decode_attention_append(*args, k_new, v_new, slots_d, ws, stream=self.stream)
                else:
                    B.radix_decode_attention(*args, ws, stream=self.stream)
            if e0 is not None:
                kv = np.asarray(positions, dtype=np.float64) + 1
                eb, ekv = q.element_size(), self.k_pool.element_size()
                row = 2 * self.hkv * self.d * ekv + 4
                nbytes = float(np.sum(kv * row)) + 2.0 * n * self.hq * self.d * eb
                distinct = nbytes - float(max(n - 1, 0) * shared_len * row)
                self.events.append(("decode", e0, self._event(), {"tokens": n, "bytes": nbytes,
                                                                   "distinct_bytes": distinct}))
            return o

    def run_mixed(self, ext_rows, prefix_lens, extend_lens, q, k_new, v_new, out_cache_loc, dec_rows, positions,
                  slots, qd, kd, vd):
        """An iteration with extend chunks and decode rows as one attention
        launch: store the chunks' K/V, append the decode rows' slots and K/V,
        then radix_mixed_attention over the extend requests followed by the
        decode rows (prefix = position, one row each).  Returns (extend o,
        decode o)."""
        if self.device is None:
            return None, None
        n_e, n_d = len(ext_rows), len(dec_rows)
        with torch.cuda.stream(self.stream):
            loc = self._to_dev(out_cache_loc)
            e0 = self._event() if self.events is not None else None
            self._store(k_new, v_new, loc)
            if e0 is not None:
                self.events.append(("kv_store", e0, self._event(), {"rows": int(loc.numel())}))
            rows_all = np.concatenate([np.asarray(ext_rows, np.int32), np.asarray(dec_rows, np.int32)])
            pl_all = np.concatenate([np.asarray(prefix_lens, np.int32), np.asarray(positions, np.int32)])
            el_all = np.concatenate([np.asarray(extend_lens, np.int32), np.ones(n_d, np.int32)])
            qo = np.zeros(n_e + n_d + 1, dtype=np.int32)
            qo[1:] = np.cumsum(el_all)
            n = n_e + n_d
            meta = self._to_dev(np.concatenate([rows_all, pl_all, el_all, qo, np.asarray(slots, np.int32)]))
            d_rows, d_pl, d_el = meta[:n], meta[n:2 * n], meta[2 * n:3 * n]
            d_qo, d_slots = meta[3 * n:4 * n + 1], meta[4 * n + 1:]
            d_drows, d_pos = d_rows[n_e:], d_pl[n_e:]   # a decode row's prefix length is its position
            qall = torch.cat([q, qd])
            o = torch.empty_like(qall)
            e0 = self._event() if self.events is not None else None
            if self.kv_fp8_scales:
                B.decode_append_fp8(self.r2t_dev, d_drows, d_pos, d_slots, self.k_pool, self.v_pool, kd, vd,
                                    *self.kv_fp8_scales, stream=self.stream)
                B.radix_mixed_attention_fp8kv(qall, o, self.k_pool, self.v_pool, self.r2t_dev, d_rows, d_pl, d_el,
                                              d_qo, n_e, int(max(extend_lens)), 1, self.sm_scale,
                                              *self.kv_fp8_scales, stream=self.stream)
            else:
                B.decode_append(self.r2t_dev, d_drows, d_pos, d_slots, self.k_pool, self.v_pool, kd, vd,
                                stream=self.stream)
                B.radix_mixed_attention(qall, o, self.k_pool, self.v_pool, self.r2t_dev, d_rows, d_pl, d_el, d_qo,
                                        n_e, int(max(extend_lens)), 1, self.sm_scale, stream=self.stream)
            if e0 is not None:
                pl = np.asarray(prefix_lens, dtype=np.float64)
                el = np.asarray(extend_lens, dtype=np.float64)
                kv = np.asarray(positions, dtype=np.float64) + 1
                flops = 4.0 * self.d * self.hq * float(np.sum(el * pl + el * (el + 1) / 2) + np.sum(kv))
                self.events.append(("mixed", e0, self._event(), {"tokens": int(el.sum()) + n_d,
                                                                  "ext_tokens": int(el.sum()), "dec_tokens": n_d,
                                                                  "flops": flops}))
            t_e = int(np.sum(extend_lens))
            return o[:t_e], o[t_e:]

@dataclass
class _Run:
    req: object
    row: int
    prefix_len: int
    node: int
    admit_iter: int  # iteration whose extend completed the prompt (decode starts after it)
    generated: int = 0
    done: int = 0    # prompt tokens whose K/V are in the pool
    chunks: int = 0  # extend chunks run so far


class Scheduler:
    """Drives requests (objects with rid, prompt, gen, after) through a
    RadixRuntime.  ``record(kind, rid, step, o)`` receives every attention
    output (kind 'ext' or 'dec'); ``trace`` collects the host decisions."""

    def __init__(self, rt, requests, qkv_source, max_running=256, max_extend_tokens=16384,
                 skip_extend_attention=False, record=None, keep_dumps=False, policy="fcfs", graphs=None,
                 chunk_size=None, mixed=False, shared_decode=False, shared_min=256):
        if rt.max_reqs < max_running:
            raise ValueError("the slot table needs a row per running request")
        if policy not in ("fcfs", "lspf"):
            raise ValueError(f"unknown policy {policy!r}")
        self.policy = policy
        if chunk_size is not None and chunk_size < 1:
            raise ValueError("chunk_size must be positive")
        self.chunk_size = chunk_size
        self.prefilling = []  # admitted requests with prompt tokens still to extend
        self.graphs = graphs  # a DecodeGraphs: decode steps replay captured graphs when the batch fits
        # mixed: an iteration's extend chunks and decode rows share one
        # attention launch (radix_mixed_attention) unless a request finishes
        # right after its extend: its freed slots could be handed to this
        # iteration's decode rows and overwritten before the launch reads them.
        self.mixed = bool(mixed)
        self.mixed_launches = 0
        # shared_decode: a decode batch whose slot rows all begin with the same
        # shared_min or more slots (requests that matched a common cached
        # prefix) reads that common part once (radix_decode_attention_shared).
        self.shared_decode = bool(shared_decode)
        self.shared_min = int(shared_min)
        self.shared_decodes = 0
        self.rt = rt
        self.pending = list(requests)
        self.qkv = qkv_source
        self.max_running = max_running
        self.max_extend_tokens = max_extend_tokens
        self.skip_extend_attention = skip_extend_attention
        self.record = record
        self.keep_dumps = keep_dumps
        self.finished = set()
        self.waiting, self.running = [], []
        self.cached_tokens = self.prefill_tokens = 0
        self.iterations, self.dumps = [], []
        self.request_slots = {}

    def _arrive(self):
        still = []
        for r in self.pending:
            if all(a in self.finished for a in r.after):
                self.waiting.append(r)
            else:
                still.append(r)
        self.pending = still

    def _pages_left(self, total_len, held):
        """Slots a request of total_len positions holding held of them still
        needs: whole pages."""
        p = self.rt.page_size
        return (-(-total_len // p) - (-(-held // p))) * p

    def _finish(self, run, rec):
        rt = self.rt
        full = list(run.req.prompt) + list(run.req.gen)
        row = rt.r2t_host[run.row, :len(full)].copy()
        # whole pages into the tree; the tree's duplicates and the trailing
        # partial page back to the pool
        aligned = len(full) - len(full) % rt.page_size
        present = B.rt_insert(rt.tree, full[:aligned], row[:aligned])
        dups = row[run.prefix_len:present] if present > run.prefix_len else row[:0]
        dups = np.concatenate([dups, row[aligned:]])
        if dups.size:
            B.rt_pool_free(rt.pool, dups)
        B.rt_unlock(rt.tree, run.node)
        self.request_slots[run.req.rid] = [int(x) for x in row]
        rec["finished"].append((run.req.rid, present, [int(x) for x in dups]))
        self.finished.add(run.req.rid)
        rt.free_rows.append(run.row)

    def step(self, it):
        rt = self.rt
        rec = {"admitted": [], "extend_loc": [], "extend_freed": [], "decode": [], "decode_freed": [],
               "finished": []}
        chunked = self.chunk_size is not None
        reserved = sum(self._pages_left(len(r.req.prompt) + len(r.req.gen), len(r.req.prompt) + r.generated)
                       for r in self.running)
        reserved += sum(self._pages_left(len(r.req.prompt) + len(r.req.gen), r.done) for r in self.prefilling)
        budget = self.chunk_size if chunked else self.max_extend_tokens
        chunks = []  # (run, first token, tokens) of this iteration's extend, in launch order
        for r in self.prefilling:
            if budget <= 0:
                break
            n = min(len(r.req.prompt) - r.done, budget)
            chunks.append((r, r.done, n))
            budget -= n
        admitted = []
        order = self.waiting
        if self.policy == "lspf" and self.waiting:
            lens = [B.rt_match_prefix(rt.tree, r.prompt)[0].size for r in self.waiting]
            order = [self.waiting[i] for i in np.lexsort((np.arange(len(lens)), -np.asarray(lens)))]
        for req in list(order):
            if len(self.running) + len(self.prefilling) + len(admitted) >= self.max_running:
                break
            if chunked and budget <= 0:
                break
            slots, node = B.rt_match_prefix(rt.tree, req.prompt)
            B.rt_lock(rt.tree, node)
            p = len(slots)
            e = len(req.prompt) - p
            need = self._pages_left(len(req.prompt) + len(req.gen), p)
            avail = B.rt_pool_available(rt.pool) + B.rt_evictable_size(rt.tree) - reserved
            if need > avail or (not chunked and admitted and e > budget):
                B.rt_unlock(rt.tree, node)
                break
            self.waiting.remove(req)
            row = rt.free_rows.pop(0)
            rt.r2t_host[row, :p] = slots
            run = _Run(req, row, p, node, it, done=p)
            admitted.append(run)
            reserved += need
            n = min(e, budget) if chunked else e
            if n > 0:
                chunks.append((run, p, n))
            budget -= n
            rec["admitted"].append((req.rid, p, e))
            self.cached_tokens += p
            self.prefill_tokens += len(req.prompt)

        total = sum(n for _, _, n in chunks)
        if total > 0:
            # slots by the page rule, written into the host rows as well
            loc, evicted = B.rt_alloc_positions(rt.tree, [r.row for r, _, _ in chunks],
                                                [start for _, start, _ in chunks], [n for _, _, n in chunks],
                                                rt.r2t_host)
            rec["extend_loc"] = [int(x) for x in loc]
            rec["extend_freed_tokens"] = evicted
        else:
            loc = np.zeros(0, dtype=np.int32)
        if chunked:
            rec["chunks"] = [(r.req.rid, start, n) for r, start, n in chunks]
        off = 0
        for r, start, n in chunks:
            rt.r2t_host[r.row, start:start + n] = loc[off:off + n]
            off += n
            r.done = start + n
        # device rows: the computed prefix of every request touched this iteration
        touched = list({id(r): r for r in [c[0] for c in chunks] + admitted}.values())
        rt.upload_rows([r.row for r in touched], [r.done for r in touched])
        ext = None  # this iteration's extend launch, deferred when it may join the decode rows
        if total > 0 and rt.device is not None:
            qs, ks, vs = [], [], []
            for r, start, n in chunks:
                q, k, v = self.qkv(r.req.rid, r.req.prompt, np.arange(start, start + n))
                qs.append(q)
                ks.append(k)
                vs.append(v)
            ext = ([r.row for r, _, _ in chunks], [start for _, start, _ in chunks], [n for _, _, n in chunks],
                   torch.cat(qs), torch.cat(ks), torch.cat(vs), loc, [(r.req.rid, r.chunks, n) for r, _, n in chunks])
        for r, _, _ in chunks:
            r.chunks += 1
        new_ids = {id(r) for r in admitted}
        completing = [r for r in [c[0] for c in chunks if id(c[0]) not in new_ids] + admitted
                      if r.done == len(r.req.prompt)]
        if ext is not None and not (self.mixed and not self.skip_extend_attention and
                                    all(len(r.req.gen) > 0 for r in completing)):
            self._launch_extend(ext)
            ext = None
        for r in [c[0] for c in chunks if id(c[0]) not in new_ids] + admitted:
            if r.done < len(r.req.prompt):
                if id(r) in new_ids:
                    self.prefilling.append(r)
                continue
            if id(r) not in new_ids:
                self.prefilling = [x for x in self.prefilling if x is not r]
            r.admit_iter = it
            if len(r.req.gen) == 0:
                self._finish(r, rec)
            else:
                self.running.append(r)

        dec = [r for r in self.running if r.admit_iter < it]
        if dec:
            positions = np.array([len(r.req.prompt) + r.generated for r in dec], dtype=np.int32)
            rows = np.array([r.row for r in dec], dtype=np.int32)
            slots, evicted = B.rt_alloc_positions(rt.tree, rows, positions, np.ones(len(dec), np.int32), rt.r2t_host)
            rec["decode_freed_tokens"] = evicted
            for r, s, pos in zip(dec, slots, positions):
                rec["decode"].append((r.req.rid, int(pos), int(s)))
            o = None
            if rt.device is not None:
                qs, ks, vs = [], [], []
                for r, pos in zip(dec, positions):
                    seq = list(r.req.prompt) + list(r.req.gen[:r.generated + 1])
                    q, k, v = self.qkv(r.req.rid, seq, np.array([pos]))
                    qs.append(q)
                    ks.append(k)
                    vs.append(v)
                q, k, v = torch.cat(qs), torch.cat(ks), torch.cat(vs)
                if ext is not None:
                    rows_e, starts, ns, qe, ke, ve, loc_e, tags = ext
                    o_e, o = rt.run_mixed(rows_e, starts, ns, qe, ke, ve, loc_e, rows, positions, slots, q, k, v)
                    self._record_extend(o_e, tags)
                    self.mixed_launches += 1
                    ext = None
                else:
                    shared = self._common_slots(rows, positions) if self.shared_decode else 0
                    if shared >= self.shared_min:
                        o = rt.run_decode(rows, positions, slots, q, k, v, shared_len=shared)
                        self.shared_decodes += 1
                    else:
                        o = self.graphs.run(rows, positions, slots, q, k, v) if self.graphs is not None else None
                        if o is None:
                            o = rt.run_decode(rows, positions, slots, q, k, v)
            if o is not None and self.record is not None:
                for i, r in enumerate(dec):
                    self.record("dec", r.req.rid, r.generated, o[i:i + 1])
            for r in dec:
                r.generated += 1
            done = [r for r in dec if r.generated == len(r.req.gen)]
            for r in done:
                self.running.remove(r)
                self._finish(r, rec)
        if ext is not None:  # no decode rows this iteration
            self._launch_extend(ext)
        # Host rows and pinned staging are reused by later iterations.
        if rt.stream is not None:
            rt.stream.synchronize()
        self.iterations.append(rec)
        if self.keep_dumps:
            self.dumps.append(B.rt_tree_dump(rt.tree))

    def _common_slots(self, rows, positions):
        """Length of the common leading run of the decode rows' slots (the
        K/V every request of the batch reads), at most the shortest context
        before the new tokens."""
        if len(rows) < 2:
            return 0
        L = int(np.min(positions))
        if L <= 0:
            return 0
        m = self.rt.r2t_host[np.asarray(rows), :L]
        eq = (m == m[0]).all(axis=0)
        return L if bool(eq.all()) else int(np.argmin(eq))

    def _launch_extend(self, ext):
        rows, starts, ns, q, k, v, loc, tags = ext
        o = self.rt.run_extend(rows, starts, ns, q, k, v, loc, attention=not self.skip_extend_attention)
        self._record_extend(o, tags)

    def _record_extend(self, o, tags):
        if o is None or self.record is None:
            return
        off = 0
        for rid, chunk, n in tags:
            self.record("ext", rid, chunk, o[off:off + n])
            off += n

    def run(self, max_iterations=100000):
        self._arrive()
        it = 0
        while self.waiting or self.running or self.pending or self.prefilling:
            if it >= max_iterations:
                raise RuntimeError("workload did not drain")
            self.step(it)
            self._arrive()
            it += 1
        return self
