"""Benchmark of the RadixAttention hot path on one MI355X.

Default workload (few-shot shared prefix at the Llama-3-8B attention shape:
32 query heads, 8 KV heads, head dim 128, bf16): a warm-up request puts a
1024-token prefix into the radix tree; then every step serves one batch of
64 fresh requests = that prefix + 128 distinct suffix tokens, through the
whole path:

  host   rt_admit_batch     match each request, lock its path, allocate the
                            suffix slots (evicting LRU leaves on a deficit),
                            fill its req_to_token row
  device kv_store_extend    scatter the suffix K/V into the pool at the slots
                            the req_to_token rows hold
  device extend attention   suffix rows against prefix + suffix K/V
  host   rt_decode_slots    one slot per request for its first generated token
  device decode attention   radix_decode_attention_shared_append: the new
                            token's req_to_token entry and K/V row are
                            written by the decode's own launches; the batch
                            is one group sharing the prefix's slots, read
                            once for all 64 queries; each request's own tail
                            split-K (--decode plain: split-K over whole
                            contexts, radix_decode_attention_append)
  host   rt_finish_batch    insert prompt + token, free duplicates, unlock

Q/K/V of every step are generated into HBM before the timed region.  After
the warm-up steps, about 200 ms of replays of the last warm-up step's
launches (same rows, same values) let the GPU's clocks settle at their
level under the step's own load before the timed steps (the first few dozen
steps otherwise run 10-20 % slower).  Suffix token ids are drawn
over the Llama-3 vocabulary with first tokens distinct over the whole run,
so no suffix matches an earlier one: every step extends 64 x 128 rows.

Output: one JSON line (metric, value = extend + decode tokens per second of
whole steps, roofline of the extend kernel from HIP events on its stream,
ceilings measured on the box, CPU oracle baseline on a bounded sample, also
on one thread).  ``--workload long_context`` or ``fork`` time decode steps
instead, ``chat`` the multi-turn workload through the scheduler (extra
lines, not the headline); decode rooflines count distinct bytes.
"""

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "extend+decode attention tokens/s at Llama-3-8B shape; % HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def profiled_traffic(unit):
    """HBM bytes per call of `unit` (one kernel, or the kernels of one
    library call summed) from the committed rocprofv3 counter runs
    (profiles/traffic.json), or None once any of its source files has
    changed since those counters were taken."""
    import hashlib
    try:
        data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        ent = data[unit]
        for path, want in zip(ent["sources"], ent["source_sha256s"]):
            if hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest() != want:
                return None
        return (ent["fetch_kib"] * data["fetch_factor"] + ent["write_kib"] * data["write_factor"]) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--time-every", type=int, default=1,
                    help="few_shot: HIP timing events around the extend launch of every K-th timed step")
    ap.add_argument("--workload", default="few_shot", choices=["few_shot", "long_context", "fork", "chat", "decode_graph"])
    ap.add_argument("--policy", default="fcfs", choices=["fcfs", "lspf"],
                    help="admission order of the chat workload's scheduler")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="K/V pool format (fp8 = OCP E4M3 codes, scales 1)")
    ap.add_argument("--chunk-size", type=int, default=None,
                    help="chunked prefill for the chat workload: extend tokens per scheduler iteration")
    ap.add_argument("--decode", choices=["plain", "shared"], default=None,
                    help="decode path of few_shot, long_context and fork: plain = radix_decode_attention (split-K "
                         "over each request's whole context), shared = radix_decode_attention_shared (K/V that a "
                         "group of requests shares read once per group); default shared")
    ap.add_argument("--mixed", action="store_true",
                    help="chat workload: an iteration's extend chunks and decode rows share one attention launch")
    ap.add_argument("--page-size", type=int, default=1,
                    help="KV slots per pool page (few_shot and chat); 1 = token-granular")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=192, help="few_shot: requests in the oracle's timed sample")
    return ap.parse_args()


# --------------------------------------------------------------- few-shot --
class FewShotBench:
    B, PREFIX, SUFFIX = 64, 1024, 128
    HQ, HKV, D = 32, 8, 128
    SLOTS = 262144
    SEED = 1
    VOCAB = 128256   # Llama-3 tokenizer

    def __init__(self, n_batches, torch, B_mod, gen_t, kv_dtype="bf16", page_size=1, shared_decode=False):
        self.fp8 = kv_dtype == "fp8"
        self.shared_decode = shared_decode
        self.page_size = int(page_size)
        self.torch = torch
        self.Bm = B_mod
        self.gen_t = gen_t
        self.dev = torch.device("cuda:0")
        # One stream for the whole step: the stream current at construction,
        # so that torch's row copy (on the current stream) and the library's
        # launches (on self.stream) stay in order without a per-step stream
        # switch.  (A separate copy stream that overlaps the copy with the
        # previous step's kernels measured no faster.)
        self.stream = torch.cuda.current_stream(self.dev)
        rng = np.random.Generator(np.random.PCG64(self.SEED))
        self.prefix = rng.integers(0, 1000, size=self.PREFIX).astype(np.int32)
        # every batch: 64 suffixes of 128 tokens + 1 generated token each,
        # ids over the Llama-3 vocabulary; the suffixes' first tokens are
        # pairwise distinct over the whole run, so no suffix matches an
        # earlier one and every request extends exactly SUFFIX rows
        firsts = rng.choice(self.VOCAB, size=n_batches * self.B, replace=False).astype(np.int32)
        self.suffix = []
        for i in range(n_batches):
            sfx = rng.integers(0, self.VOCAB, size=(self.B, self.SUFFIX + 1)).astype(np.int32)
            sfx[:, 0] = firsts[i * self.B:(i + 1) * self.B]
            self.suffix.append(sfx)
        self.stride = self.PREFIX + self.SUFFIX + 1
        bf16 = torch.bfloat16
        self.pool = B_mod.rt_pool_create(self.SLOTS, self.page_size)
        self.tree = B_mod.rt_tree_create(self.pool)
        pool_dt = torch.uint8 if self.fp8 else bf16
        self.k_pool = torch.zeros((self.SLOTS + 1, self.HKV, self.D), dtype=pool_dt, device=self.dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        # two row sets of 64 so that host writes for step i+1 never touch rows still being copied for step i
        # Per row set: B slot-table rows, then 5 rows whose columns from
        # PREFIX on carry the step's metadata (prefix_lens, extend_lens,
        # qo_indptr, rows, decode slots), so that one copy of the columns
        # from PREFIX on moves a step's changes (below).
        P0, B = self.PREFIX, self.B
        assert self.stride - P0 >= B + 1
        self.set_rows = B + 5
        while (self.set_rows * self.stride) % 4:   # each row set starts 16-byte aligned
            self.set_rows += 1
        self.r2t_host_t = torch.zeros((2 * self.set_rows, self.stride), dtype=torch.int32, pin_memory=True)
        self.r2t_host = self.r2t_host_t.numpy()
        self.r2t_dev = torch.zeros((2 * self.set_rows, self.stride), dtype=torch.int32, device=self.dev)
        lens = (B, B, B + 1, B, B)
        meta = lambda t, rs: tuple(t[rs * self.set_rows + B + k, P0:P0 + n] for k, n in enumerate(lens))
        # host and device views of each row set's metadata: prefix_lens,
        # extend_lens, qo_indptr, rows, decode slots
        self.meta_host = [meta(self.r2t_host, rs) for rs in range(2)]
        self.meta_views = [meta(self.r2t_dev, rs) for rs in range(2)]
        self.copy_done = [torch.cuda.Event(), torch.cuda.Event()]
        # (device, pinned host) views of each row set, whole and from column
        # PREFIX on, for the per-step copy
        sets = [slice(rs * self.set_rows, (rs + 1) * self.set_rows) for rs in range(2)]
        self.copy_views = [(self.r2t_dev[sl], self.r2t_host_t[sl], self.r2t_dev[sl, P0:], self.r2t_host_t[sl, P0:])
                           for sl in sets]
        self.rows_whole = [False, False]   # row set uploaded whole since its prefix columns last changed
        self.prefix_slots = None           # the shared prefix's slots as last uploaded
        self.copy_mark = [None, None]   # event whose completion frees each row set's staging
        self.rows = [np.arange(rs * self.set_rows, rs * self.set_rows + self.B, dtype=np.int32) for rs in range(2)]
        self.dec_pos = np.full(self.B, self.PREFIX + self.SUFFIX, dtype=np.int32)
        self.ws = torch.empty(B_mod.radix_decode_workspace_bytes(self.B, self.HQ, self.HKV, self.D, self.stride),
                              dtype=torch.uint8, device=self.dev)
        # Shared decode: the batch is one group; every request holds the
        # cached prefix's slots at positions 0 .. PREFIX-1 (each step checks
        # that the prefix is still matched), and its own slots after them.
        self.sl_dev = torch.full((self.B,), self.PREFIX, dtype=torch.int32, device=self.dev)
        self.gs_dev = torch.tensor([0, self.B], dtype=torch.int32, device=self.dev)
        self.ws_shared = torch.empty(B_mod.radix_decode_shared_workspace_bytes(
            self.B, self.HQ, self.HKV, self.D, 1, self.B, self.PREFIX, self.SUFFIX + 1), dtype=torch.uint8,
            device=self.dev)
        self.o_ext = torch.empty((self.B * self.SUFFIX, self.HQ, self.D), dtype=bf16, device=self.dev)
        self.o_dec = torch.empty((self.B, self.HQ, self.D), dtype=bf16, device=self.dev)
        self.sm_scale = 1.0 / np.sqrt(self.D)
        self.pos_dev = torch.full((self.B,), self.PREFIX + self.SUFFIX, dtype=torch.int32, device=self.dev)
        self.row_base = np.arange(self.B, dtype=np.int32) * self.SUFFIX
        self.ext_events = []
        self.flops = []
        self.ext_tokens = []
        self.dec_bytes = []
        self.host_s = []
        self.step_lens = []
        self.ext_lens = []     # (pl, el) of the steps whose extend launch carries timing events
        self.wait_s = []       # host time blocked on a row set's staging (the GPU is behind)
        self.dec_distinct = []
        self.ext_rows = []

    def gen_inputs(self, n_batches):
        """Q/K/V of every suffix position and of the generated token, in HBM."""
        torch, T = self.torch, self.gen_t
        from synth import chain_start, prefix_hashes_rows_np
        bf16 = torch.bfloat16
        ph = prefix_hashes_rows_np(self.prefix[None, :], [chain_start(self.SEED)])
        self.inputs = []
        self.tokens = []
        n = self.PREFIX + self.SUFFIX
        self.tok_off = np.arange(0, self.B * n + 1, n, dtype=np.int64)
        self.full_off = np.arange(0, self.B * (n + 1) + 1, n + 1, dtype=np.int64)
        for i in range(n_batches):
            hn = prefix_hashes_rows_np(self.suffix[i], np.full(self.B, ph[0, -1], dtype=np.uint64))
            h = torch.from_numpy(hn.view(np.int64)).to(self.dev)    # [64, 129]
            hs, hd = h[:, :self.SUFFIX].reshape(-1), h[:, self.SUFFIX].contiguous()
            q = T.qkv_values_t(hs, 1, range(self.HQ), self.D, self.SEED, bf16)
            k = T.qkv_values_t(hs, 2, range(self.HKV), self.D, self.SEED, bf16)
            v = T.qkv_values_t(hs, 3, range(self.HKV), self.D, self.SEED, bf16)
            qd = T.qkv_values_t(hd, 1, range(self.HQ), self.D, self.SEED, bf16)
            kd = T.qkv_values_t(hd, 2, range(self.HKV), self.D, self.SEED, bf16)
            vd = T.qkv_values_t(hd, 3, range(self.HKV), self.D, self.SEED, bf16)
            self.inputs.append((q, k, v, qd, kd, vd))
            # the batch's token ids as the requests arrive: prompts, then prompts + generated token
            prompts = np.concatenate([np.broadcast_to(self.prefix, (self.B, self.PREFIX)),
                                      self.suffix[i][:, :self.SUFFIX]], axis=1)
            full = np.concatenate([prompts, self.suffix[i][:, self.SUFFIX:self.SUFFIX + 1]], axis=1)
            self.tokens.append((prompts.reshape(-1).copy(), full.reshape(-1).copy()))
        torch.cuda.synchronize()

    def warm_prefix(self):
        """The warm-up request: extend the 1024-token prefix and insert it."""
        torch, Bm, T = self.torch, self.Bm, self.gen_t
        from synth import chain_start, prefix_hashes_rows_np
        bf16 = torch.bfloat16
        hn = prefix_hashes_rows_np(self.prefix[None, :], [chain_start(self.SEED)])
        h = torch.from_numpy(hn.view(np.int64).reshape(-1)).to(self.dev)
        q = T.qkv_values_t(h, 1, range(self.HQ), self.D, self.SEED, bf16)
        k = T.qkv_values_t(h, 2, range(self.HKV), self.D, self.SEED, bf16)
        v = T.qkv_values_t(h, 3, range(self.HKV), self.D, self.SEED, bf16)
        toks = self.prefix
        off = np.array([0, self.PREFIX], dtype=np.int64)
        rows = np.array([0], dtype=np.int32)
        pl, el, nodes, loc = Bm.rt_admit_batch(self.tree, toks, off, self.r2t_host, rows)
        with torch.cuda.stream(self.stream):
            self.r2t_dev[0, :self.PREFIX].copy_(self.r2t_host_t[0, :self.PREFIX])
            dloc = torch.from_numpy(loc).to(self.dev)
            self._store(k, v, dloc)
            o = torch.empty_like(q)
            meta = torch.tensor([0, self.PREFIX, 0, self.PREFIX, 0], dtype=torch.int32, device=self.dev)
            self._extend(q, o, meta[4:5], meta[0:1], meta[1:2], meta[2:4], self.PREFIX)
        self.stream.synchronize()
        Bm.rt_finish_batch(self.tree, toks, off, self.r2t_host, rows, pl, nodes)

    def settle_clocks(self, ms=200.0):
        """Untimed, when no warm-up step runs (else settle_on_step): repeat
        an extend launch of the batch's own shape (64
        requests x 128 rows over 1152 keys, the first batch's queries) for
        about ``ms`` milliseconds, so that the GPU's clocks reach the level
        they hold under this load before any step runs; without it the first
        few dozen steps run 10-15 % slower.  Its requests use the second row
        set, which no step has used yet: each row holds the prefix's slots
        and, at the suffix positions, the slots of prefix positions 0..127
        (cached K/V, read only); the output goes to scratch.  The first step
        that uses that row set rewrites it."""
        torch, B, P, S = self.torch, self.B, self.PREFIX, self.SUFFIX
        rows = self.rows[1]
        pre = self.r2t_host[0, :P].copy()
        self.r2t_host[rows, :P] = pre
        self.r2t_host[rows, P:P + S] = pre[:S]
        lo, hi = self.set_rows, 2 * self.set_rows
        self.r2t_dev[lo:hi].copy_(self.r2t_host_t[lo:hi])
        meta = torch.from_numpy(np.concatenate([rows, np.full(B, P), np.full(B, S), np.arange(B + 1) * S])
                                .astype(np.int32)).to(self.dev)
        d_rows, d_pl, d_el, d_qo = meta[:B], meta[B:2 * B], meta[2 * B:3 * B], meta[3 * B:]
        q = self.inputs[0][0]
        o = torch.empty_like(q)
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(8):
                self._extend(q, o, d_rows, d_pl, d_el, d_qo, S)
            self.stream.synchronize()

    def _store_extend(self, k, v, rows, pl, el, qo, max_e):
        f = self.Bm.kv_store_extend_fp8 if self.fp8 else self.Bm.kv_store_extend
        f(self.k_pool, self.v_pool, k, v, self.r2t_dev, rows, pl, el, qo, max_e, stream=self.stream)

    def _store(self, k, v, loc):
        if self.fp8:
            self.Bm.kv_store_fp8(self.k_pool, self.v_pool, k, v, loc, stream=self.stream)
        else:
            self.Bm.kv_store(self.k_pool, self.v_pool, k, v, loc, stream=self.stream)

    def _extend(self, q, o, rows, pl, el, qo, max_e):
        f = self.Bm.radix_extend_attention_fp8kv if self.fp8 else self.Bm.radix_extend_attention
        f(q, o, self.k_pool, self.v_pool, self.r2t_dev, rows, pl, el, qo, max_e, self.sm_scale, stream=self.stream)

    def _decode(self, qd, kd, vd, d_rows, d_pos, d_dslots):
        """The decode step: each request's new token (K/V row kd / vd, slot
        d_dslots) is stored and attended to by the decode call's own
        launches (the _append entry points)."""
        B, S, P0 = self.B, self.SUFFIX, self.PREFIX
        Bm = self.Bm
        if self.shared_decode:
            dec = Bm.radix_decode_attention_shared_append_fp8kv if self.fp8 else Bm.radix_decode_attention_shared_append
            dec(qd, self.o_dec, self.k_pool, self.v_pool, self.r2t_dev, d_rows, d_pos, self.sl_dev, self.gs_dev, B,
                P0, S + 1, self.sm_scale, kd, vd, d_dslots, self.ws_shared, stream=self.stream)
        else:
            dec = Bm.radix_decode_attention_append_fp8kv if self.fp8 else Bm.radix_decode_attention_append
            dec(qd, self.o_dec, self.k_pool, self.v_pool, self.r2t_dev, d_rows, d_pos, P0 + S + 1, self.sm_scale,
                kd, vd, d_dslots,
                self.ws, stream=self.stream)

    def settle_on_step(self, i, ms=200.0):
        """Untimed, after the warm-up steps: step i's launches (the K/V
        scatter, extend and decode (with its append) of the last
        warm-up step, whose rows, metadata and K/V are still in place; every
        launch rewrites the same values) again and again for about ``ms``
        milliseconds, so that the timed steps start at the clock the chip
        holds under the step's own mix of work.  An extend-only settle
        (settle_clocks) leaves it in a state the steps then drift away from
        for some 20 ms: over 80 timed steps after it the extend went from
        175 to 204 us (step 15) and back down to 168 us."""
        Bm = self.Bm
        q, k, v, qd, kd, vd = self.inputs[i]
        d_pl, d_el, d_qo, d_rows, d_dslots = self.meta_views[i % 2]
        d_pos = self.pos_dev
        max_e = self.last_max_e
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(4):
                self._store_extend(k, v, d_rows, d_pl, d_el, d_qo, max_e)
                self._extend(q, self.o_ext, d_rows, d_pl, d_el, d_qo, max_e)
                self._decode(qd, kd, vd, d_rows, d_pos, d_dslots)
            self.stream.synchronize()

    def replay_decode(self, i, reps=10):
        """Untimed, after the timed steps: the decode call of step i (the
        last one, whose rows and K/V are still in place; its append rewrites
        the same entry and row) again, reps times, each bracketed by HIP
        events; returns the mean in seconds."""
        torch = self.torch
        d_pl, d_el, d_qo, d_rows, d_dslots = self.meta_views[i % 2]
        qd, kd, vd = self.inputs[i][3:6]
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            self._decode(qd, kd, vd, d_rows, self.pos_dev, d_dslots)
            e1.record(self.stream)
            ms.append((e0, e1))
        self.stream.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ms])) / 1e3

    def step(self, i, timed, ev=None):
        """One step; ``ev`` = two timing events (before and after the extend
        launch) recorded on the stream when given.  Each event costs the
        stream a few microseconds, so the decode is timed afterwards by
        replaying it (replay_decode)."""
        t_host = time.perf_counter()
        torch, Bm = self.torch, self.Bm
        B, S, P0 = self.B, self.SUFFIX, self.PREFIX
        q, k, v, qd, kd, vd = self.inputs[i]
        rs = i % 2
        waited = 0.0
        if self.copy_mark[rs] is not None:
            self.copy_mark[rs].synchronize()       # host staging of this row set is free again
            waited = time.perf_counter() - t_host
            if timed:
                self.wait_s.append(waited)
        rows = self.rows[rs]
        toks, full = self.tokens[i]
        pl, el, nodes, loc = Bm.rt_admit_batch(self.tree, toks, self.tok_off, self.r2t_host, rows)
        if int(pl.min()) < P0:
            raise RuntimeError("the shared prefix left the cache; the pool is too small for this run")
        h_pl, h_el, h_qo, h_rows, h_dslots = self.meta_host[rs]
        h_pl[:] = pl
        h_el[:] = el
        # request b's new rows are the last el[b] of its S rows of q / k / v
        h_qo[:B] = self.row_base + (pl - P0)
        h_qo[B] = B * S
        h_rows[:] = rows
        # one decode slot per request, at position P0 + S
        h_dslots[:] = Bm.rt_decode_slots_batch(self.tree, rows, self.dec_pos, self.r2t_host)
        d_pl, d_el, d_qo, d_rows, d_dslots = self.meta_views[rs]
        max_e = int(el.max())
        # every launch names self.stream
        # Rows and metadata, by a kernel on the step's stream that reads the
        # pinned staging (no hand-over to a DMA engine and back).  Every
        # request matched the whole prefix (checked above) through the same
        # tree nodes, so columns 0 .. P0-1 of its row hold the prefix's
        # slots, which stay fixed while the prefix is cached: once a row set
        # has gone up whole with those slots, only the columns from P0 on
        # change.
        dev_all, host_all, dev_tail, host_tail = self.copy_views[rs]
        if self.prefix_slots is None or not np.array_equal(self.r2t_host[rows[0], :P0], self.prefix_slots):
            self.prefix_slots = self.r2t_host[rows[0], :P0].copy()
            self.rows_whole = [False, False]
        if self.rows_whole[rs]:
            Bm.rt_copy_from_host_2d(dev_tail, host_tail, stream=self.stream)
        else:
            Bm.rt_copy_from_host(dev_all, host_all, stream=self.stream)
            self.rows_whole[rs] = True
        self._store_extend(k, v, d_rows, d_pl, d_el, d_qo, max_e)
        # the marker that frees this row set's staging: a timed step's first
        # timing event follows the copy on the stream, so it serves; other
        # steps record one of their own
        if ev is not None:
            ev[0].record(self.stream)
            self.copy_mark[rs] = ev[0]
        else:
            self.copy_done[rs].record(self.stream)
            self.copy_mark[rs] = self.copy_done[rs]
        self._extend(q, self.o_ext, d_rows, d_pl, d_el, d_qo, max_e)
        if ev is not None:
            ev[1].record(self.stream)
        # decode step: the new token's slot-table entry and K/V row are
        # written by the decode's own launches
        self._decode(qd, kd, vd, d_rows, self.pos_dev, d_dslots)
        # finish: prompt + generated token into the tree
        Bm.rt_finish_batch(self.tree, full, self.full_off, self.r2t_host, rows, pl, nodes)
        self.last_prefix_lens = pl
        self.last_max_e = max_e
        if timed:
            # flops and bytes follow from (pl, el) after the timed region
            if ev is not None:
                self.ext_events.append((ev[0], ev[1]))
                self.ext_lens.append((pl, el))
            self.step_lens.append((pl, el))
            self.host_s.append(time.perf_counter() - t_host - waited)
        return int(el.sum()) + B

    def accounting(self):
        """Extend flops of every step whose extend launch was timed; decode
        bytes of every timed step."""
        P0, S, B = self.PREFIX, self.SUFFIX, self.B
        eb = 1 if self.fp8 else 2
        for pl, el in self.ext_lens:
            rows_keys = float(np.sum(pl.astype(np.float64) * el + el.astype(np.float64) * (el + 1) / 2))
            self.flops.append(4.0 * self.D * self.HQ * rows_keys)
            self.ext_rows.append(int(el.sum()))
        # the decode's own append: each new token's K and V rows read (bf16)
        # and written into the pool
        append = B * self.HKV * self.D * (2 + eb) * 2
        for pl, el in self.step_lens:
            self.ext_tokens.append(int(el.sum()) + B)
            self.dec_bytes.append(B * (P0 + S + 1) * (self.HKV * self.D * eb * 2 + 4) + 2 * B * self.HQ * self.D * 2
                                  + append)
            # the prefix once, every request's own tail
            self.dec_distinct.append(P0 * self.HKV * self.D * eb * 2 + B * (S + 1) * (self.HKV * self.D * eb * 2 + 4)
                                     + 2 * B * self.HQ * self.D * 2 + append)


def run_few_shot(args, torch):
    from prefix_shared_kv_rt_amd import binding as Bm
    from synth import torch_gen
    n = args.warmup + args.steps
    fb = FewShotBench(n, torch, Bm, torch_gen, kv_dtype=args.kv_dtype, page_size=args.page_size,
                      shared_decode=(args.decode or "shared") == "shared")
    fb.gen_inputs(n)
    fb.warm_prefix()
    # Collect before the clock settle: a collector pass between the warm-up
    # and the timed steps idles the GPU long enough for its clocks to drop.
    # Disabled until the timed steps end: a pass inside them would stall the
    # host, not the path.
    gc.collect()
    gc.disable()
    if args.warmup > 0:
        for i in range(args.warmup):
            fb.step(i, timed=False)
        fb.settle_on_step(args.warmup - 1)
    else:
        fb.settle_clocks()
    fb.stream.synchronize()
    torch.cuda.synchronize()
    # timing events around the extend launch of every time_every-th step
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] if k % args.time_every == 0 else None
           for k in range(args.steps)]
    t0 = time.perf_counter()
    tokens = 0
    for i in range(args.warmup, n):
        tokens += fb.step(i, timed=True, ev=evs[i - args.warmup])
    fb.stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    fb.accounting()
    ext_ms = [a.elapsed_time(b) for a, b in fb.ext_events]
    dec_avg_s = fb.replay_decode(n - 1)
    ext_avg_s = float(np.mean(ext_ms)) / 1e3
    dec_traffic = (profiled_traffic("decode_shared_bf16_few_shot")
                   if fb.shared_decode and not fb.fp8 and args.page_size == 1 else None)
    flops_avg = float(np.mean(fb.flops))
    achieved_tflops = flops_avg / ext_avg_s / 1e12
    result = {
        "metric": METRIC,
        "value": tokens / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "few-shot shared prefix, Llama-3-8B attention shape: 64 requests x (1024 shared + 128 "
                        "distinct tokens) per step, one extend pass + one decode step, tree match/insert on host",
            "batch": fb.B, "prefix_len": fb.PREFIX, "suffix_len": fb.SUFFIX, "num_q_heads": fb.HQ,
            "num_kv_heads": fb.HKV, "head_dim": fb.D, "pool_slots": fb.SLOTS,
            "kv_dtype": "fp8_e4m3" if fb.fp8 else "bf16", "page_size": fb.page_size,
            "decode": "radix_decode_attention_shared_append" if fb.shared_decode else "radix_decode_attention_append",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "radix_extend_attention_fp8kv (extend_bf16<128, 1, true, false>)" if fb.fp8 else
                      "radix_extend_attention (extend_bf16<128, 1, false, false>)",
            "achieved": achieved_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS,
            "traffic": None if fb.fp8 else profiled_traffic("extend_bf16"),
            "flops_per_launch": flops_avg,
            "avg_launch_us": ext_avg_s * 1e6,
        },
        "kernels": {
            "extend_us": ext_avg_s * 1e6,
            "extend_rows_per_step": float(np.mean(fb.ext_rows)),
            "extend_tokens_per_s": float(np.mean(fb.ext_rows)) / ext_avg_s,
            "decode_us": dec_avg_s * 1e6,   # decode attention, replayed after the timed steps
            # bytes each request's whole context would move (the shared
            # prefix counted once per request: an upper bound, not HBM traffic)
            "decode_per_request_gbs": float(np.mean(fb.dec_bytes)) / dec_avg_s / 1e9,
            # bytes the step must read at least once (prefix once, every tail)
            "decode_distinct_gbs": float(np.mean(fb.dec_distinct)) / dec_avg_s / 1e9,
            "decode_distinct_frac": float(np.mean(fb.dec_distinct)) / dec_avg_s / 1e9 / PEAK_HBM_GBS,
            # the decode call's HBM traffic from the committed counter runs
            # (None once its sources changed), over the same event time
            "decode_traffic_frac": (dec_traffic / dec_avg_s / 1e9 / PEAK_HBM_GBS) if dec_traffic else None,
            # host time to run one step's tree work and enqueue its GPU work,
            # without the time blocked waiting for the GPU to release a row
            # set's staging (the step is host-bound when this nears
            # ms_per_step)
            "host_us_per_step": float(np.mean(fb.host_s)) * 1e6,
            "host_wait_us_per_step": float(np.mean(fb.wait_s)) * 1e6 if fb.wait_s else 0.0,
            "extend_timed_steps": len(fb.ext_events),
        },
    }
    return result, fb


class DecodeBench:
    """Decode steps of a batch whose prompts are already in the pool.

    long_context: 32 requests, 16384 shared + 16384 private prompt tokens,
    Hq 64 / Hkv 8 / D 128.  fork: 16 prompts of 2048 tokens, each matched
    whole by 8 branches (batch 128), Hq 32 / Hkv 8 / D 128.  Prompt K/V are
    scattered into the pool with kv_store (no extend attention); each timed
    step allocates one slot per request and runs decode attention over the
    whole context, whose launches also write each request's slot-table entry
    and K/V row (the _append decode entry points)."""

    def __init__(self, name, torch, Bm, gen_t, n_steps, kv_dtype="bf16", shared_decode=False):
        self.torch, self.Bm, self.T = torch, Bm, gen_t
        self.fp8 = kv_dtype == "fp8"
        self.shared_decode = shared_decode
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.Stream(self.dev)
        self.name = name
        if name == "long_context":
            self.SEED, self.HQ, self.HKV, self.D = 4, 64, 8, 128
            self.B, self.groups, self.shared, self.private = 32, 1, 16384, 16384
            self.SLOTS = 1 << 20
        else:  # fork
            self.SEED, self.HQ, self.HKV, self.D = 2, 32, 8, 128
            self.B, self.groups, self.shared, self.private = 128, 16, 2048, 0
            self.SLOTS = 262144
        self.n_steps = n_steps
        rng = np.random.Generator(np.random.PCG64(self.SEED))
        self.prompt_len = self.shared + self.private
        # group g's shared part; request b belongs to group b // (B / groups)
        self.shared_toks = rng.integers(0, 1000, size=(self.groups, self.shared)).astype(np.int32)
        self.private_toks = rng.integers(0, 1000, size=(self.B, self.private)).astype(np.int32)
        self.gen_toks = rng.integers(0, 1000, size=(self.B, n_steps)).astype(np.int32)
        self.stride = self.prompt_len + n_steps
        self.pool = Bm.rt_pool_create(self.SLOTS)
        self.tree = Bm.rt_tree_create(self.pool)
        pool_dt = torch.uint8 if self.fp8 else torch.bfloat16
        self.k_pool = torch.zeros((self.SLOTS + 1, self.HKV, self.D), dtype=pool_dt, device=self.dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.r2t_host = np.zeros((self.B + self.groups, self.stride), dtype=np.int32)
        self.r2t_dev = torch.zeros((self.B + self.groups, self.stride), dtype=torch.int32, device=self.dev)
        self.sm_scale = 1.0 / np.sqrt(self.D)

    def _values(self, hashes, kind, heads):
        return self.T.qkv_values_t(hashes, kind, range(heads), self.D, self.SEED, self.torch.bfloat16)

    def _dev_hashes(self, h):
        return self.torch.from_numpy(np.ascontiguousarray(h).view(np.int64)).to(self.dev)

    def _store(self, hashes, slots):
        """Scatter generated K/V of positions with these (host) hashes into the pool."""
        torch = self.torch
        for lo in range(0, hashes.size, 16384):
            h = self._dev_hashes(hashes[lo:lo + 16384])
            loc = torch.from_numpy(np.ascontiguousarray(slots[lo:lo + 16384])).to(self.dev)
            store = self.Bm.kv_store_fp8 if self.fp8 else self.Bm.kv_store
            store(self.k_pool, self.v_pool, self._values(h, 2, self.HKV), self._values(h, 3, self.HKV), loc,
                  stream=self.torch.cuda.current_stream())

    def cold_extend(self, sh_hash, rows, reps=5):
        """Fork: the 16 cold prompts' extend pass (P = 0, E = 2048 each)
        through kv_store and radix_extend_attention, as a serving step runs
        it; the K/V it stores are the ones the branches decode against.
        Repeated ``reps`` times after one untimed pass (the repeats rewrite
        the same slots and outputs); returns the mean time per pass."""
        torch, Bm = self.torch, self.Bm
        n = self.groups * self.shared
        h = self._dev_hashes(sh_hash.reshape(-1))
        q = self._values(h, 1, self.HQ)
        k = self._values(h, 2, self.HKV)
        v = self._values(h, 3, self.HKV)
        o = torch.empty_like(q)
        g = self.groups
        meta = torch.from_numpy(np.concatenate([rows, np.zeros(g), np.full(g, self.shared),
                                                np.arange(g + 1) * self.shared]).astype(np.int32)).to(self.dev)
        d_rows, d_pl, d_el, d_qo = meta[:g], meta[g:2 * g], meta[2 * g:3 * g], meta[3 * g:]
        r2t_dev = self.r2t_dev
        r2t_dev.copy_(torch.from_numpy(self.r2t_host))
        store = Bm.kv_store_extend_fp8 if self.fp8 else Bm.kv_store_extend
        ext = Bm.radix_extend_attention_fp8kv if self.fp8 else Bm.radix_extend_attention
        evs = []
        with torch.cuda.stream(self.stream):
            for r in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                store(self.k_pool, self.v_pool, k, v, r2t_dev, d_rows, d_pl, d_el, d_qo, self.shared,
                      stream=self.stream)
                e0.record(self.stream)
                ext(q, o, self.k_pool, self.v_pool, r2t_dev, d_rows, d_pl, d_el, d_qo, self.shared, self.sm_scale,
                    stream=self.stream)
                e1.record(self.stream)
                if r > 0:
                    evs.append((e0, e1))
        self.stream.synchronize()
        self.cold_o = o
        assert n == q.shape[0]
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3

    def setup(self):
        torch, Bm, T = self.torch, self.Bm, self.T
        per = self.B // self.groups
        # shared prompts: admitted, stored and inserted first (prompt-only requests)
        from synth import chain_start, prefix_hashes_rows_np
        sh_hash = prefix_hashes_rows_np(self.shared_toks, np.full(self.groups, chain_start(self.SEED), dtype=np.uint64))
        toks = self.shared_toks.reshape(-1)
        off = np.arange(0, self.groups * self.shared + 1, self.shared, dtype=np.int64)
        rows = np.arange(self.B, self.B + self.groups, dtype=np.int32)
        pl, el, nodes, loc = Bm.rt_admit_batch(self.tree, toks, off, self.r2t_host, rows)
        self.cold_extend_s = None
        if self.name == "fork":
            # cold prompts: the real extend pass (scatter + extend attention)
            self.cold_extend_s = self.cold_extend(sh_hash, rows)
        else:
            self._store(sh_hash.reshape(-1), loc)
        Bm.rt_finish_batch(self.tree, toks, off, self.r2t_host, rows, pl, nodes)
        # the decoding requests: match the shared part, store their private part
        prompts = np.concatenate([np.repeat(self.shared_toks, per, axis=0), self.private_toks], axis=1)
        toks = prompts.reshape(-1)
        off = np.arange(0, self.B * self.prompt_len + 1, self.prompt_len, dtype=np.int64)
        rows = np.arange(self.B, dtype=np.int32)
        self.pl, el, self.nodes, loc = Bm.rt_admit_batch(self.tree, toks, off, self.r2t_host, rows)
        assert (self.pl == self.shared).all()
        start = np.repeat(sh_hash[:, -1], per)                                    # [B]
        if self.private:
            ph = prefix_hashes_rows_np(self.private_toks, start)
            self._store(ph.reshape(-1), loc)
            start = ph[:, -1]
        # decode inputs for every step
        gh = self._dev_hashes(prefix_hashes_rows_np(self.gen_toks, start))         # [B, steps]
        self.q = [self._values(gh[:, s].contiguous(), 1, self.HQ) for s in range(self.n_steps)]
        # per-step positions and new slots: one pinned staging row per step
        # (never reused within a run, so no step waits for an earlier copy)
        # and its device row, copied by a kernel on the step's stream
        self.meta_host_t = torch.zeros((self.n_steps, 2 * self.B), dtype=torch.int32, pin_memory=True)
        self.meta_host = self.meta_host_t.numpy()
        self.meta_dev = torch.zeros((self.n_steps, 2 * self.B), dtype=torch.int32, device=self.dev)
        self.k = [self._values(gh[:, s].contiguous(), 2, self.HKV) for s in range(self.n_steps)]
        self.v = [self._values(gh[:, s].contiguous(), 3, self.HKV) for s in range(self.n_steps)]
        self.r2t_dev.copy_(torch.from_numpy(self.r2t_host))
        self.rows_dev = torch.arange(self.B, dtype=torch.int32, device=self.dev)
        self.o = torch.empty((self.B, self.HQ, self.D), dtype=torch.bfloat16, device=self.dev)
        self.ws = torch.empty(Bm.radix_decode_workspace_bytes(self.B, self.HQ, self.HKV, self.D, self.stride),
                              dtype=torch.uint8, device=self.dev)
        if self.shared_decode:
            # group g = requests g*per .. (g+1)*per - 1, which share the first `shared` slots of their rows
            self.sl_dev = torch.full((self.B,), self.shared, dtype=torch.int32, device=self.dev)
            self.gs_dev = torch.arange(0, self.B + 1, per, dtype=torch.int32, device=self.dev)
            need = max(Bm.radix_decode_shared_workspace_bytes(self.B, self.HQ, self.HKV, self.D, self.groups, per,
                                                              self.shared, self.private + s + 1)
                       for s in range(self.n_steps))
            self.ws_shared = torch.empty(need, dtype=torch.uint8, device=self.dev)
        self.events = []
        torch.cuda.synchronize()

    def settle_clocks(self, ms=200.0):
        """Untimed, when no warm-up step runs (else settle_on_step): decode
        attention over the prompts alone (pool reads, a scratch output) for about ``ms`` milliseconds, so that the clocks
        reach their level under sustained load before any step runs."""
        torch, Bm = self.torch, self.Bm
        d_pos = torch.full((self.B,), self.prompt_len - 1, dtype=torch.int32, device=self.dev)
        o = torch.empty_like(self.o)
        decode = Bm.radix_decode_attention_fp8kv if self.fp8 else Bm.radix_decode_attention
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(8):
                decode(self.q[0], o, self.k_pool, self.v_pool, self.r2t_dev, self.rows_dev, d_pos, self.prompt_len,
                       self.sm_scale, self.ws, stream=self.stream)
            self.stream.synchronize()

    def settle_on_step(self, s, ms=200.0):
        """Untimed, after the warm-up steps: step s's launches (slot-table
        scatter, K/V store and decode attention of the last warm-up step,
        whose metadata and K/V stay in place; each launch rewrites the same
        values) again and again for about ``ms`` milliseconds, so that the
        timed steps start at the clock the chip holds under their own work."""
        torch, Bm = self.torch, self.Bm
        meta = self.meta_dev[s]
        d_pos, d_slots = meta[:self.B], meta[self.B:]
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(8):
                self.launch_step(s, d_pos, d_slots)
            self.stream.synchronize()

    def launch_step(self, s, d_pos, d_slots):
        """Step s's GPU work after its metadata copy, on the bench's stream."""
        self.launch_decode(s, d_pos, d_slots)

    def launch_decode(self, s, d_pos, d_slots):
        """Decode with the new tokens' append (slot-table entry and K/V row
        of each request) in the decode's own launches."""
        Bm = self.Bm   # FP8 pools: scales 1 (the binding's defaults)
        if self.shared_decode:
            decode = Bm.radix_decode_attention_shared_append_fp8kv if self.fp8 else \
                Bm.radix_decode_attention_shared_append
            decode(self.q[s], self.o, self.k_pool, self.v_pool, self.r2t_dev, self.rows_dev, d_pos, self.sl_dev,
                   self.gs_dev, self.B // self.groups, self.shared, self.private + s + 1, self.sm_scale, self.k[s],
                   self.v[s], d_slots, self.ws_shared, stream=self.stream)
        else:
            decode = Bm.radix_decode_attention_append_fp8kv if self.fp8 else Bm.radix_decode_attention_append
            decode(self.q[s], self.o, self.k_pool, self.v_pool, self.r2t_dev, self.rows_dev, d_pos,
                   self.prompt_len + s + 1, self.sm_scale, self.k[s], self.v[s], d_slots, self.ws,
                   stream=self.stream)

    def step(self, s, timed):
        torch, Bm = self.torch, self.Bm
        pos = np.full(self.B, self.prompt_len + s, dtype=np.int32)
        rows = np.arange(self.B, dtype=np.int32)
        slots = Bm.rt_decode_slots_batch(self.tree, rows, pos, self.r2t_host)
        with torch.cuda.stream(self.stream):
            self.meta_host[s, :self.B] = pos
            self.meta_host[s, self.B:] = slots
            meta = self.meta_dev[s]
            Bm.rt_copy_from_host(meta, self.meta_host_t[s], stream=self.stream)
            d_pos, d_slots = meta[:self.B], meta[self.B:]
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
            self.launch_decode(s, d_pos, d_slots)
            if timed:
                e1.record(self.stream)
                self.events.append((e0, e1, int(pos[0]) + 1))
        return self.B


def run_decode_bench(args, torch):
    from prefix_shared_kv_rt_amd import binding as Bm
    from synth import torch_gen
    n = args.warmup + args.steps
    db = DecodeBench(args.workload, torch, Bm, torch_gen, n, kv_dtype=args.kv_dtype,
                     shared_decode=(args.decode or "shared") == "shared")
    db.setup()
    gc.collect()     # before the clock settle (see run_few_shot)
    gc.disable()
    if args.warmup > 0:
        for s in range(args.warmup):
            db.step(s, timed=False)
        db.settle_on_step(args.warmup - 1)
    else:
        db.settle_clocks()
    db.stream.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tokens = 0
    for s in range(args.warmup, n):
        tokens += db.step(s, timed=True)
    db.stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    ms = [a.elapsed_time(b) for a, b, _ in db.events]
    avg_s = float(np.mean(ms)) / 1e3
    kv = np.mean([k for _, _, k in db.events])
    row = db.HKV * db.D * (1 if db.fp8 else 2)   # one K (or V) pool row
    # every request's whole context (the shared part once per request: what
    # the plain decode's waves request, much of it served by L2 / MALL)
    # the decode's own append: each new token's K and V rows read (bf16) and
    # written into the pool
    append = db.B * 2 * (db.HKV * db.D * 2 + row)
    per_request = db.B * kv * (2 * row + 4) + 2 * db.B * db.HQ * db.D * 2 + append
    # what a step must read at least once: each group's shared part once,
    # every request's own tail, q and o
    distinct = (db.groups * db.shared * 2 * row + db.B * (kv - db.shared) * (2 * row + 4)
                + 2 * db.B * db.HQ * db.D * 2 + append)
    achieved = distinct / avg_s / 1e9
    frac = achieved / PEAK_HBM_GBS
    assert frac <= 1.0, f"decode roofline above HBM peak ({frac:.3f}): the byte count is wrong"
    label = ("long-context decode: 32 requests x (16384 shared + 16384 private) context, Hq 64 / Hkv 8 / D 128"
             if db.name == "long_context" else
             "fork decode: 16 prompts x 2048 tokens, 8 branches each (batch 128), Hq 32 / Hkv 8 / D 128")
    result = {
        "metric": METRIC + " (decode)", "value": tokens / wall, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": label, "batch": db.B, "num_q_heads": db.HQ, "num_kv_heads": db.HKV,
                   "head_dim": db.D, "pool_slots": db.SLOTS, "kv_dtype": "fp8_e4m3" if db.fp8 else "bf16",
                   "shared_decode": bool(db.shared_decode)},
        "roofline": {"bound": "hbm",
                     "kernel": ("radix_decode_attention_shared_append" if db.shared_decode
                                else "radix_decode_attention_append")
                               + ("_fp8kv" if db.fp8 else "")
                               + (" (shared pass + private split + combine)" if db.shared_decode
                                  else " (split + combine)") + "; bytes = distinct bytes",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": frac,
                     "traffic": profiled_traffic(("decode_shared" if db.shared_decode else "decode_split")
                                                 + ("_fp8" if db.fp8 else "_bf16") + "_" + db.name),
                     "bytes_per_launch": distinct, "per_request_bytes_per_launch": per_request,
                     "avg_launch_us": avg_s * 1e6},
    }
    traffic = result["roofline"]["traffic"]
    if traffic:   # the counters' bytes over the same launch time
        result["roofline"]["traffic_gbs"] = traffic / avg_s / 1e9
        result["roofline"]["traffic_frac"] = traffic / avg_s / 1e9 / PEAK_HBM_GBS
    if db.cold_extend_s is not None:
        g, e = db.groups, db.shared
        flops = 4.0 * db.D * db.HQ * g * e * (e + 1) / 2
        tf = flops / db.cold_extend_s / 1e12
        result["cold_extend"] = {"what": f"{g} cold prompts x {e} tokens (P = 0): kv_store_extend + "
                                         "radix_extend_attention, extend timed (HIP events, mean of 5 passes)",
                                 "us": db.cold_extend_s * 1e6, "flops": flops, "tflops": tf,
                                 "mfma_frac": tf / PEAK_BF16_TFLOPS}
    return result


def run_chat(args, torch):
    """The multi-turn chat workload through the scheduler once: 256 sessions
    x 4 turns on a shared 512-token system prompt, U{128..384} user tokens
    and 128 generated tokens per turn, pool at 60 % of the working set (so
    eviction and re-extension happen).  Every kernel is timed with HIP
    events; mixed tokens/s = (extend + decode tokens) / summed kernel time."""
    from prefix_shared_kv_rt_amd.runtime import RadixRuntime, Scheduler
    from synth import workloads
    from synth.sources import QKVSource
    wl = workloads.paged(workloads.chat(), args.page_size)
    rt = RadixRuntime(wl.num_slots, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, torch.bfloat16, 256, wl.max_ctx,
                      kv_fp8_scales=(1.0, 1.0) if args.kv_dtype == "fp8" else None, page_size=wl.page_size)
    src = QKVSource(wl.seed, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, torch.bfloat16)
    rt.events = []
    sch = Scheduler(rt, wl.requests, src, max_running=256, max_extend_tokens=16384, policy=args.policy,
                    chunk_size=args.chunk_size, mixed=args.mixed, shared_decode=args.decode == "shared")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks = [0]
    sch._arrive()
    it = 0
    while sch.waiting or sch.running or sch.pending or sch.prefilling:
        sch.step(it)
        sch._arrive()
        marks.append(len(rt.events))
        it += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # GPU time of each iteration that decoded: how long running requests wait per token
    it_ms = []
    for a, b in zip(marks[:-1], marks[1:]):
        evs = rt.events[a:b]
        if any(kind in ("decode", "mixed") for kind, _, _, _ in evs):
            it_ms.append(sum(x.elapsed_time(y) for _, x, y, _ in evs))
    per = {}
    for kind, a, b, info in rt.events:
        d = per.setdefault(kind, {"launches": 0, "ms": 0.0, "tokens": 0, "flops": 0.0, "bytes": 0.0, "rows": 0,
                                  "distinct_bytes": 0.0})
        d["launches"] += 1
        d["ms"] += a.elapsed_time(b)
        for k in ("tokens", "flops", "bytes", "rows", "distinct_bytes"):
            d[k] += info.get(k, 0)
    rt.close()
    ext, dec, mix = per.get("extend", {}), per.get("decode", {}), per.get("mixed", {})
    kernel_s = sum(d["ms"] for d in per.values()) / 1e3
    tokens = ext.get("tokens", 0) + dec.get("tokens", 0) + mix.get("tokens", 0)
    byrid = {r.rid: r for r in wl.requests}
    evicted = sum(it.get("extend_freed_tokens", 0) + it.get("decode_freed_tokens", 0) for it in sch.iterations)
    re_extended = 0
    for it in sch.iterations:
        for rid, p, e in it["admitted"]:
            for a in byrid[rid].after:
                prev = byrid[a]
                re_extended += max(0, min(len(byrid[rid].prompt), len(prev.prompt) + len(prev.gen)) - p)
    ext_tf = ext.get("flops", 0.0) / max(ext.get("ms", 0.0), 1e-9) / 1e9
    dec_gbs = dec.get("bytes", 0.0) / max(dec.get("ms", 0.0), 1e-9) / 1e6
    # roofline of the kernel kind with the most summed time
    dom = max(per, key=lambda k: per[k]["ms"])
    d = per[dom]
    if dom == "decode":
        ach = d["distinct_bytes"] / (d["ms"] / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "radix_decode_attention (all decode launches); bytes = distinct bytes",
                "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}
    else:
        ach = d["flops"] / (d["ms"] / 1e3) / 1e12
        roof = {"bound": "mfma", "kernel": f"radix_{dom}_attention (all {dom} launches)", "achieved": ach,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS}
    roof.update({"traffic": None, "launches": d["launches"], "avg_launch_us": d["ms"] * 1e3 / d["launches"]})
    assert roof["frac"] <= 1.0, roof
    return {
        "metric": METRIC + " (chat, mixed)", "value": tokens / kernel_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": len(sch.iterations), "warmup": 0, "ms_per_step": wall / len(sch.iterations) * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "multi-turn chat: 512-token system prompt, 256 sessions x 4 turns, "
                               "U{128..384} user + 128 generated tokens per turn, pool 60% of the working set; "
                               "one pass of the whole workload, a step = one scheduler iteration",
                   "policy": args.policy, "chunk_size": args.chunk_size, "page_size": wl.page_size,
                   "mixed_launch": bool(args.mixed), "decode": args.decode or "plain",
                   "kv_dtype": "fp8_e4m3" if args.kv_dtype == "fp8" else "bf16",
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "pool_slots": wl.num_slots},
        "roofline": roof,
        "wall_tokens_per_s": tokens / wall,
        "kernels": {k: {"launches": d["launches"], "ms": d["ms"]} for k, d in per.items()},
        "extend": {"tokens": ext.get("tokens", 0), "tflops": ext_tf, "mfma_frac": ext_tf / PEAK_BF16_TFLOPS},
        "decode": {"tokens": dec.get("tokens", 0), "gbs": dec_gbs, "hbm_frac": dec_gbs / PEAK_HBM_GBS,
                   "distinct_gbs": dec.get("distinct_bytes", 0.0) / max(dec.get("ms", 0.0), 1e-9) / 1e6,
                   "shared_launches": sch.shared_decodes},
        "mixed": {"launches": mix.get("launches", 0), "tokens": mix.get("tokens", 0),
                  "tflops": mix.get("flops", 0.0) / max(mix.get("ms", 0.0), 1e-9) / 1e9},
        "hit_rate": {"cached": sch.cached_tokens, "prefill": sch.prefill_tokens,
                     "ratio": sch.cached_tokens / max(sch.prefill_tokens, 1)},
        "evicted_tokens": evicted, "re_extended_tokens": re_extended,
        "decode_iteration_gpu_ms": {"p50": float(np.percentile(it_ms, 50)), "p99": float(np.percentile(it_ms, 99)),
                                    "max": float(np.max(it_ms))} if it_ms else None,
    }


def run_decode_graph(args, torch):
    """Decode-step latency, eager launches against replayed HIP graphs, at the
    Llama-3-8B shape with 2048-token contexts and batch 1..128.  A step is what
    a serving loop does per generated token: stage the batch's rows,
    positions and new slots, append the new tokens, attend, synchronise.  The
    eager step also uploads its index vectors one by one; the graph step reads
    the new Q/K/V from its static buffers, where a producer writes them."""
    from prefix_shared_kv_rt_amd.graphs import DecodeGraphs
    from prefix_shared_kv_rt_amd.runtime import RadixRuntime
    HQ, HKV, D, CTX, SLOTS = 32, 8, 128, 2304, 1 << 19
    sizes = [1, 4, 16, 64, 128]
    fp8 = args.kv_dtype == "fp8"
    rt = RadixRuntime(SLOTS, HQ, HKV, D, torch.bfloat16, 129, CTX, kv_fp8_scales=(1.0, 1.0) if fp8 else None)
    g = torch.Generator(device="cuda").manual_seed(7)
    if fp8:  # codes of N(0, 1) values, as an FP8 store leaves them
        for pool in (rt.k_pool, rt.v_pool):
            vals = torch.randn(pool[1:].shape, generator=g, device="cuda")
            pool[1:] = vals.to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        rt.k_pool[1:] = torch.randn(rt.k_pool[1:].shape, generator=g, device="cuda").to(torch.bfloat16)
        rt.v_pool[1:] = torch.randn(rt.v_pool[1:].shape, generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(7)
    for r in range(128):
        rt.r2t_host[r, :] = rng.integers(1, SLOTS // 2, CTX)
    rt.r2t_dev.copy_(torch.from_numpy(rt.r2t_host))
    t0 = time.perf_counter()
    graphs = DecodeGraphs(rt, max_batch=128)
    capture_s = time.perf_counter() - t0
    table = {}
    steps = max(args.steps, 20)
    for n in sizes:
        rows = np.arange(n, dtype=np.int32)
        pos = np.full(n, 2047, dtype=np.int32)
        slots = (SLOTS // 2 + np.arange(n)).astype(np.int32)
        q = torch.randn((n, HQ, D), device="cuda").to(torch.bfloat16)
        k = torch.randn((n, HKV, D), device="cuda").to(torch.bfloat16)
        v = torch.randn((n, HKV, D), device="cuda").to(torch.bfloat16)
        res = {}
        gq, gk, gv = graphs.inputs(n)  # a producer would write the new tokens' Q/K/V here
        gq.copy_(q), gk.copy_(k), gv.copy_(v)
        for mode in ("eager", "graph"):
            run = (lambda: rt.run_decode(rows, pos, slots, q, k, v)) if mode == "eager" else \
                  (lambda: graphs.run(rows, pos, slots))
            for _ in range(args.warmup + 2):
                run()
                rt.stream.synchronize()
            t1 = time.perf_counter()
            for _ in range(steps):
                run()
                rt.stream.synchronize()
            res[mode] = (time.perf_counter() - t1) / steps * 1e6
        table[n] = {"eager_us": res["eager"], "graph_us": res["graph"], "speedup": res["eager"] / res["graph"]}
    rt.close()
    return {
        "metric": METRIC + " (decode step latency, graphs)", "value": 1e6 / table[1]["graph_us"],
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": table[1]["graph_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode steps of batch 1..128 at 2048-token contexts, Hq 32 / Hkv 8 / D 128; "
                               "value = batch-1 tokens/s with graphs; each step synchronised",
                   "num_q_heads": HQ, "num_kv_heads": HKV, "head_dim": D, "graph_sizes": graphs.sizes,
                   "kv_dtype": "fp8_e4m3" if fp8 else "bf16"},
        "capture_s": capture_s,
        "latency": table,
    }


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(args):
    """The oracle, unchanged, on a bounded sample of the same workload
    (about 10-30 s of CPU work), timed on this host's cores, plus the same
    kind of sample on one thread.  Tokens/s = attention outputs recomputed
    (one query row = one token) / oracle wall time (tree work included)."""
    from synth import workloads
    cores = _oracle_threads()
    wl_name = args.workload
    if wl_name == "few_shot":
        wl = workloads.few_shot(batch=args.cpu_sample, decode_steps=1)
        want = lambda kind, rid, step: rid != 0
        per_output = lambda k: 128 if k[0] == "ext" else 1
        sample = (f"{args.cpu_sample} few-shot requests (1024 shared + 128 distinct tokens + 1 decode step) after "
                  f"the warm-up prefix")
        wl1, want1 = workloads.few_shot(batch=16, decode_steps=1), want
        sample1 = "16 few-shot requests"
    elif wl_name == "fork":
        wl = workloads.fork()
        want = lambda kind, rid, step: kind == "dec" and step in (0, 127, 255) and (rid - 16) % 8 == 0
        per_output = lambda k: 1
        sample = ("fork: the tree over all 16 prompts x 8 branches x 256 steps; attention of one branch per prompt "
                  "(16) at decode steps 0, 127, 255")
        wl1 = workloads.fork()
        want1 = lambda kind, rid, step: kind == "dec" and step == 0 and (rid - 16) % 8 == 0
        sample1 = "fork tree + 16 branches at step 0"
    elif wl_name == "long_context":
        wl = workloads.long_context(decode_steps=1)
        want = lambda kind, rid, step: kind == "dec" and step == 0 and rid in (1, 32)
        per_output = lambda k: 1
        sample = "long context: requests 1 and 32 (32769-key contexts) at decode step 0"
        wl1 = wl
        want1 = lambda kind, rid, step: kind == "dec" and step == 0 and rid == 1
        sample1 = "long context: request 1 at decode step 0"
    elif wl_name == "chat":
        wl = workloads.chat()
        want = lambda kind, rid, step: kind == "dec" and rid % 16 == 0 and step in (0, 64)
        per_output = lambda k: 1
        sample = ("chat: the tree and scheduler over all 256 sessions x 4 turns; attention of every 16th request's "
                  "decode rows at steps 0 and 64")
        wl1 = wl
        want1 = lambda kind, rid, step: kind == "dec" and rid % 64 == 0 and step == 0
        sample1 = "chat tree + every 64th request's decode row at step 0"
    else:
        return None

    def run(w, f, threads):
        from oracle.runner import run_workload
        import contextlib
        ctx = contextlib.nullcontext()
        if threads is not None:
            from threadpoolctl import threadpool_limits
            ctx = threadpool_limits(limits=threads)
        with ctx:
            t0 = time.perf_counter()
            tr = run_workload(w, want=f)
            dt = time.perf_counter() - t0
        return dt, sum(per_output(k) for k in tr.outputs)

    dt, toks = run(wl, want, None)
    dt1, toks1 = run(wl1, want1, 1)
    return {"value": toks / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample}; naive tree + float64 full recompute; {toks} tokens in {dt:.1f} s",
            "one_thread": {"value": toks1 / dt1, "unit": "tokens/s", "cores": 1,
                           "sample": f"{sample1}; {toks1} tokens in {dt1:.1f} s"}}


def ceilings(torch):
    """Ceilings measured on this GPU in the same run, beside the published
    peaks: a plain copy (kv_store over 262144 rows of 2 KiB: 1 GiB read and
    1 GiB written) and a large bf16 GEMM (torch / hipBLASLt, 8192^3).  (A
    read-only stream through torch reductions measured 0.9-4.0 TB/s, below
    what the decode kernels reach, so it is not reported as a ceiling.)"""
    from prefix_shared_kv_rt_amd import binding as Bm
    dev = torch.device("cuda:0")
    n, hkv, d = 262144, 8, 128
    pool_k = torch.empty((n + 1, hkv, d), dtype=torch.bfloat16, device=dev)
    pool_v = torch.empty_like(pool_k)
    src_k = torch.randn((n, hkv, d), device=dev).to(torch.bfloat16)
    src_v = torch.randn((n, hkv, d), device=dev).to(torch.bfloat16)
    loc = torch.arange(1, n + 1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)

    def timed(f, reps):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            f()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    t_copy = timed(lambda: Bm.kv_store(pool_k, pool_v, src_k, src_v, loc, stream=st), 20)
    copy_bytes = 4.0 * n * hkv * d * 2
    a = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    bm = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(a, bm), 20)
    del pool_k, pool_v, src_k, src_v, a, bm
    torch.cuda.empty_cache()
    return {"copy_gbs": copy_bytes / t_copy / 1e9, "copy_frac_of_peak": copy_bytes / t_copy / 1e9 / PEAK_HBM_GBS,
            "bf16_gemm_tflops": 2.0 * 8192 ** 3 / t_mm / 1e12,
            "bf16_gemm_frac_of_peak": 2.0 * 8192 ** 3 / t_mm / 1e12 / PEAK_BF16_TFLOPS,
            "what": "measured after the timed steps: kv_store copy of 1 GiB (read) + 1 GiB (write); "
                    "torch.matmul bf16 8192^3"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.workload == "few_shot":
        result, _ = run_few_shot(args, torch)
    elif args.workload == "chat":
        result = run_chat(args, torch)
    elif args.workload == "decode_graph":
        result = run_decode_graph(args, torch)
    else:
        result = run_decode_bench(args, torch)
    if args.workload != "decode_graph":
        result["ceilings"] = ceilings(torch)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(args)
        if cb is not None:
            result["cpu_baseline"] = cb
    print(json.dumps(result))


if __name__ == "__main__":
    main()
