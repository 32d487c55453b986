"""Decode steps replayed from HIP graphs.

The v0.2 handbook (section "CUDA Graph enabled by default") describes the
scheme this follows:

* one graph per batch size in a fixed list, 1, 2, 4 and then every multiple
  of 8, captured once after two warm-up runs;
* static input buffers sized for the largest batch, which every graph's
  kernels read; a step copies its batch into the front of them;
* a smaller batch is padded up to the next captured size with dummy requests
  of length 1 whose new token is written to slot 0, the pool's reserved
  dummy slot, and the padded outputs are dropped;
* batches larger than the largest captured size run eagerly.

A decode step here is one host-to-device copy of the batch's indices (rows,
positions, new slots: one pinned block) and the replay of three kernels on
the runtime's stream: the append of the new tokens (slot table and K/V in
one launch; for FP8 pools the K/V rows are encoded on the way) and decode
attention (split and combine).  The new tokens' Q/K/V
are read from static buffers that a producer fills in place (``inputs``) or
that ``run`` copies into.  The decode kernels' split plan depends on the batch
size and the maximum context length, both fixed at capture: the graphs use
the runtime's full context length (``max_ctx``), so any step whose requests
fit the slot table can replay them; chunks past a request's length are empty
and weigh nothing in the combine.

Nothing inside a captured region allocates or clears memory: the dummy
inputs are written by ordinary copies before the replay.
"""

import numpy as np
import torch

from . import binding as B


def default_batch_sizes(max_batch):
    sizes = [s for s in [1, 2, 4] + list(range(8, max_batch + 1, 8)) if s <= max_batch]
    if not sizes or sizes[-1] != max_batch:
        sizes.append(max_batch)
    return sizes


class DecodeGraphs:
    """Captured decode steps for a ``RadixRuntime``.  Takes the runtime's last
    slot-table row as the dummy requests' row (it is removed from the free
    rows), so the runtime needs one more row than its running requests."""

    def __init__(self, rt, max_batch=None, batch_sizes=None):
        if rt.device is None:
            raise ValueError("decode graphs need a device runtime")
        if rt.max_reqs - 1 in rt.free_rows:
            rt.free_rows.remove(rt.max_reqs - 1)
        else:
            raise ValueError("the slot table's last row is in use; create the graphs before scheduling")
        self.rt = rt
        self.dummy_row = rt.max_reqs - 1
        max_batch = int(max_batch if max_batch is not None else rt.max_reqs - 1)
        self.sizes = sorted(batch_sizes) if batch_sizes else default_batch_sizes(max_batch)
        self.max_bs = self.sizes[-1]
        self.max_kv = rt.max_ctx
        dev = rt.device
        bs = self.max_bs
        # rows, positions and new slots of the padded batch, one device block
        # filled by one copy from one pinned host block
        self.idx = torch.zeros((3, bs), dtype=torch.int32, device=dev)
        self.idx[0].fill_(self.dummy_row)
        self.q = torch.zeros((bs, rt.hq, rt.d), dtype=rt.dtype, device=dev)
        self.k = torch.zeros((bs, rt.hkv, rt.d), dtype=rt.dtype, device=dev)
        self.v = torch.zeros((bs, rt.hkv, rt.d), dtype=rt.dtype, device=dev)
        self.o = torch.zeros((bs, rt.hq, rt.d), dtype=rt.dtype, device=dev)
        nbytes = max(B.radix_decode_workspace_bytes(s, rt.hq, rt.hkv, rt.d, self.max_kv) for s in self.sizes)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.stage = torch.zeros((3, bs), dtype=torch.int32, pin_memory=True)
        self.stage_np = self.stage.numpy()
        self.stage_np[0] = self.dummy_row
        self.copied = None
        self.graphs = {}
        self.replays = 0
        self._capture_all()

    def _launch(self, bs, stream):
        rt = self.rt
        rows, pos, slots = self.idx[0, :bs], self.idx[1, :bs], self.idx[2, :bs]
        if rt.kv_fp8_scales:   # append and decode in the decode's launches
            B.radix_decode_attention_append_fp8kv(self.q[:bs], self.o[:bs], rt.k_pool, rt.v_pool, rt.r2t_dev, rows,
                                                  pos, self.max_kv, rt.sm_scale, self.k[:bs], self.v[:bs], slots,
                                                  self.ws, *rt.kv_fp8_scales, stream=stream)
        elif rt.dtype == torch.bfloat16:
            B.radix_decode_attention_append(self.q[:bs], self.o[:bs], rt.k_pool, rt.v_pool, rt.r2t_dev, rows, pos,
                                            self.max_kv, rt.sm_scale, self.k[:bs], self.v[:bs], slots, self.ws,
                                            stream=stream)
        else:
            B.decode_append(rt.r2t_dev, rows, pos, slots, rt.k_pool, rt.v_pool, self.k[:bs], self.v[:bs],
                            stream=stream)
            B.radix_decode_attention(self.q[:bs], self.o[:bs], rt.k_pool, rt.v_pool, rt.r2t_dev, rows, pos,
                                     self.max_kv, rt.sm_scale, self.ws, stream=stream)

    def _capture_all(self):
        rt = self.rt
        # The dummy row's first entry is slot 0; dummy steps (position 0)
        # rewrite it with slot 0 and read only it.
        rt.r2t_dev[self.dummy_row].zero_()
        side = torch.cuda.Stream(device=rt.device)
        side.wait_stream(rt.stream)
        with torch.cuda.stream(side):
            for bs in self.sizes:
                for _ in range(2):
                    self._launch(bs, side)
                side.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    self._launch(bs, torch.cuda.current_stream())
                self.graphs[bs] = g
        side.synchronize()
        rt.stream.wait_stream(side)

    def padded_size(self, n):
        for s in self.sizes:
            if s >= n:
                return s
        return None

    def inputs(self, n):
        """Views of the static Q/K/V buffers for a step of n requests, for a
        producer to write the new tokens' values in place (then call run
        without q, k, v).  The previous step must have completed."""
        return self.q[:n], self.k[:n], self.v[:n]

    def run(self, rows, positions, slots, q=None, k=None, v=None):
        """One decode step of len(rows) requests; returns o [n, Hq, D] (a view
        of the static output buffer, valid until the next step), or None when
        the batch is larger than the largest captured size or a context is
        longer than the captured one."""
        n = len(rows)
        bs = self.padded_size(n)
        if bs is None or int(max(positions)) + 1 > self.max_kv:
            return None
        rt = self.rt
        if self.copied is not None:
            self.copied.synchronize()
        st = self.stage_np
        st[0, :n], st[0, n:bs] = rows, self.dummy_row
        st[1, :n], st[1, n:bs] = positions, 0
        st[2, :n], st[2, n:bs] = slots, 0
        with torch.cuda.stream(rt.stream):
            self.idx.copy_(self.stage, non_blocking=True)
            self.copied = torch.cuda.Event()
            self.copied.record(rt.stream)
            if q is not None:
                self.q[:n].copy_(q)
                self.k[:n].copy_(k)
                self.v[:n].copy_(v)
            e0 = rt._event() if rt.events is not None else None
            self.graphs[bs].replay()
            if e0 is not None:
                kv = np.asarray(positions, dtype=np.float64) + 1
                eb, ekv = self.q.element_size(), rt.k_pool.element_size()
                nbytes = float(np.sum(kv * (2 * rt.hkv * rt.d * ekv + 4))) + 2.0 * n * rt.hq * rt.d * eb
                rt.events.append(("decode", e0, rt._event(), {"tokens": n, "bytes": nbytes, "graph_batch": bs}))
        self.replays += 1
        return self.o[:n]
