"""Device-resident Q/K/V inputs for a request's positions, from the seeded
generator in ``synth.gen`` (values depend only on the token prefix)."""

import numpy as np
import torch

from .gen import KIND_K, KIND_Q, KIND_V, chain_start, prefix_hashes_from_np, qkv_values_np


class QKVSource:
    """Callable (rid, tokens, positions) -> (q [n, Hq, D], k [n, Hkv, D],
    v [n, Hkv, D]) device tensors.  A request's hash chain is cached and
    extended as its sequence grows."""

    def __init__(self, seed, num_q_heads, num_kv_heads, head_dim, dtype, device="cuda"):
        self.seed = seed
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.dtype = dtype
        self.device = device
        self._chains = {}
        self._start = chain_start(seed)

    def hashes(self, rid, tokens, upto):
        have = self._chains.get(rid)
        if have is None:
            have = np.zeros(0, dtype=np.uint64)
        if have.size < upto:
            start = have[-1] if have.size else np.uint64(self._start)
            more = prefix_hashes_from_np(list(tokens)[have.size:upto], start)
            have = np.concatenate([have, more])
            self._chains[rid] = have
        return have[:upto]

    def host_values(self, rid, tokens, positions):
        positions = np.asarray(positions, dtype=np.int64)
        h = self.hashes(rid, tokens, int(positions.max()) + 1)[positions]
        q = qkv_values_np(h, KIND_Q, range(self.hq), self.d, self.seed)
        k = qkv_values_np(h, KIND_K, range(self.hkv), self.d, self.seed)
        v = qkv_values_np(h, KIND_V, range(self.hkv), self.d, self.seed)
        return q, k, v

    def __call__(self, rid, tokens, positions):
        q, k, v = self.host_values(rid, tokens, positions)
        dev = lambda a: torch.from_numpy(a).to(self.dtype).to(self.device)
        return dev(q), dev(k), dev(v)
