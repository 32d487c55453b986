"""The same generator as ``synth.gen`` written with torch int64 tensor ops,
so that large inputs can be produced directly in device memory.

int64 addition and multiplication wrap modulo 2**64 in two's complement,
which is the same ring as uint64; right shifts are made logical by
masking.  The results equal ``synth.gen`` bit for bit (checked in tests).
"""

import torch

from .gen import value_keys_np, chain_start


def _s64(u):
    u &= (1 << 64) - 1
    return u - (1 << 64) if u >= (1 << 63) else u


_GAMMA = _s64(0x9E3779B97F4A7C15)
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)


def _lsr(z, k):
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64_t(x):
    z = x + _GAMMA
    z = (z ^ _lsr(z, 30)) * _M1
    z = (z ^ _lsr(z, 27)) * _M2
    return z ^ _lsr(z, 31)


def prefix_hashes_t(tokens, seed=None, start_hash=None):
    """Rolling prefix hashes of a batch of equal-length token rows.

    tokens: int64 tensor [R, L] (any device).  Returns int64 [R, L]."""
    R, L = tokens.shape
    if start_hash is None:
        start_hash = chain_start(seed)
    h = torch.full((R,), _s64(int(start_hash)), dtype=torch.int64, device=tokens.device)
    out = torch.empty((R, L), dtype=torch.int64, device=tokens.device)
    for i in range(L):
        h = splitmix64_t(h ^ (tokens[:, i] + 1))
        out[:, i] = h
    return out


def qkv_values_t(hashes, kind, heads, head_dim, seed, dtype=torch.float32):
    """[N, len(heads), head_dim] values for int64 prefix hashes ``hashes``."""
    keys_np = value_keys_np(kind, heads, head_dim, seed).astype("int64", copy=False)
    keys = torch.from_numpy(keys_np.view("int64")).to(hashes.device)
    x = splitmix64_t(hashes.reshape(-1, 1, 1) ^ keys.unsqueeze(0))
    a = x & 63
    b = _lsr(x, 6) & 63
    c = _lsr(x, 12) & 63
    s = 2 * (a + b + c) - 189
    return (s.to(torch.float32) / 64.0).to(dtype)
