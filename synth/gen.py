"""Integer-only counter-based value generator (numpy implementation).

splitmix64 is Steele, Lea and Flood's SplitMix64 finaliser ("Fast splittable
pseudorandom number generators", OOPSLA 2014): add the golden-ratio
increment, then two xor-shift-multiply rounds and a final xor-shift.
"""

import numpy as np

MASK64 = (1 << 64) - 1
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

KIND_Q, KIND_K, KIND_V = 1, 2, 3

# Salt that separates the hash chain from the per-(kind, head, dim) keys.
_CHAIN_SALT = 0x243F6A8885A308D3
_KEY_SALT = 0x13198A2E03707344


def splitmix64_np(x):
    """SplitMix64 finaliser applied elementwise to a uint64 array."""
    z = np.asarray(x, dtype=np.uint64) + _GAMMA
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _chain_start(seed):
    return splitmix64_np(np.array([(seed * 0x2545F4914F6CDD1D + _CHAIN_SALT) & MASK64],
                                  dtype=np.uint64))[0]


def prefix_hashes_from_np(tokens, start_hash):
    """Continue the rolling hash from ``start_hash`` (the hash of the
    position before tokens[0]).  Returns uint64 [len(tokens)]."""
    toks = np.asarray(tokens, dtype=np.int64)
    out = np.empty(toks.shape[0], dtype=np.uint64)
    h = np.uint64(start_hash)
    with np.errstate(over="ignore"):
        for i in range(toks.shape[0]):
            h = splitmix64_np(np.array([h ^ np.uint64(int(toks[i]) + 1)], dtype=np.uint64))[0]
            out[i] = h
    return out


def prefix_hashes_rows_np(tokens, start_hashes):
    """Rolling hashes of several rows at once: tokens int [R, L], start_hashes
    uint64 [R] (hash before each row's first token).  Returns uint64 [R, L]."""
    toks = np.asarray(tokens, dtype=np.int64)
    R, L = toks.shape
    out = np.empty((R, L), dtype=np.uint64)
    h = np.asarray(start_hashes, dtype=np.uint64).copy()
    t1 = (toks + 1).astype(np.uint64)
    with np.errstate(over="ignore"):
        for i in range(L):
            h = splitmix64_np(h ^ t1[:, i])
            out[:, i] = h
    return out


def prefix_hashes_np(tokens, seed):
    """Rolling hash of tokens[0..i] for every i (uint64 [len(tokens)])."""
    return prefix_hashes_from_np(tokens, _chain_start(seed))


def chain_start(seed):
    """Hash of the empty prefix for ``seed``."""
    return int(_chain_start(seed))


def value_keys_np(kind, heads, head_dim, seed):
    """uint64 [len(heads), head_dim] per-(kind, head, dim) keys."""
    heads = np.asarray(heads, dtype=np.uint64)
    dims = np.arange(head_dim, dtype=np.uint64)
    c = (np.uint64(kind) << np.uint64(40)) | (heads[:, None] << np.uint64(20)) | dims[None, :]
    s = np.uint64((seed * 0x9E3779B97F4A7C15 + _KEY_SALT) & MASK64)
    return splitmix64_np(c ^ s)


def _bits_to_values(x):
    a = (x & np.uint64(63)).astype(np.int32)
    b = ((x >> np.uint64(6)) & np.uint64(63)).astype(np.int32)
    c = ((x >> np.uint64(12)) & np.uint64(63)).astype(np.int32)
    s = 2 * (a + b + c) - 189
    return s.astype(np.float32) / np.float32(64.0)


def qkv_values_np(hashes, kind, heads, head_dim, seed):
    """float32 [len(hashes), len(heads), head_dim] values for positions whose
    prefix hashes are ``hashes``.  Values are exact in bf16."""
    h = np.asarray(hashes, dtype=np.uint64)
    keys = value_keys_np(kind, heads, head_dim, seed)
    x = splitmix64_np(h[:, None, None] ^ keys[None, :, :])
    return _bits_to_values(x)
