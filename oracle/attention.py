"""Causal scaled-dot-product attention in float64 (oracle).

The pages never print the attention formula; they say that a request's
cached prefix KV is reused and only the uncached suffix is prefilled
(SGLang explainer, section 04, "hit then prefill only the suffix"; SGLang
paper summary, section 3, "Reuse opportunities": KV depends only on the
prefix tokens).  The plainest reading, used here, is standard causal
attention: query row at position p and query head h attends keys 0..p of
KV head h // (Hq / Hkv), with scores q.k * sm_scale, a max-subtracted
softmax, and a weighted sum of V rows.  No rotary embedding, no soft cap,
no window: the inputs stand for post-projection Q/K/V.

``recompute_rows`` is the oracle for both kernels: it regenerates Q/K/V for
every position from the token sequence (no pool, no slot table, no reuse)
and evaluates the rows asked for.
"""

import numpy as np

from synth import KIND_K, KIND_Q, KIND_V, prefix_hashes_np, qkv_values_np


def causal_attention(q, k, v, q_pos, sm_scale):
    """q: [R, Hq, D]; k, v: [Lk, Hkv, D]; q_pos: [R] key bound per row
    (row r sees keys 0..q_pos[r]).  Returns float64 [R, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    R, Hq, D = q.shape
    Lk, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    out = np.zeros((R, Hq, D), dtype=np.float64)
    future = np.arange(Lk)[None, :] > q_pos[:, None]
    for h in range(Hq):
        kv = h // group
        s = (q[:, h, :] @ k[:, kv, :].T) * sm_scale
        s = np.where(future, -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        out[:, h, :] = (p @ v[:, kv, :]) / p.sum(axis=1, keepdims=True)
    return out


def regenerate_qkv(tokens, positions, num_q_heads, num_kv_heads, head_dim, seed):
    """Fresh Q for ``positions`` and K/V for positions 0..max(positions)."""
    positions = np.asarray(positions, dtype=np.int64)
    n = int(positions.max()) + 1
    hashes = prefix_hashes_np(list(tokens)[:n], seed)
    q = qkv_values_np(hashes[positions], KIND_Q, range(num_q_heads), head_dim, seed)
    k = qkv_values_np(hashes, KIND_K, range(num_kv_heads), head_dim, seed)
    v = qkv_values_np(hashes, KIND_V, range(num_kv_heads), head_dim, seed)
    return q, k, v


def recompute_rows(tokens, positions, num_q_heads, num_kv_heads, head_dim, seed, sm_scale, kv_fp8_scales=None):
    """Attention output (float64 [len(positions), Hq, D]) of the given
    positions of one sequence, from fully recomputed Q/K/V.  With
    ``kv_fp8_scales = (k_scale, v_scale)`` the K and V rows are first
    replaced by what an FP8 (E4M3) pool holds for them (``oracle.fp8``)."""
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size == 0:
        return np.zeros((0, num_q_heads, head_dim))
    q, k, v = regenerate_qkv(tokens, positions, num_q_heads, num_kv_heads, head_dim, seed)
    if kv_fp8_scales is not None:
        from .fp8 import stored_values
        k = stored_values(k, kv_fp8_scales[0])
        v = stored_values(v, kv_fp8_scales[1])
    return causal_attention(q, k, v, positions, sm_scale)
