"""Pins for the float64 attention oracle and the KV scatter oracle."""

import math

import numpy as np
import pytest

from oracle.attention import causal_attention, recompute_rows, regenerate_qkv
from oracle.kv_store import kv_store
from synth import KIND_K, KIND_V, prefix_hashes_np, qkv_values_np


def _brute(q, k, v, q_pos, scale):
    """Literal definition with Python loops and math.exp."""
    R, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.zeros((R, Hq, D))
    for r in range(R):
        for h in range(Hq):
            kv = h // g
            scores = []
            for i in range(q_pos[r] + 1):
                scores.append(sum(float(q[r, h, d]) * float(k[i, kv, d]) for d in range(D)) * scale)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = sum(w)
            for d in range(D):
                out[r, h, d] = sum(w[i] * float(v[i, kv, d]) for i in range(len(w))) / z
    return out


@pytest.mark.parametrize("hq,hkv,d,lk", [(1, 1, 3, 5), (2, 1, 4, 6), (2, 2, 8, 4), (4, 2, 5, 6)])
def test_brute_force_equals_vectorised(hq, hkv, d, lk):
    rng = np.random.default_rng(hq * 100 + d)
    q = rng.normal(size=(lk, hq, d))
    k = rng.normal(size=(lk, hkv, d))
    v = rng.normal(size=(lk, hkv, d))
    pos = np.arange(lk)
    scale = 1 / math.sqrt(d)
    got = causal_attention(q, k, v, pos, scale)
    assert np.max(np.abs(got - _brute(q, k, v, pos, scale))) < 1e-14
    # non-contiguous query positions (an extend that starts after a prefix)
    pos2 = np.array([lk - 1, 2, 3])
    got2 = causal_attention(q[:3], k, v, pos2, scale)
    assert np.max(np.abs(got2 - _brute(q[:3], k, v, pos2, scale))) < 1e-14


def test_zero_query_gives_running_mean_of_visible_values():
    rng = np.random.default_rng(1)
    k = rng.normal(size=(7, 2, 4))
    v = rng.normal(size=(7, 2, 4))
    q = np.zeros((7, 2, 4))
    out = causal_attention(q, k, v, np.arange(7), 0.5)
    for p in range(7):
        assert np.allclose(out[p], v[:p + 1].mean(axis=0), atol=1e-15)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    k = np.tile(rng.normal(size=(1, 1, 6)), (5, 1, 1))
    v = rng.normal(size=(5, 1, 6))
    q = rng.normal(size=(1, 1, 6))
    out = causal_attention(q, k, v, [4], 0.3)
    assert np.allclose(out[0, 0], v[:, 0].mean(axis=0), atol=1e-14)


def test_dominant_score_selects_its_value_row():
    d = 4
    k = np.zeros((6, 1, d))
    k[3, 0, 0] = 100.0  # score gap of 100 * scale = 50 over every other key
    v = np.arange(6 * d, dtype=np.float64).reshape(6, 1, d)
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    out = causal_attention(q, k, v, [5], 0.5)
    assert np.allclose(out[0, 0], v[3, 0], atol=1e-18 + 1e-12)
    # the same key in the future of the query is invisible
    out2 = causal_attention(q, k, v, [2], 0.5)
    assert np.allclose(out2[0, 0], v[:3, 0].mean(axis=0))


def test_future_keys_do_not_matter():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(4, 2, 5))
    k = rng.normal(size=(9, 2, 5))
    v = rng.normal(size=(9, 2, 5))
    pos = np.array([0, 3, 5, 6])
    a = causal_attention(q, k, v, pos, 0.4)
    k2, v2 = k.copy(), v.copy()
    k2[7:] = 1e3
    v2[7:] = -1e3
    b = causal_attention(q, k2, v2, pos, 0.4)
    assert np.array_equal(a, b)


def test_gqa_equals_mha_with_repeated_kv_and_uses_contiguous_groups():
    rng = np.random.default_rng(4)
    hq, hkv, d, lk = 8, 2, 6, 7
    q = rng.normal(size=(lk, hq, d))
    k = rng.normal(size=(lk, hkv, d))
    v = rng.normal(size=(lk, hkv, d))
    gqa = causal_attention(q, k, v, np.arange(lk), 0.3)
    mha = causal_attention(q, np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1),
                           np.arange(lk), 0.3)
    assert np.max(np.abs(gqa - mha)) < 1e-15
    # q heads 0..3 use kv head 0: changing kv head 1 leaves them untouched
    k2 = k.copy()
    k2[:, 1] = rng.normal(size=(lk, d))
    other = causal_attention(q, k2, v, np.arange(lk), 0.3)
    assert np.array_equal(other[:, :4], gqa[:, :4])
    assert not np.allclose(other[:, 4:], gqa[:, 4:])


def test_scale_enters_the_scores():
    rng = np.random.default_rng(5)
    q = rng.normal(size=(3, 1, 4))
    k = rng.normal(size=(3, 1, 4))
    v = rng.normal(size=(3, 1, 4))
    a = causal_attention(q, k, v, np.arange(3), 0.25)
    b = causal_attention(2 * q, k, v, np.arange(3), 0.125)
    c = causal_attention(q, k, v, np.arange(3), 0.5)
    assert np.allclose(a, b, atol=1e-15)
    assert not np.allclose(a, c)


def test_reuse_invariant_extend_rows_equal_full_prefill_rows():
    """KV depends only on the prefix: rows P..L-1 computed for an extend equal
    the same rows of a full prefill; the last row is the decode output."""
    toks = list(np.random.default_rng(6).integers(0, 1000, size=40))
    full = recompute_rows(toks, np.arange(40), 4, 2, 16, 9, 0.25)
    ext = recompute_rows(toks, np.arange(25, 40), 4, 2, 16, 9, 0.25)
    dec = recompute_rows(toks, [39], 4, 2, 16, 9, 0.25)
    # equal up to the summation order of the matrix products
    assert np.max(np.abs(full[25:] - ext)) < 1e-13
    assert np.max(np.abs(full[39:] - dec)) < 1e-13


def test_cached_prefix_from_a_permuted_pool_equals_recompute():
    """Reuse through a pool: K/V of a shared prefix stored by one request at
    scattered slots, gathered back for another request, give the same
    attention as recomputing everything."""
    rng = np.random.default_rng(7)
    seed, hq, hkv, d = 3, 4, 2, 8
    shared = list(rng.integers(0, 1000, size=12))
    a = shared + list(rng.integers(0, 1000, size=5))
    b = shared + list(rng.integers(0, 1000, size=6))
    n_slots = 64
    kp = np.zeros((n_slots + 1, hkv, d))
    vp = np.zeros((n_slots + 1, hkv, d))
    slots_a = list(rng.permutation(np.arange(1, n_slots + 1))[:len(a)])
    ha = prefix_hashes_np(a, seed)
    kp = kv_store(kp, qkv_values_np(ha, KIND_K, range(hkv), d, seed), slots_a)
    vp = kv_store(vp, qkv_values_np(ha, KIND_V, range(hkv), d, seed), slots_a)
    free = [s for s in range(1, n_slots + 1) if s not in slots_a]
    slots_b = slots_a[:12] + free[:len(b) - 12]
    hb = prefix_hashes_np(b, seed)
    kp = kv_store(kp, qkv_values_np(hb[12:], KIND_K, range(hkv), d, seed), slots_b[12:])
    vp = kv_store(vp, qkv_values_np(hb[12:], KIND_V, range(hkv), d, seed), slots_b[12:])
    q, _, _ = regenerate_qkv(b, np.arange(12, len(b)), hq, hkv, d, seed)
    via_pool = causal_attention(q, kp[slots_b], vp[slots_b], np.arange(12, len(b)), 0.3)
    want = recompute_rows(b, np.arange(12, len(b)), hq, hkv, d, seed, 0.3)
    assert np.max(np.abs(via_pool - want)) < 1e-13


def test_kv_store_replaces_exactly_the_listed_rows():
    rng = np.random.default_rng(8)
    pool = rng.normal(size=(10, 2, 3))
    new = rng.normal(size=(3, 2, 3))
    out = kv_store(pool, new, [7, 2, 5])
    for s in range(10):
        want = {7: new[0], 2: new[1], 5: new[2]}.get(s, pool[s])
        assert np.array_equal(out[s], want)
