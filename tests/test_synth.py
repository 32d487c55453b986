"""The shared input generator: exactness, the prefix property, and the
numpy/torch agreement the GPU-side inputs rely on."""

import numpy as np
import torch

from synth import KIND_K, KIND_Q, prefix_hashes_np, qkv_values_np, splitmix64_np
from synth import torch_gen
from synth import workloads


def test_splitmix64_published_vector():
    # SplitMix64 from state 0: the first output of the generator whose state
    # advances by the golden-ratio gamma is 0xE220A8397B1DCDAF.
    assert int(splitmix64_np(np.array([0], dtype=np.uint64))[0]) == 0xE220A8397B1DCDAF


def test_values_exact_in_bf16_and_near_standard_normal():
    toks = np.random.default_rng(0).integers(0, 1000, size=2000)
    v = qkv_values_np(prefix_hashes_np(toks, 5), KIND_K, range(4), 64, 5)
    assert np.array_equal(torch.from_numpy(v).to(torch.bfloat16).float().numpy(), v)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    s = v * 64
    assert np.all(np.abs(s) <= 189) and np.all(s % 2 == 1)


def test_shared_prefix_gives_identical_values_and_divergence_changes_them():
    a = [5, 6, 7, 8, 9]
    b = [5, 6, 7, 1, 9]
    va = qkv_values_np(prefix_hashes_np(a, 1), KIND_Q, range(2), 8, 1)
    vb = qkv_values_np(prefix_hashes_np(b, 1), KIND_Q, range(2), 8, 1)
    assert np.array_equal(va[:3], vb[:3])
    assert not np.array_equal(va[3:], vb[3:])


def test_torch_generator_matches_numpy_bit_for_bit():
    toks = np.random.default_rng(1).integers(0, 1000, size=(3, 64))
    hn = np.stack([prefix_hashes_np(t, 11) for t in toks])
    ht = torch_gen.prefix_hashes_t(torch.from_numpy(toks), seed=11)
    assert np.array_equal(hn.view(np.int64), ht.numpy())
    vn = qkv_values_np(hn.reshape(-1), KIND_K, [0, 2, 7], 32, 11)
    vt = torch_gen.qkv_values_t(ht.reshape(-1), KIND_K, [0, 2, 7], 32, 11)
    assert np.array_equal(vn, vt.numpy())


def test_workload_shapes():
    t = workloads.tiny(512)
    assert len(t.requests) == 4 and all(len(r.prompt) == 48 and len(r.gen) == 8 for r in t.requests)
    assert len({r.prompt[32] for r in t.requests}) == 4
    assert len(workloads.tiny(160).requests) == 8
    f = workloads.few_shot(batch=4, decode_steps=1)
    assert [len(r.prompt) for r in f.requests] == [1024] + [1152] * 4
    c = workloads.chat(sessions=4)
    assert len(c.requests) == 1 + 16


def test_row_hash_chains_equal_single_chains():
    from synth import chain_start, prefix_hashes_rows_np
    toks = np.random.default_rng(2).integers(0, 1000, size=(4, 33))
    rows = prefix_hashes_rows_np(toks, [chain_start(3)] * 4)
    assert np.array_equal(rows, np.stack([prefix_hashes_np(t, 3) for t in toks]))
