"""The oracle scheduler on the small workloads: hit-rate integers against
Theorem 3.1, conservation of slots, and the eviction script of the tiny
workload with a 160-slot pool."""

import random

import numpy as np
import pytest

from oracle.hit_rate import distinct_prefix_tokens, hit_rate, optimal_hit_rate
from oracle.runner import run_workload
from synth import workloads


def _slots_conserved(tr, num_slots):
    tree_slots = []
    for line in tr.final_dump.splitlines():
        v = line.split(" v=")[1]
        tree_slots += [int(s) for s in v.split(",")] if v else []
    assert sorted(tree_slots + tr.free_list) == list(range(1, num_slots + 1))


def test_tiny_512_reaches_theorem_optimum():
    wl = workloads.tiny(512)
    tr = run_workload(wl, attention=False)
    assert (tr.cached_tokens, tr.prefill_tokens) == (96, 192)
    assert tr.cached_tokens * 1 == int(optimal_hit_rate([r.prompt for r in wl.requests]) * 192)
    _slots_conserved(tr, 512)
    # nothing was evicted
    assert all(not r["extend_freed"] and not r["decode_freed"] for r in tr.iterations)


def test_tiny_160_eviction_script():
    """Wave 2 needs 4 x (16 + 8) slots with 32 free: the extend allocation
    of 64 evicts r0's tail then r1's leaf (48 tokens); the 4th decode step
    evicts r2's leaf; the shared prefix and r3's leaf survive."""
    wl = workloads.tiny(160)
    tr = run_workload(wl, attention=False)
    assert (tr.cached_tokens, tr.prefill_tokens) == (96 + 128, 192 + 192)
    rs = tr.request_slots
    wave2 = next(i for i, r in enumerate(tr.iterations) if any(a[0] == 4 for a in r["admitted"]))
    rec = tr.iterations[wave2]
    assert [a[1:] for a in rec["admitted"]] == [(32, 16)] * 4
    assert rec["extend_freed"] == rs[0][32:] + rs[1][32:]
    evict_steps = [i for i, r in enumerate(tr.iterations) if r["decode_freed"]]
    assert len(evict_steps) == 1 and evict_steps[0] == wave2 + 5  # wave-2 decode step 4
    assert tr.iterations[evict_steps[0]]["decode_freed"] == rs[2][32:]
    _slots_conserved(tr, 160)
    survivors = tr.final_dump
    assert ",".join(map(str, rs[3][32:])) in survivors
    for r in (0, 1, 2):
        assert ",".join(map(str, rs[r][32:])) not in survivors


def test_few_shot_and_chat_drain_and_conserve():
    wl = workloads.few_shot(batch=6, prefix_len=64, suffix_len=16, decode_steps=2, num_slots=1000)
    tr = run_workload(wl, attention=False)
    assert tr.cached_tokens == 6 * 64 and tr.prefill_tokens == 64 + 6 * 80
    _slots_conserved(tr, 1000)
    wl = workloads.chat(sessions=6, turns=3, system_len=40, user_lo=8, user_hi=20, gen_len=6)
    tr = run_workload(wl, attention=False)
    _slots_conserved(tr, wl.num_slots)
    assert tr.prefill_tokens == sum(len(r.prompt) for r in wl.requests)
    # a 60% pool forces eviction and re-extension
    assert any(r["extend_freed"] or r["decode_freed"] for r in tr.iterations)


def test_outputs_are_recomputed_rows():
    wl = workloads.tiny(512)
    tr = run_workload(wl, attention=True)
    assert tr.outputs[("ext", 0, 0)].shape == (48, 4, 64)
    assert tr.outputs[("ext", 1, 0)].shape == (16, 4, 64)
    assert tr.outputs[("dec", 2, 7)].shape == (1, 4, 64)
    # r1's extend rows equal the corresponding rows of a full prefill of r1
    from oracle.attention import recompute_rows
    r1 = wl.requests[1]
    full = recompute_rows(r1.prompt, np.arange(48), 4, 4, 64, wl.seed, wl.sm_scale)
    assert np.max(np.abs(full[32:] - tr.outputs[("ext", 1, 0)])) < 1e-13


def _trie_prompts(rng, n):
    """Prompts that share prefixes at several depths: each extends a random
    earlier prompt's prefix (or starts fresh) with new tokens."""
    prompts = []
    for _ in range(n):
        if prompts and rng.random() < 0.8:
            base = rng.choice(prompts)
            head = base[:rng.randint(1, len(base))]
        else:
            head = []
        prompts.append(head + [rng.randrange(1000) for _ in range(rng.randint(1, 12))])
    return [p for i, p in enumerate(prompts) if p not in prompts[:i]]


def _batch(prompts):
    reqs = [workloads.Request(i, list(p), [], ()) for i, p in enumerate(prompts)]
    return workloads.Workload("batch", 0, 1, 1, 8, "f32", max(len(p) for p in prompts), reqs,
                              max_ctx=max(len(p) for p in prompts))


@pytest.mark.parametrize("seed", range(10))
def test_lspf_offline_batch_reaches_theorem_optimum(seed):
    """Theorem 3.1 through the scheduler: a whole batch waiting at once,
    served one request per iteration in longest-shared-prefix-first order
    with a pool exactly as large as the longest request, computes every
    edge of the prompt tree once -- hit rate == H_opt -- whatever the
    arrival order."""
    rng = random.Random(seed)
    prompts = _trie_prompts(rng, 30)
    rng.shuffle(prompts)
    tr = run_workload(_batch(prompts), attention=False, max_running=1, policy="lspf")
    assert tr.prefill_tokens - tr.cached_tokens == distinct_prefix_tokens(prompts)
    assert hit_rate(tr.cached_tokens, tr.prefill_tokens) == optimal_hit_rate(prompts)


def test_lspf_groups_the_explainers_interleaved_queue():
    """The explainer's A1, B1, A2, B2 queue with room for one prefix: arrival
    order recomputes both prefixes, longest-shared-prefix-first serves A2
    right after A1 and B2 right after B1."""
    a, b = list(range(0, 20)), list(range(100, 120))
    prompts = [a + [1], b + [1], a + [2], b + [2]]
    fcfs = run_workload(_batch(prompts), attention=False, max_running=1)
    lspf = run_workload(_batch(prompts), attention=False, max_running=1, policy="lspf")
    assert fcfs.cached_tokens == 0
    assert lspf.cached_tokens == 40
    order = [it["admitted"][0][0] for it in lspf.iterations]
    assert order == [0, 2, 1, 3]


def test_chunked_prefill_script():
    """Chunked prefill on a hand-worked case: A (100-token prompt, 3 output
    tokens) and B (10-token prompt, 2 output tokens) arrive together, chunks
    of 32.  A takes the whole budget for three iterations, its 4-token tail
    leaves room for B's whole prompt in the fourth, both decode from the
    fifth; B finishes after 2 steps and A after 3."""
    a = workloads.Request(0, list(range(1, 101)), [7, 8, 9], ())
    b = workloads.Request(1, list(range(500, 510)), [5, 6], ())
    wl = workloads.Workload("chunks", 0, 1, 1, 8, "f32", 1000, [a, b], max_ctx=110)
    tr = run_workload(wl, attention=False, chunk_size=32)
    chunks = [it["chunks"] for it in tr.iterations]
    assert chunks[:4] == [[(0, 0, 32)], [(0, 32, 32)], [(0, 64, 32)], [(0, 96, 4), (1, 0, 10)]]
    assert [it["admitted"] for it in tr.iterations[:4]] == [[(0, 0, 100)], [], [], [(1, 0, 10)]]
    dec = [[(rid, pos) for rid, pos, _ in it["decode"]] for it in tr.iterations]
    assert dec[:4] == [[], [], [], []]
    assert dec[4:] == [[(0, 100), (1, 10)], [(0, 101), (1, 11)], [(0, 102)]]
    fin = [[f[0] for f in it["finished"]] for it in tr.iterations]
    assert fin[5] == [1] and fin[6] == [0]
    # the slots of A's chunks are consecutive allocations from the FIFO pool
    assert tr.request_slots[0][:100] == list(range(1, 101))


@pytest.mark.parametrize("chunk", [7, 64, 100000])
def test_chunked_prefill_keeps_hit_rate_and_slots(chunk):
    """On the tiny workload (no eviction at 512 slots) chunking changes when
    tokens are computed, not what is cached: the hit-rate integers, every
    request's final slot count and the conservation of slots hold for any
    chunk size; a chunk larger than every iteration's demand reproduces the
    unchunked extend allocations."""
    wl = workloads.tiny(512)
    base = run_workload(wl, attention=False)
    tr = run_workload(wl, attention=False, chunk_size=chunk)
    assert (tr.cached_tokens, tr.prefill_tokens) == (base.cached_tokens, base.prefill_tokens)
    assert {k: len(v) for k, v in tr.request_slots.items()} == {k: len(v) for k, v in base.request_slots.items()}
    _slots_conserved(tr, 512)
    for it in tr.iterations:
        assert sum(n for _, _, n in it["chunks"]) <= chunk
    if chunk == 100000:
        assert [it["extend_loc"] for it in tr.iterations] == [it["extend_loc"] for it in base.iterations]
