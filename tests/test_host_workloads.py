"""Host decisions of the runtime (C++ tree + pool through the C ABI, batch
scheduler) against the oracle on the full-size workloads: admitted batches,
prefix lengths, every allocated slot, evictions, finishes, hit-rate
integers, the final tree and the final free list must be identical.  No GPU:
the runtime runs its host half only."""

import time

import pytest

from oracle.runner import run_workload
from prefix_shared_kv_rt_amd import binding as B
from prefix_shared_kv_rt_amd.runtime import RadixRuntime, Scheduler
from synth import workloads


def _host_compare(wl, max_running=256, max_extend_tokens=16384, policy="fcfs", chunk_size=None):
    t0 = time.time()
    ora = run_workload(wl, attention=False, max_running=max_running, max_extend_tokens=max_extend_tokens,
                       policy=policy, chunk_size=chunk_size)
    t1 = time.time()
    rt = RadixRuntime(wl.num_slots, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, None,
                      max(max_running, 8), wl.max_ctx, device=None, page_size=wl.page_size)
    sch = Scheduler(rt, wl.requests, None, max_running=max_running, max_extend_tokens=max_extend_tokens,
                    policy=policy, chunk_size=chunk_size).run()
    t2 = time.time()
    print(f"{wl.name} ({policy}): oracle {t1 - t0:.1f}s, runtime {t2 - t1:.1f}s, {len(ora.iterations)} iterations, "
          f"hit {ora.cached_tokens}/{ora.prefill_tokens}", flush=True)
    assert (sch.cached_tokens, sch.prefill_tokens) == (ora.cached_tokens, ora.prefill_tokens)
    assert len(sch.iterations) == len(ora.iterations)
    for i, (a, b) in enumerate(zip(sch.iterations, ora.iterations)):
        assert a["admitted"] == b["admitted"], i
        assert a["extend_loc"] == b["extend_loc"], i
        assert a.get("extend_freed_tokens", 0) == len(b["extend_freed"]), i
        assert a["decode"] == b["decode"], i
        assert a.get("decode_freed_tokens", 0) == len(b["decode_freed"]), i
        assert a["finished"] == b["finished"], i
        assert a.get("chunks") == b.get("chunks"), i
    assert sch.request_slots == ora.request_slots
    assert B.rt_tree_dump(rt.tree) == ora.final_dump
    assert list(B.rt_pool_free_list(rt.pool)) == ora.free_list
    rt.close()
    return ora


@pytest.mark.parametrize("pool", [512, 160])
def test_tiny(pool):
    ora = _host_compare(workloads.tiny(pool))
    assert (ora.cached_tokens, ora.prefill_tokens) == ((96, 192) if pool == 512 else (224, 384))


def test_few_shot_full():
    ora = _host_compare(workloads.few_shot())
    assert ora.cached_tokens == 64 * 1024 and ora.prefill_tokens == 1024 + 64 * 1152


def test_fork_full():
    ora = _host_compare(workloads.fork())
    assert ora.cached_tokens == 128 * 2048 and ora.prefill_tokens == 144 * 2048


def test_long_context_full():
    ora = _host_compare(workloads.long_context())
    assert ora.cached_tokens == 32 * 16384


def test_chat_full_with_eviction():
    wl = workloads.chat()
    ora = _host_compare(wl)
    evicted = sum(len(it["extend_freed"]) + len(it["decode_freed"]) for it in ora.iterations)
    assert evicted > 0
    # re-extension: some turn matched less than the whole history its previous
    # turn inserted (part of it was evicted in between)
    by_rid = {r.rid: r for r in wl.requests}
    matched = {rid: p for it in ora.iterations for rid, p, _ in it["admitted"]}
    redo = [r.rid for r in wl.requests if r.after and r.after[0] != 0 and
            matched[r.rid] < len(by_rid[r.after[0]].prompt) + len(by_rid[r.after[0]].gen)]
    assert redo


@pytest.mark.parametrize("pool", [512, 160])
def test_tiny_lspf(pool):
    _host_compare(workloads.tiny(pool), policy="lspf")


def test_chat_full_lspf():
    """Longest-shared-prefix-first on the full chat workload: identical host
    decisions, and the cache-aware order keeps more of the history cached
    than arrival order does."""
    wl = workloads.chat()
    lspf = _host_compare(wl, policy="lspf")
    fcfs = run_workload(wl, attention=False)
    assert lspf.cached_tokens > fcfs.cached_tokens


@pytest.mark.parametrize("pool,chunk", [(512, 7), (160, 16), (160, 5)])
def test_tiny_chunked(pool, chunk):
    _host_compare(workloads.tiny(pool), chunk_size=chunk)


def test_chat_full_chunked():
    _host_compare(workloads.chat(), chunk_size=512)


def test_long_context_chunked():
    """32 prompts of 32768 tokens through 8192-token chunks: every prompt
    takes four iterations, and decode runs beside the next prompts' chunks."""
    ora = _host_compare(workloads.long_context(), chunk_size=8192)
    assert all(sum(n for _, _, n in it["chunks"]) <= 8192 for it in ora.iterations)
    assert any(it["chunks"] and it["decode"] for it in ora.iterations)


@pytest.mark.parametrize("page", [2, 4])
@pytest.mark.parametrize("pool", [512, 160])
def test_tiny_paged(pool, page):
    _host_compare(workloads.paged(workloads.tiny(pool), page))


@pytest.mark.parametrize("page", [4, 16])
def test_small_chat_paged(page):
    wl = workloads.paged(workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6), page)
    ora = _host_compare(wl, max_running=4, max_extend_tokens=128)
    assert any(it["extend_freed"] or it["decode_freed"] for it in ora.iterations)
    ora = _host_compare(wl, max_running=4, max_extend_tokens=128, policy="lspf")
    ora = _host_compare(wl, max_running=4, chunk_size=24)


def test_few_shot_full_paged():
    ora = _host_compare(workloads.paged(workloads.few_shot(), 16))
    assert ora.cached_tokens == 64 * 1024 and ora.prefill_tokens == 1024 + 64 * 1152


def test_chat_full_paged_with_eviction():
    wl = workloads.paged(workloads.chat(), 16)
    ora = _host_compare(wl)
    assert sum(len(it["extend_freed"]) + len(it["decode_freed"]) for it in ora.iterations) > 0
