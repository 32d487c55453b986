"""Workload parity on the GPU: the runtime (C++ tree + HIP kernels) and the
oracle (naive tree + float64 full recompute) run the same seeded workload;
host decisions must be bit-identical and attention within tolerance."""

import numpy as np
import pytest
import torch

from oracle.runner import run_workload
from prefix_shared_kv_rt_amd.graphs import DecodeGraphs
from prefix_shared_kv_rt_amd.runtime import RadixRuntime, Scheduler
from synth import workloads
from synth.sources import QKVSource

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {"f32": 1e-4, "bf16": 2e-2}


def run_both(wl, want=None, max_running=256, max_extend_tokens=16384, max_reqs=None, policy="fcfs", graphs=False,
             chunk_size=None, kv_fp8_scales=None, mixed=False, shared_decode=False, shared_min=256):
    ora = run_workload(wl, want=want, max_running=max_running, max_extend_tokens=max_extend_tokens, policy=policy,
                       chunk_size=chunk_size, kv_fp8_scales=kv_fp8_scales)
    outs = {}

    def record(kind, rid, step, o):
        if want is None or want(kind, rid, step):
            outs[(kind, rid, step)] = o.float().cpu().numpy()

    rt = RadixRuntime(wl.num_slots, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, TORCH_DT[wl.dtype],
                      max_reqs or max(max_running, 8), wl.max_ctx, kv_fp8_scales=kv_fp8_scales,
                      page_size=wl.page_size)
    src = QKVSource(wl.seed, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, TORCH_DT[wl.dtype])
    dg = DecodeGraphs(rt, max_batch=max_running) if graphs else None
    sch = Scheduler(rt, wl.requests, src, max_running=max_running, max_extend_tokens=max_extend_tokens,
                    skip_extend_attention=wl.skip_extend_attention, record=record, policy=policy, graphs=dg,
                    chunk_size=chunk_size, mixed=mixed, shared_decode=shared_decode,
                    shared_min=shared_min).run()
    if graphs:
        assert dg.replays > 0
    from prefix_shared_kv_rt_amd import binding as B
    final_dump = B.rt_tree_dump(rt.tree)
    free_list = list(B.rt_pool_free_list(rt.pool))
    rt.close()
    return ora, sch, outs, final_dump, free_list


def check_host_identical(ora, sch, final_dump, free_list):
    assert (sch.cached_tokens, sch.prefill_tokens) == (ora.cached_tokens, ora.prefill_tokens)
    assert len(sch.iterations) == len(ora.iterations)
    for a, b in zip(sch.iterations, ora.iterations):
        assert a["admitted"] == b["admitted"]
        assert a["extend_loc"] == b["extend_loc"]
        assert a.get("extend_freed_tokens", 0) == len(b["extend_freed"])
        assert a["decode"] == b["decode"]
        assert a.get("decode_freed_tokens", 0) == len(b["decode_freed"])
        assert a["finished"] == b["finished"]
        assert a.get("chunks") == b.get("chunks")
    assert sch.request_slots == ora.request_slots
    assert final_dump == ora.final_dump
    assert free_list == ora.free_list


def check_outputs(ora, outs, tol):
    assert set(outs) == set(ora.outputs)
    worst = 0.0
    for key, want in ora.outputs.items():
        worst = max(worst, float(np.max(np.abs(outs[key].astype(np.float64) - want))))
    print(f"  {len(outs)} outputs, max abs err {worst:.3e}", flush=True)
    assert worst <= tol


@pytest.mark.parametrize("pool", [512, 160])
def test_tiny_workload(pool):
    print(f"tiny workload pool={pool}", flush=True)
    wl = workloads.tiny(pool)
    ora, sch, outs, dump, free = run_both(wl)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["f32"])
    assert (sch.cached_tokens, sch.prefill_tokens) == ((96, 192) if pool == 512 else (224, 384))


def test_tiny_workload_in_bf16():
    print("tiny workload bf16", flush=True)
    wl = workloads.tiny(160)
    wl.dtype = "bf16"
    ora, sch, outs, dump, free = run_both(wl)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


def test_small_few_shot_bf16():
    print("few-shot (8 x [256 + 64], 2 decode steps)", flush=True)
    wl = workloads.few_shot(batch=8, prefix_len=256, suffix_len=64, decode_steps=2, num_slots=4096)
    ora, sch, outs, dump, free = run_both(wl)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


@pytest.mark.parametrize("policy,graphs,chunk", [("fcfs", False, None), ("lspf", False, None), ("fcfs", True, None),
                                                 ("fcfs", False, 24)])
def test_small_chat_with_eviction_bf16(policy, graphs, chunk):
    print(f"chat (6 sessions x 3 turns, pool 60%, {policy}, graphs {graphs}, chunk {chunk})", flush=True)
    wl = workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6)
    sel = lambda kind, rid, step: kind == "ext" or step in (0, 5)
    ora, sch, outs, dump, free = run_both(wl, want=sel, max_running=4, max_extend_tokens=128, policy=policy,
                                          graphs=graphs, chunk_size=chunk)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])
    assert any(len(it["extend_freed"]) or len(it["decode_freed"]) for it in ora.iterations)


@pytest.mark.timeout(900)
def test_chat_full_size_sampled():
    """The full multi-turn chat workload (256 sessions x 4 turns, pool at 60%
    of the working set, eviction and re-extension): every host decision
    bit-exact, attention of sampled requests (every 64th) within tolerance."""
    print("chat full size", flush=True)
    wl = workloads.chat()
    sel = lambda kind, rid, step: rid % 64 == 5 and (kind == "ext" or step in (0, 127))
    ora, sch, outs, dump, free = run_both(wl, want=sel)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


def test_chunked_prefill_few_shot_bf16():
    """Prompts of 1024 + 96 tokens through 160-token chunks beside decode:
    every chunk's rows against the oracle's rows of the same positions."""
    print("few-shot 6 x (1024 + 96), chunks of 160", flush=True)
    wl = workloads.few_shot(batch=6, suffix_len=96, decode_steps=4, num_slots=8192)
    ora, sch, outs, dump, free = run_both(wl, chunk_size=160)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])
    assert max(len(it["chunks"]) for it in ora.iterations) > 1


@pytest.mark.parametrize("scales,graphs", [((1.0, 1.0), False), ((0.5, 2.0), False), ((0.5, 2.0), True)])
def test_small_chat_fp8_pool(scales, graphs):
    """The small chat workload with FP8 pools (decode steps eager or replayed
    from HIP graphs): host decisions as with bf16, attention against the
    oracle over the values the FP8 pool holds."""
    print(f"chat (6 sessions x 3 turns, pool 60%, fp8 pool {scales}, graphs {graphs})", flush=True)
    wl = workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6)
    sel = lambda kind, rid, step: kind == "ext" or step in (0, 5)
    ora, sch, outs, dump, free = run_both(wl, want=sel, max_running=4, max_extend_tokens=128, kv_fp8_scales=scales,
                                          graphs=graphs)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


@pytest.mark.parametrize("page,graphs,chunk", [(16, False, None), (4, True, None), (16, False, 24)])
def test_small_chat_paged(page, graphs, chunk):
    """Pools of pages: slots by the page rule in the slot table, the same
    kernels; host decisions bit-exact and attention within tolerance."""
    print(f"chat (6 sessions x 3 turns, pool 60%, pages of {page}, graphs {graphs}, chunk {chunk})", flush=True)
    wl = workloads.paged(workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6),
                         page)
    sel = lambda kind, rid, step: kind == "ext" or step in (0, 5)
    ora, sch, outs, dump, free = run_both(wl, want=sel, max_running=4, max_extend_tokens=128, graphs=graphs,
                                          chunk_size=chunk)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


def test_small_few_shot_paged():
    print("few-shot (8 x [256 + 64], 2 decode steps), pages of 16", flush=True)
    wl = workloads.paged(workloads.few_shot(batch=8, prefix_len=256, suffix_len=64, decode_steps=2,
                                            num_slots=4096), 16)
    ora, sch, outs, dump, free = run_both(wl)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


@pytest.mark.parametrize("chunk,page,fp8,graphs", [(None, 1, False, False), (24, 1, False, True), (24, 16, False, False),
                                                   (None, 4, True, False)])
def test_small_chat_mixed_launch(chunk, page, fp8, graphs):
    """Iterations with extend chunks and decode rows run them as one
    radix_mixed_attention launch: host decisions as always, every extend
    and decode output against the oracle's."""
    print(f"chat mixed launch (chunk {chunk}, pages of {page}, fp8 {fp8}, graphs {graphs})", flush=True)
    wl = workloads.paged(workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6), page)
    scales = (0.5, 2.0) if fp8 else None
    ora, sch, outs, dump, free = run_both(wl, max_running=4, max_extend_tokens=128, chunk_size=chunk,
                                          kv_fp8_scales=scales, mixed=True, graphs=graphs)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])
    print(f"  {sch.mixed_launches} mixed launches", flush=True)
    assert sch.mixed_launches > 0


def test_small_fork_mixed_falls_back_when_a_prompt_finishes():
    """Fork heads finish right after their extend while earlier branches
    decode: those iterations keep separate launches (the heads' freed slots
    may be handed to the decode rows); results as the oracle's."""
    print("fork 6 prompts x 200 tokens x 3 branches x 4 steps, mixed", flush=True)
    wl = workloads.fork(prompts=6, prompt_len=200, branches=3, decode_steps=4, num_slots=4096)
    ora, sch, outs, dump, free = run_both(wl, max_running=8, max_extend_tokens=400, mixed=True)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])


@pytest.mark.parametrize("page,fp8", [(1, False), (16, False), (1, True)])
def test_small_chat_shared_decode(page, fp8):
    """Decode batches whose slot rows begin with a common run (the system
    prompt every session matched) go through radix_decode_attention_shared:
    host decisions as always, every output against the oracle's."""
    print(f"chat shared decode (pages of {page}, fp8 {fp8})", flush=True)
    wl = workloads.paged(workloads.chat(sessions=6, turns=3, system_len=64, user_lo=16, user_hi=48, gen_len=6), page)
    sel = lambda kind, rid, step: kind == "dec" or step == 0
    ora, sch, outs, dump, free = run_both(wl, want=sel, max_running=4, max_extend_tokens=128,
                                          kv_fp8_scales=(0.5, 2.0) if fp8 else None, shared_decode=True,
                                          shared_min=16)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])
    print(f"  {sch.shared_decodes} shared decodes", flush=True)
    assert sch.shared_decodes > 0


def test_small_few_shot_shared_decode():
    print("few-shot (8 x [256 + 64], 2 decode steps), shared decode", flush=True)
    wl = workloads.few_shot(batch=8, prefix_len=256, suffix_len=64, decode_steps=2, num_slots=4096)
    ora, sch, outs, dump, free = run_both(wl, shared_decode=True, shared_min=64)
    check_host_identical(ora, sch, dump, free)
    check_outputs(ora, outs, TOL["bf16"])
    assert sch.shared_decodes > 0
