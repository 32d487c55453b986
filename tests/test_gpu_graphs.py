"""Decode steps replayed from captured HIP graphs: every replay against the
same decode launched eagerly over the graph's own buffers (bit for bit),
against the float64 oracle over the pool's contents, and against the
runtime's own eager step, with eager work and synchronisation between
replays; padding to the captured sizes; fallback beyond the largest size."""

import numpy as np
import pytest
import torch

from oracle.attention import causal_attention
from oracle.fp8 import dequantize, store_codes
from prefix_shared_kv_rt_amd import binding as B
from prefix_shared_kv_rt_amd.graphs import DecodeGraphs, default_batch_sizes
from prefix_shared_kv_rt_amd.runtime import RadixRuntime

pytestmark = pytest.mark.gpu

HQ, HKV, D, SLOTS, ROWS, CTX = 8, 2, 128, 8192, 20, 300


def _runtime(seed):
    rt = RadixRuntime(SLOTS, HQ, HKV, D, torch.bfloat16, ROWS, CTX)
    g = torch.Generator(device="cuda").manual_seed(seed)
    rt.k_pool[1:] = torch.randn(rt.k_pool[1:].shape, generator=g, device="cuda").to(torch.bfloat16)
    rt.v_pool[1:] = torch.randn(rt.v_pool[1:].shape, generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    # each row's context: distinct slots from the first half of the pool; the
    # new tokens' slots come from the second half
    for r in range(ROWS):
        rt.r2t_host[r, :] = rng.permutation(np.arange(1, SLOTS // 2))[:CTX]
    rt.r2t_dev.copy_(torch.from_numpy(rt.r2t_host))
    return rt


def _runtime_fp8(seed, scales):
    rt = RadixRuntime(SLOTS, HQ, HKV, D, torch.bfloat16, ROWS, CTX, kv_fp8_scales=scales)
    rng = np.random.default_rng(seed)
    # pools hold the codes of N(0, 1) rows, as kv_store_fp8 would leave them
    for pool, scale in ((rt.k_pool, scales[0]), (rt.v_pool, scales[1])):
        pool[1:] = torch.from_numpy(store_codes(rng.standard_normal((SLOTS, HKV, D)), scale)).cuda()
    for r in range(ROWS):
        rt.r2t_host[r, :] = rng.permutation(np.arange(1, SLOTS // 2))[:CTX]
    rt.r2t_dev.copy_(torch.from_numpy(rt.r2t_host))
    return rt


def _oracle(rt, rows, positions, q):
    """The float64 oracle's decode attention over the K/V gathered through
    the device slot table (for FP8 pools: the values the stored codes stand
    for)."""
    r2t = rt.r2t_dev.cpu().numpy()
    if rt.kv_fp8_scales:
        kp = dequantize(rt.k_pool.cpu().numpy(), rt.kv_fp8_scales[0])
        vp = dequantize(rt.v_pool.cpu().numpy(), rt.kv_fp8_scales[1])
    else:
        kp, vp = rt.k_pool.float().cpu().numpy(), rt.v_pool.float().cpu().numpy()
    qh = q.float().cpu().numpy().astype(np.float64)
    out = []
    for i, (r, p) in enumerate(zip(rows, positions)):
        sl = r2t[r, :p + 1].astype(np.int64)
        out.append(causal_attention(qh[i:i + 1], kp[sl].astype(np.float64), vp[sl].astype(np.float64),
                                    np.array([p]), rt.sm_scale)[0])
    return np.stack(out)


def _eager_over_graph_buffers(rt, graphs, n):
    """The decode attention a replay of n requests ran (padded batch, the
    graphs' full context length), launched eagerly into a fresh output."""
    bs = graphs.padded_size(n)
    o = torch.full_like(graphs.o[:bs], float("nan"))
    ws = torch.empty_like(graphs.ws)
    rows, pos = graphs.idx[0, :bs], graphs.idx[1, :bs]
    if rt.kv_fp8_scales:
        B.radix_decode_attention_fp8kv(graphs.q[:bs], o, rt.k_pool, rt.v_pool, rt.r2t_dev, rows, pos, graphs.max_kv,
                                       rt.sm_scale, ws, *rt.kv_fp8_scales, stream=rt.stream)
    else:
        B.radix_decode_attention(graphs.q[:bs], o, rt.k_pool, rt.v_pool, rt.r2t_dev, rows, pos, graphs.max_kv,
                                 rt.sm_scale, ws, stream=rt.stream)
    rt.stream.synchronize()
    return o[:n]


def test_default_sizes_follow_the_handbook_list():
    assert default_batch_sizes(128) == [1, 2, 4] + list(range(8, 129, 8))
    assert default_batch_sizes(20) == [1, 2, 4, 8, 16, 20]


@pytest.mark.parametrize("pool", ["bf16", "fp8"])
def test_graph_replays_match_eager_and_reference(pool):
    rt = _runtime(0) if pool == "bf16" else _runtime_fp8(0, (0.5, 2.0))
    graphs = DecodeGraphs(rt, max_batch=16)
    assert graphs.sizes == [1, 2, 4, 8, 16]
    rng = np.random.default_rng(1)
    free = np.arange(SLOTS // 2, SLOTS + 1)
    for trial, n in enumerate([1, 3, 8, 13, 16, 5, 2, 16]):
        print(f"trial {trial}: batch {n}", flush=True)
        rows = rng.choice(np.array(rt.free_rows), n, replace=False).astype(np.int32)
        positions = rng.integers(0, CTX - 1, n).astype(np.int32)
        slots = rng.choice(free, n, replace=False).astype(np.int32)
        q = torch.randn((n, HQ, D), device="cuda").to(torch.bfloat16)
        k = torch.randn((n, HKV, D), device="cuda").to(torch.bfloat16)
        v = torch.randn((n, HKV, D), device="cuda").to(torch.bfloat16)
        eager = rt.run_decode(rows, positions, slots, q, k, v).float()
        rt.stream.synchronize()
        # eager work between replays
        _ = (torch.randn(1024, device="cuda") * 2).sum().item()
        out_bf16 = graphs.run(rows, positions, slots, q, k, v)
        rt.stream.synchronize()
        out = out_bf16.float()
        assert graphs.replays == trial + 1
        # the same launches eagerly: bit for bit
        again = _eager_over_graph_buffers(rt, graphs, n)
        assert torch.equal(out_bf16.view(torch.int16), again.view(torch.int16))
        want = _oracle(rt, rows, positions, q)
        assert np.abs(out.cpu().numpy() - want).max() <= 2e-2
        # the runtime's eager step (its own split plan): equal up to rounding
        assert (out - eager).abs().max().item() <= 2e-2
    # past the largest captured size: the caller falls back to eager
    n = 17
    rows = np.array(rt.free_rows[:n], dtype=np.int32)
    assert graphs.run(rows, np.zeros(n, np.int32), np.arange(1, n + 1, dtype=np.int32),
                      torch.zeros((n, HQ, D), device="cuda", dtype=torch.bfloat16),
                      torch.zeros((n, HKV, D), device="cuda", dtype=torch.bfloat16),
                      torch.zeros((n, HKV, D), device="cuda", dtype=torch.bfloat16)) is None
    rt.close()


def test_graphs_reserve_the_dummy_row():
    rt = _runtime(2)
    DecodeGraphs(rt, max_batch=4)
    assert ROWS - 1 not in rt.free_rows
    # the dummy requests read and write only slot 0 through that row
    assert int(rt.r2t_dev[ROWS - 1, 0].item()) == 0
    rt.close()
