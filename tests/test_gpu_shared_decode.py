"""The shared-prefix decode on the GPU: requests in groups whose slot rows
share their first S_g entries; radix_decode_attention_shared against the
float64 oracle over each request's whole context and against the plain
split-K decode (bf16 and FP8 pools, GQA groups, both head dims, ragged shared
lengths, groups of one, fully shared contexts)."""

import numpy as np
import pytest
import torch

from prefix_shared_kv_rt_amd import binding as B
from tests.gpu_util import host_values, i32, max_err, oracle_rows, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2


def make_shared_case(rng, groups, hq, hkv, d, extra_slots=29, permute_rows=True):
    """groups: list of (shared length S_g, [private length of each member]).
    Each member's context is the group's S_g shared positions (one set of
    slots and K/V values per group) followed by its own private positions.
    Returns pools, slot table, row indices and per-request metadata."""
    members = [(gi, p) for gi, (sg, privs) in enumerate(groups) for p in privs]
    total = sum(sg for sg, _ in groups) + sum(p for _, p in members)
    num_slots = total + extra_slots
    perm = rng.permutation(np.arange(1, num_slots + 1))
    kpool = np.zeros((num_slots + 1, hkv, d))
    vpool = np.zeros((num_slots + 1, hkv, d))
    off = 0
    shared = []
    for sg, _ in groups:
        sl = perm[off:off + sg]
        off += sg
        k, v = host_values(rng, (sg, hkv, d), "bf16"), host_values(rng, (sg, hkv, d), "bf16")
        kpool[sl], vpool[sl] = k, v
        shared.append((sl, k, v))
    n = len(members)
    ctx = [groups[gi][0] + p for gi, p in members]
    stride = max(sg for sg, _ in groups) + max(max(1, p) for _, p in members) + 7
    r2t = np.zeros((n + 5, stride), dtype=np.int32)
    rows = (rng.permutation(n + 5)[:n] if permute_rows else np.arange(n)).astype(np.int32)
    ks, vs = [], []
    for b, (gi, p) in enumerate(members):
        sl = perm[off:off + p]
        off += p
        k, v = host_values(rng, (p, hkv, d), "bf16"), host_values(rng, (p, hkv, d), "bf16")
        kpool[sl], vpool[sl] = k, v
        r2t[rows[b], :groups[gi][0]] = shared[gi][0]
        r2t[rows[b], groups[gi][0]:ctx[b]] = sl
        ks.append(np.concatenate([shared[gi][1], k]))
        vs.append(np.concatenate([shared[gi][2], v]))
    gs = np.zeros(len(groups) + 1, dtype=np.int32)
    gs[1:] = np.cumsum([len(privs) for _, privs in groups])
    return dict(kpool=kpool, vpool=vpool, r2t=r2t, rows=rows, k=ks, v=vs,
                prefix_lens=np.array(ctx, dtype=np.int32) - 1,
                shared_lens=np.array([groups[gi][0] for gi, _ in members], dtype=np.int32), group_start=gs,
                max_group=max(len(privs) for _, privs in groups), max_shared=max(sg for sg, _ in groups),
                max_private=max(max(1, p) for _, p in members))


CASES = [
    # (groups, hq, hkv, d)
    ([(1024, [1 + (7 * i) % 130 for i in range(64)])], 32, 8, 128),          # few-shot shaped
    ([(2048, [1 + i % 5 for i in range(8)]) for _ in range(16)], 32, 8, 128),  # fork shaped
    ([(0, [40]), (77, [3, 1, 200]), (0, [1, 2]), (300, [1])], 12, 4, 64),   # ragged, groups of one
    ([(513, [0, 0, 5, 64])], 64, 8, 128),                                     # contexts wholly shared
    ([(8192, [100, 1, 37, 250])], 16, 2, 128),                                # long shared part
]


def _run(case, q, hq, hkv, d, fp8=None):
    kp, vp = case["kp"], case["vp"]
    ws = torch.empty(B.radix_decode_shared_workspace_bytes(q.shape[0], hq, hkv, d, len(case["group_start"]) - 1,
                                                           case["max_group"], case["max_shared"],
                                                           case["max_private"]), dtype=torch.uint8, device="cuda")
    o = torch.full_like(q, float("nan"))
    args = (q, o, kp, vp, i32(case["r2t"]), i32(case["rows"]), i32(case["prefix_lens"]), i32(case["shared_lens"]),
            i32(case["group_start"]), case["max_group"], case["max_shared"], case["max_private"], 1.0 / np.sqrt(d), ws)
    if fp8:
        B.radix_decode_attention_shared_fp8kv(*args, *fp8)
    else:
        B.radix_decode_attention_shared(*args)
    return o


def _run_plain(case, q, hq, hkv, d, fp8=None):
    kp, vp = case["kp"], case["vp"]
    max_kv = int(case["prefix_lens"].max()) + 1
    ws = torch.empty(B.radix_decode_workspace_bytes(q.shape[0], hq, hkv, d, max_kv), dtype=torch.uint8, device="cuda")
    o = torch.full_like(q, float("nan"))
    args = (q, o, kp, vp, i32(case["r2t"]), i32(case["rows"]), i32(case["prefix_lens"]), max_kv, 1.0 / np.sqrt(d), ws)
    if fp8:
        B.radix_decode_attention_fp8kv(*args, *fp8)
    else:
        B.radix_decode_attention(*args)
    return o


@pytest.fixture(params=["one launch", "two launches", "two streams"])
def streams(request, monkeypatch):
    """How the shared pass runs beside the private split: in one launch with
    it (the default for private chunks of up to 1024 keys below 128 MiB of
    private K/V), as a launch of its own before it on the caller's stream
    (RADIXRT_SHARED_FUSED=0), or forked onto the
    library's second stream (RADIXRT_FORK_MIN_BYTES=0)."""
    monkeypatch.delenv("RADIXRT_FORK_MIN_BYTES", raising=False)
    monkeypatch.delenv("RADIXRT_SHARED_FUSED", raising=False)
    if request.param == "two launches":
        monkeypatch.setenv("RADIXRT_SHARED_FUSED", "0")
    elif request.param == "two streams":
        monkeypatch.setenv("RADIXRT_FORK_MIN_BYTES", "0")
    return request.param


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_shared_decode_matches_oracle_and_plain_decode(ci, streams):
    groups, hq, hkv, d = CASES[ci]
    print(f"shared decode case {ci} ({streams}): {len(groups)} groups, hq={hq} hkv={hkv} d={d}", flush=True)
    rng = np.random.default_rng(900 + ci)
    case = make_shared_case(rng, groups, hq, hkv, d)
    case["kp"], case["vp"] = to_dev(case["kpool"], "bf16"), to_dev(case["vpool"], "bf16")
    n = len(case["prefix_lens"])
    q_host = host_values(rng, (n, hq, d), "bf16")
    q = to_dev(q_host, "bf16")
    o = _run(case, q, hq, hkv, d)
    o_plain = _run_plain(case, q, hq, hkv, d)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(n):
        pos = int(case["prefix_lens"][b])
        want = oracle_rows(q_host[b:b + 1], case["k"][b], case["v"][b], np.array([pos]), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[b:b + 1], want))
    diff = float((o.float() - o_plain.float()).abs().max())
    print(f"  max abs err {worst:.3e}, against the plain decode {diff:.3e}", flush=True)
    assert worst <= TOL
    assert diff <= TOL


@pytest.mark.parametrize("ci,scales", [(0, (1.0, 1.0)), (2, (0.5, 2.0))])
def test_shared_decode_fp8_pool_matches_plain_fp8_decode(ci, scales):
    groups, hq, hkv, d = CASES[ci]
    print(f"shared decode fp8 case {ci} scales {scales}", flush=True)
    rng = np.random.default_rng(950 + ci)
    case = make_shared_case(rng, groups, hq, hkv, d)
    # E4M3 codes of the bf16 values at the given scales
    kb, vb = to_dev(case["kpool"], "bf16"), to_dev(case["vpool"], "bf16")
    case["kp"] = torch.zeros(kb.shape, dtype=torch.uint8, device="cuda")
    case["vp"] = torch.zeros_like(case["kp"])
    loc = torch.arange(kb.shape[0], dtype=torch.int32, device="cuda")
    B.kv_store_fp8(case["kp"], case["vp"], kb, vb, loc, *scales)
    n = len(case["prefix_lens"])
    q = to_dev(host_values(rng, (n, hq, d), "bf16"), "bf16")
    o = _run(case, q, hq, hkv, d, fp8=scales)
    o_plain = _run_plain(case, q, hq, hkv, d, fp8=scales)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    diff = float((o.float() - o_plain.float()).abs().max())
    print(f"  against the plain fp8 decode {diff:.3e}", flush=True)
    assert diff <= TOL


def test_shared_decode_rejects_bad_arguments():
    q = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((10, 2, 64), dtype=torch.bfloat16, device="cuda")
    r2t, z, gs = i32(np.zeros((4, 16))), i32(np.zeros(4)), i32(np.array([0, 4]))
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for mg, ms, mp in [(0, 4, 4), (4, -1, 4), (4, 4, 0), (4, 12, 8)]:   # the last one exceeds the stride
        with pytest.raises(B.RadixRTError):
            B.radix_decode_attention_shared(q, q, kp, kp, r2t, None, z, z, gs, mg, ms, mp, 0.125, ws)
    with pytest.raises(B.RadixRTError):  # workspace too small
        B.radix_decode_attention_shared(q, q, kp, kp, r2t, None, z, z, gs, 4, 4, 4, 0.125, ws[:16])


@pytest.mark.parametrize("ci", [0, 2])
def test_shared_decode_replays_from_a_captured_graph(ci, streams):
    """Captured in a HIP graph, the shared decode (on one stream, or with its
    shared pass forked onto the library's second stream and joined back)
    replays bit for bit what the eager call computes, with eager work and
    synchronisation between replays; the eager call matches the oracle."""
    groups, hq, hkv, d = CASES[ci]
    print(f"shared decode graph case {ci} ({streams})", flush=True)
    rng = np.random.default_rng(990 + ci)
    case = make_shared_case(rng, groups, hq, hkv, d)
    kp, vp = to_dev(case["kpool"], "bf16"), to_dev(case["vpool"], "bf16")
    n = len(case["prefix_lens"])
    q_host = host_values(rng, (n, hq, d), "bf16")
    q = to_dev(q_host, "bf16")
    dev = [i32(case[k]) for k in ("r2t", "rows", "prefix_lens", "shared_lens", "group_start")]
    ws = torch.empty(B.radix_decode_shared_workspace_bytes(n, hq, hkv, d, len(case["group_start"]) - 1,
                                                           case["max_group"], case["max_shared"],
                                                           case["max_private"]), dtype=torch.uint8, device="cuda")

    def call(o):
        B.radix_decode_attention_shared(q, o, kp, vp, *dev, case["max_group"], case["max_shared"],
                                        case["max_private"], 1.0 / np.sqrt(d), ws)

    eager = torch.full_like(q, float("nan"))
    call(eager)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(n):
        pos = int(case["prefix_lens"][b])
        want = oracle_rows(q_host[b:b + 1], case["k"][b], case["v"][b], np.array([pos]), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(eager[b:b + 1], want))
    assert worst <= TOL
    out = torch.full_like(q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)          # warm-up on the capturing stream
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call(out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        _ = (torch.randn(4096, device="cuda") * 2).sum().item()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


def test_shared_decode_long_private_tails(streams, monkeypatch):
    """Private tails long enough that each (request, KV head) splits them
    into two chunks of more than 1024 keys (64 requests x Hkv 8 = 512 units,
    tails of 2100..2399 keys, D 64).  The library sends such chunks to the
    two-launch path; the single launch, forced here through
    RADIXRT_SHARED_FUSED=force, streams each chunk through its ring of 1024
    slot indices, refilled window by window."""
    if streams == "one launch":
        monkeypatch.setenv("RADIXRT_SHARED_FUSED", "force")
    groups = [(96, [2100 + (37 * i) % 300 for i in range(64)])]
    hq, hkv, d = 8, 8, 64
    print(f"shared decode, long private tails ({streams})", flush=True)
    rng = np.random.default_rng(1234)
    case = make_shared_case(rng, groups, hq, hkv, d)
    case["kp"], case["vp"] = to_dev(case["kpool"], "bf16"), to_dev(case["vpool"], "bf16")
    n = len(case["prefix_lens"])
    q_host = host_values(rng, (n, hq, d), "bf16")
    q = to_dev(q_host, "bf16")
    o = _run(case, q, hq, hkv, d)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(0, n, 7):
        pos = int(case["prefix_lens"][b])
        want = oracle_rows(q_host[b:b + 1], case["k"][b], case["v"][b], np.array([pos]), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[b:b + 1], want))
    print(f"  max abs err {worst:.3e}", flush=True)
    assert worst <= TOL
