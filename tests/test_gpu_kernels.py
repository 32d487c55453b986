"""Kernel parity on the GPU: kv_store bit-exact; extend and decode attention
against the float64 oracle on seeded inputs (several tiles, ragged tails,
GQA groups, both head dims, both dtypes); split and slot-placement
invariance."""

import numpy as np
import pytest
import torch

from prefix_shared_kv_rt_amd import binding as B
from tests.gpu_util import DT, TOL, host_values, i32, make_pool_case, max_err, oracle_rows, to_dev

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hkv,d", [(8, 128), (4, 64), (1, 128)])
def test_kv_store_bit_exact(dtype, hkv, d):
    _announce(f"kv_store {dtype} hkv={hkv} d={d}")
    rng = np.random.default_rng(hkv * 1000 + d)
    n_slots, T = 3000, 777
    kp = torch.from_numpy(rng.standard_normal((n_slots + 1, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    vp = torch.from_numpy(rng.standard_normal((n_slots + 1, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    kn = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    vn = torch.from_numpy(rng.standard_normal((T, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    loc = rng.permutation(np.arange(1, n_slots + 1))[:T]
    want_k, want_v = kp.cpu().clone(), vp.cpu().clone()
    want_k[torch.from_numpy(loc)] = kn.cpu()
    want_v[torch.from_numpy(loc)] = vn.cpu()
    B.kv_store(kp, vp, kn, vn, i32(loc))
    torch.cuda.synchronize()
    assert torch.equal(kp.cpu().view(torch.int16 if dtype == "bf16" else torch.int32),
                       want_k.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(vp.cpu().view(torch.int16 if dtype == "bf16" else torch.int32),
                       want_v.view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 8, 128), ("f32", 2, 64)])
def test_decode_append_bit_exact(dtype, hkv, d):
    """The fused append equals the slot-table scatter plus kv_store, bit for
    bit, including padding rows that all write slot 0 through one row."""
    _announce(f"decode_append {dtype} hkv={hkv} d={d}")
    rng = np.random.default_rng(5 + d)
    n_slots, n, stride, rows_n = 2000, 300, 97, 400
    kp = torch.from_numpy(rng.standard_normal((n_slots + 1, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    vp = torch.from_numpy(rng.standard_normal((n_slots + 1, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    kn = torch.from_numpy(rng.standard_normal((n, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    vn = torch.from_numpy(rng.standard_normal((n, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    rows = rng.permutation(rows_n - 1)[:n].astype(np.int32)
    pos = rng.integers(0, stride, n).astype(np.int32)
    slots = rng.permutation(np.arange(1, n_slots + 1))[:n].astype(np.int32)
    rows[-5:], pos[-5:], slots[-5:] = rows_n - 1, 0, 0  # padding: one dummy row, slot 0
    r2t = torch.from_numpy(rng.integers(1, n_slots, (rows_n, stride)).astype(np.int32)).cuda()
    want_r2t, want_k, want_v = r2t.clone(), kp.clone(), vp.clone()
    B.req_to_token_scatter(want_r2t, i32(rows), i32(pos), i32(slots))
    B.kv_store(want_k, want_v, kn[:-5], vn[:-5], i32(slots[:-5]))
    B.decode_append(r2t, i32(rows), i32(pos), i32(slots), kp, vp, kn, vn)
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(r2t.cpu(), want_r2t.cpu())
    # every row but slot 0 must match exactly; slot 0 holds, element by
    # element, the value of one of the padding rows that all wrote it
    assert torch.equal(kp[1:].cpu().view(view), want_k[1:].cpu().view(view))
    assert torch.equal(vp[1:].cpu().view(view), want_v[1:].cpu().view(view))
    pad_k, got = kn[-5:].cpu().view(view), kp[0].cpu().view(view)
    assert bool((got[None] == pad_k).any(dim=0).all())


def _run_extend(case, q_host, prefix_lens, extend_lens, hq, hkv, d, dtype, use_rows=True):
    qo = np.zeros(len(prefix_lens) + 1, dtype=np.int32)
    qo[1:] = np.cumsum(extend_lens)
    q = to_dev(q_host, dtype)
    o = torch.full_like(q, float("nan"))
    kp, vp = to_dev(case["kpool"], dtype), to_dev(case["vpool"], dtype)
    r2t = i32(case["r2t"])
    rows = i32(case["rows"]) if use_rows else None
    if not use_rows:
        r2t = i32(case["r2t"][case["rows"]])
    B.radix_extend_attention(q, o, kp, vp, r2t, rows, i32(prefix_lens), i32(extend_lens), i32(qo),
                             max(extend_lens) if len(extend_lens) else 0, 1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    return o


EXTEND_CASES = [
    # (prefix_lens, extend_lens, hq, hkv, d)
    ([0, 5, 70, 130], [200, 1, 63, 129], 32, 8, 128),
    ([1024, 1024], [128, 77], 32, 8, 128),
    ([0, 17, 300], [3, 250, 40], 8, 8, 128),
    ([64, 0], [100, 33], 8, 1, 128),
    ([10, 200, 0], [90, 45, 130], 12, 4, 64),
    ([0], [300], 4, 4, 64),
    ([50, 3], [0, 70], 32, 8, 128),
    # keys beyond two 1024-key index segments, a wave with no rows left
    ([2500, 7, 1900], [70, 2, 300], 32, 8, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ci", range(len(EXTEND_CASES)))
def test_extend_matches_oracle(dtype, ci):
    prefix_lens, extend_lens, hq, hkv, d = EXTEND_CASES[ci]
    _announce(f"extend {dtype} case {ci}: P={prefix_lens} E={extend_lens} hq={hq} hkv={hkv} d={d}")
    rng = np.random.default_rng(ci + (100 if dtype == "bf16" else 0))
    case = make_pool_case(rng, prefix_lens, extend_lens, hq, hkv, d, dtype)
    q_host = host_values(rng, (sum(extend_lens), hq, d), dtype)
    o = _run_extend(case, q_host, prefix_lens, extend_lens, hq, hkv, d, dtype, use_rows=(ci % 2 == 0))
    off, worst = 0, 0.0
    for b, (p, e) in enumerate(zip(prefix_lens, extend_lens)):
        if e == 0:
            continue
        want = oracle_rows(q_host[off:off + e], case["k"][b], case["v"][b], np.arange(p, p + e), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[off:off + e], want))
        off += e
    print(f"  max abs err {worst:.3e}")
    assert worst <= TOL[dtype]


def _run_decode(case, q_host, prefix_lens, hq, hkv, d, dtype, rows=None, r2t=None):
    q = to_dev(q_host, dtype)
    o = torch.full_like(q, float("nan"))
    kp, vp = to_dev(case["kpool"], dtype), to_dev(case["vpool"], dtype)
    max_kv = max(prefix_lens) + 1
    ws = torch.empty(B.radix_decode_workspace_bytes(len(prefix_lens), hq, hkv, d, max_kv), dtype=torch.uint8,
                     device="cuda")
    B.radix_decode_attention(q, o, kp, vp, i32(case["r2t"] if r2t is None else r2t),
                             i32(case["rows"] if rows is None else rows), i32(prefix_lens), max_kv,
                             1.0 / np.sqrt(d), ws)
    torch.cuda.synchronize()
    return o


DECODE_CASES = [
    ([0, 1, 15, 16, 17, 63, 64, 65], 32, 8, 128),
    ([2048, 2100, 2303, 1], 32, 8, 128),
    ([5000, 777, 3333], 64, 8, 128),
    ([40, 600, 1200], 16, 16, 64),
    ([513, 1024, 31], 8, 1, 128),
    # 1536 (request, KV head) units: one chunk of up to 4096 keys each (the
    # longest the plan makes), then two of 4000, ragged last blocks
    ([4095, 4000, 2100] + [1 + (7 * i) % 40 for i in range(93)], 64, 16, 128),
    ([7999, 4095, 17] + [3 + (5 * i) % 29 for i in range(189)], 32, 8, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ci", range(len(DECODE_CASES)))
def test_decode_matches_oracle(dtype, ci):
    prefix_lens, hq, hkv, d = DECODE_CASES[ci]
    _announce(f"decode {dtype} case {ci}: P={prefix_lens} hq={hq} hkv={hkv} d={d}")
    rng = np.random.default_rng(50 + ci + (100 if dtype == "bf16" else 0))
    case = make_pool_case(rng, prefix_lens, [1] * len(prefix_lens), hq, hkv, d, dtype)
    q_host = host_values(rng, (len(prefix_lens), hq, d), dtype)
    o = _run_decode(case, q_host, prefix_lens, hq, hkv, d, dtype)
    worst = 0.0
    for b, p in enumerate(prefix_lens):
        want = oracle_rows(q_host[b:b + 1], case["k"][b], case["v"][b], np.array([p]), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[b:b + 1], want))
    print(f"  max abs err {worst:.3e}")
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_split_count_does_not_change_result(dtype):
    """The same three requests decoded alone (many context chunks each) and
    inside a batch of 300 (few chunks): equal up to fp32 rounding."""
    _announce(f"decode split invariance {dtype}")
    rng = np.random.default_rng(7)
    hq, hkv, d = 32, 8, 128
    lens = [3000, 1500, 2222]
    case = make_pool_case(rng, lens, [1] * 3, hq, hkv, d, dtype)
    q_host = host_values(rng, (3, hq, d), dtype)
    alone = _run_decode(case, q_host, lens, hq, hkv, d, dtype).float()
    big = 300
    rows = np.concatenate([case["rows"], np.full(big - 3, case["rows"][0], dtype=np.int32)])
    q_big = np.concatenate([q_host, np.repeat(q_host[:1], big - 3, axis=0)])
    batched = _run_decode(case, q_big, lens + [lens[0]] * (big - 3), hq, hkv, d, dtype, rows=rows)[:3].float()
    diff = float((alone - batched).abs().max())
    print(f"  split diff {diff:.3e}")
    assert diff <= (1e-5 if dtype == "f32" else 1e-2)


def test_slot_placement_does_not_change_result():
    """Permuting where the K/V rows live in the pool gives bit-identical
    outputs (the kernels' arithmetic does not depend on slot numbers)."""
    _announce("slot placement invariance")
    hq, hkv, d, dtype = 32, 8, 128, "bf16"
    P, E = [300, 40], [70, 130]
    a = make_pool_case(np.random.default_rng(3), P, E, hq, hkv, d, dtype, place_rng=np.random.default_rng(1))
    b = make_pool_case(np.random.default_rng(3), P, E, hq, hkv, d, dtype, extra_slots=500,
                       place_rng=np.random.default_rng(2))
    # same values (same value stream), different slots and rows
    assert not np.array_equal(a["r2t"], b["r2t"])
    assert all(np.array_equal(x, y) for x, y in zip(a["k"], b["k"]))
    q_host = host_values(np.random.default_rng(9), (sum(E), hq, d), dtype)
    oa = _run_extend(a, q_host, P, E, hq, hkv, d, dtype)
    ob = _run_extend(b, q_host, P, E, hq, hkv, d, dtype)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    qd = host_values(np.random.default_rng(10), (2, hq, d), dtype)
    da = _run_decode(a, qd, [P[0] + E[0] - 1, P[1] + E[1] - 1], hq, hkv, d, dtype)
    db = _run_decode(b, qd, [P[0] + E[0] - 1, P[1] + E[1] - 1], hq, hkv, d, dtype)
    assert torch.equal(da.view(torch.int16), db.view(torch.int16))


def test_gqa_equals_mha_with_repeated_kv():
    _announce("gqa == mha with repeated kv")
    rng = np.random.default_rng(11)
    hq, hkv, d, dtype = 16, 4, 128, "bf16"
    P, E = [90, 0], [60, 150]
    case = make_pool_case(rng, P, E, hq, hkv, d, dtype)
    q_host = host_values(rng, (sum(E), hq, d), dtype)
    o_gqa = _run_extend(case, q_host, P, E, hq, hkv, d, dtype)
    rep = dict(case)
    rep["kpool"] = np.repeat(case["kpool"], hq // hkv, axis=1)
    rep["vpool"] = np.repeat(case["vpool"], hq // hkv, axis=1)
    o_mha = _run_extend(rep, q_host, P, E, hq, hq, d, dtype)
    assert float((o_gqa.float() - o_mha.float()).abs().max()) <= 1e-2


def test_bad_arguments_are_rejected_before_launch():
    q = torch.zeros((4, 8, 96), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((10, 2, 96), dtype=torch.bfloat16, device="cuda")
    r2t = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    lens = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(B.RadixRTError):
        B.radix_extend_attention(q, q, kp, kp, r2t, None, lens, lens, lens, 4, 0.1)
    with pytest.raises(B.RadixRTError):
        B.radix_decode_attention(q, q, kp, kp, r2t, None, lens, 100, 0.1, torch.empty(16, device="cuda"))


@pytest.mark.parametrize("trend", [+1.0, -1.0])
def test_extend_and_decode_with_steep_score_trends(trend):
    """Scores that rise (or fall) steeply along the context move each row's
    running max by far more than the kernels' rescale slack, tile after tile."""
    _announce(f"steep score trend {trend}")
    rng = np.random.default_rng(21)
    hq, hkv, d, dtype = 8, 2, 128, "bf16"
    P, E = [700, 0, 260], [90, 150, 1]
    case = make_pool_case(rng, P, E, hq, hkv, d, dtype)
    qdir = np.zeros(d)
    qdir[:8] = 1.0
    for b in range(len(P)):
        n = P[b] + E[b]
        ramp = trend * np.linspace(0, 24, n)[:, None, None] * qdir[None, None, :]
        for arr, pool in ((case["k"][b], case["kpool"]),):
            arr += ramp
            arr[:] = torch.from_numpy(arr.astype(np.float32)).to(torch.bfloat16).double().numpy()
        sl = case["r2t"][case["rows"][b], :n]
        case["kpool"][sl] = case["k"][b]
    q_host = host_values(rng, (sum(E), hq, d), dtype)
    q_host[:, :, :8] = np.abs(q_host[:, :, :8]) + 1.0
    o = _run_extend(case, q_host, P, E, hq, hkv, d, dtype)
    off, worst = 0, 0.0
    for b, (p, e) in enumerate(zip(P, E)):
        want = oracle_rows(q_host[off:off + e], case["k"][b], case["v"][b], np.arange(p, p + e), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[off:off + e], want))
        off += e
    qd = q_host[:len(P)].copy()
    od = _run_decode(case, qd, [p + e - 1 for p, e in zip(P, E)], hq, hkv, d, dtype)
    for b, (p, e) in enumerate(zip(P, E)):
        want = oracle_rows(qd[b:b + 1], case["k"][b], case["v"][b], np.array([p + e - 1]), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(od[b:b + 1], want))
    print(f"  max abs err {worst:.3e}")
    assert worst <= TOL[dtype]
