"""Decode with the step's append folded into its launches
(radix_decode_attention_append, radix_decode_attention_shared_append and
their FP8-pool forms): each request's new token, the key at position
prefix_lens[b], arrives as K/V input rows and a fresh slot; the call must
leave the pools and the slot table as decode_append would and return what
the decode call returns after it (bit for bit: same kernels, same plan), and
match the float64 oracle over the whole context."""

import numpy as np
import pytest
import torch

from prefix_shared_kv_rt_amd import binding as B
from tests.gpu_util import host_values, i32, max_err, oracle_rows, to_dev
from tests.test_gpu_shared_decode import make_shared_case, streams  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu
TOL = 2e-2

CASES = [
    # (groups, hq, hkv, d); every member has a private part (its new token)
    ([(1024, [1 + (7 * i) % 130 for i in range(64)])], 32, 8, 128),           # few-shot shaped
    ([(2048, [1 + i % 5 for i in range(8)]) for _ in range(16)], 32, 8, 128),   # fork shaped
    ([(0, [40]), (77, [3, 1, 200]), (0, [1, 2]), (300, [1])], 12, 4, 64),    # ragged, groups of one
]


def _prepare(ci, seed, fp8_scales=None):
    """A shared-prefix case whose last position per request is its new token:
    the token's K/V become inputs, its slot moves to a fresh slot that holds
    garbage, and its slot-table entry is cleared (both are the call's job)."""
    groups, hq, hkv, d = CASES[ci]
    rng = np.random.default_rng(seed)
    n = sum(len(p) for _, p in groups)
    case = make_shared_case(rng, groups, hq, hkv, d, extra_slots=n + 16)
    pos = case["prefix_lens"]
    used = set(np.unique(case["r2t"]).tolist())
    free = np.array([s for s in range(1, case["kpool"].shape[0]) if s not in used], dtype=np.int32)
    new_slots = rng.permutation(free)[:n].astype(np.int32)
    k_new = np.stack([case["k"][b][-1] for b in range(n)])
    v_new = np.stack([case["v"][b][-1] for b in range(n)])
    r2t = case["r2t"].copy()
    r2t[case["rows"], pos] = 0
    kpool, vpool = case["kpool"].copy(), case["vpool"].copy()
    kpool[new_slots] = 1e4     # garbage: the call must overwrite it before reading
    vpool[new_slots] = -1e4
    kb, vb = to_dev(kpool, "bf16"), to_dev(vpool, "bf16")
    if fp8_scales:
        kp = torch.zeros(kb.shape, dtype=torch.uint8, device="cuda")
        vp = torch.zeros_like(kp)
        loc = torch.arange(kb.shape[0], dtype=torch.int32, device="cuda")
        B.kv_store_fp8(kp, vp, kb, vb, loc, *fp8_scales)
    else:
        kp, vp = kb, vb
    q_host = host_values(rng, (n, hq, d), "bf16")
    return dict(case=case, hq=hq, hkv=hkv, d=d, n=n, kp=kp, vp=vp, r2t=r2t, new_slots=new_slots,
                k_new=to_dev(k_new, "bf16"), v_new=to_dev(v_new, "bf16"), q_host=q_host, q=to_dev(q_host, "bf16"))


def _shared_args(p, kp, vp, r2t_dev, o, ws):
    c = p["case"]
    return (p["q"], o, kp, vp, r2t_dev, i32(c["rows"]), i32(c["prefix_lens"]), i32(c["shared_lens"]),
            i32(c["group_start"]), c["max_group"], c["max_shared"], c["max_private"], 1.0 / np.sqrt(p["d"]))


def _shared_ws(p):
    c = p["case"]
    return torch.empty(B.radix_decode_shared_workspace_bytes(p["n"], p["hq"], p["hkv"], p["d"],
                                                             len(c["group_start"]) - 1, c["max_group"],
                                                             c["max_shared"], c["max_private"]),
                       dtype=torch.uint8, device="cuda")


def _plain_ws(p):
    max_kv = int(p["case"]["prefix_lens"].max()) + 1
    return torch.empty(B.radix_decode_workspace_bytes(p["n"], p["hq"], p["hkv"], p["d"], max_kv),
                       dtype=torch.uint8, device="cuda"), max_kv


def _run(p, shared, fused, fp8_scales):
    """The call under test (fused) or decode_append + the decode call; returns
    (o, k_pool, v_pool, req_to_token) after it."""
    c = p["case"]
    kp, vp, r2t_dev = p["kp"].clone(), p["vp"].clone(), i32(p["r2t"])
    o = torch.full_like(p["q"], float("nan"))
    slots = i32(p["new_slots"])
    rows, pos = i32(c["rows"]), i32(c["prefix_lens"])
    sc = fp8_scales or ()
    if not fused:
        if fp8_scales:
            B.decode_append_fp8(r2t_dev, rows, pos, slots, kp, vp, p["k_new"], p["v_new"], *fp8_scales)
        else:
            B.decode_append(r2t_dev, rows, pos, slots, kp, vp, p["k_new"], p["v_new"])
    if shared:
        ws = _shared_ws(p)
        args = _shared_args(p, kp, vp, r2t_dev, o, ws)
        if fused:
            f = B.radix_decode_attention_shared_append_fp8kv if fp8_scales else B.radix_decode_attention_shared_append
            f(*args, p["k_new"], p["v_new"], slots, ws, *sc)
        else:
            f = B.radix_decode_attention_shared_fp8kv if fp8_scales else B.radix_decode_attention_shared
            f(*args, ws, *sc)
    else:
        ws, max_kv = _plain_ws(p)
        args = (p["q"], o, kp, vp, r2t_dev, rows, pos, max_kv, 1.0 / np.sqrt(p["d"]))
        if fused:
            f = B.radix_decode_attention_append_fp8kv if fp8_scales else B.radix_decode_attention_append
            f(*args, p["k_new"], p["v_new"], slots, ws, *sc)
        else:
            f = B.radix_decode_attention_fp8kv if fp8_scales else B.radix_decode_attention
            f(*args, ws, *sc)
    torch.cuda.synchronize()
    return o, kp, vp, r2t_dev


def _check(p, shared, fp8_scales, label):
    o, kp, vp, r2t = _run(p, shared, True, fp8_scales)
    o_ref, kp_ref, vp_ref, r2t_ref = _run(p, shared, False, fp8_scales)
    c = p["case"]
    assert torch.equal(r2t, r2t_ref), "slot table differs from decode_append's"
    assert torch.equal(kp.view(torch.uint8), kp_ref.view(torch.uint8)), "K pool differs from decode_append's"
    assert torch.equal(vp.view(torch.uint8), vp_ref.view(torch.uint8)), "V pool differs from decode_append's"
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "output differs from append + decode"
    worst = 0.0
    if not fp8_scales:
        for b in range(p["n"]):
            want = oracle_rows(p["q_host"][b:b + 1], c["k"][b], c["v"][b], np.array([int(c["prefix_lens"][b])]),
                               1.0 / np.sqrt(p["d"]))
            worst = max(worst, max_err(o[b:b + 1], want))
    print(f"  {label}: bit-identical to append + decode; max abs err against the oracle {worst:.3e}", flush=True)
    assert worst <= TOL


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_shared_decode_append(ci, streams):
    print(f"shared decode with append, case {ci} ({streams})", flush=True)
    _check(_prepare(ci, 3100 + ci), True, None, "shared")


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_plain_decode_append(ci):
    print(f"plain decode with append, case {ci}", flush=True)
    _check(_prepare(ci, 3200 + ci), False, None, "plain")


@pytest.mark.parametrize("ci,scales", [(0, (1.0, 1.0)), (2, (0.5, 2.0))])
def test_decode_append_fp8_pools(ci, scales, streams):
    print(f"fp8 decode with append, case {ci}, scales {scales} ({streams})", flush=True)
    _check(_prepare(ci, 3300 + ci, scales), True, scales, "shared fp8")
    if streams == "one launch":
        _check(_prepare(ci, 3400 + ci, scales), False, scales, "plain fp8")


def test_shared_decode_append_long_private_tails(streams, monkeypatch):
    """Private tails split into chunks of more than 1024 keys: in the single
    launch (forced) the new token's slot index arrives through the index
    ring's refill, not its first fill."""
    if streams == "one launch":
        monkeypatch.setenv("RADIXRT_SHARED_FUSED", "force")
    global CASES
    saved = CASES
    CASES = [([(96, [2100 + (37 * i) % 300 for i in range(64)])], 8, 8, 64)]
    try:
        print(f"shared decode with append, long private tails ({streams})", flush=True)
        _check(_prepare(0, 3500), True, None, "long tails")
    finally:
        CASES = saved


def test_decode_append_rejects_missing_inputs():
    q = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((10, 2, 64), dtype=torch.bfloat16, device="cuda")
    r2t, z = i32(np.zeros((4, 16))), i32(np.zeros(4))
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.RadixRTError):   # no new slots
        B.radix_decode_attention_append(q, q, kp, kp, r2t, None, z, 8, 0.125, q, q, None, ws)
    with pytest.raises(B.RadixRTError):   # no K rows
        B.radix_decode_attention_append(q, q, kp, kp, r2t, None, z, 8, 0.125, None, q, z, ws)
