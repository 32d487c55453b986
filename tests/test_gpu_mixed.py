"""The table-driven extend scatter and the mixed extend + decode launch on the
GPU: kv_store_extend equals kv_store over the same slots bit for bit;
radix_mixed_attention equals radix_extend_attention over the same batch bit
for bit and the float64 oracle within tolerance; the scheduler's mixed
iterations keep every host decision and output of the oracle's workload."""

import numpy as np
import pytest
import torch

from prefix_shared_kv_rt_amd import binding as B
from tests.gpu_util import DT, TOL, host_values, i32, make_pool_case, max_err, oracle_rows, to_dev

pytestmark = pytest.mark.gpu

VIEW = {"bf16": torch.int16, "f32": torch.int32}


def _store_case(rng, dtype, hkv, d, gaps):
    """Pools, a slot table whose rows hold distinct slots, and an extend
    batch (ragged, some requests empty) whose source rows sit at qo[b]
    (with unused rows between requests when ``gaps``)."""
    n_slots, n_rows, stride = 9000, 40, 400
    pl = rng.integers(0, 200, 23).astype(np.int32)
    el = rng.integers(0, 190, 23).astype(np.int32)
    el[[3, 11]] = 0
    el[5] = 1
    rows = rng.permutation(n_rows)[:23].astype(np.int32)
    r2t = np.zeros((n_rows, stride), dtype=np.int32)
    perm = rng.permutation(np.arange(1, n_slots + 1))
    off = 0
    for b in range(23):
        n = pl[b] + el[b]
        r2t[rows[b], :n] = perm[off:off + n]
        off += n
    gap = rng.integers(0, 9, 23) if gaps else np.zeros(23, dtype=np.int64)
    qo = np.zeros(24, dtype=np.int32)
    qo[1:] = np.cumsum(el + gap)
    qo[:23] += gap.astype(np.int32)          # request b's rows start after its gap
    total = int(qo[23])
    src = DT[dtype] if dtype != "fp8" else torch.bfloat16
    kn = torch.from_numpy(rng.standard_normal((total, hkv, d)).astype(np.float32)).to(src).cuda()
    vn = torch.from_numpy(rng.standard_normal((total, hkv, d)).astype(np.float32)).to(src).cuda()
    loc = np.concatenate([r2t[rows[b], pl[b]:pl[b] + el[b]] for b in range(23)])
    src_rows = np.concatenate([np.arange(qo[b], qo[b] + el[b]) for b in range(23)])
    return dict(n_slots=n_slots, pl=pl, el=el, rows=rows, r2t=r2t, qo=qo, kn=kn, vn=vn, loc=loc,
                src_rows=torch.from_numpy(src_rows).cuda())


@pytest.mark.parametrize("dtype,hkv,d,gaps", [("bf16", 8, 128, True), ("bf16", 2, 64, False), ("f32", 4, 128, True)])
def test_kv_store_extend_bit_exact(dtype, hkv, d, gaps):
    print(f"kv_store_extend {dtype} hkv={hkv} d={d} gaps={gaps}", flush=True)
    rng = np.random.default_rng(hkv * 7 + d + gaps)
    c = _store_case(rng, dtype, hkv, d, gaps)
    kp = torch.from_numpy(rng.standard_normal((c["n_slots"] + 1, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    vp = torch.from_numpy(rng.standard_normal((c["n_slots"] + 1, hkv, d)).astype(np.float32)).to(DT[dtype]).cuda()
    want_k, want_v = kp.clone(), vp.clone()
    B.kv_store(want_k, want_v, c["kn"][c["src_rows"]].contiguous(), c["vn"][c["src_rows"]].contiguous(),
               i32(c["loc"]))
    B.kv_store_extend(kp, vp, c["kn"], c["vn"], i32(c["r2t"]), i32(c["rows"]), i32(c["pl"]), i32(c["el"]),
                      i32(c["qo"]), int(c["el"].max()))
    torch.cuda.synchronize()
    assert torch.equal(kp.cpu().view(VIEW[dtype]), want_k.cpu().view(VIEW[dtype]))
    assert torch.equal(vp.cpu().view(VIEW[dtype]), want_v.cpu().view(VIEW[dtype]))


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.37, 2.5)])
def test_kv_store_extend_fp8_bit_exact(scales):
    print(f"kv_store_extend_fp8 scales={scales}", flush=True)
    rng = np.random.default_rng(31)
    hkv, d = 8, 128
    c = _store_case(rng, "fp8", hkv, d, True)
    kp = torch.from_numpy(rng.integers(0, 256, (c["n_slots"] + 1, hkv, d)).astype(np.uint8)).cuda()
    vp = torch.from_numpy(rng.integers(0, 256, (c["n_slots"] + 1, hkv, d)).astype(np.uint8)).cuda()
    want_k, want_v = kp.clone(), vp.clone()
    B.kv_store_fp8(want_k, want_v, c["kn"][c["src_rows"]].contiguous(), c["vn"][c["src_rows"]].contiguous(),
                   i32(c["loc"]), *scales)
    B.kv_store_extend_fp8(kp, vp, c["kn"], c["vn"], i32(c["r2t"]), i32(c["rows"]),
                          i32(c["pl"]), i32(c["el"]), i32(c["qo"]), int(c["el"].max()), *scales)
    torch.cuda.synchronize()
    assert torch.equal(kp.cpu(), want_k.cpu())
    assert torch.equal(vp.cpu(), want_v.cpu())


# (extend prefix lens, extend lens, decode positions, tail lens, hq, hkv, d)
MIXED_CASES = [
    ([0, 300, 1024], [200, 129, 64], [5, 0, 700, 1500, 64, 2047], None, 32, 8, 128),
    ([17], [1000], list(range(0, 300, 7)), None, 32, 8, 128),
    ([], [], [1, 130, 900], None, 32, 8, 128),                      # decode rows only
    ([40, 0, 3], [90, 0, 33], [], None, 8, 2, 64),                   # extend only
    ([10, 200], [70, 45], [12, 64, 257], [1, 3, 2], 12, 4, 64),      # short tails longer than one row
    ([0, 64], [130, 1], [100, 3000], None, 8, 1, 128),
]


def _mixed_inputs(ci, dtype):
    epl, eel, dpos, tails, hq, hkv, d = MIXED_CASES[ci]
    tails = tails if tails is not None else [1] * len(dpos)
    pl = list(epl) + list(dpos)
    el = list(eel) + list(tails)
    rng = np.random.default_rng(400 + ci + (50 if dtype == "bf16" else 0))
    case = make_pool_case(rng, pl, el, hq, hkv, d, "bf16" if dtype == "fp8" else dtype)
    q_host = host_values(rng, (sum(el), hq, d), "bf16" if dtype == "fp8" else dtype)
    qo = np.zeros(len(pl) + 1, dtype=np.int32)
    qo[1:] = np.cumsum(el)
    return epl, eel, pl, el, hq, hkv, d, case, q_host, qo


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ci", range(len(MIXED_CASES)))
def test_mixed_launch_matches_extend_and_oracle(dtype, ci):
    epl, eel, pl, el, hq, hkv, d, case, q_host, qo = _mixed_inputs(ci, dtype)
    print(f"mixed {dtype} case {ci}: {len(epl)} extend + {len(pl) - len(epl)} short, hq={hq} hkv={hkv} d={d}",
          flush=True)
    q = to_dev(q_host, dtype)
    kp, vp = to_dev(case["kpool"], dtype), to_dev(case["vpool"], dtype)
    args = (kp, vp, i32(case["r2t"]), i32(case["rows"]), i32(pl), i32(el), i32(qo))
    o_mix = torch.full_like(q, float("nan"))
    o_ext = torch.full_like(q, float("nan"))
    n_e = len(epl)
    max_e = max(eel) if eel else 0
    max_t = max(el[n_e:]) if len(el) > n_e else 0
    B.radix_mixed_attention(q, o_mix, *args, n_e, max_e, max_t, 1.0 / np.sqrt(d))
    B.radix_extend_attention(q, o_ext, *args, max(el), 1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    assert torch.equal(o_mix.cpu().view(VIEW[dtype]), o_ext.cpu().view(VIEW[dtype]))
    worst = 0.0
    for b, (p, e) in enumerate(zip(pl, el)):
        if e == 0:
            continue
        want = oracle_rows(q_host[qo[b]:qo[b] + e], case["k"][b], case["v"][b], np.arange(p, p + e),
                           1.0 / np.sqrt(d))
        worst = max(worst, max_err(o_mix[qo[b]:qo[b] + e], want))
    print(f"  max abs err {worst:.3e}", flush=True)
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("ci", [0, 4])
def test_mixed_launch_fp8_matches_extend(ci):
    epl, eel, pl, el, hq, hkv, d, case, q_host, qo = _mixed_inputs(ci, "fp8")
    print(f"mixed fp8 case {ci}", flush=True)
    rng = np.random.default_rng(77 + ci)
    n = case["kpool"].shape[0]
    kp = torch.from_numpy(rng.integers(0, 126, (n, hkv, d)).astype(np.uint8)).cuda()   # finite E4M3 codes
    vp = torch.from_numpy(rng.integers(0, 126, (n, hkv, d)).astype(np.uint8)).cuda()
    kp ^= torch.from_numpy((rng.integers(0, 2, (n, hkv, d)) * 128).astype(np.uint8)).cuda()
    q = to_dev(q_host, "bf16")
    args = (kp, vp, i32(case["r2t"]), i32(case["rows"]), i32(pl), i32(el), i32(qo))
    o_mix, o_ext = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
    n_e = len(epl)
    B.radix_mixed_attention_fp8kv(q, o_mix, *args, n_e, max(eel) if eel else 0, max(el[n_e:]) if len(el) > n_e else 0,
                                  1.0 / np.sqrt(d), 0.05, 0.5)
    B.radix_extend_attention_fp8kv(q, o_ext, *args, max(el), 1.0 / np.sqrt(d), 0.05, 0.5)
    torch.cuda.synchronize()
    assert not torch.isnan(o_mix.float()).any()
    assert torch.equal(o_mix.cpu().view(torch.int16), o_ext.cpu().view(torch.int16))


def test_mixed_launch_rejects_bad_counts():
    q = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((10, 2, 64), dtype=torch.bfloat16, device="cuda")
    z = i32(np.zeros(5))
    r2t = i32(np.zeros((4, 8)))
    for n_e, me, mt in [(-1, 1, 1), (5, 1, 1), (2, -1, 1), (2, 1, -1)]:
        with pytest.raises(B.RadixRTError):
            B.radix_mixed_attention(q, q, kp, kp, r2t, None, z[:4], z[:4], z, n_e, me, mt, 0.125)
