"""FP8 (E4M3) K/V pools on the GPU: the store kernel against the oracle's
codes bit for bit, and extend and decode attention over FP8 pools against
float64 attention on the values those codes stand for."""

import numpy as np
import pytest
import torch

from oracle.fp8 import dequantize, kv_store_fp8 as oracle_store, store_codes
from prefix_shared_kv_rt_amd import binding as B
from tests.gpu_util import host_values, i32, make_pool_case, max_err, oracle_rows, to_dev

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("hkv,d,k_scale,v_scale", [(8, 128, 1.0, 1.0), (2, 64, 0.37, 3.0)])
def test_kv_store_fp8_bit_exact(hkv, d, k_scale, v_scale):
    _announce(f"kv_store_fp8 hkv={hkv} d={d} scales {k_scale} {v_scale}")
    rng = np.random.default_rng(hkv + d)
    n_slots, T = 1500, 611
    mags = np.array([1e-4, 1e-2, 1.0, 30.0, 300.0, 3000.0])
    k = rng.standard_normal((T, hkv, d)) * mags[rng.integers(0, len(mags), (T, hkv, 1))]
    v = rng.standard_normal((T, hkv, d)) * mags[rng.integers(0, len(mags), (T, hkv, 1))]
    k[0, 0, :4] = [np.inf, -np.inf, np.nan, -0.0]
    kn = torch.from_numpy(k.astype(np.float32)).to(torch.bfloat16)
    vn = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    loc = rng.permutation(np.arange(1, n_slots + 1))[:T].astype(np.int32)
    pool0 = rng.integers(0, 256, (n_slots + 1, hkv, d)).astype(np.uint8)
    kp, vp = torch.from_numpy(pool0).cuda(), torch.from_numpy(pool0.copy()).cuda()
    B.kv_store_fp8(kp, vp, kn.cuda(), vn.cuda(), i32(loc), k_scale, v_scale)
    torch.cuda.synchronize()
    want_k = oracle_store(pool0, kn.float().numpy(), loc, k_scale)
    want_v = oracle_store(pool0, vn.float().numpy(), loc, v_scale)
    got_k, got_v = kp.cpu().numpy(), vp.cpu().numpy()
    # NaN codes agree up to the sign bit (the NaN's sign is not specified)
    nan_k = (want_k & 0x7F) == 0x7F
    assert np.array_equal((got_k & 0x7F) == 0x7F, nan_k)
    assert np.array_equal(got_k[~nan_k], want_k[~nan_k])
    assert np.array_equal(got_v, want_v)


@pytest.mark.parametrize("hkv,d,k_scale,v_scale", [(8, 128, 1.0, 1.0), (2, 64, 0.37, 3.0)])
def test_decode_append_fp8_bit_exact(hkv, d, k_scale, v_scale):
    """The fused FP8 append writes the slot-table entries and the oracle's
    E4M3 codes of the new rows; padding rows that all write slot 0 through
    one row leave there, 8-byte piece by piece, the codes of one of them."""
    _announce(f"decode_append_fp8 hkv={hkv} d={d} scales {k_scale} {v_scale}")
    rng = np.random.default_rng(40 + d)
    n_slots, n, stride, rows_n = 2000, 300, 97, 400
    pool0 = rng.integers(0, 256, (n_slots + 1, hkv, d)).astype(np.uint8)
    kn = torch.from_numpy((rng.standard_normal((n, hkv, d)) * 5).astype(np.float32)).to(torch.bfloat16)
    vn = torch.from_numpy((rng.standard_normal((n, hkv, d)) * 5).astype(np.float32)).to(torch.bfloat16)
    rows = rng.permutation(rows_n - 1)[:n].astype(np.int32)
    pos = rng.integers(0, stride, n).astype(np.int32)
    slots = rng.permutation(np.arange(1, n_slots + 1))[:n].astype(np.int32)
    rows[-5:], pos[-5:], slots[-5:] = rows_n - 1, 0, 0
    r2t0 = rng.integers(1, n_slots, (rows_n, stride)).astype(np.int32)
    r2t = torch.from_numpy(r2t0).cuda()
    kp, vp = torch.from_numpy(pool0).cuda(), torch.from_numpy(pool0.copy()).cuda()
    B.decode_append_fp8(r2t, i32(rows), i32(pos), i32(slots), kp, vp, kn.cuda(), vn.cuda(), k_scale, v_scale)
    torch.cuda.synchronize()
    want_r2t = r2t0.copy()
    want_r2t[rows, pos] = slots
    assert np.array_equal(r2t.cpu().numpy(), want_r2t)
    for pool, new, scale in ((kp, kn, k_scale), (vp, vn, v_scale)):
        got = pool.cpu().numpy()
        want = oracle_store(pool0, new[:-5].float().numpy(), slots[:-5], scale)
        assert np.array_equal(got[1:], want[1:])
        pad = store_codes(new[-5:].float().numpy(), scale).reshape(5, -1, 8)
        g0 = got[0].reshape(-1, 8)
        assert bool((g0[None] == pad).all(axis=2).any(axis=0).all())


def test_decode_append_fp8_rejects_bad_scale():
    r2t = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    pool = torch.zeros((4, 1, 128), dtype=torch.uint8, device="cuda")
    kn = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.RadixRTError):
        B.decode_append_fp8(r2t, i32([0]), i32([0]), i32([1]), pool, pool, kn, kn, -1.0, 1.0)


FP8_DECODE_CASES = [
    ([0, 1, 15, 16, 17, 63, 64, 65], 32, 8, 128, 1.0, 1.0),
    ([2048, 2100, 2303, 1], 32, 8, 128, 0.5, 2.0),
    ([5000, 777, 3333], 64, 8, 128, 1.0, 0.25),
    ([40, 600, 1200], 16, 16, 64, 1.5, 1.0),
]


@pytest.mark.parametrize("ci", range(len(FP8_DECODE_CASES)))
def test_decode_fp8_matches_oracle(ci):
    prefix_lens, hq, hkv, d, ks, vs = FP8_DECODE_CASES[ci]
    _announce(f"decode fp8 case {ci}: P={prefix_lens} hq={hq} hkv={hkv} d={d} scales {ks} {vs}")
    rng = np.random.default_rng(500 + ci)
    case = make_pool_case(rng, prefix_lens, [1] * len(prefix_lens), hq, hkv, d, "bf16")
    kc, vc = store_codes(case["kpool"], ks), store_codes(case["vpool"], vs)
    q_host = host_values(rng, (len(prefix_lens), hq, d), "bf16")
    q = to_dev(q_host, "bf16")
    o = torch.full_like(q, float("nan"))
    max_kv = max(prefix_lens) + 1
    ws = torch.empty(B.radix_decode_workspace_bytes(len(prefix_lens), hq, hkv, d, max_kv), dtype=torch.uint8,
                     device="cuda")
    B.radix_decode_attention_fp8kv(q, o, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), i32(case["r2t"]),
                                   i32(case["rows"]), i32(prefix_lens), max_kv, 1.0 / np.sqrt(d), ws, ks, vs)
    torch.cuda.synchronize()
    kvals, vvals = dequantize(kc, ks), dequantize(vc, vs)
    worst = 0.0
    for b, p in enumerate(prefix_lens):
        sl = case["r2t"][case["rows"][b], :p + 1]
        want = oracle_rows(q_host[b:b + 1], kvals[sl], vvals[sl], np.array([p]), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[b:b + 1], want))
    print(f"  max abs err {worst:.3e}")
    assert worst <= 2e-2


def test_decode_fp8_rejects_bad_scale():
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((4, 1, 128), dtype=torch.uint8, device="cuda")
    r2t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.RadixRTError):
        B.radix_decode_attention_fp8kv(q, q.clone(), pool, pool, r2t, None, i32([0]), 1, 0.1, ws, 0.0, 1.0)


FP8_EXTEND_CASES = [
    # (prefix_lens, extend_lens, hq, hkv, d, k_scale, v_scale)
    ([0, 5, 70, 130], [200, 1, 63, 129], 32, 8, 128, 1.0, 1.0),
    ([1024, 1024], [128, 77], 32, 8, 128, 0.5, 2.0),
    ([10, 200, 0], [90, 45, 130], 12, 4, 64, 1.0, 0.25),
    ([50, 3], [0, 70], 32, 8, 128, 3.0, 1.0),
]


@pytest.mark.parametrize("ci", range(len(FP8_EXTEND_CASES)))
def test_extend_fp8_matches_oracle(ci):
    prefix_lens, extend_lens, hq, hkv, d, ks, vs = FP8_EXTEND_CASES[ci]
    _announce(f"extend fp8 case {ci}: P={prefix_lens} E={extend_lens} hq={hq} hkv={hkv} d={d} scales {ks} {vs}")
    rng = np.random.default_rng(700 + ci)
    case = make_pool_case(rng, prefix_lens, extend_lens, hq, hkv, d, "bf16")
    kc, vc = store_codes(case["kpool"], ks), store_codes(case["vpool"], vs)
    q_host = host_values(rng, (sum(extend_lens), hq, d), "bf16")
    qo = np.zeros(len(prefix_lens) + 1, dtype=np.int32)
    qo[1:] = np.cumsum(extend_lens)
    q = to_dev(q_host, "bf16")
    o = torch.full_like(q, float("nan"))
    B.radix_extend_attention_fp8kv(q, o, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), i32(case["r2t"]),
                                   i32(case["rows"]), i32(prefix_lens), i32(extend_lens), i32(qo), max(extend_lens),
                                   1.0 / np.sqrt(d), ks, vs)
    torch.cuda.synchronize()
    kvals, vvals = dequantize(kc, ks), dequantize(vc, vs)
    off, worst = 0, 0.0
    for b, (p, e) in enumerate(zip(prefix_lens, extend_lens)):
        if e == 0:
            continue
        sl = case["r2t"][case["rows"][b], :p + e]
        want = oracle_rows(q_host[off:off + e], kvals[sl], vvals[sl], np.arange(p, p + e), 1.0 / np.sqrt(d))
        worst = max(worst, max_err(o[off:off + e], want))
        off += e
    print(f"  max abs err {worst:.3e}")
    assert worst <= 2e-2
