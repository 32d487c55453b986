"""radix_decode_attention_noalloc (split-K workspace in the library's own
device array) against radix_decode_attention with a caller workspace: the
same kernels on the same inputs, so the outputs must be bit-identical; the
float64 oracle checks both.  Two calls in a row, the second smaller (the
array keeps the first call's partials), and sizes beyond the array's
maximum refused before any launch."""

import numpy as np
import pytest
import torch

from prefix_shared_kv_rt_amd import binding as B
from tests.gpu_util import TOL, host_values, i32, make_pool_case, max_err, oracle_rows, to_dev

pytestmark = pytest.mark.gpu


def _decode_both(case, q_host, pos, hq, hkv, d, dtype):
    """Outputs of the workspace entry point and of the no-alloc one."""
    q = to_dev(q_host, dtype)
    kp, vp = to_dev(case["kpool"], dtype), to_dev(case["vpool"], dtype)
    r2t, rows, plens = i32(case["r2t"]), i32(case["rows"]), i32(pos)
    max_kv = max(pos) + 1
    ws = torch.empty(B.radix_decode_workspace_bytes(len(pos), hq, hkv, d, max_kv), dtype=torch.uint8, device="cuda")
    o_ws = torch.full_like(q, float("nan"))
    o_na = torch.full_like(q, float("nan"))
    B.radix_decode_attention(q, o_ws, kp, vp, r2t, rows, plens, max_kv, 1.0 / np.sqrt(d), ws)
    B.radix_decode_attention_noalloc(q, o_na, kp, vp, r2t, rows, plens, max_kv, 1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    return o_ws, o_na


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_matches_workspace_decode_twice(dtype):
    hq, hkv, d = 32, 8, 128
    # first call: ragged contexts up to 2.3 K keys; second: fewer, shorter requests
    for call, (P, E) in enumerate((([300, 1500, 77, 2049, 5, 640], [1, 2, 1, 250, 3, 1]),
                                   ([40, 9, 700], [1, 1, 2]))):
        print(f"noalloc decode {dtype} call {call}: P={P} E={E}", flush=True)
        rng = np.random.default_rng(70 + call + (10 if dtype == "bf16" else 0))
        case = make_pool_case(rng, P, E, hq, hkv, d, dtype)
        pos = [p + e - 1 for p, e in zip(P, E)]
        q_host = host_values(rng, (len(P), hq, d), dtype)
        o_ws, o_na = _decode_both(case, q_host, pos, hq, hkv, d, dtype)
        view = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(o_ws.view(view), o_na.view(view)), "no-alloc output differs from the workspace entry point"
        worst = 0.0
        for b, p in enumerate(pos):
            want = oracle_rows(q_host[b:b + 1], case["k"][b], case["v"][b], np.array([p]), 1.0 / np.sqrt(d))
            worst = max(worst, max_err(o_na[b:b + 1], want))
        print(f"  max abs err {worst:.3e}")
        assert worst <= TOL[dtype]


def test_noalloc_decode_refuses_sizes_beyond_its_array():
    # Valid, in-bounds arguments (every request one key, slot 0) whose
    # workspace, sized by max_kv, exceeds the array.
    hq, hkv, d = 64, 8, 128
    batch, max_kv = 256, 8192
    need = B.radix_decode_workspace_bytes(batch, hq, hkv, d, max_kv)
    assert need > B.NOALLOC_MAX_WORKSPACE_BYTES
    q = torch.zeros((batch, hq, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    pool = torch.zeros((4, hkv, d), dtype=torch.bfloat16, device="cuda")
    r2t = torch.zeros((batch, max_kv), dtype=torch.int32, device="cuda")
    lens = torch.zeros(batch, dtype=torch.int32, device="cuda")
    with pytest.raises(B.RadixRTError, match="scratch array"):
        B.radix_decode_attention_noalloc(q, o, pool, pool, r2t, None, lens, max_kv, 0.1)
    torch.cuda.synchronize()
