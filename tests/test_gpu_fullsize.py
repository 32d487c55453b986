"""Parity at the full workload sizes, in the launch configuration bench.py
times (its own classes drive the same kernels with the same grids): sampled
outputs against the oracle's float64 full recompute of those rows."""

import numpy as np
import pytest
import torch

import bench
from oracle.attention import recompute_rows
from prefix_shared_kv_rt_amd import binding as B
from synth import torch_gen

pytestmark = pytest.mark.gpu
TOL = 2e-2


SAMPLED = (0, 9, 18, 27, 36, 45, 54, 63)   # requests checked in every step


def check_few_shot(fb, i, o_ext, o_dec, prefix_lens):
    """Sampled outputs of batch i (host copies o_ext, o_dec) against the
    oracle's full recompute: for each sampled request the first extend row
    actually computed (position = matched prefix), a middle one, the last,
    and the decode row."""
    fp8 = (1.0, 1.0) if fb.fp8 else None
    worst = 0.0
    for b in SAMPLED:
        toks = list(fb.prefix) + list(fb.suffix[i][b])
        p = int(prefix_lens[b])  # rows below p were cached, not recomputed
        rows = sorted({p, (p + fb.PREFIX + fb.SUFFIX) // 2, fb.PREFIX + fb.SUFFIX - 1})
        want = recompute_rows(toks, rows, fb.HQ, fb.HKV, fb.D, fb.SEED, fb.sm_scale, kv_fp8_scales=fp8)
        got = o_ext[[b * fb.SUFFIX + (r - fb.PREFIX) for r in rows]]
        worst = max(worst, float(np.abs(got - want).max()))
        want_d = recompute_rows(toks, [fb.PREFIX + fb.SUFFIX], fb.HQ, fb.HKV, fb.D, fb.SEED, fb.sm_scale,
                                kv_fp8_scales=fp8)
        worst = max(worst, float(np.abs(o_dec[b:b + 1] - want_d).max()))
    return {"max_abs_err": worst, "tol": TOL, "ok": worst <= TOL}


@pytest.mark.parametrize("kv_dtype,page,shared", [("bf16", 1, False), ("fp8", 1, False), ("bf16", 16, False),
                                                  ("bf16", 1, True), ("fp8", 1, True)])
def test_few_shot_full_size_bench_path(kv_dtype, page, shared):
    """64 requests x (1024 shared + 128 distinct) per step, run as bench.py
    runs them: warm-up steps, the clock settle that replays the last one's
    launches, then more steps, all back to back with no synchronisation
    between them (the row sets' staging alternates as in the timed loop);
    each step's outputs are copied on the step's stream right after its
    kernels (the decode with its append folded in).  Eight requests per step are checked: the extend
    rows actually computed and the decode row (bf16 pool, or FP8 E4M3 pool at
    unit scales against attention over the values the FP8 pool holds; token
    slots or pages of 16).  Every suffix starts with its own token, so each
    request matches exactly the 1024-token prefix."""
    print(f"few-shot full size, {kv_dtype} pool, pages of {page}, shared decode {shared}", flush=True)
    n = 5
    fb = bench.FewShotBench(n, torch, B, torch_gen, kv_dtype=kv_dtype, page_size=page, shared_decode=shared)
    fb.gen_inputs(n)
    fb.warm_prefix()
    outs = []
    for i in range(n):
        fb.step(i, timed=False)
        with torch.cuda.stream(fb.stream):
            outs.append((fb.o_ext.clone(), fb.o_dec.clone(), fb.last_prefix_lens.copy()))
        if i == 1:
            fb.settle_on_step(1, ms=20.0)   # rewrites step 1's rows and outputs with the same values
            with torch.cuda.stream(fb.stream):
                outs.append((fb.o_ext.clone(), fb.o_dec.clone(), fb.last_prefix_lens.copy()))
    fb.stream.synchronize()
    worst = 0.0
    steps = [0, 1, 1, 2, 3, 4]   # the third copy: step 1's outputs after the settle's replays
    for i, (o_ext, o_dec, pl) in zip(steps, outs):
        assert (pl == fb.PREFIX).all()
        res = check_few_shot(fb, i, o_ext.float().cpu().numpy(), o_dec.float().cpu().numpy(), pl)
        print(f"  step {i}: {res}", flush=True)
        worst = max(worst, res["max_abs_err"])
    assert worst <= TOL


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,steps,sample_steps,kv_dtype,shared", [
    ("fork", 256, (0, 127, 255), "bf16", False),
    ("long_context", 128, (0, 64, 127), "bf16", False),
    ("long_context", 128, (0, 127), "fp8", False),
    ("fork", 256, (0, 255), "bf16", True),
    ("long_context", 128, (0, 127), "bf16", True),
])
def test_decode_full_size_bench_path(name, steps, sample_steps, kv_dtype, shared):
    print(f"{name} full size, {steps} decode steps, {kv_dtype} pool, shared decode {shared}", flush=True)
    db = bench.DecodeBench(name, torch, B, torch_gen, steps, kv_dtype=kv_dtype, shared_decode=shared)
    db.setup()
    saved = {}
    for s in range(steps):
        db.step(s, timed=False)
        if s == 3:
            db.settle_on_step(3, ms=20.0)   # the bench's clock settle: step 3's launches replayed
        if s in sample_steps:
            db.stream.synchronize()
            saved[s] = db.o.float().cpu().numpy()
    per = db.B // db.groups
    worst = 0.0
    for b in (0, db.B - 1):
        toks = list(db.shared_toks[b // per]) + list(db.private_toks[b]) + list(db.gen_toks[b])
        pos = [db.prompt_len + s for s in sample_steps]
        want = recompute_rows(toks, pos, db.HQ, db.HKV, db.D, db.SEED, db.sm_scale,
                              kv_fp8_scales=(1.0, 1.0) if kv_dtype == "fp8" else None)
        for k, s in enumerate(sample_steps):
            worst = max(worst, float(np.abs(saved[s][b] - want[k]).max()))
    print(f"  max abs err {worst:.3e}", flush=True)
    assert worst <= TOL
