"""Host-side logic of bench.py (no GPU): the one-GPU guard, the flop and
byte accounting of the few-shot step, and the rule that counter traffic is
reported only while its source files are unchanged."""

import json
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_few_shot_accounting_counts_causal_pairs_and_distinct_bytes():
    """The extend flops are 4 D Hq times the causal (row, key) pairs of the
    rows actually computed; the decode's distinct bytes are the prefix once,
    every request's tail (K, V and its slot index), q and o, and the new
    tokens' K/V rows read and written (bf16 pool, few-shot sizes)."""
    fb = types.SimpleNamespace(PREFIX=1024, SUFFIX=128, B=64, HQ=32, HKV=8, D=128, fp8=False,
                               flops=[], ext_rows=[], ext_tokens=[], dec_bytes=[], dec_distinct=[])
    pl = np.full(64, 1024, dtype=np.int32)
    el = np.full(64, 128, dtype=np.int32)
    el[3] = 100          # a request that matched 28 suffix tokens computes fewer rows
    pl[3] = 1052
    fb.ext_lens = [(pl, el)]
    fb.step_lens = [(pl, el)]
    bench.FewShotBench.accounting(fb)
    pairs = sum(sum(p + j + 1 for j in range(e)) for p, e in zip(pl.tolist(), el.tolist()))
    assert fb.flops == [4.0 * 128 * 32 * pairs]
    assert fb.ext_rows == [int(el.sum())]
    assert fb.ext_tokens == [int(el.sum()) + 64]
    row = 8 * 128 * 2                                   # one K (or V) pool row, bf16
    want = 1024 * 2 * row + 64 * 129 * (2 * row + 4) + 2 * 64 * 32 * 128 * 2 + 64 * 2 * (8 * 128 * 2 + row)
    assert fb.dec_distinct == [want]
    assert fb.dec_bytes[0] > fb.dec_distinct[0]         # the prefix once per request


def test_counter_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    import hashlib
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({
        "fetch_factor": 2.0, "write_factor": 1.0,
        "unit": {"sources": ["k.hip"], "source_sha256s": [digest], "fetch_kib": 10.0, "write_kib": 5.0}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("unit") == (10.0 * 2.0 + 5.0) * 1024.0
    assert bench.profiled_traffic("missing") is None
    src.write_text("kernel source, edited\n")
    assert bench.profiled_traffic("unit") is None

