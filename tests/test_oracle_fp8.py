"""The oracle's FP8 (OCP E4M3) pool format against what the format's
definition fixes: named code values, round-to-nearest-even at midpoints,
saturation, subnormal underflow, and PyTorch's own float8_e4m3fn decoder and
encoder inside the finite range."""

import numpy as np
import pytest
import torch

from oracle.fp8 import dequantize, e4m3_values, kv_store_fp8, quantize_e4m3, store_codes


def test_named_codes():
    v = e4m3_values()
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6          # smallest normal
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254


def test_decode_matches_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    v = e4m3_values()
    assert np.array_equal(np.isnan(ref), np.isnan(v))
    assert np.array_equal(ref[~np.isnan(ref)], v[~np.isnan(v)])


def test_every_finite_code_round_trips():
    v = e4m3_values()
    codes = np.array([c for c in range(256) if np.isfinite(v[c])], dtype=np.uint8)
    assert np.array_equal(quantize_e4m3(v[codes]), codes)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),        # midpoint of 1.0 (m=0) and 1.125 (m=1): even mantissa
    (1.1875, 0x3A),        # midpoint of 1.125 (m=1) and 1.25 (m=2): even mantissa
    (1.07, 0x39),          # nearer to 1.125
    (-1.0625, 0xB8),
    (460.0, 0x7E),         # past the largest finite value: saturates
    (1e30, 0x7E), (-np.inf, 0xFE), (np.inf, 0x7E),
    (2.0 ** -11, 0x00),    # a quarter of the smallest subnormal
    (2.0 ** -10, 0x00),    # midpoint of 0 and 2^-9: even (zero)
    (1.5 * 2.0 ** -10, 0x01),
    (3 * 2.0 ** -10, 0x02),  # midpoint of 2^-9 (m=1) and 2^-8 (m=2): even
    (7.5 * 2.0 ** -9, 0x08),  # midpoint of the largest subnormal and the smallest normal: even (normal m=0)
])
def test_rounding_and_saturation(x, code):
    assert int(quantize_e4m3(np.array([x]))[0]) == code


def test_nan_stays_nan():
    c = quantize_e4m3(np.array([np.nan]))[0]
    assert c & 0x7F == 0x7F


def test_quantize_matches_torch_inside_the_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (0.01, 1.0, 30.0, 150.0)])
    x = x[np.abs(x) < 440].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quantize_e4m3(x), ref)


def test_scale_and_store():
    rows = np.array([[[1.0, -3.0, 500.0, 0.3]]], dtype=np.float32)
    codes = store_codes(rows, 0.5)          # values doubled before rounding
    assert list(codes.reshape(-1)) == [0x40, 0xCC, 0x7E, list(quantize_e4m3(np.array([0.6], np.float32)))[0]]
    assert dequantize(np.array([0x40]), 0.5)[0] == 1.0
    pool = np.zeros((5, 1, 4), dtype=np.uint8)
    out = kv_store_fp8(pool, rows, [3], 0.5)
    assert np.array_equal(out[3], codes[0]) and not out[[0, 1, 2, 4]].any()


def test_attention_reads_the_stored_values():
    """With K/V values that E4M3 holds exactly (small multiples of 1/8), the
    FP8 pool changes nothing; in general it equals attention over the
    round-tripped rows."""
    from oracle.attention import causal_attention, recompute_rows, regenerate_qkv
    toks = list(range(1, 40))
    pos = np.array([10, 38])
    a = recompute_rows(toks, pos, 4, 2, 16, 3, 0.25, kv_fp8_scales=(1.0, 1.0))
    q, k, v = regenerate_qkv(toks, pos, 4, 2, 16, 3)
    b = causal_attention(q, dequantize(store_codes(k, 1.0), 1.0), dequantize(store_codes(v, 1.0), 1.0), pos, 0.25)
    assert np.array_equal(a, b)
    rng = np.random.default_rng(1)
    k8 = rng.integers(-16, 17, k.shape) / 8.0
    v8 = rng.integers(-16, 17, v.shape) / 8.0
    assert np.array_equal(dequantize(store_codes(k8, 1.0), 1.0), k8)
    assert np.array_equal(dequantize(store_codes(v8, 0.5), 0.5), v8)
