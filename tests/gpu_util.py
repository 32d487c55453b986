"""Helpers for the GPU tests: seeded host inputs for the kernels and the
comparison against the float64 oracle."""

import numpy as np
import torch

from oracle.attention import causal_attention

DT = {"bf16": torch.bfloat16, "f32": torch.float32}
TOL = {"bf16": 2e-2, "f32": 1e-4}


def host_values(rng, shape, dtype):
    """N(0,1) values already rounded to the kernel's input dtype, as float64."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(DT[dtype])
    return x.float().numpy().astype(np.float64)


def make_pool_case(rng, prefix_lens, extend_lens, hq, hkv, d, dtype, extra_slots=37, stride_pad=5,
                   place_rng=None):
    """Random K/V for every position of every request, scattered to random
    distinct pool slots (drawn from ``place_rng`` if given, so that the same
    values can be placed differently).  Returns host arrays + slot table."""
    place = place_rng if place_rng is not None else rng
    B = len(prefix_lens)
    lens = [p + e for p, e in zip(prefix_lens, extend_lens)]
    total = sum(lens)
    num_slots = total + extra_slots
    perm = place.permutation(np.arange(1, num_slots + 1))[:total]
    stride = max(lens) + stride_pad
    r2t = np.zeros((B + 3, stride), dtype=np.int32)
    rows = place.permutation(B + 3)[:B].astype(np.int32)
    kpool = np.zeros((num_slots + 1, hkv, d))
    vpool = np.zeros((num_slots + 1, hkv, d))
    seqs_k, seqs_v, off = [], [], 0
    for b in range(B):
        k = host_values(rng, (lens[b], hkv, d), dtype)
        v = host_values(rng, (lens[b], hkv, d), dtype)
        sl = perm[off:off + lens[b]]
        off += lens[b]
        r2t[rows[b], :lens[b]] = sl
        kpool[sl] = k
        vpool[sl] = v
        seqs_k.append(k)
        seqs_v.append(v)
    return dict(num_slots=num_slots, r2t=r2t, rows=rows, kpool=kpool, vpool=vpool, k=seqs_k, v=seqs_v,
                stride=stride, lens=lens)


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DT[dtype]).cuda()


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def max_err(got, want):
    return float(np.max(np.abs(got.float().cpu().numpy().astype(np.float64) - want))) if want.size else 0.0


def oracle_rows(q, k, v, positions, scale):
    return causal_attention(q, k, v, positions, scale)
