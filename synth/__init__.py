"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws token streams and Q/K/V values.  It contains none of the
RadixAttention arithmetic (no tree, no pool, no attention): both the CPU
oracle and the HIP path take what it produces as plain inputs.

Q/K/V values.  The method's premise (SGLang paper summary, section 3,
"Reuse opportunities"; SGLang explainer, section 04) is that the K/V of a
token depends only on the tokens up to and including it.  The generator
makes that literal: the value of (kind, head, dim) at sequence position i
is a fixed function of the seed and a rolling hash of tokens[0..i].  Two
requests that share a prefix therefore see bit-identical Q/K/V on it, and
recomputing a prefix gives exactly what a cache would have stored.

Every value is s/64 for an odd integer s in [-189, 189]: the sum of three
independent uniform odd integers in [-63, 63].  That is an Irwin-Hall(3)
approximation of N(0, 1) (mean 0, variance 4095/4096) whose values are all
exact in bfloat16 and float32, and whose generation uses integer
operations only, so the numpy and torch implementations below agree bit
for bit on any device.
"""

from .gen import (
    MASK64,
    splitmix64_np,
    prefix_hashes_np,
    prefix_hashes_from_np,
    prefix_hashes_rows_np,
    chain_start,
    value_keys_np,
    qkv_values_np,
    KIND_Q,
    KIND_K,
    KIND_V,
)

__all__ = [
    "MASK64",
    "splitmix64_np",
    "prefix_hashes_np",
    "prefix_hashes_from_np",
    "prefix_hashes_rows_np",
    "chain_start",
    "value_keys_np",
    "qkv_values_np",
    "KIND_Q",
    "KIND_K",
    "KIND_V",
]
