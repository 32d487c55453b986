// Work-order and LDS-layout helpers shared by the attention kernels that
// stage K/V tiles in LDS (extend.hip, extend_wide.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace rtk {

// MI355X places workgroup i on XCD i % 8.  xcd_slice maps block `bid` of
// `nblk` to a work index such that each XCD runs one contiguous slice of the
// work list: work items that read the same K/V rows (requests sharing a
// cached prefix under one KV head) then meet them in that XCD's L2.
__device__ __forceinline__ int xcd_slice(int bid, int nblk) {
  const int xcd = bid & 7, local = bid >> 3;
  const int q = nblk >> 3, r = nblk & 7;
  return xcd * q + min(xcd, r) + local;
}

// LDS tile layout: rows (keys) of D*2 bytes, unpadded; the 16-byte chunks of
// row k are permuted by chunk ^ f(k).  f is a bijection on the low 4 bits of
// k chosen so that both access patterns are free of bank conflicts whether
// the LDS serves 128 or 256 bytes per cycle: 8 or 16 consecutive keys read at
// one chunk index (the K operand) land on distinct bank groups, and so do 4
// consecutive keys read at 2 or 4 consecutive chunks (the transpose reads).
__device__ __forceinline__ int swz_f(int k) {
  return ((0xCA60 >> (4 * (k & 3))) & 0xF) ^ ((k >> 2) & 1) ^ (((k >> 3) & 1) << 1);
}
// Byte offset of logical 16-byte chunk `chunk` of row `key` in a tile of
// bf16 rows of D elements.
template <int D>
__device__ __forceinline__ int swz(int key, int chunk) {
  constexpr int kRowBytes = 2 * D, kCPR = kRowBytes / 16;
  return key * kRowBytes + ((chunk ^ (swz_f(key) & (kCPR - 1))) << 4);
}

}  // namespace rtk
