// kv_store: scatter the new tokens' K and V rows into the token-granular
// pool at their out_cache_loc slots (SGLang v0.2 handbook chapter, "CUDA
// Graph" section: out_cache_loc names where this step's new K/V go).
//
// A pool row is num_kv_heads * head_dim elements (2 KiB for 8 x 128 bf16),
// contiguous.  Each thread moves 16-byte pieces; consecutive threads take
// consecutive pieces of a row, so each wave reads and writes whole 128-byte
// lines.  The copy is a pure byte move: bit-exact for any dtype.

#include "dev_common.h"
#include "radixrt.h"
#include "rt_internal.h"

namespace {

using rtk::u32x4;

__global__ void __launch_bounds__(256) kv_store_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                       const char* __restrict__ k_new,
                                                       const char* __restrict__ v_new,
                                                       const int32_t* __restrict__ loc, int64_t n_tokens,
                                                       int64_t row_bytes) {
  const int64_t pieces_per_row = row_bytes >> 4;
  const int64_t total = n_tokens * pieces_per_row;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; p < total; p += stride) {
    const int64_t t = p / pieces_per_row;
    const int64_t off = (p - t * pieces_per_row) << 4;
    const int64_t slot = loc[t];
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + t * row_bytes + off);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + t * row_bytes + off);
    *reinterpret_cast<u32x4*>(k_pool + slot * row_bytes + off) = kv;
    *reinterpret_cast<u32x4*>(v_pool + slot * row_bytes + off) = vv;
  }
}

// One decode step's appends: block t writes token t's slot into the slot
// table and copies its K and V rows into the pool.
__global__ void __launch_bounds__(256) decode_append_kernel(int32_t* __restrict__ r2t, int64_t stride,
                                                            const int32_t* __restrict__ rows,
                                                            const int32_t* __restrict__ pos,
                                                            const int32_t* __restrict__ slots,
                                                            char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                            const char* __restrict__ k_new,
                                                            const char* __restrict__ v_new, int n,
                                                            int64_t row_bytes) {
  const int64_t pieces = row_bytes >> 4;
  for (int t = blockIdx.x; t < n; t += gridDim.x) {
    const int64_t slot = slots[t];
    if (threadIdx.x == 0) r2t[int64_t(rows[t]) * stride + pos[t]] = int32_t(slot);
    for (int64_t p = threadIdx.x; p < pieces; p += blockDim.x) {
      const int64_t off = p << 4;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + t * row_bytes + off);
      const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + t * row_bytes + off);
      *reinterpret_cast<u32x4*>(k_pool + slot * row_bytes + off) = kv;
      *reinterpret_cast<u32x4*>(v_pool + slot * row_bytes + off) = vv;
    }
  }
}

}  // namespace

extern "C" int decode_append(int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* rows,
                             const int32_t* positions, const int32_t* slots, int32_t n, void* k_pool,
                             void* v_pool, const void* k_new, const void* v_new, int32_t num_kv_heads,
                             int32_t head_dim, int dtype, void* stream) {
  if (n < 0 || req_to_token_stride < 1 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128) ||
      (dtype != RT_F32 && dtype != RT_BF16))
    return rt::fail(RT_ERR_INVALID, "decode_append: bad size, shape or dtype");
  if (n == 0) return RT_OK;
  if (!req_to_token || !rows || !positions || !slots || !k_pool || !v_pool || !k_new || !v_new)
    return rt::fail(RT_ERR_INVALID, "decode_append: null pointer");
  const int64_t row_bytes = int64_t(num_kv_heads) * head_dim * (dtype == RT_BF16 ? 2 : 4);
  const uint32_t grid = uint32_t(n < 4096 ? n : 4096);
  hipLaunchKernelGGL(decode_append_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, req_to_token,
                     int64_t(req_to_token_stride), rows, positions, slots, (char*)k_pool, (char*)v_pool,
                     (const char*)k_new, (const char*)v_new, int(n), row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string("decode_append launch: ") + hipGetErrorString(e));
  return RT_OK;
}

extern "C" int kv_store(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                        const int32_t* out_cache_loc, int32_t n_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int dtype, void* stream) {
  if (n_tokens < 0 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128) ||
      (dtype != RT_F32 && dtype != RT_BF16))
    return rt::fail(RT_ERR_INVALID, "kv_store: bad shape or dtype");
  if (n_tokens == 0) return RT_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !out_cache_loc)
    return rt::fail(RT_ERR_INVALID, "kv_store: null pointer");
  const int64_t eb = dtype == RT_BF16 ? 2 : 4;
  const int64_t row_bytes = int64_t(num_kv_heads) * head_dim * eb;
  const int64_t total = int64_t(n_tokens) * (row_bytes >> 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(kv_store_kernel, dim3(uint32_t(blocks)), dim3(256), 0, (hipStream_t)stream,
                     (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, out_cache_loc,
                     int64_t(n_tokens), row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string("kv_store launch: ") + hipGetErrorString(e));
  return RT_OK;
}
