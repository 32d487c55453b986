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

using rtk::u32x2;
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

// bf16 rows in, FP8 rows out: 8 values per piece (16 bytes read, 8 written).
__global__ void __launch_bounds__(256) kv_store_fp8_kernel(uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                           const char* __restrict__ k_new,
                                                           const char* __restrict__ v_new,
                                                           const int32_t* __restrict__ loc, int64_t n_tokens,
                                                           int64_t row_elems, float k_inv, float v_inv) {
  const int64_t pieces_per_row = row_elems >> 3;
  const int64_t total = n_tokens * pieces_per_row;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; p < total; p += stride) {
    const int64_t t = p / pieces_per_row;
    const int64_t e = (p - t * pieces_per_row) << 3;
    const int64_t slot = loc[t];
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + (t * row_elems + e) * 2);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + (t * row_elems + e) * 2);
    u32x2 ko = {0u, 0u}, vo = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t kb = (kw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const uint32_t vb = (vw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      ko[i >> 2] |= rtk::f32_to_e4m3(__uint_as_float(kb << 16) * k_inv) << (8 * (i & 3));
      vo[i >> 2] |= rtk::f32_to_e4m3(__uint_as_float(vb << 16) * v_inv) << (8 * (i & 3));
    }
    *reinterpret_cast<u32x2*>(k_pool + slot * row_elems + e) = ko;
    *reinterpret_cast<u32x2*>(v_pool + slot * row_elems + e) = vo;
  }
}

// decode_append for FP8 pools: block t writes token t's slot into the slot
// table and stores its K and V rows as E4M3 codes (8 values per piece).
__global__ void __launch_bounds__(256) decode_append_fp8_kernel(int32_t* __restrict__ r2t, int64_t stride,
                                                                const int32_t* __restrict__ rows,
                                                                const int32_t* __restrict__ pos,
                                                                const int32_t* __restrict__ slots,
                                                                uint8_t* __restrict__ k_pool,
                                                                uint8_t* __restrict__ v_pool,
                                                                const char* __restrict__ k_new,
                                                                const char* __restrict__ v_new, int n,
                                                                int64_t row_elems, float k_inv, float v_inv) {
  const int64_t pieces = row_elems >> 3;
  for (int t = blockIdx.x; t < n; t += gridDim.x) {
    const int64_t slot = slots[t];
    if (threadIdx.x == 0) r2t[int64_t(rows[t]) * stride + pos[t]] = int32_t(slot);
    for (int64_t p = threadIdx.x; p < pieces; p += blockDim.x) {
      const int64_t e = p << 3;
      const u32x4 kw = *reinterpret_cast<const u32x4*>(k_new + (t * row_elems + e) * 2);
      const u32x4 vw = *reinterpret_cast<const u32x4*>(v_new + (t * row_elems + e) * 2);
      u32x2 ko = {0u, 0u}, vo = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t kb = (kw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
        const uint32_t vb = (vw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
        ko[i >> 2] |= rtk::f32_to_e4m3(__uint_as_float(kb << 16) * k_inv) << (8 * (i & 3));
        vo[i >> 2] |= rtk::f32_to_e4m3(__uint_as_float(vb << 16) * v_inv) << (8 * (i & 3));
      }
      *reinterpret_cast<u32x2*>(k_pool + slot * row_elems + e) = ko;
      *reinterpret_cast<u32x2*>(v_pool + slot * row_elems + e) = vo;
    }
  }
}

}  // namespace

extern "C" int decode_append_fp8(int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* rows,
                                 const int32_t* positions, const int32_t* slots, int32_t n, void* k_pool,
                                 void* v_pool, const void* k_new, const void* v_new, int32_t num_kv_heads,
                                 int32_t head_dim, float k_scale, float v_scale, void* stream) {
  if (n < 0 || req_to_token_stride < 1 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128) ||
      !(k_scale > 0.f) || !(v_scale > 0.f))
    return rt::fail(RT_ERR_INVALID, "decode_append_fp8: bad size, shape or scale");
  if (n == 0) return RT_OK;
  if (!req_to_token || !rows || !positions || !slots || !k_pool || !v_pool || !k_new || !v_new)
    return rt::fail(RT_ERR_INVALID, "decode_append_fp8: null pointer");
  const int64_t row_elems = int64_t(num_kv_heads) * head_dim;
  const uint32_t grid = uint32_t(n < 4096 ? n : 4096);
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  hipLaunchKernelGGL(decode_append_fp8_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, req_to_token,
                     int64_t(req_to_token_stride), rows, positions, slots, (uint8_t*)k_pool, (uint8_t*)v_pool,
                     (const char*)k_new, (const char*)v_new, int(n), row_elems, k_inv, v_inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return rt::fail(RT_ERR_HIP, std::string("decode_append_fp8 launch: ") + hipGetErrorString(e));
  return RT_OK;
}

extern "C" int kv_store_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                            const int32_t* out_cache_loc, int32_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                            float k_scale, float v_scale, void* stream) {
  if (n_tokens < 0 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128) || !(k_scale > 0.f) ||
      !(v_scale > 0.f))
    return rt::fail(RT_ERR_INVALID, "kv_store_fp8: bad shape or scale");
  if (n_tokens == 0) return RT_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !out_cache_loc)
    return rt::fail(RT_ERR_INVALID, "kv_store_fp8: null pointer");
  const int64_t row_elems = int64_t(num_kv_heads) * head_dim;
  const int64_t total = int64_t(n_tokens) * (row_elems >> 3);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  hipLaunchKernelGGL(kv_store_fp8_kernel, dim3(uint32_t(blocks)), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)k_pool, (uint8_t*)v_pool, (const char*)k_new, (const char*)v_new, out_cache_loc,
                     int64_t(n_tokens), row_elems, k_inv, v_inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string("kv_store_fp8 launch: ") + hipGetErrorString(e));
  return RT_OK;
}

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
