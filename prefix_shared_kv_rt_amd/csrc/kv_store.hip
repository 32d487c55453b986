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


// Extend scatter driven by the slot table: block (x, b) moves extend rows
// j0 .. j0 + kExtTok - 1 of request b (j0 = x * kExtTok); row j of request b
// is source row qo[b] + j and lands at slot r2t[row_b][prefix_lens[b] + j].
// Threads walk the block's rows as consecutive 16-byte source pieces, so a
// wave reads and writes whole lines.  FP8 pools take 8 bf16 values per piece
// and store their 8 codes.
constexpr int kExtTok = 8;

template <bool FP8>
__global__ void __launch_bounds__(256) kv_store_extend_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ r2t, int64_t stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ qo_indptr, uint32_t pieces,
    int64_t src_row_bytes, int64_t dst_row_bytes, float k_inv, float v_inv) {
  const int b = blockIdx.y;
  const int j0 = blockIdx.x * kExtTok;
  const int E = extend_lens[b];
  if (j0 >= E) return;
  const uint32_t n = uint32_t(min(kExtTok, E - j0));
  const int64_t row = rpi ? rpi[b] : b;
  const int32_t* slots = r2t + row * stride + prefix_lens[b] + j0;
  const int64_t src0 = int64_t(qo_indptr[b]) + j0;
  const uint32_t total = n * pieces;
  // kUnroll pieces per thread per round, all loaded before any is stored, so
  // each thread keeps 2 * kUnroll 16-byte loads in flight.
  constexpr int kUnroll = 4;
  for (uint32_t base = threadIdx.x; base < total; base += kUnroll * blockDim.x) {
    u32x4 kw[kUnroll], vw[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t idx = base + u * blockDim.x;
      if (idx < total) {
        const uint32_t t = idx / pieces;
        const uint32_t pc = idx - t * pieces;
        const int64_t src = (src0 + t) * src_row_bytes + int64_t(pc) * 16;
        kw[u] = *reinterpret_cast<const u32x4*>(k_new + src);
        vw[u] = *reinterpret_cast<const u32x4*>(v_new + src);
        dst[u] = int64_t(slots[t]) * dst_row_bytes + int64_t(pc) * (FP8 ? 8 : 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (base + u * blockDim.x >= total) break;
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(k_pool + dst[u]) = kw[u];
        *reinterpret_cast<u32x4*>(v_pool + dst[u]) = vw[u];
      } else {
        u32x2 ko = {0u, 0u}, vo = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t kb = (kw[u][i >> 1] >> (16 * (i & 1))) & 0xffffu;
          const uint32_t vb = (vw[u][i >> 1] >> (16 * (i & 1))) & 0xffffu;
          ko[i >> 2] |= rtk::f32_to_e4m3(__uint_as_float(kb << 16) * k_inv) << (8 * (i & 3));
          vo[i >> 2] |= rtk::f32_to_e4m3(__uint_as_float(vb << 16) * v_inv) << (8 * (i & 3));
        }
        *reinterpret_cast<u32x2*>(k_pool + dst[u]) = ko;
        *reinterpret_cast<u32x2*>(v_pool + dst[u]) = vo;
      }
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

namespace {

int store_extend(const char* name, bool fp8, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                 const int32_t* req_to_token, int32_t stride, const int32_t* req_pool_indices,
                 const int32_t* prefix_lens, const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                 int32_t max_extend_len, int32_t num_kv_heads, int32_t head_dim, int64_t eb, float k_inv,
                 float v_inv, void* stream) {
  if (batch < 0 || max_extend_len < 0 || stride < 1 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128))
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": bad size or shape");
  if (batch > 65535) return rt::fail(RT_ERR_INVALID, std::string(name) + ": batch above 65535");
  if (batch == 0 || max_extend_len == 0) return RT_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !req_to_token || !prefix_lens || !extend_lens || !qo_indptr)
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": null pointer");
  const int64_t row_elems = int64_t(num_kv_heads) * head_dim;
  const int64_t src_row_bytes = row_elems * eb;
  const uint32_t pieces = uint32_t(src_row_bytes / 16);
  const dim3 grid{uint32_t((int64_t(max_extend_len) + kExtTok - 1) / kExtTok), uint32_t(batch)};
  if (fp8)
    hipLaunchKernelGGL(kv_store_extend_kernel<true>, grid, dim3(256), 0, (hipStream_t)stream, (char*)k_pool,
                       (char*)v_pool, (const char*)k_new, (const char*)v_new, req_to_token, int64_t(stride),
                       req_pool_indices, prefix_lens, extend_lens, qo_indptr, pieces, src_row_bytes, row_elems,
                       k_inv, v_inv);
  else
    hipLaunchKernelGGL(kv_store_extend_kernel<false>, grid, dim3(256), 0, (hipStream_t)stream, (char*)k_pool,
                       (char*)v_pool, (const char*)k_new, (const char*)v_new, req_to_token, int64_t(stride),
                       req_pool_indices, prefix_lens, extend_lens, qo_indptr, pieces, src_row_bytes, src_row_bytes,
                       k_inv, v_inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string(name) + " launch: " + hipGetErrorString(e));
  return RT_OK;
}

}  // namespace

extern "C" int kv_store_extend(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                               const int32_t* req_to_token, int32_t req_to_token_stride,
                               const int32_t* req_pool_indices, const int32_t* prefix_lens,
                               const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                               int32_t max_extend_len, int32_t num_kv_heads, int32_t head_dim, int dtype,
                               void* stream) {
  if (dtype != RT_F32 && dtype != RT_BF16) return rt::fail(RT_ERR_INVALID, "kv_store_extend: bad dtype");
  return store_extend("kv_store_extend", false, k_pool, v_pool, k_new, v_new, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch, max_extend_len, num_kv_heads,
                      head_dim, dtype == RT_BF16 ? 2 : 4, 1.f, 1.f, stream);
}

extern "C" int kv_store_extend_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                   const int32_t* req_to_token, int32_t req_to_token_stride,
                                   const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                   const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                   int32_t max_extend_len, int32_t num_kv_heads, int32_t head_dim, float k_scale,
                                   float v_scale, void* stream) {
  if (!(k_scale > 0.f) || !(v_scale > 0.f)) return rt::fail(RT_ERR_INVALID, "kv_store_extend_fp8: bad scale");
  return store_extend("kv_store_extend_fp8", true, k_pool, v_pool, k_new, v_new, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch, max_extend_len, num_kv_heads,
                      head_dim, 2, 1.0f / k_scale, 1.0f / v_scale, stream);
}
