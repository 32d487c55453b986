// req_to_token_scatter: write one slot per request into the device slot
// table, req_to_token[rows[i]][positions[i]] = slots[i] (the per-step
// update of the v0.2 runtime's req_to_token table by out_cache_loc, SGLang
// v0.2 handbook chapter, "CUDA Graph" section).
//
// rt_copy_from_host: the step's host-built rows and metadata move to the
// device with a kernel on the caller's stream that reads pinned host memory
// directly.  An asynchronous host-to-device copy runs on a DMA engine, and
// the hand-over between that engine and the compute queue leaves the GPU
// idle on both sides of the copy; the kernel keeps the whole step on one
// queue.

#include <algorithm>
#include <cstdint>

#include "dev_common.h"
#include "radixrt.h"
#include "rt_internal.h"

namespace {
__global__ void __launch_bounds__(256) r2t_scatter_kernel(int32_t* __restrict__ r2t, int64_t stride,
                                                          const int32_t* __restrict__ rows,
                                                          const int32_t* __restrict__ pos,
                                                          const int32_t* __restrict__ slots, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) r2t[int64_t(rows[i]) * stride + pos[i]] = slots[i];
}

// height rows of width bytes, at the given pitches; 16-byte pieces when
// every row start is 16-byte aligned (vec), else 4-byte words.  The grid
// strides over the pieces of all rows.
__global__ void __launch_bounds__(256) host_copy_kernel(char* __restrict__ dst, int64_t dst_pitch,
                                                        const char* __restrict__ src, int64_t src_pitch,
                                                        int64_t width, int64_t height, bool vec) {
  const int64_t step = int64_t(gridDim.x) * blockDim.x;
  const int64_t t0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_row = vec ? width / 16 : width / 4;
  const int64_t total = per_row * height;
  for (int64_t i = t0; i < total; i += step) {
    const int64_t r = i / per_row, c = i - r * per_row;
    if (vec)
      *reinterpret_cast<rtk::u32x4*>(dst + r * dst_pitch + c * 16) =
          *reinterpret_cast<const rtk::u32x4*>(src + r * src_pitch + c * 16);
    else
      *reinterpret_cast<uint32_t*>(dst + r * dst_pitch + c * 4) =
          *reinterpret_cast<const uint32_t*>(src + r * src_pitch + c * 4);
  }
}
}  // namespace

namespace {
// Host-side checks of a copy (nothing is launched); on success *dsrc is the
// device mapping of src.
int check_copy(const char* name, void* dst, int64_t dst_pitch, const void* src, int64_t src_pitch, int64_t width,
               int64_t height, const void** dsrc) {
  if (width < 0 || height < 0 || width % 4 != 0 || dst_pitch % 4 != 0 || src_pitch % 4 != 0 ||
      (height > 1 && (dst_pitch < width || src_pitch < width)))
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": sizes or pitches not multiples of 4, or pitch < width");
  *dsrc = nullptr;
  if (width == 0 || height == 0) return RT_OK;
  if (!dst || !src) return rt::fail(RT_ERR_INVALID, std::string(name) + ": null pointer");
  if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 3)
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": pointers not 4-byte aligned");
  const int64_t src_span = (height - 1) * src_pitch + width;  // bytes from the first to past the last read
  const int64_t dst_span = (height - 1) * dst_pitch + width;
  // src: pinned host memory whose allocation (as the runtime records it)
  // holds the whole range; the kernel reads it through its device mapping.
  hipPointerAttribute_t sattr{};
  void* sbase = nullptr;
  size_t ssize = 0;
  void* mapped = nullptr;
  const bool src_ok = hipPointerGetAttributes(&sattr, src) == hipSuccess && sattr.type == hipMemoryTypeHost &&
                      hipMemGetAddressRange(&sbase, &ssize, const_cast<void*>(src)) == hipSuccess &&
                      static_cast<const char*>(src) >= static_cast<char*>(sbase) &&
                      static_cast<const char*>(src) + src_span <= static_cast<char*>(sbase) + ssize &&
                      hipHostGetDevicePointer(&mapped, const_cast<void*>(src), 0) == hipSuccess && mapped;
  if (!src_ok) {
    (void)hipGetLastError();
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": source is not inside one pinned host allocation");
  }
  // dst: device memory whose allocation holds the whole range.
  hipPointerAttribute_t attr{};
  void* base = nullptr;
  size_t size = 0;
  const bool dev_ok = hipPointerGetAttributes(&attr, dst) == hipSuccess && attr.type == hipMemoryTypeDevice &&
                      hipMemGetAddressRange(&base, &size, dst) == hipSuccess &&
                      static_cast<char*>(dst) + dst_span <= static_cast<char*>(base) + size;
  if (!dev_ok) {
    (void)hipGetLastError();
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": destination is not device memory holding the range");
  }
  *dsrc = mapped;
  return RT_OK;
}

int copy_from_host(const char* name, void* dst, int64_t dst_pitch, const void* src, int64_t src_pitch,
                   int64_t width, int64_t height, void* stream) {
  const void* dsrc = nullptr;
  const int rc = check_copy(name, dst, dst_pitch, src, src_pitch, width, height, &dsrc);
  if (rc != RT_OK || width == 0 || height == 0) return rc;
  const bool vec = ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(dsrc) | uintptr_t(width) |
                     uintptr_t(height > 1 ? dst_pitch | src_pitch : 0)) & 15) == 0;
  const int64_t pieces = (vec ? width / 16 : width / 4) * height;
  const uint32_t blocks = uint32_t(std::min<int64_t>(1024, std::max<int64_t>(1, (pieces + 255) / 256)));
  hipLaunchKernelGGL(host_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, static_cast<char*>(dst),
                     dst_pitch, static_cast<const char*>(dsrc), src_pitch, width, height, vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string(name) + " launch: " + hipGetErrorString(e));
  return RT_OK;
}
}  // namespace

extern "C" int rt_copy_from_host_check(void* dst, int64_t dst_pitch, const void* src, int64_t src_pitch,
                                       int64_t width, int64_t height) {
  const void* dsrc = nullptr;
  return check_copy("rt_copy_from_host_check", dst, dst_pitch, src, src_pitch, width, height, &dsrc);
}

extern "C" int rt_copy_from_host(void* dst, const void* src, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 4 != 0) return rt::fail(RT_ERR_INVALID, "rt_copy_from_host: bytes not a multiple of 4");
  return copy_from_host("rt_copy_from_host", dst, bytes, src, bytes, bytes, 1, stream);
}

extern "C" int rt_copy_from_host_2d(void* dst, int64_t dst_pitch, const void* src, int64_t src_pitch,
                                    int64_t width, int64_t height, void* stream) {
  return copy_from_host("rt_copy_from_host_2d", dst, dst_pitch, src, src_pitch, width, height, stream);
}

extern "C" int req_to_token_scatter(int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* rows,
                                    const int32_t* positions, const int32_t* slots, int32_t n, void* stream) {
  if (n < 0 || req_to_token_stride < 1) return rt::fail(RT_ERR_INVALID, "req_to_token_scatter: bad size");
  if (n == 0) return RT_OK;
  if (!req_to_token || !rows || !positions || !slots)
    return rt::fail(RT_ERR_INVALID, "req_to_token_scatter: null pointer");
  hipLaunchKernelGGL(r2t_scatter_kernel, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     req_to_token, int64_t(req_to_token_stride), rows, positions, slots, int(n));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return rt::fail(RT_ERR_HIP, std::string("req_to_token_scatter launch: ") + hipGetErrorString(e));
  return RT_OK;
}
