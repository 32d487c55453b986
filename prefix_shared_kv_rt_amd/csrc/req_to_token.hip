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

// 16-byte pieces when both ends are 16-byte aligned (vec), else 4-byte
// words; the grid strides over the pieces.
__global__ void __launch_bounds__(256) host_copy_kernel(char* __restrict__ dst, const char* __restrict__ src,
                                                        int64_t bytes, bool vec) {
  const int64_t step = int64_t(gridDim.x) * blockDim.x;
  const int64_t t0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n16 = bytes / 16;
    for (int64_t i = t0; i < n16; i += step)
      reinterpret_cast<rtk::u32x4*>(dst)[i] = reinterpret_cast<const rtk::u32x4*>(src)[i];
    done = n16 * 16;
  }
  const int64_t n4 = (bytes - done) / 4;
  for (int64_t i = t0; i < n4; i += step)
    reinterpret_cast<uint32_t*>(dst + done)[i] = reinterpret_cast<const uint32_t*>(src + done)[i];
}
}  // namespace

extern "C" int rt_copy_from_host(void* dst, const void* src, int64_t bytes, void* stream) {
  const char* name = "rt_copy_from_host";
  if (bytes < 0 || bytes % 4 != 0) return rt::fail(RT_ERR_INVALID, std::string(name) + ": bytes not a multiple of 4");
  if (bytes == 0) return RT_OK;
  if (!dst || !src) return rt::fail(RT_ERR_INVALID, std::string(name) + ": null pointer");
  if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 3)
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": pointers not 4-byte aligned");
  // The kernel reads src through its device mapping.  Both ends of the range
  // must resolve to one pinned allocation; anything else is refused here.
  void* dsrc = nullptr;
  void* dlast = nullptr;
  char* last = const_cast<char*>(static_cast<const char*>(src)) + (bytes - 1);
  const hipError_t e0 = hipHostGetDevicePointer(&dsrc, const_cast<void*>(src), 0);
  const hipError_t e1 = e0 == hipSuccess ? hipHostGetDevicePointer(&dlast, last, 0) : e0;
  if (e0 != hipSuccess || e1 != hipSuccess || !dsrc || static_cast<char*>(dlast) != static_cast<char*>(dsrc) + (bytes - 1)) {
    (void)hipGetLastError();
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": source is not inside one pinned host allocation");
  }
  // dst must be device memory whose allocation holds the whole range.
  hipPointerAttribute_t attr{};
  void* base = nullptr;
  size_t size = 0;
  const bool dev_ok = hipPointerGetAttributes(&attr, dst) == hipSuccess && attr.type == hipMemoryTypeDevice &&
                      hipMemGetAddressRange(&base, &size, dst) == hipSuccess &&
                      static_cast<char*>(dst) + bytes <= static_cast<char*>(base) + size;
  if (!dev_ok) {
    (void)hipGetLastError();
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": destination is not device memory holding bytes");
  }
  const bool vec = ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(dsrc)) & 15) == 0;
  const int64_t pieces = vec ? bytes / 16 : bytes / 4;
  const uint32_t blocks = uint32_t(std::min<int64_t>(1024, std::max<int64_t>(1, (pieces + 255) / 256)));
  hipLaunchKernelGGL(host_copy_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, static_cast<char*>(dst),
                     static_cast<const char*>(dsrc), bytes, vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string(name) + " launch: " + hipGetErrorString(e));
  return RT_OK;
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
