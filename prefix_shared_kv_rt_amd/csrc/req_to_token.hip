// req_to_token_scatter: write one slot per request into the device slot
// table, req_to_token[rows[i]][positions[i]] = slots[i] (the per-step
// update of the v0.2 runtime's req_to_token table by out_cache_loc, SGLang
// v0.2 handbook chapter, "CUDA Graph" section).

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
}  // namespace

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
