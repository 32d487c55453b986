// radix_decode_attention: batched decode attention over the token pool.
//
// Each request has one query row (its newest token, whose K/V the scatter
// kernel already wrote, or, in the _append entry points, the decode launch
// writes itself) and attends its whole context: keys 0..prefix_len,
// gathered through the request's req_to_token row (the per-request slot
// table of the SGLang v0.2 handbook chapter, "CUDA Graph" section).  The
// cached prefix found by the radix tree is read in place, never recomputed
// (SGLang explainer, section 04).
//
// Decode is bound by HBM bandwidth: every K/V row of every request is read
// once per step and used for only a few multiply-adds.  The design is built
// around moving those bytes:
//  * Split-K: the context is cut into chunks; one wavefront owns one
//    (request, KV head, chunk) and keeps an online-softmax state; a second
//    kernel merges the chunks exactly from their (max, sum, accumulator).
//  * GQA grouping: the wavefront computes all G = Hq / Hkv query heads of
//    its KV head at once, so each K/V row is fetched once per group.
//  * A chunk's slot indices are staged in the wave's LDS once, so the
//    dependent index->row load chain costs one round trip per chunk, and the
//    rows of the next 16-key block are in flight while one is consumed.
//  * bf16: the G x 16-key score tile and the PV update are MFMA
//    contractions (16x16x32 for Q K^T, 16x16x16 for P V) whose operands are
//    loaded straight from HBM in the MFMA lane layout: K rows as 64-byte
//    runs, V rows whole (each lane takes D/16 consecutive dims, 16 bytes at
//    D = 128, of 4 keys: the PV contraction dimension is the key, and the
//    dims are regrouped in registers).
//  * fp32 inputs take a plain VALU path (one lane per dim, wave-wide dot
//    products); it exists for full-precision checks, not for speed.

#include <math.h>

#include <stdlib.h>

#include <algorithm>
#include <type_traits>
#include <mutex>
#include <string>

#include "decode_split.h"
#include "dev_common.h"
#include "radixrt.h"
#include "rt_internal.h"

namespace {

using namespace rtk;

struct DecodePlan {
  int splits;  // context chunks per (request, KV head)
  int chunk;   // keys per chunk (multiple of 16, at most kMaxChunk)
};

// Slot indices of one chunk are staged in LDS (16 KiB at 4096 keys).  On
// MI355X, all-private decode of 32 x 16385 keys (Hkv 8, D 128, bf16) takes
// 374 us with chunks of up to 4096 keys (6 per request and head) against
// 399 us with up to 2048 (9): fewer, longer streams per wave read HBM closer
// to a plain streaming read of the same bytes (6.3 TB/s).
constexpr int kMaxChunk = 4096;
constexpr int64_t kMaxKvLen = 2097152;  // longest context a decode call accepts
// FP8 pools move half the bytes per key, so a wave streams a chunk's keys
// with less in flight; shorter chunks (more items) keep HBM busier on long
// contexts (32 x 32897 keys: 24 chunks in 327 us against 17 in 358 us).
constexpr int kMaxChunkFp8 = 1408;
constexpr int kMaxChunkFp8Lds = 2048;  // longest FP8 chunk: kMaxKvLen / 1024 splits
static_assert(kMaxKvLen <= int64_t(1024) * kMaxChunkFp8Lds && kMaxChunkFp8 <= kMaxChunkFp8Lds &&
                  kMaxChunkFp8Lds <= kMaxChunk,
              "a plan's chunk must fit the kernel's staged index array");
// About six work items per CU: fewer, longer chunks amortise each item's
// index staging, Q load and partial write.  On MI355X, 1536 is faster than
// 6144 for few-shot (35 against 45 us), fork (108 against 112 us) and long
// context (574 against 582 us) decode; 512 or fewer starve few-shot.
constexpr int kTargetItems = 1536;

// Chunk the context into about kTargetItems (chunk, KV head, request) work
// items; chunks hold at least 64 keys and at most max_chunk (at most
// kMaxChunk in any case).  Depends only on the call's sizes and pool format.
DecodePlan plan_decode(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len, int max_chunk = kMaxChunk,
                       int target_items = kTargetItems) {
  const int64_t units = int64_t(batch) * num_kv_heads;
  int64_t s = (target_items + units - 1) / units;
  s = std::max<int64_t>(s, (max_kv_len + max_chunk - 1) / max_chunk);
  s = std::min<int64_t>(s, std::max(1, (max_kv_len + 63) / 64));
  s = std::max<int64_t>(std::min<int64_t>(s, 1024), 1);
  int chunk = int((max_kv_len + s - 1) / s);
  chunk = (chunk + 15) / 16 * 16;
  const int splits = (max_kv_len + chunk - 1) / chunk;
  return {splits, chunk};
}

// The shared-prefix decode: pass A (the extend kernel's partial mode) cuts
// the longest shared part into n_a chunks of chunk_a keys (a multiple of the
// extend tile, 128..2048 keys, about 256 items of (query tile, group, KV
// head, chunk)); pass B is the split plan over the longest private tail.
// Partial slots 0 .. n_a - 1 of each (request, head) hold pass A's chunks,
// n_a .. n_a + b.splits - 1 pass B's.
struct SharedPlan {
  int n_a, chunk_a;
  DecodePlan b;
  int total() const { return n_a + b.splits; }
};
constexpr int kSharedRows = 128;  // query rows per item of the extend kernel
#ifndef RT_SHARED_ITEMS
#define RT_SHARED_ITEMS 256
#endif
#ifndef RT_SHARED_MIN_CHUNK
#define RT_SHARED_MIN_CHUNK 128
#endif
constexpr int kSharedItems = RT_SHARED_ITEMS;        // target work items of the shared pass
// Target work items of the private pass.  Long-context private tails (32 x
// 16385 keys beside the overlapped shared pass): 1024 or 512 -> 416 us per
// call, 1536 -> 421, 3072 -> 446; few-shot tails (130 keys) are the same
// 30-31 us for all four.
constexpr int kPrivateItems = 1024;
constexpr int kSharedMinChunk = RT_SHARED_MIN_CHUNK;  // shortest shared chunk (keys)
SharedPlan plan_shared(int32_t batch, int32_t Hq, int32_t Hkv, int32_t n_groups, int32_t max_group_size,
                       int32_t max_shared_len, int32_t max_private_len, int max_chunk) {
  SharedPlan sp{0, 64, plan_decode(batch, Hkv, std::max(max_private_len, 1), max_chunk, kPrivateItems)};
  if (max_shared_len > 0) {
    const int64_t n_qt = (int64_t(max_group_size) * (Hq / Hkv) + kSharedRows - 1) / kSharedRows;
    const int64_t units = std::max<int64_t>(1, n_qt * n_groups * Hkv);
    int64_t c = (kSharedItems + units - 1) / units;
    c = std::max<int64_t>(c, (max_shared_len + 2047) / 2048);
    c = std::min<int64_t>(c, std::max<int64_t>(1, (max_shared_len + kSharedMinChunk - 1) / kSharedMinChunk));
    int chunk = int((max_shared_len + c - 1) / c);
    chunk = (chunk + 63) / 64 * 64;
    sp.chunk_a = chunk;
    sp.n_a = (max_shared_len + chunk - 1) / chunk;
  }
  return sp;
}

// ----------------------------------------------------------------- bf16 --
// Persistent waves, one per 64-thread workgroup: the grid holds as many
// waves as fit on the chip (rtk::dec::split_items has the item order).
template <int D, bool KV8, bool APP = false>
__global__ void __launch_bounds__(64) decode_split_bf16(
    const char* __restrict__ q, const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const int32_t* __restrict__ req_to_token, int64_t stride, const int32_t* __restrict__ rpi,
    const int32_t* __restrict__ prefix_lens, int B, int Hq, int Hkv, int G, int S, int chunk, float scale_log2,
    float v_scale, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    const int32_t* __restrict__ key_start, int s_off, int S_total, rt::AppendArgs app) {
  // FP8 chunks hold at most 1408 keys, or 2048 when a context needs more
  // than 1024 of them: the smaller array keeps LDS from limiting occupancy.
  __shared__ int32_t s_idx[KV8 ? kMaxChunkFp8Lds : kMaxChunk];
  rtk::dec::split_items<D, KV8, 0, APP>(blockIdx.x & 7, blockIdx.x >> 3, gridDim.x >> 3, threadIdx.x, s_idx, q, k_pool,
                                v_pool, req_to_token, stride, rpi, prefix_lens, B, Hq, Hkv, G, S, chunk, scale_log2,
                                v_scale, ws_acc, ws_ml, key_start, s_off, S_total, app);
}

// ----------------------------------------------------------------- fp32 --
template <int D>
__global__ void __launch_bounds__(64) decode_split_f32(
    const float* __restrict__ q, const float* __restrict__ k_pool, const float* __restrict__ v_pool,
    const int32_t* __restrict__ req_to_token, int64_t stride, const int32_t* __restrict__ rpi,
    const int32_t* __restrict__ prefix_lens, int Hq, int Hkv, int G, int S, int chunk, float scale_log2,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
  constexpr int PER = D / 64;  // dims per lane
  const int lane = threadIdx.x;
  int item = blockIdx.x;
  const int s = item % S;
  item /= S;
  const int h = item % Hq;
  const int b = item / Hq;
  const int kvh = h / G;
  const int kv_len = prefix_lens[b] + 1;
  const int start = s * chunk;
  const int end = min(kv_len, start + chunk);
  const int32_t* idx_row = req_to_token + int64_t(rpi ? rpi[b] : b) * stride;
  const int64_t row = int64_t(Hkv) * D;

  float qd[PER], acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    qd[i] = q[(int64_t(b) * Hq + h) * D + lane + 64 * i];
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int key = start; key < end; ++key) {
    const int64_t slot = idx_row[key];
    const float* kr = k_pool + slot * row + int64_t(kvh) * D;
    const float* vr = v_pool + slot * row + int64_t(kvh) * D;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) part = fmaf(qd[i], kr[lane + 64 * i], part);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += shfl_xor(part, off);
    const float sc = part * scale_log2;
    const float m_new = fmaxf(m, sc);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(p, vr[lane + 64 * i], acc[i] * alpha);
    m = m_new;
  }
  const int64_t part = (int64_t(b) * Hq + h) * S + s;
  if (lane == 0) {
    ws_ml[part * 2 + 0] = m;
    ws_ml[part * 2 + 1] = l;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) ws_acc[part * D + lane + 64 * i] = acc[i];
}

// -------------------------------------------------------------- combine --
// One wave per (request, query head): merges the S split partials exactly,
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
// Lane s (mod 64) reads partial s's (m, l), so the max and the weights take
// wave reductions instead of a loop; the accumulators are then read eight
// partials at a time (a short last batch padded with weight-0 repeats) with
// every load issued before the multiply-adds, so a long split costs a few
// memory round trips, not one per partial; up to kCombineFast partials are
// read in one batch beside their (m, l).
constexpr int kCombineFast = 16;  // splits up to this many take the one-round-trip path
template <int D, bool BF16>
__global__ void __launch_bounds__(64) decode_combine(const float* __restrict__ ws_acc,
                                                     const float* __restrict__ ws_ml, int S,
                                                     void* __restrict__ out) {
  constexpr int PER = D / 64;
  constexpr int U = 8;  // partials per batch of loads
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;  // b * Hq + h
  const float* ml = ws_ml + bh * S * 2;
  const float* acc_s = ws_acc + bh * S * D + lane;
  if (S <= kCombineFast) {
    // Short splits: every partial's accumulator loads go out with the
    // (m, l) loads, so the whole merge waits for one memory round trip.
    float a[kCombineFast][PER];
#pragma unroll
    for (int u = 0; u < kCombineFast; ++u) {
      const int64_t sp = min(u, S - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) a[u][i] = acc_s[sp * D + 64 * i];
    }
    const float m_s = lane < S ? ml[2 * lane] : -INFINITY;
    const float l_s = lane < S ? ml[2 * lane + 1] : 0.f;
    float mx = m_s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
    const float w = lane < S ? exp2f(m_s - mx) : 0.f;
    float L = w * l_s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += shfl_xor(L, off);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
#pragma unroll
    for (int u = 0; u < kCombineFast; ++u) {
      // lanes past S hold weight 0, so the repeated loads of partial S - 1 add nothing
      const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(wu, a[u][i], acc[i]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float v = acc[i] * inv;
      if (BF16)
        reinterpret_cast<uint16_t*>(out)[bh * D + lane + 64 * i] = uint16_t(f32_to_bf16_bits(v));
      else
        reinterpret_cast<float*>(out)[bh * D + lane + 64 * i] = v;
    }
    return;
  }
  float mmax = -INFINITY;
  for (int s = lane; s < S; s += 64) mmax = fmaxf(mmax, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, shfl_xor(mmax, off));
  float L = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    // weight of partial s0 + lane; empty chunks have m = -inf -> 0
    const int n = min(64, S - s0);
    const float w = lane < n ? exp2f(ml[2 * (s0 + lane)] - mmax) : 0.f;
    float lw = lane < n ? w * ml[2 * (s0 + lane) + 1] : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lw += shfl_xor(lw, off);
    L += lw;
    // batches of U partials; a short last batch repeats partial n - 1 with
    // weight 0, so every batch issues all its loads at once
    for (int j = 0; j < n; j += U) {
      float a[U][PER];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t sp = s0 + min(j + u, n - 1);
#pragma unroll
        for (int i = 0; i < PER; ++i) a[u][i] = acc_s[sp * D + 64 * i];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int src = min(j + u, 63);
        float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), src));
        if (j + u >= n) wu = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(wu, a[u][i], acc[i]);
      }
    }
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float v = acc[i] * inv;
    if (BF16)
      reinterpret_cast<uint16_t*>(out)[bh * D + lane + 64 * i] = uint16_t(f32_to_bf16_bits(v));
    else
      reinterpret_cast<float*>(out)[bh * D + lane + 64 * i] = v;
  }
}

// Resident 64-thread blocks of the bf16 split kernel on this device
// (occupancy x compute units, a multiple of 8), queried once per device.
template <int D, bool KV8, bool APP = false>
int resident_waves() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 2048;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_bf16<D, KV8, APP>, 64, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
        cus < 1)
      return 2048;
    cached[dev] = std::max(8, (per_cu * cus) / 8 * 8);
  }
  return cached[dev];
}

// Pool formats of launch_decode: the two public dtypes plus FP8 K/V under
// bf16 q/o.
constexpr int kModeFp8Kv = 100;

template <int D>
hipError_t launch_decode(const void* q, void* o, const void* k_pool, const void* v_pool, const int32_t* r2t,
                   int64_t stride, const int32_t* rpi, const int32_t* plens, int B, int Hq, int Hkv,
                   DecodePlan pl, float scale_log2, float v_scale, int mode, float* ws_acc, float* ws_ml,
                   hipStream_t st, const int32_t* key_start = nullptr, int s_off = 0, int S_total = 0,
                   hipEvent_t combine_after = nullptr, const rt::AppendArgs& app = rt::AppendArgs()) {
  // combine_after (optional): work on another stream that also writes
  // partials; the combine waits for it.  Returns the wait's status.
  const int G = Hq / Hkv;
  if (S_total == 0) S_total = pl.splits;
  // the chunk's slot indices must fit the kernel's LDS array
  if (pl.chunk > (mode == kModeFp8Kv ? kMaxChunkFp8Lds : kMaxChunk)) return hipErrorInvalidValue;
  if (mode == RT_BF16 || mode == kModeFp8Kv) {
    const int64_t items = int64_t(B) * Hkv * pl.splits;
#define RT_SPLIT_LAUNCH(K8, AP)                                                                                  \
  do {                                                                                                           \
    const int64_t grid = std::min<int64_t>(resident_waves<D, K8, AP>(), (items + 7) / 8 * 8);                   \
    hipLaunchKernelGGL((decode_split_bf16<D, K8, AP>), dim3(uint32_t(grid)), dim3(64), 0, st, (const char*)q,   \
                       (const char*)k_pool, (const char*)v_pool, r2t, stride, rpi, plens, B, Hq, Hkv, G, pl.splits, \
                       pl.chunk, scale_log2, K8 ? v_scale : 1.0f, ws_acc, ws_ml, key_start, s_off, S_total, app);  \
  } while (0)
    if (mode == RT_BF16) {
      if (app.slots) RT_SPLIT_LAUNCH(false, true); else RT_SPLIT_LAUNCH(false, false);
    } else {
      if (app.slots) RT_SPLIT_LAUNCH(true, true); else RT_SPLIT_LAUNCH(true, false);
    }
#undef RT_SPLIT_LAUNCH
    if (combine_after) {
      const hipError_t we = hipStreamWaitEvent(st, combine_after, 0);
      if (we != hipSuccess) return we;
    }
    hipLaunchKernelGGL((decode_combine<D, true>), dim3(uint32_t(int64_t(B) * Hq)), dim3(64), 0, st, ws_acc,
                       ws_ml, S_total, o);
  } else {
    const uint32_t grid = uint32_t(int64_t(B) * Hq * pl.splits);
    hipLaunchKernelGGL(decode_split_f32<D>, dim3(grid), dim3(64), 0, st, (const float*)q,
                       (const float*)k_pool, (const float*)v_pool, r2t, stride, rpi, plens, Hq, Hkv, G,
                       pl.splits, pl.chunk, scale_log2, ws_acc, ws_ml);
    hipLaunchKernelGGL((decode_combine<D, false>), dim3(uint32_t(int64_t(B) * Hq)), dim3(64), 0, st, ws_acc,
                       ws_ml, pl.splits, o);
  }
  return hipSuccess;
}

int decode_entry(const char* name, const void* q, void* o, const void* k_pool, const void* v_pool,
                 const int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* req_pool_indices,
                 const int32_t* prefix_lens, int32_t batch, int32_t max_kv_len, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, float sm_scale, float k_scale, float v_scale, int mode,
                 void* workspace, int64_t workspace_bytes, void* stream,
                 const rt::AppendArgs& app = rt::AppendArgs()) {
  const std::string fn(name);
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || max_kv_len < 1 || req_to_token_stride < max_kv_len ||
      !(sm_scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return rt::fail(RT_ERR_INVALID, fn + ": bad shape, stride or scale");
  if (int64_t(max_kv_len) > kMaxKvLen)
    return rt::fail(RT_ERR_INVALID, fn + ": max_kv_len above 2097152");
  if (mode != RT_F32 && num_q_heads / num_kv_heads > 16)
    return rt::fail(RT_ERR_INVALID, fn + ": the bf16 path supports at most 16 query heads per KV head");
  if (batch == 0) return RT_OK;
  if (!q || !o || !k_pool || !v_pool || !req_to_token || !prefix_lens || !workspace ||
      (app.slots && (!app.k_new || !app.v_new)))
    return rt::fail(RT_ERR_INVALID, fn + ": null pointer");
  if (app.slots && mode == RT_F32) return rt::fail(RT_ERR_INVALID, fn + ": bf16 or FP8 pools only");
  const int64_t need = radix_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_kv_len);
  if (workspace_bytes < need)
    return rt::fail(RT_ERR_INVALID, fn + ": workspace too small (need " + std::to_string(need) + ")");
  const DecodePlan pl = plan_decode(batch, num_kv_heads, max_kv_len, mode == kModeFp8Kv ? kMaxChunkFp8 : kMaxChunk);
  float* ws_acc = static_cast<float*>(workspace);
  float* ws_ml = ws_acc + int64_t(batch) * num_q_heads * pl.splits * head_dim;
  const float scale_log2 = sm_scale * k_scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  const hipError_t le =
      head_dim == 128
          ? launch_decode<128>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices,
                               prefix_lens, batch, num_q_heads, num_kv_heads, pl, scale_log2, v_scale, mode, ws_acc,
                               ws_ml, st, nullptr, 0, 0, nullptr, app)
          : launch_decode<64>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices,
                              prefix_lens, batch, num_q_heads, num_kv_heads, pl, scale_log2, v_scale, mode, ws_acc,
                              ws_ml, st, nullptr, 0, 0, nullptr, app);
  if (le != hipSuccess) return rt::fail(RT_ERR_HIP, fn + ": " + hipGetErrorString(le));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, fn + " launch: " + hipGetErrorString(e));
  return RT_OK;
}

}  // namespace

extern "C" int64_t radix_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_kv_len) {
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || max_kv_len < 1)
    return -1;
  if (batch == 0) return 0;
  // enough for either pool format's plan
  const int splits = std::max(plan_decode(batch, num_kv_heads, max_kv_len).splits,
                              plan_decode(batch, num_kv_heads, max_kv_len, kMaxChunkFp8).splits);
  return int64_t(batch) * num_q_heads * splits * (head_dim + 2) * int64_t(sizeof(float));
}

extern "C" int radix_decode_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                                      const int32_t* req_to_token, int32_t req_to_token_stride,
                                      const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                      const int32_t* extend_lens, int32_t batch, int32_t max_kv_len,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float sm_scale, int dtype, void* workspace, int64_t workspace_bytes,
                                      void* stream) {
  (void)extend_lens;  // decode rows are one token each by definition
  if (dtype != RT_F32 && dtype != RT_BF16) return rt::fail(RT_ERR_INVALID, "radix_decode_attention: bad dtype");
  return decode_entry("radix_decode_attention", q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, batch, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                      sm_scale, 1.0f, 1.0f, dtype, workspace, workspace_bytes, stream);
}

extern "C" int radix_decode_attention_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                            const int32_t* req_to_token, int32_t req_to_token_stride,
                                            const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                            int32_t batch, int32_t max_kv_len, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim, float sm_scale, float k_scale,
                                            float v_scale, void* workspace, int64_t workspace_bytes, void* stream) {
  return decode_entry("radix_decode_attention_fp8kv", q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, batch, max_kv_len, num_q_heads, num_kv_heads, head_dim,
                      sm_scale, k_scale, v_scale, kModeFp8Kv, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------- no allocation --
// radix_decode_attention_noalloc: the split-K partials go to `scratch`, a
// file-scope device array of kNoAllocScratchBytes that every GPU the
// library runs on holds until the process ends.  In host code `scratch` is
// only a stand-in symbol; its device address on the current GPU comes from
// hipGetSymbolAddress, looked up once per device (the entry point's first
// call there) and kept.  The split kernel writes every partial slot the
// combine reads (empty chunks included), so nothing needs clearing between
// calls.
namespace {

constexpr int64_t kNoAllocScratchBytes = RT_NOALLOC_MAX_WORKSPACE_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, or nullptr (error recorded).
void* scratch_on_device(const char* name) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    rt::fail(RT_ERR_HIP, std::string(name) + ": no usable current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      rt::fail(RT_ERR_HIP, std::string(name) + ": scratch address: " + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// The shared-prefix decode runs its shared pass (MFMA-bound) on a second
// stream of the library's, beside the private split (HBM-bound) on the
// caller's stream, when the private tails are long enough to hide it: each
// hop between the two hardware queues costs about 10 us on MI355X, which
// only pays when the split itself is long (32 requests x 16384 private
// keys: 421 us against 437 us on one stream; few-shot and fork batches,
// whose splits take under 10 us, measured slower with the hops).  Each
// device gets one such stream and a fork and a join event, made on first
// use.  The mutex keeps one call's record/wait sequence whole when several
// host threads call at once.
// The threshold (K/V bytes of the private tails) can be set per call through
// the environment variable RADIXRT_FORK_MIN_BYTES (0: always two streams).
constexpr int64_t kForkMinPrivateBytes = int64_t(128) << 20;
// The single-launch path (shared pass and private split in one launch) is
// on by default for private chunks up to rt::fused_max_private_chunk();
// RADIXRT_SHARED_FUSED=0 turns it off (the two then run as two launches),
// =force uses it for any private chunk length.
int shared_fused_mode() {  // 0 off, 1 default, 2 forced
  const char* e = getenv("RADIXRT_SHARED_FUSED");
  if (!e) return 1;
  if (std::string(e) == "0") return 0;
  if (std::string(e) == "force") return 2;
  return 1;
}

int64_t fork_min_private_bytes() {
  const char* e = getenv("RADIXRT_FORK_MIN_BYTES");
  if (!e || !*e) return kForkMinPrivateBytes;
  char* end = nullptr;
  const long long v = strtoll(e, &end, 10);
  return (end && *end == 0 && v >= 0) ? int64_t(v) : kForkMinPrivateBytes;
}
struct ForkJoin {
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_fj_mu;
ForkJoin g_fj[kMaxDevices];

// The current device's fork/join set, or nullptr (error recorded).  Called
// with g_fj_mu held.
ForkJoin* fork_join_on_device(const std::string& name) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    rt::fail(RT_ERR_HIP, name + ": no usable current device");
    return nullptr;
  }
  ForkJoin& f = g_fj[dev];
  if (!f.aux) {
    hipStream_t aux = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&aux, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (b) (void)hipEventDestroy(b);
      if (a) (void)hipEventDestroy(a);
      if (aux) (void)hipStreamDestroy(aux);
      rt::fail(RT_ERR_HIP, name + ": second stream: " + hipGetErrorString(e));
      return nullptr;
    }
    f.fork = a;
    f.join = b;
    f.aux = aux;
  }
  return &f;
}

}  // namespace

extern "C" int radix_decode_attention_noalloc(const void* q, void* o, const void* k_pool, const void* v_pool,
                                              const int32_t* req_to_token, int32_t req_to_token_stride,
                                              const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                              const int32_t* extend_lens, int32_t batch, int32_t max_kv_len,
                                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                              float sm_scale, int dtype, void* stream) {
  (void)extend_lens;
  static const char* kName = "radix_decode_attention_noalloc";
  if (dtype != RT_F32 && dtype != RT_BF16) return rt::fail(RT_ERR_INVALID, std::string(kName) + ": bad dtype");
  const int64_t need = radix_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_kv_len);
  if (need < 0) return rt::fail(RT_ERR_INVALID, std::string(kName) + ": bad shape");
  if (need > kNoAllocScratchBytes)
    return rt::fail(RT_ERR_INVALID, std::string(kName) + ": these sizes need " + std::to_string(need) +
                                        " bytes of split-K workspace, above the library's " +
                                        std::to_string(kNoAllocScratchBytes) + "-byte scratch array");
  if (batch == 0) return RT_OK;
  void* ws = scratch_on_device(kName);
  if (!ws) return RT_ERR_HIP;
  return decode_entry(kName, q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      batch, max_kv_len, num_q_heads, num_kv_heads, head_dim, sm_scale, 1.0f, 1.0f, dtype, ws,
                      kNoAllocScratchBytes, stream);
}

namespace {

int shared_entry(const char* name, const void* q, void* o, const void* k_pool, const void* v_pool,
                 const int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* req_pool_indices,
                 const int32_t* prefix_lens, const int32_t* shared_lens, const int32_t* group_start, int32_t batch,
                 int32_t n_groups, int32_t max_group_size, int32_t max_shared_len, int32_t max_private_len,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale, float k_scale,
                 float v_scale, bool kv8, void* workspace, int64_t workspace_bytes, void* stream,
                 const rt::AppendArgs& app = rt::AppendArgs()) {
  const std::string fn(name);
  if (batch < 0 || n_groups < 0 || (batch > 0 && (n_groups < 1 || n_groups > batch)) || max_group_size < 1 ||
      max_shared_len < 0 || max_private_len < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 16 || (head_dim != 64 && head_dim != 128) ||
      int64_t(req_to_token_stride) < int64_t(max_shared_len) + max_private_len || !(sm_scale > 0.f) ||
      !(k_scale > 0.f) || !(v_scale > 0.f))
    return rt::fail(RT_ERR_INVALID, fn + ": bad shape, count, stride or scale");
  if (int64_t(max_shared_len) + max_private_len > kMaxKvLen)
    return rt::fail(RT_ERR_INVALID, fn + ": context above 2097152");
  if (batch == 0) return RT_OK;
  if (!q || !o || !k_pool || !v_pool || !req_to_token || !prefix_lens || !shared_lens || !group_start ||
      !workspace || (app.slots && (!app.k_new || !app.v_new)))
    return rt::fail(RT_ERR_INVALID, fn + ": null pointer");
  const int64_t need = radix_decode_shared_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, n_groups,
                                                           max_group_size, max_shared_len, max_private_len);
  if (need < 0 || workspace_bytes < need)
    return rt::fail(RT_ERR_INVALID, fn + ": workspace too small (need " + std::to_string(need) + ")");
  const SharedPlan sp = plan_shared(batch, num_q_heads, num_kv_heads, n_groups, max_group_size, max_shared_len,
                                    max_private_len, kv8 ? kMaxChunkFp8 : kMaxChunk);
  float* ws_acc = static_cast<float*>(workspace);
  float* ws_ml = ws_acc + int64_t(batch) * num_q_heads * sp.total() * head_dim;
  const float scale_log2 = sm_scale * k_scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  // Shared pass on the caller's stream, or, for long private tails, on the
  // library's second stream, forked from and joined back into the caller's:
  // the caller's later work still follows all of it.
  std::unique_lock<std::mutex> lock(g_fj_mu, std::defer_lock);
  hipEvent_t join = nullptr;
  const int64_t private_bytes =
      int64_t(batch) * max_private_len * num_kv_heads * head_dim * (kv8 ? 1 : 2) * 2;
  const int fused = shared_fused_mode();
  if (sp.n_a > 0 && private_bytes < fork_min_private_bytes() &&
      (fused == 2 || (fused == 1 && sp.b.chunk <= rt::fused_max_private_chunk()))) {
    const int rc = rt::launch_shared_fused(q, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices,
                                           prefix_lens, shared_lens, group_start, n_groups, max_group_size, sp.n_a,
                                           sp.chunk_a, batch, sp.b.splits, sp.b.chunk, sp.total(), num_q_heads,
                                           num_kv_heads, head_dim, scale_log2, v_scale, kv8, ws_acc, ws_ml, stream,
                                           app);
    if (rc != RT_OK) return rc;
    if (head_dim == 128)
      hipLaunchKernelGGL((decode_combine<128, true>), dim3(uint32_t(int64_t(batch) * num_q_heads)), dim3(64), 0, st,
                         ws_acc, ws_ml, sp.total(), o);
    else
      hipLaunchKernelGGL((decode_combine<64, true>), dim3(uint32_t(int64_t(batch) * num_q_heads)), dim3(64), 0, st,
                         ws_acc, ws_ml, sp.total(), o);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return rt::fail(RT_ERR_HIP, fn + " launch: " + hipGetErrorString(e));
    return RT_OK;
  }
  if (sp.n_a > 0 && private_bytes < fork_min_private_bytes()) {
    const int rc = rt::launch_extend_shared_part(q, k_pool, v_pool, req_to_token, req_to_token_stride,
                                                 req_pool_indices, shared_lens, group_start, n_groups, max_group_size,
                                                 sp.n_a, sp.chunk_a, sp.total(), num_q_heads, num_kv_heads, head_dim,
                                                 scale_log2, v_scale, kv8, ws_acc, ws_ml, stream);
    if (rc != RT_OK) return rc;
  } else if (sp.n_a > 0) {
    lock.lock();
    ForkJoin* fj = fork_join_on_device(fn);
    if (!fj) return RT_ERR_HIP;
    hipError_t e = hipEventRecord(fj->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(fj->aux, fj->fork, 0);
    if (e != hipSuccess) return rt::fail(RT_ERR_HIP, fn + " fork: " + hipGetErrorString(e));
    const int rc = rt::launch_extend_shared_part(q, k_pool, v_pool, req_to_token, req_to_token_stride,
                                                 req_pool_indices, shared_lens, group_start, n_groups, max_group_size,
                                                 sp.n_a, sp.chunk_a, sp.total(), num_q_heads, num_kv_heads, head_dim,
                                                 scale_log2, v_scale, kv8, ws_acc, ws_ml, fj->aux);
    // the join is recorded even after a failed launch, so the caller's
    // stream never waits on a fork that has no join
    e = hipEventRecord(fj->join, fj->aux);
    if (rc != RT_OK) return rc;
    if (e != hipSuccess) return rt::fail(RT_ERR_HIP, fn + " join: " + hipGetErrorString(e));
    join = fj->join;
  }
  const int mode = kv8 ? kModeFp8Kv : RT_BF16;
  hipError_t we;
  if (head_dim == 128)
    we = launch_decode<128>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                       batch, num_q_heads, num_kv_heads, sp.b, scale_log2, v_scale, mode, ws_acc, ws_ml, st,
                       shared_lens, sp.n_a, sp.total(), join, app);
  else
    we = launch_decode<64>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      batch, num_q_heads, num_kv_heads, sp.b, scale_log2, v_scale, mode, ws_acc, ws_ml, st,
                      shared_lens, sp.n_a, sp.total(), join, app);
  if (we != hipSuccess) return rt::fail(RT_ERR_HIP, fn + ": " + hipGetErrorString(we));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, fn + " launch: " + hipGetErrorString(e));
  return RT_OK;
}

}  // namespace

extern "C" int64_t radix_decode_shared_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                       int32_t head_dim, int32_t n_groups, int32_t max_group_size,
                                                       int32_t max_shared_len, int32_t max_private_len) {
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || n_groups < 0 || max_group_size < 1 ||
      max_shared_len < 0 || max_private_len < 1)
    return -1;
  const int splits = std::max(
      plan_shared(batch, num_q_heads, num_kv_heads, n_groups, max_group_size, max_shared_len, max_private_len,
                  kMaxChunk).total(),
      plan_shared(batch, num_q_heads, num_kv_heads, n_groups, max_group_size, max_shared_len, max_private_len,
                  kMaxChunkFp8).total());
  return int64_t(batch) * num_q_heads * splits * (head_dim + 2) * int64_t(sizeof(float));
}

extern "C" int radix_decode_attention_shared(const void* q, void* o, const void* k_pool, const void* v_pool,
                                             const int32_t* req_to_token, int32_t req_to_token_stride,
                                             const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                             const int32_t* shared_lens, const int32_t* group_start, int32_t batch,
                                             int32_t n_groups, int32_t max_group_size, int32_t max_shared_len,
                                             int32_t max_private_len, int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, float sm_scale, void* workspace,
                                             int64_t workspace_bytes, void* stream) {
  return shared_entry("radix_decode_attention_shared", q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, shared_lens, group_start, batch, n_groups, max_group_size,
                      max_shared_len, max_private_len, num_q_heads, num_kv_heads, head_dim, sm_scale, 1.f, 1.f,
                      false, workspace, workspace_bytes, stream);
}

extern "C" int radix_decode_attention_shared_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                                   const int32_t* req_to_token, int32_t req_to_token_stride,
                                                   const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                                   const int32_t* shared_lens, const int32_t* group_start,
                                                   int32_t batch, int32_t n_groups, int32_t max_group_size,
                                                   int32_t max_shared_len, int32_t max_private_len,
                                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                   float sm_scale, float k_scale, float v_scale, void* workspace,
                                                   int64_t workspace_bytes, void* stream) {
  return shared_entry("radix_decode_attention_shared_fp8kv", q, o, k_pool, v_pool, req_to_token,
                      req_to_token_stride, req_pool_indices, prefix_lens, shared_lens, group_start, batch, n_groups,
                      max_group_size, max_shared_len, max_private_len, num_q_heads, num_kv_heads, head_dim, sm_scale,
                      k_scale, v_scale, true, workspace, workspace_bytes, stream);
}

// ------------------------------------------------ decode with the append --
namespace {
rt::AppendArgs append_args(int32_t* req_to_token, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* new_slots, float k_scale, float v_scale) {
  rt::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = new_slots;
  a.r2t = req_to_token;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_inv = 1.f / k_scale;
  a.v_inv = 1.f / v_scale;
  return a;
}
}  // namespace

extern "C" int radix_decode_attention_append(const void* q, void* o, void* k_pool, void* v_pool,
                                             int32_t* req_to_token, int32_t req_to_token_stride,
                                             const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                             int32_t batch, int32_t max_kv_len, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                             const void* k_new, const void* v_new, const int32_t* new_slots,
                                             void* workspace, int64_t workspace_bytes, void* stream) {
  static const char* kName = "radix_decode_attention_append";
  if (!new_slots) return rt::fail(RT_ERR_INVALID, std::string(kName) + ": null pointer");
  return decode_entry(kName, q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      batch, max_kv_len, num_q_heads, num_kv_heads, head_dim, sm_scale, 1.f, 1.f, RT_BF16, workspace,
                      workspace_bytes, stream,
                      append_args(req_to_token, k_pool, v_pool, k_new, v_new, new_slots, 1.f, 1.f));
}

extern "C" int radix_decode_attention_append_fp8kv(const void* q, void* o, void* k_pool, void* v_pool,
                                                   int32_t* req_to_token, int32_t req_to_token_stride,
                                                   const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                                   int32_t batch, int32_t max_kv_len, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                                   float k_scale, float v_scale, const void* k_new,
                                                   const void* v_new, const int32_t* new_slots, void* workspace,
                                                   int64_t workspace_bytes, void* stream) {
  static const char* kName = "radix_decode_attention_append_fp8kv";
  if (!new_slots) return rt::fail(RT_ERR_INVALID, std::string(kName) + ": null pointer");
  return decode_entry(kName, q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      batch, max_kv_len, num_q_heads, num_kv_heads, head_dim, sm_scale, k_scale, v_scale, kModeFp8Kv,
                      workspace, workspace_bytes, stream,
                      append_args(req_to_token, k_pool, v_pool, k_new, v_new, new_slots, k_scale, v_scale));
}

extern "C" int radix_decode_attention_shared_append(
    const void* q, void* o, void* k_pool, void* v_pool, int32_t* req_to_token, int32_t req_to_token_stride,
    const int32_t* req_pool_indices, const int32_t* prefix_lens, const int32_t* shared_lens,
    const int32_t* group_start, int32_t batch, int32_t n_groups, int32_t max_group_size, int32_t max_shared_len,
    int32_t max_private_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
    const void* k_new, const void* v_new, const int32_t* new_slots, void* workspace, int64_t workspace_bytes,
    void* stream) {
  static const char* kName = "radix_decode_attention_shared_append";
  if (!new_slots) return rt::fail(RT_ERR_INVALID, std::string(kName) + ": null pointer");
  return shared_entry(kName, q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      shared_lens, group_start, batch, n_groups, max_group_size, max_shared_len, max_private_len,
                      num_q_heads, num_kv_heads, head_dim, sm_scale, 1.f, 1.f, false, workspace, workspace_bytes,
                      stream, append_args(req_to_token, k_pool, v_pool, k_new, v_new, new_slots, 1.f, 1.f));
}

extern "C" int radix_decode_attention_shared_append_fp8kv(
    const void* q, void* o, void* k_pool, void* v_pool, int32_t* req_to_token, int32_t req_to_token_stride,
    const int32_t* req_pool_indices, const int32_t* prefix_lens, const int32_t* shared_lens,
    const int32_t* group_start, int32_t batch, int32_t n_groups, int32_t max_group_size, int32_t max_shared_len,
    int32_t max_private_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
    float k_scale, float v_scale, const void* k_new, const void* v_new, const int32_t* new_slots, void* workspace,
    int64_t workspace_bytes, void* stream) {
  static const char* kName = "radix_decode_attention_shared_append_fp8kv";
  if (!new_slots) return rt::fail(RT_ERR_INVALID, std::string(kName) + ": null pointer");
  return shared_entry(kName, q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      shared_lens, group_start, batch, n_groups, max_group_size, max_shared_len, max_private_len,
                      num_q_heads, num_kv_heads, head_dim, sm_scale, k_scale, v_scale, true, workspace,
                      workspace_bytes, stream,
                      append_args(req_to_token, k_pool, v_pool, k_new, v_new, new_slots, k_scale, v_scale));
}
