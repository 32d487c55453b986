// radix_decode_attention: batched decode attention over the token pool.
//
// Each request has one query row (its newest token, whose K/V the scatter
// kernel already wrote) and attends its whole context: keys 0..prefix_len,
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
//  * The per-chunk slot indices are staged in LDS in runs of 512, so the
//    dependent index->row load chain costs one round trip per run, and the
//    next 16-key block's rows are requested before the current block is
//    consumed.
//  * bf16: the G x 16-key score tile and the PV update are MFMA
//    contractions (16x16x32 for Q K^T, 16x16x16 for P V) whose operands are
//    loaded straight from HBM in the MFMA lane layout: K rows as 64-byte
//    runs, V rows as 128-byte runs of 4 dims per lane (the PV contraction
//    dimension is the key, so each lane takes 4 dims of 4 keys and the dims
//    are regrouped in registers).
//  * fp32 inputs take a plain VALU path (one lane per dim, wave-wide dot
//    products); it exists for full-precision checks, not for speed.

#include <math.h>

#include "dev_common.h"
#include "radixrt.h"
#include "rt_internal.h"

namespace {

using namespace rtk;

constexpr int kIdxRun = 512;  // slot indices staged per LDS run (per wave)

struct DecodePlan {
  int splits;
  int chunk;
};

// Chunking depends only on (batch, max_kv_len) so the workspace size is
// known without the head layout: aim for >= 512 (request, chunk) pairs,
// chunks of at least 64 keys, at most 64 chunks per request.
DecodePlan plan_decode(int32_t batch, int32_t max_kv_len) {
  int s = (512 + batch - 1) / batch;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  int chunk = (max_kv_len + s - 1) / s;
  chunk = (chunk + 15) / 16 * 16;
  if (chunk < 64) chunk = 64;
  int splits = (max_kv_len + chunk - 1) / chunk;
  if (splits < 1) splits = 1;
  return {splits, chunk};
}

// ----------------------------------------------------------------- bf16 --
template <int D>
__global__ void __launch_bounds__(64) decode_split_bf16(
    const char* __restrict__ q, const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const int32_t* __restrict__ req_to_token, int64_t stride, const int32_t* __restrict__ rpi,
    const int32_t* __restrict__ prefix_lens, int Hq, int Hkv, int G, int S, int chunk, float scale_log2,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
  constexpr int KS = D / 32;      // 32-dim steps of the score contraction
  constexpr int VH = D / 64;      // 64-dim halves of the PV update
  __shared__ int32_t s_idx[kIdxRun];

  const int lane = threadIdx.x;
  const int col = lane & 15;      // MFMA column: query head within the group / key within block
  const int grp = lane >> 4;      // MFMA k-group
  int item = blockIdx.x;
  const int s = item % S;
  item /= S;
  const int kvh = item % Hkv;
  const int b = item / Hkv;

  const int kv_len = prefix_lens[b] + 1;
  const int start = s * chunk;
  const int end = min(kv_len, start + chunk);
  const int64_t row_bytes = int64_t(Hkv) * D * 2;
  const int32_t* idx_row = req_to_token + int64_t(rpi ? rpi[b] : b) * stride;
  const char* kbase = k_pool + int64_t(kvh) * D * 2;
  const char* vbase = v_pool + int64_t(kvh) * D * 2;

  // Q^T operand: column = query head kvh*G + col, k = dims 32*ks + 8*grp + t.
  bf16x8 qop[KS];
  if (col < G) {
    const char* qp = q + (int64_t(b) * Hq + kvh * G + col) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = as_bf16x8(ld16(qp + (32 * ks + 8 * grp) * 2));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = as_bf16x8(u32x4{0, 0, 0, 0});
  }

  floatx4 o[VH * 4];
#pragma unroll
  for (int i = 0; i < VH * 4; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  for (int run = start; run < end; run += kIdxRun) {
    const int run_end = min(end, run + kIdxRun);
    __syncthreads();
    for (int i = lane; i < run_end - run; i += 64) s_idx[i] = idx_row[run + i];
    __syncthreads();

    // Operand registers of one 16-key block.
    u32x4 kreg[KS];
    u32x2 vreg[VH][4];
    auto load_block = [&](int kb) {
      const int kk = kb + col;
      if (kk < run_end) {
        const char* kp = kbase + int64_t(s_idx[kk - run]) * row_bytes + (8 * grp) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kreg[ks] = ld16(kp + 64 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kreg[ks] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kv = kb + 4 * grp + t;
        if (kv < run_end) {
          const char* vp = vbase + int64_t(s_idx[kv - run]) * row_bytes + (4 * col) * 2;
#pragma unroll
          for (int h = 0; h < VH; ++h) vreg[h][t] = ld8(vp + 128 * h);
        } else {
#pragma unroll
          for (int h = 0; h < VH; ++h) vreg[h][t] = u32x2{0, 0};
        }
      }
    };

    load_block(run);
    for (int kb = run; kb < run_end; kb += 16) {
      // Consume the current block's registers into MFMA operands, then
      // start the next block's loads before the dependent math.
      floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc = mfma_16x16x32(as_bf16x8(kreg[ks]), qop[ks], sacc);
      bf16x4 vop[VH][4];
#pragma unroll
      for (int h = 0; h < VH; ++h) {
        vop[h][0] = as_bf16x4(u32x2{pack_lo16(vreg[h][0].x, vreg[h][1].x), pack_lo16(vreg[h][2].x, vreg[h][3].x)});
        vop[h][1] = as_bf16x4(u32x2{pack_hi16(vreg[h][0].x, vreg[h][1].x), pack_hi16(vreg[h][2].x, vreg[h][3].x)});
        vop[h][2] = as_bf16x4(u32x2{pack_lo16(vreg[h][0].y, vreg[h][1].y), pack_lo16(vreg[h][2].y, vreg[h][3].y)});
        vop[h][3] = as_bf16x4(u32x2{pack_hi16(vreg[h][0].y, vreg[h][1].y), pack_hi16(vreg[h][2].y, vreg[h][3].y)});
      }
      if (kb + 16 < run_end) load_block(kb + 16);

      // Scores of keys kb + 4*grp + v for head `col` (log2 domain).
      float sv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[v] = (kb + 4 * grp + v < run_end) ? sacc[v] * scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = __builtin_amdgcn_exp2f(sv[v] - m_new);
      l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m = m_new;
#pragma unroll
      for (int i = 0; i < VH * 4; ++i) o[i] *= alpha;
      const bf16x4 pop = as_bf16x4(u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
#pragma unroll
      for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[h * 4 + r] = mfma_16x16x16(vop[h][r], pop, o[h * 4 + r]);
    }
  }

  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (col < G) {
    const int64_t part = (int64_t(b) * Hq + kvh * G + col) * S + s;
    if (grp == 0) {
      ws_ml[part * 2 + 0] = m;
      ws_ml[part * 2 + 1] = l;
    }
    float* acc = ws_acc + part * D;
    // Tile (h, r) row i holds dim 64h + 4i + r; this lane holds rows i = 4*grp + v.
#pragma unroll
    for (int h = 0; h < VH; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        floatx4 w = {o[h * 4 + 0][v], o[h * 4 + 1][v], o[h * 4 + 2][v], o[h * 4 + 3][v]};
        *reinterpret_cast<floatx4*>(acc + 64 * h + 16 * grp + 4 * v) = w;
      }
  }
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
template <int D, bool BF16>
__global__ void __launch_bounds__(64) decode_combine(const float* __restrict__ ws_acc,
                                                     const float* __restrict__ ws_ml, int S,
                                                     void* __restrict__ out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;  // b * Hq + h
  const float* ml = ws_ml + bh * S * 2;
  float mmax = -INFINITY;
  for (int s = 0; s < S; ++s) mmax = fmaxf(mmax, ml[2 * s]);
  float L = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s = 0; s < S; ++s) {
    const float w = exp2f(ml[2 * s] - mmax);  // empty chunks have m = -inf -> 0
    L = fmaf(w, ml[2 * s + 1], L);
    const float* a = ws_acc + (bh * S + s) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, a[lane + 64 * i], acc[i]);
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

template <int D>
void launch_decode(const void* q, void* o, const void* k_pool, const void* v_pool, const int32_t* r2t,
                   int64_t stride, const int32_t* rpi, const int32_t* plens, int B, int Hq, int Hkv,
                   DecodePlan pl, float scale_log2, int dtype, float* ws_acc, float* ws_ml, hipStream_t st) {
  const int G = Hq / Hkv;
  if (dtype == RT_BF16) {
    const uint32_t grid = uint32_t(int64_t(B) * Hkv * pl.splits);
    hipLaunchKernelGGL(decode_split_bf16<D>, dim3(grid), dim3(64), 0, st, (const char*)q, (const char*)k_pool,
                       (const char*)v_pool, r2t, stride, rpi, plens, Hq, Hkv, G, pl.splits, pl.chunk,
                       scale_log2, ws_acc, ws_ml);
    hipLaunchKernelGGL((decode_combine<D, true>), dim3(uint32_t(int64_t(B) * Hq)), dim3(64), 0, st, ws_acc,
                       ws_ml, pl.splits, o);
  } else {
    const uint32_t grid = uint32_t(int64_t(B) * Hq * pl.splits);
    hipLaunchKernelGGL(decode_split_f32<D>, dim3(grid), dim3(64), 0, st, (const float*)q,
                       (const float*)k_pool, (const float*)v_pool, r2t, stride, rpi, plens, Hq, Hkv, G,
                       pl.splits, pl.chunk, scale_log2, ws_acc, ws_ml);
    hipLaunchKernelGGL((decode_combine<D, false>), dim3(uint32_t(int64_t(B) * Hq)), dim3(64), 0, st, ws_acc,
                       ws_ml, pl.splits, o);
  }
}

}  // namespace

extern "C" int64_t radix_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                                int32_t max_kv_len) {
  if (batch < 0 || num_q_heads < 1 || (head_dim != 64 && head_dim != 128) || max_kv_len < 1) return -1;
  if (batch == 0) return 0;
  DecodePlan pl = plan_decode(batch, max_kv_len);
  return int64_t(batch) * num_q_heads * pl.splits * (head_dim + 2) * int64_t(sizeof(float));
}

extern "C" int radix_decode_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                                      const int32_t* req_to_token, int32_t req_to_token_stride,
                                      const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                      const int32_t* extend_lens, int32_t batch, int32_t max_kv_len,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float sm_scale, int dtype, void* workspace, int64_t workspace_bytes,
                                      void* stream) {
  (void)extend_lens;  // decode rows are one token each by definition
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || (dtype != RT_F32 && dtype != RT_BF16) || max_kv_len < 1 ||
      req_to_token_stride < max_kv_len || !(sm_scale > 0.f))
    return rt::fail(RT_ERR_INVALID, "radix_decode_attention: bad shape, dtype, stride or scale");
  if (dtype == RT_BF16 && num_q_heads / num_kv_heads > 16)
    return rt::fail(RT_ERR_INVALID, "radix_decode_attention: bf16 path supports at most 16 query heads per KV head");
  if (batch == 0) return RT_OK;
  if (!q || !o || !k_pool || !v_pool || !req_to_token || !prefix_lens || !workspace)
    return rt::fail(RT_ERR_INVALID, "radix_decode_attention: null pointer");
  const int64_t need = radix_decode_workspace_bytes(batch, num_q_heads, head_dim, max_kv_len);
  if (workspace_bytes < need)
    return rt::fail(RT_ERR_INVALID, "radix_decode_attention: workspace too small (need " + std::to_string(need) + ")");
  const DecodePlan pl = plan_decode(batch, max_kv_len);
  float* ws_acc = static_cast<float*>(workspace);
  float* ws_ml = ws_acc + int64_t(batch) * num_q_heads * pl.splits * head_dim;
  const float scale_log2 = sm_scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128)
    launch_decode<128>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                       batch, num_q_heads, num_kv_heads, pl, scale_log2, dtype, ws_acc, ws_ml, st);
  else
    launch_decode<64>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride, req_pool_indices, prefix_lens,
                      batch, num_q_heads, num_kv_heads, pl, scale_log2, dtype, ws_acc, ws_ml, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return rt::fail(RT_ERR_HIP, std::string("radix_decode_attention launch: ") + hipGetErrorString(e));
  return RT_OK;
}
