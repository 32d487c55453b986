// The split-K decode's work loop for one wave, shared by the split kernel
// (decode.hip) and the single-launch shared-prefix decode (extend.hip).
// Included by those two translation units only.
#pragma once

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "dev_common.h"
#include "rt_internal.h"

namespace rtk {
namespace dec {

constexpr float kSlack = 8.f;  // log2 headroom of the lazy softmax rescale

// Persistent waves: the grid holds as many waves as fit on the chip; work
// items (chunk s, KV head h, request b) are ordered with b innermost and cut
// into 8 contiguous slices, one per XCD (the hardware places block i on XCD
// i % 8).  Requests that share a cached prefix read the same slots for the
// same (s, h), so their concurrent waves on one XCD meet those rows in L2.
// One 16-key block's operands as loaded: bf16 pools hold them as the MFMA
// takes them; FP8 pools hold half the bytes, widened to bf16 when consumed.
// A lane's V piece: D/16 consecutive elements of one row (16 bytes for bf16
// at D = 128).
template <int D, bool KV8> struct VPiece;
template <> struct VPiece<128, false> { using T = u32x4; };
template <> struct VPiece<64, false> { using T = u32x2; };
template <> struct VPiece<128, true> { using T = u32x2; };
template <> struct VPiece<64, true> { using T = uint32_t; };
template <int D, bool KV8>
struct DecBlock {
  typename std::conditional<KV8, u32x2, u32x4>::type k[D / 32];  // key kb + col, dims 32*ks + 8*grp .. +7
  typename VPiece<D, KV8>::T v[4];  // V row kb + 4*grp + t, dims (D/16)*col .. +D/16-1
};

// Work items (chunk s, KV head h, request b) are numbered with b innermost
// and cut into 8 contiguous slices, one per XCD; the calling wave takes items
// local, local + per_xcd, ... of slice `xcd` (the XCD it runs on).  s_idx:
// this wave's LDS array of slot indices: with WIN = 0 it holds a whole chunk;
// with WIN (a power of two) it is a ring of WIN entries, two windows of
// WIN / 2 keys, and the wave fetches each next window's indices while it
// streams the current one (so a chunk may be any length).  Needs only its
// own wave: it uses no workgroup barrier.
//
// APP (with app.slots != nullptr): the launch also appends each
// request's new token, the key at position prefix_lens[b].  The item whose
// chunk holds that key takes its slot from app.slots[b] (the table entry is
// not written yet), first stores the token's K and V rows of its KV head at
// that slot and, for KV head 0, the slot-table entry, and waits for those
// stores before its loads; no other item reads that key.
template <int D, bool KV8, int WIN = 0, bool APP = false>
__device__ __forceinline__ void split_items(
    int xcd, int local, int per_xcd, int lane, int32_t* s_idx, const char* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const int32_t* __restrict__ req_to_token,
    int64_t stride, const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens, int B, int Hq,
    int Hkv, int G, int S, int chunk, float scale_log2, float v_scale, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, const int32_t* __restrict__ key_start, int s_off, int S_total,
    const rt::AppendArgs& app = rt::AppendArgs()) {
  // key_start (optional): request b's chunks cover keys key_start[b] ..
  // prefix_lens[b] (the shared-prefix decode's private tails); its partials
  // go to split slots s_off .. s_off + S - 1 of S_total (default: S).
  if (S_total == 0) S_total = S;
  constexpr int KS = D / 32;      // 32-dim steps of the score contraction
  constexpr int VW = D / 16;      // V elements per lane and key; also the PV update's 16-row tiles
  constexpr int EB = KV8 ? 1 : 2; // bytes per pool element
  const int col = lane & 15;      // MFMA column: query head within the group / key within block
  const int grp = lane >> 4;      // MFMA k-group
  const int64_t row_bytes = int64_t(Hkv) * D * EB;

  // This wave's share of its XCD's slice of the item list.
  const int n_items = B * Hkv * S;
  const int q8 = n_items >> 3, r8 = n_items & 7;
  const int lo = xcd * q8 + min(xcd, r8);
  const int hi_item = lo + q8 + (xcd < r8 ? 1 : 0);

  for (int item = lo + local; item < hi_item; item += per_xcd) {
    const int b = item % B;
    const int kvh = (item / B) % Hkv;
    const int s = item / (B * Hkv);
    const int kv_len = prefix_lens[b] + 1;
    const int start = (key_start ? key_start[b] : 0) + s * chunk;
    const int end = min(kv_len, start + chunk);
    const int64_t row = rpi ? rpi[b] : b;
    const int32_t* idx_row = req_to_token + row * stride;
    const char* kbase = k_pool + (int64_t(kvh) * D + 8 * grp) * EB;
    const char* vbase = v_pool + (int64_t(kvh) * D + VW * col) * EB;

    // Q^T operand: column = query head kvh*G + col, k = dims 32*ks + 8*grp + t.
    // Its loads go out before the slot indices' below, so the two round
    // trips overlap.
    bf16x8 qop[KS];
    if (col < G) {
      const char* qp = q + (int64_t(b) * Hq + kvh * G + col) * D * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[ks] = as_bf16x8(ld16(qp + (32 * ks + 8 * grp) * 2));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[ks] = as_bf16x8(u32x4{0, 0, 0, 0});
    }

    // Slot indices of the whole chunk into this wave's LDS, once.  The
    // workgroup is this one wave, whose LDS accesses complete in program
    // order, so no barrier (and no wait for the Q loads) is needed between
    // the previous item's index reads, these writes and the reads below.
    // Sixteen loads per lane go out before the first store, so a chunk of up
    // to 1024 keys costs one memory round trip (one per 1024 keys after).
    static_assert(WIN == 0 || (WIN >= 128 && (WIN & (WIN - 1)) == 0), "the index ring is a power of two");
    constexpr int H = WIN / 2;           // keys per window of the ring
    const int n_keys = end - start;
    const int32_t* src = idx_row + start;
    // Appending: the chunk holding the new token (its last key) reads that
    // key's slot from app.slots.
    const bool owner = APP && start < kv_len && end == kv_len;
    const int own = owner ? n_keys - 1 : -1;
    const int32_t new_slot = owner ? app.slots[b] : 0;
    __builtin_amdgcn_wave_barrier();
    {
      const int n = WIN ? min(n_keys, WIN) : n_keys;   // the ring's first two windows
      constexpr int U = 16;
      for (int base = 0; base < n; base += 64 * U) {
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = base + 64 * u + lane;
          v[u] = i < n ? src[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = base + 64 * u + lane;
          if (i < n) s_idx[i] = v[u];
        }
      }
      // the new token's entry (LDS accesses of one wave complete in order)
      if (APP && own >= 0 && own < n && lane == 0) s_idx[own] = new_slot;
    }
    __builtin_amdgcn_wave_barrier();

    if (APP && owner) {
      // The new token's K and V rows of this KV head (D / 8 lanes, 8
      // elements each), its slot-table entry (KV head 0), then a wait for
      // the stores: this wave's loads below read that row back.
      const int64_t src_off = (int64_t(b) * Hkv + kvh) * D * 2;
      const int64_t dst_off = int64_t(new_slot) * row_bytes + int64_t(kvh) * D * EB;
      if (lane < D / 8) {
        const u32x4 kw = ld16(static_cast<const char*>(app.k_new) + src_off + 16 * lane);
        const u32x4 vw = ld16(static_cast<const char*>(app.v_new) + src_off + 16 * lane);
        char* kd = static_cast<char*>(app.k_pool) + dst_off;
        char* vd = static_cast<char*>(app.v_pool) + dst_off;
        if constexpr (KV8) {
          u32x2 ko = {0u, 0u}, vo = {0u, 0u};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t kb16 = (kw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
            const uint32_t vb16 = (vw[i >> 1] >> (16 * (i & 1))) & 0xffffu;
            ko[i >> 2] |= f32_to_e4m3(__uint_as_float(kb16 << 16) * app.k_inv) << (8 * (i & 3));
            vo[i >> 2] |= f32_to_e4m3(__uint_as_float(vb16 << 16) * app.v_inv) << (8 * (i & 3));
          }
          *reinterpret_cast<u32x2*>(kd + 8 * lane) = ko;
          *reinterpret_cast<u32x2*>(vd + 8 * lane) = vo;
        } else {
          *reinterpret_cast<u32x4*>(kd + 16 * lane) = kw;
          *reinterpret_cast<u32x4*>(vd + 16 * lane) = vw;
        }
      }
      if (kvh == 0 && lane == 0) app.r2t[row * stride + (kv_len - 1)] = new_slot;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    floatx4 o[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    // Keys past `end` are clamped to the chunk's last key (masked below), so
    // every load is valid and the loop needs no tail branches.  A 16-key
    // block never straddles two windows (both are multiples of 16 keys from
    // `start`).
    auto slot = [&](int rel) { return uint32_t(s_idx[WIN ? (rel & (WIN - 1)) : rel]); };
    auto load = [&](DecBlock<D, KV8>& blk, int kb) {
      const int kk = min(kb + col, end - 1) - start;
      const char* kp = kbase + int64_t(slot(kk)) * row_bytes;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KV8)
          blk.k[ks] = ld8(kp + 32 * ks);
        else
          blk.k[ks] = ld16(kp + 64 * ks);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kv = min(kb + 4 * grp + t, end - 1) - start;
        blk.v[t] = *reinterpret_cast<const typename VPiece<D, KV8>::T*>(vbase + int64_t(slot(kv)) * row_bytes);
      }
    };

    auto consume = [&](const DecBlock<D, KV8>& cur, int kb) {
      floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KV8)
          sacc = mfma_16x16x32(fp8x8_to_bf16x8(cur.k[ks]), qop[ks], sacc);
        else
          sacc = mfma_16x16x32(as_bf16x8(cur.k[ks]), qop[ks], sacc);
      }
      // Scores of keys kb + 4*grp + v for head `col` (log2 domain); keys at or
      // past `end` (a block wholly past it included) contribute nothing.
      float sv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[v] = (kb + 4 * grp + v < end) ? sacc[v] * scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      // Lazy rescale: m only moves when a score exceeds it by 2^kSlack.
      if (__any(mx > m + kSlack)) {
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int i2 = 0; i2 < VW; ++i2) o[i2] *= alpha;
        m = m_new;
      }
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = __builtin_amdgcn_exp2f(sv[v] - m);
      l += (p[0] + p[1]) + (p[2] + p[3]);
      const bf16x4 pop = as_bf16x4(u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
      // PV update: tile r (0 .. VW-1) has rows i = dims VW*i + r; its A operand
      // takes element r of the four keys' pieces, as bf16 pairs.
      constexpr int NW = VW / 2;
      uint32_t w[4][NW];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (KV8 && D == 128) {
          const u32x4 x = __builtin_bit_cast(u32x4, fp8x8_to_bf16x8(cur.v[t]));
#pragma unroll
          for (int j = 0; j < NW; ++j) w[t][j] = x[j];
        } else if constexpr (KV8) {
          const u32x2 x = fp8x4_to_bf16x4(cur.v[t]);
#pragma unroll
          for (int j = 0; j < NW; ++j) w[t][j] = x[j];
        } else {
#pragma unroll
          for (int j = 0; j < NW; ++j) w[t][j] = cur.v[t][j];
        }
      }
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        o[2 * j] = mfma_16x16x16(as_bf16x4(u32x2{pack_lo16(w[0][j], w[1][j]), pack_lo16(w[2][j], w[3][j])}), pop,
                                 o[2 * j]);
        o[2 * j + 1] = mfma_16x16x16(
            as_bf16x4(u32x2{pack_hi16(w[0][j], w[1][j]), pack_hi16(w[2][j], w[3][j])}), pop, o[2 * j + 1]);
      }
    };

    // Two register buffers: the next 16-key block is always in flight while
    // one is consumed (past `end` the loads repeat the clamped last row).
    const int nb = end > start ? (end - start + 15) >> 4 : 0;
    if (nb > 0) {
      DecBlock<D, KV8> cur, nxt;
      constexpr int PU = WIN ? H / 64 : 1;   // index loads per lane per window
      int32_t pre[PU];
      int pend = -1;                         // first key (from start) of fetched, unstored indices
      load(cur, start);
      for (int i = 0; i < nb; ++i) {
        const int kb = start + 16 * i;
        if constexpr (WIN != 0) {
          // The next block opens window w = rel / H >= 1: every block of
          // window w - 1 has been loaded, so its half of the ring takes
          // window w + 1, fetched now and stored after this block.
          const int rel = kb + 16 - start;
          if (rel % H == 0 && rel >= H && rel + H < n_keys) {
            pend = rel + H;
#pragma unroll
            for (int u = 0; u < PU; ++u) {
              const int k = pend + 64 * u + lane;
              pre[u] = k < n_keys ? src[k] : 0;
            }
          }
        }
        load(nxt, kb + 16);
        consume(cur, kb);
        if constexpr (WIN != 0) {
          if (pend >= 0) {
#pragma unroll
            for (int u = 0; u < PU; ++u) {
              const int k = pend + 64 * u + lane;
              if (k < n_keys) s_idx[k & (WIN - 1)] = pre[u];
            }
            if (APP && own >= pend && own < pend + H && lane == 0) s_idx[own & (WIN - 1)] = new_slot;
            pend = -1;
          }
        }
        cur = nxt;
      }
    }

    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (col < G) {
      const int64_t part = (int64_t(b) * Hq + kvh * G + col) * S_total + s_off + s;
      if (grp == 0) {
        ws_ml[part * 2 + 0] = m;
        ws_ml[part * 2 + 1] = l;
      }
      float* acc = ws_acc + part * D;
      // This lane holds rows i = 4*grp + v of every tile r: dims VW*i + r.
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int r4 = 0; r4 < VW / 4; ++r4) {
          floatx4 w = {o[4 * r4 + 0][v], o[4 * r4 + 1][v], o[4 * r4 + 2][v], o[4 * r4 + 3][v]};
          if constexpr (KV8) w *= v_scale;
          *reinterpret_cast<floatx4*>(acc + VW * (4 * grp + v) + 4 * r4) = w;
        }
    }
  }
}

}  // namespace dec
}  // namespace rtk
