// radix_extend_attention: attention for the uncached suffix of each request.
//
// The radix tree hands each request a cached prefix of P tokens whose K/V
// already sit in the pool; only the E suffix tokens are new (SGLang
// explainer, section 04: match the longest prefix, reference the shared
// KV, prefill only the missed suffix).  Extend row j of request b attends
// keys 0..P+j, all gathered through req_to_token -- the prefix in place,
// the suffix just written by the scatter kernel.
//
// bf16 path (the hot one).  Work item = (KV head, request, tile of 128
// query rows).  The query rows of a tile are (extend row, group head) pairs
// with the G = Hq / Hkv heads of one KV head innermost, so every K/V tile
// staged in LDS serves all G heads at once.  Four wavefronts own 32 rows
// each.  Per 32-key tile:
//   * the slot indices of the item's keys are staged in LDS once per 1024
//     keys; each wave then issues direct HBM-to-LDS loads
//     (global_load_lds_dwordx4, 1 KiB per instruction) for its share of the
//     next tile's 32 K rows and 32 V rows while the current tile is used
//     (two LDS stages);
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B =
//     the wave's Q rows held in registers for the whole kernel).  With keys
//     as MFMA rows, each lane owns one query row, so the softmax max/sum
//     need only one cross-lane exchange (lane ^ 32).
//   * Online softmax in the log2 domain with a lazy rescale: the running max
//     moves only when a tile's max exceeds it by more than 2^8.  Q is
//     multiplied by scale * log2(e) once (and rounded back to bf16), and the
//     score accumulators start each tile at -m instead of 0, so the MFMA hands back
//     scores already shifted by the running max and each probability costs
//     one v_exp_f32.  Row sums add the bf16-rounded probabilities that the
//     P V product uses, two per v_dot2_f32_bf16.
//   * O^T += V^T P^T with the same MFMA.  P^T comes straight from the score
//     registers (the key order of the contraction is chosen to match the
//     score layout); V^T operands come from LDS through gfx950's transpose
//     read (ds_read_b64_tr_b16), which hands each lane 4 consecutive keys of
//     one dim -- no register shuffles.
//   * Causal masking is applied only on tiles that cross the wave's
//     diagonal; tiles beyond a wave's last row are skipped.
// Registers are held to 168 per lane so that three waves share each SIMD
// (three work items per CU, 36 KiB of LDS each): with 64-key tiles and two
// waves per SIMD the kernel measured slower, on few-shot, FP8-pool and
// ragged chat batches alike.
// Work items are laid out so that each XCD (blockIdx % 8 on MI355X) runs a
// contiguous slice of (KV head, request) items: requests that share a
// prefix read the same K/V rows and find them in that XCD's L2.
//
// fp32 path: one wavefront per (extend row, query head), lanes over dims,
// keys in order with wave-wide dot products.  For full-precision checks.

#include <math.h>

#include <algorithm>

#include "dev_common.h"
#include "radixrt.h"
#include "rt_internal.h"
#include "decode_split.h"
#include "tile_layout.h"

namespace {

using namespace rtk;

constexpr int kBN = 32;        // keys per LDS tile
// 32-row query blocks per wave.  2 halves the LDS reads per MFMA but needs
// more than 256 registers (one wave per SIMD); on gfx950 1 measures faster.
constexpr int kRB = 1;
constexpr int kWavesPerSimd = 3;  // occupancy the register budget is cut to
// Waves per workgroup.  A work item's K/V tiles are gathered once for all of
// its kWaves * 32 query rows.  8 waves halve that gather traffic but measure
// slower than 4 on MI355X: the gather is not what bounds the kernel.
constexpr int kWaves = 4;
constexpr int kSeg = 1024;     // keys whose slot indices are staged in LDS at a time
constexpr float kSlack = 8.f;  // log2 headroom of the lazy softmax rescale

template <int D>
struct ExtendCfg {
  static constexpr int kRowBytes = D * 2;                 // one K or V row of one head
  static constexpr int kCPR = kRowBytes / 16;             // 16-byte chunks per row
  static constexpr int kKPI = 64 / kCPR;                  // rows per 64-lane LDS load (1 KiB)
  static constexpr int kKB = kBN / 32;                    // 32-key blocks per tile
  static constexpr int kTile = kBN * kRowBytes;           // bytes of one K (or V) tile
  static constexpr int kKS = D / 16;                      // 16-dim steps of Q K^T
  static constexpr int kR = D / 32;                       // 32-dim tiles of O^T
};

// PART: the shared-prefix pass of radix_decode_attention_shared.  A
// "request" b is then a group of consecutive decode rows (qo_indptr =
// group_start: rows qo_indptr[b] .. qo_indptr[b+1] - 1, one query row each)
// whose slot rows agree on their first shared_lens[qo_indptr[b]] entries;
// item (query tile, group, KV head, chunk c) attends its rows to shared keys
// [c * chunk_keys, (c + 1) * chunk_keys) without a causal mask and writes the
// split-K partial (max, sum, unnormalised accumulator) of each (row, head) to
// split slot c of the decode workspace instead of an output row.
// The workgroup body; vblock / vgrid stand for blockIdx.x / gridDim.x (the
// single-launch shared decode runs it in the first vgrid workgroups of a
// larger grid).
template <int D, int RB, bool KV8, bool PART>
__device__ __forceinline__ void extend_body(
    const int vblock, const int vgrid, const char* __restrict__ q, char* __restrict__ o,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const int32_t* __restrict__ req_to_token,
    int64_t stride, const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ qo_indptr, int B1, int B2, int Hq,
    int Hkv, int G, int n_qt, int n_qt2, int seg2, float scale_log2, float v_scale, int n_chunks, int chunk_keys,
    int S_total, float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
  using C = ExtendCfg<D>;
  constexpr int kWaveRows = 32 * RB;          // query rows per wave (RB blocks of 32)
  constexpr int kItemRows = kWaves * kWaveRows;  // query rows per work item
  // Staged rows: bf16 pools stage rows as the MFMA code reads them (swizzled);
  // FP8 pools stage their D-byte rows as they are, and each tile is widened
  // once into the bf16 layout (skw / svw) for all waves.
  constexpr int kSRow = KV8 ? D : C::kRowBytes;  // staged bytes per row
  constexpr int kSCPR = kSRow / 16;              // 16-byte chunks per staged row
  constexpr int kSKPI = 64 / kSCPR;              // staged rows per 64-lane load
  constexpr int kSTileLoads = kBN / kSKPI;       // 64-lane loads per tile, K and V each
  // Loads per wave per tile.  With fewer loads than waves (FP8 rows of 64
  // dims) waves 0 .. kSTileLoads - 1 issue one each and the others none.
  constexpr int kSLoads = kSTileLoads >= kWaves ? kSTileLoads / kWaves : 1;
  static_assert(kSTileLoads % kWaves == 0 || kSTileLoads < kWaves, "tile loads must split evenly over the waves");
  // Two stages of K and V tiles: the next tile streams into one stage while
  // the other is used.  Separate arrays let the compiler see that LDS reads of
  // one stage never wait on the loads still landing in the other.
  __shared__ __attribute__((aligned(1024))) char sk0[kBN * kSRow];
  __shared__ __attribute__((aligned(1024))) char sv0[kBN * kSRow];
  __shared__ __attribute__((aligned(1024))) char sk1[kBN * kSRow];
  __shared__ __attribute__((aligned(1024))) char sv1[kBN * kSRow];
  __shared__ __attribute__((aligned(1024))) char skw[KV8 ? C::kTile : 16];
  __shared__ __attribute__((aligned(1024))) char svw[KV8 ? C::kTile : 16];
  __shared__ uint32_t s_slot[kSeg];

  // Two segments of work: n_qt query tiles for each of requests 0 .. B1-1,
  // then n_qt2 for each of the B2 short requests after them (decode rows of a
  // mixed batch).  Each segment is spread over the XCDs on its own; the first
  // ends at block seg2 (a multiple of 8 when a second segment follows, so the
  // second starts on XCD 0), and its padding blocks have no work.
  int qt, b, kvh, chunk = 0;
  if (PART) {
    const int work = xcd_slice(vblock, vgrid);
    qt = work % n_qt;
    b = (work / n_qt) % B1;
    kvh = (work / (n_qt * B1)) % Hkv;
    chunk = work / (n_qt * B1 * Hkv);
  } else if (vblock < seg2) {
    const int work = xcd_slice(vblock, seg2);
    if (work >= n_qt * B1 * Hkv) return;
    qt = work % n_qt;
    b = (work / n_qt) % B1;
    kvh = work / (n_qt * B1);
  } else {
    const int work = xcd_slice(vblock - seg2, vgrid - seg2);
    qt = work % n_qt2;
    b = B1 + (work / n_qt2) % B2;
    kvh = work / (n_qt2 * B2);
  }

  // PART: E = the group's rows, keys [key0, P) of the shared part, no mask
  // but the chunk's end.
  const int E = PART ? qo_indptr[b + 1] - qo_indptr[b] : extend_lens[b];
  const int row0 = qt * kItemRows;            // first query row of this item
  if (row0 / G >= E) return;
  const int P = PART ? min(prefix_lens[qo_indptr[b]], (chunk + 1) * chunk_keys) : prefix_lens[b];
  const int key0 = PART ? chunk * chunk_keys : 0;   // a multiple of kBN
  const int j_last = min(E - 1, (row0 + kItemRows - 1) / G);
  const int kv_end = PART ? P : P + j_last + 1;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int lane = tid & 63;
  const int r32 = lane & 31;   // this lane's query row within a 32-row block / MFMA column
  const int hi = lane >> 5;    // MFMA k-half

  // This lane's query row in each of the wave's row blocks.
  int jrow[RB], grow[RB], limit[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = row0 + wave * kWaveRows + rb * 32 + r32;
    jrow[rb] = qrow / G;
    grow[rb] = qrow - jrow[rb] * G;
    row_ok[rb] = jrow[rb] < E;
    // last visible key (invalid rows mimic the last row)
    limit[rb] = PART ? P - 1 : P + min(jrow[rb], E - 1);
  }
  const int wj_first = min((row0 + wave * kWaveRows) / G, E - 1);
  const int wj_last = min((row0 + wave * kWaveRows + kWaveRows - 1) / G, E - 1);
  const int w_min_limit = PART ? P - 1 : P + wj_first;  // keys <= this are visible to every row of the wave
  // Keys >= w_end are invisible to every row of the wave; a wave whose rows
  // all lie past the request's extend rows computes nothing.
  const int w_end = (row0 + wave * kWaveRows) / G < E ? (PART ? P : P + wj_last + 1) : 0;

  const int32_t* idx_row = req_to_token + int64_t(PART ? (rpi ? rpi[qo_indptr[b]] : qo_indptr[b])
                                                        : (rpi ? rpi[b] : b)) * stride;
  const uint32_t pool_row = uint32_t(Hkv) * kSRow;
  const char* kbase = k_pool + int64_t(kvh) * kSRow;
  const char* vbase = v_pool + int64_t(kvh) * kSRow;

  // Q^T operands (B of S^T = K Q^T): column r32 = query row, k = dims 16*ks + 8*hi + t.
  bf16x8 qop[RB][C::kKS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t tok = int64_t(qo_indptr[b]) + jrow[rb];
    const char* qp = q + (tok * Hq + int64_t(kvh) * G + grow[rb]) * C::kRowBytes + hi * 16;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      const u32x4 w = row_ok[rb] ? ld16(qp + ks * 32) : u32x4{0, 0, 0, 0};
      u32x4 s;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = pack_bf16x2(bf16_lo(w[i]) * scale_log2, bf16_hi(w[i]) * scale_log2);
      qop[rb][ks] = as_bf16x8(s);
    }
  }

  floatx16 oacc[RB][C::kR];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < C::kR; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[rb][r][i] = 0.f;
  // Scores come out of the MFMA already shifted by the running max: each
  // tile's accumulator starts at -m (all 16 entries of a lane belong to one
  // query row), so p = exp2(acc) needs no per-score arithmetic.  m starts at
  // 0 with the first computed tile forced through the rescale path.
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = 0.f;
    l[rb] = 0.f;
  }
  bool first = true;  // wave-uniform

  // Tile loads go straight from HBM to LDS (global_load_lds_dwordx4): one
  // 64-lane load fills kKPI consecutive rows (1 KiB).  Wave w issues loads
  // n = w + kWaves*it; lane i takes row kKPI*n + i/kCPR and the logical chunk that
  // the swizzle stores at physical chunk i%kCPR.  Keys past kv_end are clamped
  // to the last valid key (masked later; a real row keeps the tile finite).
  // Slot indices come from s_slot, staged per segment of kSeg keys.
  const int ld_row = lane / kSCPR;
  const int ld_pchunk = lane % kSCPR;
  int seg0 = 0;  // first key of the segment whose slot indices are in s_slot
  // Loads of one wave read the slot indices at s_slot[tile_key + krow]; the
  // staging pads the segment's last tile with the last valid key, so no clamp.
  const int krow0 = kSKPI * wave + ld_row;
  // krow = krow0 + kWaves*kSKPI*it, a multiple of 16 apart: same swizzle
  const int lchunk = KV8 ? ld_pchunk : ld_pchunk ^ (swz_f(krow0) & (C::kCPR - 1));
  const uint64_t lane_off = uint64_t(lchunk << 4);
  auto issue = [&](int tile, char* sk, char* sv) {
    if (kSTileLoads < kWaves && wave >= kSTileLoads) return;  // wave-uniform: no rows of this tile
    const uint32_t* srow = s_slot + (tile * kBN - seg0) + krow0;
#pragma unroll
    for (int it = 0; it < kSLoads; ++it) {
      const uint64_t off = uint64_t(srow[kWaves * kSKPI * it]) * pool_row + lane_off;
      const int dst = kSKPI * (wave + kWaves * it) * kSRow;
      __builtin_amdgcn_global_load_lds(kbase + off, (__attribute__((address_space(3))) void*)(sk + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vbase + off, (__attribute__((address_space(3))) void*)(sv + dst), 16, 0, 0);
    }
  };

  // K operand sources of this lane: key r32 of a 32-key block (+32 rows per
  // block), 16-byte chunk 2*ks + hi under the swizzle (which depends only on
  // the key's low 4 bits).
  int kofs[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) kofs[ks] = swz<D>(r32, 2 * ks + hi);

  // V transpose-read source of this lane: lane s = lane%16 of group gr = lane/16
  // addresses key 4*(gr/2) + s/4 and the 4-dim run at dims 16*(gr%2) + 4*(s%4)
  // (+32 per O^T tile): chunk 2*(gr%2) + (s%4)/2 (+4 per tile), half s%2.
  const int tr_key = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = (lane & 1) * 8;

  // FP8 pools: widen a staged tile into the swizzled bf16 layout, 16 codes
  // (two bf16 chunks) per unit of work.
  auto widen = [&](const char* s8, char* sw) {
    for (int u = tid; u < kBN * kSCPR; u += 64 * kWaves) {
      const int row = u / kSCPR, c = u - (u / kSCPR) * kSCPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(s8 + row * kSRow + 16 * c);
      const u32x4 lo = {fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x), fp8x2_to_bf16x2<false>(w.y),
                        fp8x2_to_bf16x2<true>(w.y)};
      const u32x4 hi = {fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z), fp8x2_to_bf16x2<false>(w.w),
                        fp8x2_to_bf16x2<true>(w.w)};
      *reinterpret_cast<u32x4*>(sw + swz<D>(row, 2 * c)) = lo;
      *reinterpret_cast<u32x4*>(sw + swz<D>(row, 2 * c + 1)) = hi;
    }
  };

  // One tile: barrier (this tile's loads have landed everywhere and the other
  // stage is free), start the next tile's loads into the other stage, then
  // compute from this one (FP8: widen it first, then a second barrier).
  int seg_end = 0;  // tiles below seg_end have their slot indices staged
  auto step = [&](int tile, const char* sk, const char* sv, char* sk_next, char* sv_next) {
    __syncthreads();
    if (tile + 1 < seg_end) issue(tile + 1, sk_next, sv_next);
    if constexpr (KV8) {
      widen(sk, skw);
      widen(sv, svw);
      __syncthreads();
      sk = skw;
      sv = svw;
    }
    const int base = tile * kBN;
    if (base >= w_end) return;                // wave-uniform: every row of this wave is done

    // ---- scores S^T[key][row] for the tile's 32-key blocks; each K operand
    // read from LDS feeds the wave's RB row blocks
    floatx16 sacc[RB][C::kKB];
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb) {
      u32x4 ka[C::kKS];
#pragma unroll
      for (int ks = 0; ks < C::kKS; ++ks)
        ka[ks] = *reinterpret_cast<const u32x4*>(sk + kb * 32 * C::kRowBytes + kofs[ks]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[rb][kb][i] = -m[rb];
#pragma unroll
        for (int ks = 0; ks < C::kKS; ++ks)
          sacc[rb][kb] = mfma_32x32x16(as_bf16x8(ka[ks]), qop[rb][ks], sacc[rb][kb]);
      }
    }
    // Lane holds keys base + 32*kb + 8*(v/4) + 4*hi + (v%4) of its query rows.
    // Only tiles that cross this wave's diagonal (or its last key) need a mask.
    const bool masked = base + kBN - 1 > w_min_limit;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (masked) {
        const int rel = base + 4 * hi - limit[rb];  // key - limit = rel + const(kb, v)
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (rel + 32 * kb + 8 * (v >> 2) + (v & 3) > 0) sacc[rb][kb][v] = -INFINITY;
      }
      float mx = sacc[rb][0][0];
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
        for (int v = (kb == 0); v < 16; ++v) mx = fmaxf(mx, sacc[rb][kb][v]);
      mx = max_lane_pair(mx);  // row max of the tile minus m
      // Lazy rescale: the reference max m only moves when some row's max
      // exceeds it by more than 2^kSlack, so probabilities stay <= 2^kSlack
      // (harmless in fp32 and bf16) and the accumulator rescale is rare.
      if (first || __any(mx > kSlack)) {
        const float m_old = first ? -INFINITY : m[rb];
        const float m_new = fmaxf(m_old, m[rb] + mx);
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
        const float shift = m_new - m[rb];
        l[rb] *= alpha;
#pragma unroll
        for (int r = 0; r < C::kR; ++r)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[rb][r][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[rb][kb][v] -= shift;
        m[rb] = m_new;
      }
    }
    first = false;

    // ---- O^T += V^T P^T, 16 keys per MFMA; each V operand read feeds the
    // wave's RB row blocks
#pragma unroll
    for (int kb = 0; kb < C::kKB; ++kb) {
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        // logical k = 8*hi + t  <->  key 32*kb + 16*sh + 8*(t/4) + 4*hi + (t%4).
        // The V^T operand (32 dims x these 8 keys) comes from two LDS
        // transpose reads of 4 keys each.
        const int k0 = 32 * kb + 16 * sh + tr_key;
        u32x2 vt[C::kR][2];
#pragma unroll
        for (int dt = 0; dt < C::kR; ++dt) {
          vt[dt][0] = ds_read_tr16(sv + swz<D>(k0, tr_chunk + 4 * dt) + tr_half);
          vt[dt][1] = ds_read_tr16(sv + swz<D>(k0 + 8, tr_chunk + 4 * dt) + tr_half);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float p[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) p[t] = __builtin_amdgcn_exp2f(sacc[rb][kb][8 * sh + t]);
          const u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
          // row sum of the rounded probabilities the MFMA uses
#pragma unroll
          for (int t = 0; t < 4; ++t) l[rb] = sum_bf16x2(pk[t], l[rb]);
          const bf16x8 pop = as_bf16x8(pk);
#pragma unroll
          for (int dt = 0; dt < C::kR; ++dt)
            oacc[rb][dt] = mfma_32x32x16(as_bf16x8(u32x4{vt[dt][0].x, vt[dt][0].y, vt[dt][1].x, vt[dt][1].y}),
                                         pop, oacc[rb][dt]);
        }
      }
    }
  };

  // Segments of kSeg keys: stage their slot indices in LDS, start tile 0 of
  // the segment, then stream its tiles through the two stages.
  const int tiles_per_seg = kSeg / kBN;
  for (int seg_tile = key0 / kBN; seg_tile < n_tiles; seg_tile += tiles_per_seg) {
    seg0 = seg_tile * kBN;
    seg_end = min(n_tiles, seg_tile + tiles_per_seg);
    __syncthreads();  // previous segment fully consumed
    for (int i = tid; i < (seg_end - seg_tile) * kBN; i += 64 * kWaves) s_slot[i] = uint32_t(idx_row[min(seg0 + i, kv_end - 1)]);
    __syncthreads();
    issue(seg_tile, sk0, sv0);
    for (int tile = seg_tile; tile < seg_end; tile += 2) {
      step(tile, sk0, sv0, sk1, sv1);
      if (tile + 1 < seg_end) step(tile + 1, sk1, sv1, sk0, sv0);
    }
  }

  // ---- normalise and store: O^T tile dt row i = dim 32*dt + i; this lane holds
  // rows i = 8*(v/4) + 4*hi + (v%4) of its query rows.
  if constexpr (PART) {
    // Split-K partial of each (row, head): max m (log2 units), sum l and
    // the unnormalised accumulator; an empty chunk writes (-inf, 0, 0).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lsum = l[rb] + __shfl_xor(l[rb], 32, 64);
      if (!row_ok[rb]) continue;
      const int64_t part = ((int64_t(qo_indptr[b]) + jrow[rb]) * Hq + int64_t(kvh) * G + grow[rb]) * S_total + chunk;
      if (hi == 0) {
        ws_ml[part * 2 + 0] = first ? -INFINITY : m[rb];
        ws_ml[part * 2 + 1] = first ? 0.f : lsum;
      }
      float* acc = ws_acc + part * D;
      const float sc = KV8 ? v_scale : 1.f;
#pragma unroll
      for (int dt = 0; dt < C::kR; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const floatx4 w = {oacc[rb][dt][4 * v4 + 0] * sc, oacc[rb][dt][4 * v4 + 1] * sc,
                             oacc[rb][dt][4 * v4 + 2] * sc, oacc[rb][dt][4 * v4 + 3] * sc};
          *reinterpret_cast<floatx4*>(acc + 32 * dt + 8 * v4 + 4 * hi) = w;
        }
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lsum = l[rb] + __shfl_xor(l[rb], 32, 64);
    if (!row_ok[rb]) continue;
    const float inv = (KV8 ? v_scale : 1.f) / lsum;
    const int64_t tok = int64_t(qo_indptr[b]) + jrow[rb];
    char* op = o + (tok * Hq + int64_t(kvh) * G + grow[rb]) * C::kRowBytes;
#pragma unroll
    for (int dt = 0; dt < C::kR; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const u32x2 w = {pack_bf16x2(oacc[rb][dt][4 * v4 + 0] * inv, oacc[rb][dt][4 * v4 + 1] * inv),
                         pack_bf16x2(oacc[rb][dt][4 * v4 + 2] * inv, oacc[rb][dt][4 * v4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + (32 * dt + 8 * v4 + 4 * hi) * 2) = w;
      }
  }
}

template <int D, int RB, bool KV8, bool PART = false>
__global__ void __launch_bounds__(64 * kWaves, RB == 1 ? kWavesPerSimd : 1) extend_bf16(
    const char* __restrict__ q, char* __restrict__ o, const char* __restrict__ k_pool,
    const char* __restrict__ v_pool, const int32_t* __restrict__ req_to_token, int64_t stride,
    const int32_t* __restrict__ rpi, const int32_t* __restrict__ prefix_lens,
    const int32_t* __restrict__ extend_lens, const int32_t* __restrict__ qo_indptr, int B1, int B2, int Hq,
    int Hkv, int G, int n_qt, int n_qt2, int seg2, float scale_log2, float v_scale, int n_chunks = 1,
    int chunk_keys = 0, int S_total = 0, float* __restrict__ ws_acc = nullptr, float* __restrict__ ws_ml = nullptr) {
  extend_body<D, RB, KV8, PART>(int(blockIdx.x), int(gridDim.x), q, o, k_pool, v_pool, req_to_token, stride, rpi,
                                prefix_lens, extend_lens, qo_indptr, B1, B2, Hq, Hkv, G, n_qt, n_qt2, seg2,
                                scale_log2, v_scale, n_chunks, chunk_keys, S_total, ws_acc, ws_ml);
}

// Single-launch shared-prefix decode: workgroups 0 .. nA - 1 run the shared
// pass (extend_body in partial mode); workgroups from nA_pad (nA rounded up
// to a multiple of 8, so that the rest start on XCD 0) on hold four split-K
// waves each, which take the private tails' items as the split kernel's
// waves do, with their slot indices in a ring of kFusedRing entries per wave
// (16 KiB per workgroup beside the shared pass's 36 KiB: three workgroups
// per CU); every partial lands in the decode workspace for the combine.
// The two parts share no data, so they run side by side on the chip instead
// of one launch after the other.
constexpr int kFusedRing = 1024;
template <int D, bool KV8, bool APP = false>
__global__ void __launch_bounds__(64 * kWaves, kWavesPerSimd) shared_decode_fused(
    const char* __restrict__ q, const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const int32_t* __restrict__ req_to_token, int64_t stride, const int32_t* __restrict__ rpi,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ shared_lens,
    const int32_t* __restrict__ group_start, int n_groups, int B, int Hq, int Hkv, int G, int n_qt, int n_chunks,
    int chunk_keys, int S_b, int chunk_b, int S_total, float scale_log2, float v_scale, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, int nA, int nA_pad, int nB, rt::AppendArgs app) {
  __shared__ int32_t s_idx[kWaves][kFusedRing];
  const int bid = int(blockIdx.x);
  if (bid < nA) {
    extend_body<D, kRB, KV8, true>(bid, nA, q, nullptr, k_pool, v_pool, req_to_token, stride, rpi, shared_lens,
                                   nullptr, group_start, n_groups, 0, Hq, Hkv, G, n_qt, 0, 0, scale_log2, v_scale,
                                   n_chunks, chunk_keys, S_total, ws_acc, ws_ml);
    return;
  }
  if (bid < nA_pad) return;
  const int j = bid - nA_pad;                                          // j % 8 is this workgroup's XCD
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  rtk::dec::split_items<D, KV8, kFusedRing, APP>(j & 7, (j >> 3) * kWaves + wave, (nB >> 3) * kWaves,
                                            int(threadIdx.x) & 63,
                                s_idx[wave], q, k_pool, v_pool, req_to_token, stride, rpi, prefix_lens, B, Hq, Hkv,
                                G, S_b, chunk_b, scale_log2, v_scale, ws_acc, ws_ml, shared_lens, n_chunks,
                                S_total, app);
}


// ----------------------------------------------------------------- fp32 --
template <int D>
__global__ void __launch_bounds__(64) extend_f32(const float* __restrict__ q, float* __restrict__ o,
                                                 const float* __restrict__ k_pool, const float* __restrict__ v_pool,
                                                 const int32_t* __restrict__ req_to_token, int64_t stride,
                                                 const int32_t* __restrict__ rpi,
                                                 const int32_t* __restrict__ prefix_lens,
                                                 const int32_t* __restrict__ extend_lens,
                                                 const int32_t* __restrict__ qo_indptr, int Hq, int Hkv, int G,
                                                 float scale_log2) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (j >= extend_lens[b]) return;
  const int kvh = h / G;
  const int n_keys = prefix_lens[b] + j + 1;
  const int32_t* idx_row = req_to_token + int64_t(rpi ? rpi[b] : b) * stride;
  const int64_t pool_row = int64_t(Hkv) * D;
  const int64_t qo = (int64_t(qo_indptr[b]) + j) * Hq + h;
  float qd[PER], acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    qd[i] = q[qo * D + lane + 64 * i];
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int key = 0; key < n_keys; ++key) {
    const int64_t slot = idx_row[key];
    const float* kr = k_pool + slot * pool_row + int64_t(kvh) * D;
    const float* vr = v_pool + slot * pool_row + int64_t(kvh) * D;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) part = fmaf(qd[i], kr[lane + 64 * i], part);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    const float sc = part * scale_log2;
    const float m_new = fmaxf(m, sc);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(p, vr[lane + 64 * i], acc[i] * alpha);
    m = m_new;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[qo * D + lane + 64 * i] = acc[i] * inv;
}

template <bool KV8>
int launch_extend_bf16(const void* q, void* o, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                       int32_t req_to_token_stride, const int32_t* req_pool_indices, const int32_t* prefix_lens,
                       const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch, int32_t num_extend,
                       int32_t max_extend_len, int32_t max_tail_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, float scale_log2, float v_scale, hipStream_t st) {
  const int G = num_q_heads / num_kv_heads;
  const int64_t item_rows = kWaves * 32 * kRB;
  const int64_t B2 = int64_t(batch) - num_extend;
  const int64_t n_qt = (int64_t(max_extend_len) * G + item_rows - 1) / item_rows;
  const int64_t n_qt2 = B2 > 0 ? (int64_t(max_tail_len) * G + item_rows - 1) / item_rows : 0;
  const int64_t n1 = n_qt * num_extend * num_kv_heads;
  const int64_t n2 = n_qt2 * B2 * num_kv_heads;
  const int64_t seg2 = n2 > 0 ? (n1 + 7) / 8 * 8 : n1;
  const int64_t grid = seg2 + n2;
  if (grid > INT32_MAX) return rt::fail(RT_ERR_INVALID, "radix_extend_attention: grid too large");
  if (grid == 0) return RT_OK;
  if (head_dim == 128)
    hipLaunchKernelGGL((extend_bf16<128, kRB, KV8>), dim3(uint32_t(grid)), dim3(64 * kWaves), 0, st,
                       (const char*)q, (char*)o, (const char*)k_pool, (const char*)v_pool, req_to_token,
                       int64_t(req_to_token_stride), req_pool_indices, prefix_lens, extend_lens, qo_indptr,
                       num_extend, int(B2), num_q_heads, num_kv_heads, G, int(n_qt), int(n_qt2), int(seg2),
                       scale_log2, v_scale);
  else
    hipLaunchKernelGGL((extend_bf16<64, kRB, KV8>), dim3(uint32_t(grid)), dim3(64 * kWaves), 0, st,
                       (const char*)q, (char*)o, (const char*)k_pool, (const char*)v_pool, req_to_token,
                       int64_t(req_to_token_stride), req_pool_indices, prefix_lens, extend_lens, qo_indptr,
                       num_extend, int(B2), num_q_heads, num_kv_heads, G, int(n_qt), int(n_qt2), int(seg2),
                       scale_log2, v_scale);
  return RT_OK;
}

}  // namespace

namespace rt {

int launch_extend_shared_part(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                              int64_t stride, const int32_t* rpi, const int32_t* shared_lens,
                              const int32_t* group_start, int n_groups, int max_group_size, int n_chunks,
                              int chunk_keys, int S_total, int Hq, int Hkv, int D, float scale_log2, float v_scale,
                              bool kv8, float* ws_acc, float* ws_ml, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int G = Hq / Hkv;
  const int64_t item_rows = kWaves * 32 * kRB;
  const int64_t n_qt = (int64_t(max_group_size) * G + item_rows - 1) / item_rows;
  const int64_t grid = n_qt * n_groups * Hkv * n_chunks;
  if (grid > INT32_MAX) return rt::fail(RT_ERR_INVALID, "radix_decode_attention_shared: grid too large");
  if (grid == 0) return RT_OK;
  if (chunk_keys % kBN != 0) return rt::fail(RT_ERR_INVALID, "shared pass: chunk not a multiple of the tile");
#define RT_SHARED_LAUNCH(DD, K8)                                                                                    \
  hipLaunchKernelGGL((extend_bf16<DD, kRB, K8, true>), dim3(uint32_t(grid)), dim3(64 * kWaves), 0, st,            \
                     (const char*)q, (char*)nullptr, (const char*)k_pool, (const char*)v_pool, req_to_token, stride, \
                     rpi, shared_lens, (const int32_t*)nullptr, group_start, n_groups, 0, Hq, Hkv, G, int(n_qt), 0,  \
                     0, scale_log2, v_scale, n_chunks, chunk_keys, S_total, ws_acc, ws_ml)
  if (D == 128) {
    if (kv8) RT_SHARED_LAUNCH(128, true); else RT_SHARED_LAUNCH(128, false);
  } else {
    if (kv8) RT_SHARED_LAUNCH(64, true); else RT_SHARED_LAUNCH(64, false);
  }
#undef RT_SHARED_LAUNCH
  return RT_OK;
}

int launch_shared_fused(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                        int64_t stride, const int32_t* rpi, const int32_t* prefix_lens, const int32_t* shared_lens,
                        const int32_t* group_start, int n_groups, int max_group_size, int n_chunks, int chunk_keys,
                        int batch, int S_b, int chunk_b, int S_total, int Hq, int Hkv, int D, float scale_log2,
                        float v_scale, bool kv8, float* ws_acc, float* ws_ml, void* stream,
                        const AppendArgs& app) {
  hipStream_t st = (hipStream_t)stream;
  const int G = Hq / Hkv;
  const int64_t item_rows = kWaves * 32 * kRB;
  const int64_t n_qt = (int64_t(max_group_size) * G + item_rows - 1) / item_rows;
  const int64_t nA = n_qt * n_groups * Hkv * n_chunks;
  const int64_t nA_pad = (nA + 7) / 8 * 8;
  const int64_t items = int64_t(batch) * Hkv * S_b;           // one split wave per private item
  const int64_t nB = ((items + kWaves - 1) / kWaves + 7) / 8 * 8;
  if (nA_pad + nB > INT32_MAX) return rt::fail(RT_ERR_INVALID, "radix_decode_attention_shared: grid too large");
  if (chunk_keys % kBN != 0) return rt::fail(RT_ERR_INVALID, "shared pass: chunk not a multiple of the tile");
  if (chunk_b < 1) return rt::fail(RT_ERR_INVALID, "single-launch shared decode: empty private chunk");
  if (nA_pad + nB == 0) return RT_OK;
#define RT_FUSED_LAUNCH1(DD, K8, AP)                                                                               \
  hipLaunchKernelGGL((shared_decode_fused<DD, K8, AP>), dim3(uint32_t(nA_pad + nB)), dim3(64 * kWaves), 0, st,    \
                     (const char*)q, (const char*)k_pool, (const char*)v_pool, req_to_token, stride, rpi,          \
                     prefix_lens, shared_lens, group_start, n_groups, batch, Hq, Hkv, G, int(n_qt), n_chunks,       \
                     chunk_keys, S_b, chunk_b, S_total, scale_log2, v_scale, ws_acc, ws_ml, int(nA), int(nA_pad),   \
                     int(nB), app)
#define RT_FUSED_LAUNCH(DD, K8)                                                                                    \
  do {                                                                                                             \
    if (app.slots) RT_FUSED_LAUNCH1(DD, K8, true); else RT_FUSED_LAUNCH1(DD, K8, false);                           \
  } while (0)
  if (D == 128) {
    if (kv8) RT_FUSED_LAUNCH(128, true); else RT_FUSED_LAUNCH(128, false);
  } else {
    if (kv8) RT_FUSED_LAUNCH(64, true); else RT_FUSED_LAUNCH(64, false);
  }
#undef RT_FUSED_LAUNCH
#undef RT_FUSED_LAUNCH1
  return RT_OK;
}

// Longer private chunks take the two-launch path: on long-context tails
// (32 x 16385 keys) the single launch measured 517-519 us against 401-402 us
// for the shared pass on a second stream beside the split kernel.
int fused_max_private_chunk() { return kFusedRing; }

}  // namespace rt

namespace {

// Shared checks and dispatch of the four entry points.  kv8: FP8 pools.
int extend_entry(const char* name, bool kv8, const void* q, void* o, const void* k_pool, const void* v_pool,
                 const int32_t* req_to_token, int32_t req_to_token_stride, const int32_t* req_pool_indices,
                 const int32_t* prefix_lens, const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                 int32_t num_extend, int32_t max_extend_len, int32_t max_tail_len, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, float sm_scale, int dtype, float k_scale, float v_scale,
                 hipStream_t st) {
  if (batch < 0 || num_extend < 0 || num_extend > batch || max_extend_len < 0 || max_tail_len < 0 ||
      num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || (dtype != RT_F32 && dtype != RT_BF16) || (kv8 && dtype != RT_BF16) ||
      req_to_token_stride < 1 || !(sm_scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": bad shape, count, dtype, stride or scale");
  if (batch == 0 || (max_extend_len == 0 && (max_tail_len == 0 || num_extend == batch))) return RT_OK;
  if (!q || !o || !k_pool || !v_pool || !req_to_token || !prefix_lens || !extend_lens || !qo_indptr)
    return rt::fail(RT_ERR_INVALID, std::string(name) + ": null pointer");
  const float scale_log2 = sm_scale * k_scale * kLog2e;
  if (dtype == RT_BF16) {
    const int rc = kv8 ? launch_extend_bf16<true>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                                                  req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch,
                                                  num_extend, max_extend_len, max_tail_len, num_q_heads,
                                                  num_kv_heads, head_dim, scale_log2, v_scale, st)
                       : launch_extend_bf16<false>(q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                                                   req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch,
                                                   num_extend, max_extend_len, max_tail_len, num_q_heads,
                                                   num_kv_heads, head_dim, scale_log2, 1.f, st);
    if (rc != RT_OK) return rc;
  } else {
    // fp32: one wave per (extend row, query head, request); one dense grid
    // over the longest extend of either part.
    const int32_t max_len = num_extend < batch ? std::max(max_extend_len, max_tail_len) : max_extend_len;
    if (max_len > 65535 * 16 || num_q_heads > 65535 || batch > 65535)
      return rt::fail(RT_ERR_INVALID, std::string(name) + ": fp32 grid too large");
    const int G = num_q_heads / num_kv_heads;
    const dim3 grid{uint32_t(max_len), uint32_t(num_q_heads), uint32_t(batch)};
    if (head_dim == 128)
      hipLaunchKernelGGL(extend_f32<128>, grid, dim3(64), 0, st, (const float*)q, (float*)o,
                         (const float*)k_pool, (const float*)v_pool, req_to_token, int64_t(req_to_token_stride),
                         req_pool_indices, prefix_lens, extend_lens, qo_indptr, num_q_heads, num_kv_heads, G,
                         scale_log2);
    else
      hipLaunchKernelGGL(extend_f32<64>, grid, dim3(64), 0, st, (const float*)q, (float*)o,
                         (const float*)k_pool, (const float*)v_pool, req_to_token, int64_t(req_to_token_stride),
                         req_pool_indices, prefix_lens, extend_lens, qo_indptr, num_q_heads, num_kv_heads, G,
                         scale_log2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt::fail(RT_ERR_HIP, std::string(name) + " launch: " + hipGetErrorString(e));
  return RT_OK;
}

}  // namespace

extern "C" int radix_extend_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                                      const int32_t* req_to_token, int32_t req_to_token_stride,
                                      const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                      const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                      int32_t max_extend_len, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float sm_scale, int dtype, void* stream) {
  return extend_entry("radix_extend_attention", false, q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch, batch, max_extend_len, 0,
                      num_q_heads, num_kv_heads, head_dim, sm_scale, dtype, 1.f, 1.f, (hipStream_t)stream);
}

extern "C" int radix_extend_attention_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                            const int32_t* req_to_token, int32_t req_to_token_stride,
                                            const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                            const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                            int32_t max_extend_len, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, float sm_scale, float k_scale, float v_scale,
                                            void* stream) {
  return extend_entry("radix_extend_attention_fp8kv", true, q, o, k_pool, v_pool, req_to_token,
                      req_to_token_stride, req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch, batch,
                      max_extend_len, 0, num_q_heads, num_kv_heads, head_dim, sm_scale, RT_BF16, k_scale, v_scale,
                      (hipStream_t)stream);
}

extern "C" int radix_mixed_attention(const void* q, void* o, const void* k_pool, const void* v_pool,
                                     const int32_t* req_to_token, int32_t req_to_token_stride,
                                     const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                     const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                     int32_t num_extend, int32_t max_extend_len, int32_t max_tail_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                     int dtype, void* stream) {
  return extend_entry("radix_mixed_attention", false, q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch, num_extend, max_extend_len,
                      max_tail_len, num_q_heads, num_kv_heads, head_dim, sm_scale, dtype, 1.f, 1.f,
                      (hipStream_t)stream);
}

extern "C" int radix_mixed_attention_fp8kv(const void* q, void* o, const void* k_pool, const void* v_pool,
                                           const int32_t* req_to_token, int32_t req_to_token_stride,
                                           const int32_t* req_pool_indices, const int32_t* prefix_lens,
                                           const int32_t* extend_lens, const int32_t* qo_indptr, int32_t batch,
                                           int32_t num_extend, int32_t max_extend_len, int32_t max_tail_len,
                                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                           float sm_scale, float k_scale, float v_scale, void* stream) {
  return extend_entry("radix_mixed_attention_fp8kv", true, q, o, k_pool, v_pool, req_to_token, req_to_token_stride,
                      req_pool_indices, prefix_lens, extend_lens, qo_indptr, batch, num_extend, max_extend_len,
                      max_tail_len, num_q_heads, num_kv_heads, head_dim, sm_scale, RT_BF16, k_scale, v_scale,
                      (hipStream_t)stream);
}
