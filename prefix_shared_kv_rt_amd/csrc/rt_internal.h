// Internal helpers shared by the library's translation units.
#pragma once

#include <stdint.h>

#include <string>

namespace rt {
// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const std::string& msg);

// Each request's new token, stored by the decode launch itself (decode_append
// folded into the attention): k_new / v_new bf16 [batch, Hkv, D] go to the
// pools at slots[b] (as E4M3 codes of x * k_inv, x * v_inv over FP8 pools)
// and slots[b] into the slot table at (row of b, prefix_lens[b]).  slots ==
// nullptr: nothing to append.
struct AppendArgs {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* slots = nullptr;
  int32_t* r2t = nullptr;
  void* k_pool = nullptr;
  void* v_pool = nullptr;
  float k_inv = 1.f, v_inv = 1.f;
};

// The shared-prefix pass of radix_decode_attention_shared (extend.hip):
// for each group of consecutive decode rows (group_start), KV head, query
// tile and chunk of chunk_keys shared keys, write the split-K partial of
// every (row, head) into split slot `chunk` of S_total.  bf16 queries; bf16
// or FP8 (kv8) pools.
int launch_extend_shared_part(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                              int64_t stride, const int32_t* rpi, const int32_t* shared_lens,
                              const int32_t* group_start, int n_groups, int max_group_size, int n_chunks,
                              int chunk_keys, int S_total, int Hq, int Hkv, int D, float scale_log2, float v_scale,
                              bool kv8, float* ws_acc, float* ws_ml, void* stream);

// The single-launch form of radix_decode_attention_shared for short private
// tails (extend.hip): the shared pass above and the split-K pass over the
// private tails (S_b chunks of chunk_b keys per request and KV head, chunk_b
// at most fused_max_private_chunk(), partial slots n_chunks ..) in one
// launch; the caller then runs the combine.
int launch_shared_fused(const void* q, const void* k_pool, const void* v_pool, const int32_t* req_to_token,
                        int64_t stride, const int32_t* rpi, const int32_t* prefix_lens, const int32_t* shared_lens,
                        const int32_t* group_start, int n_groups, int max_group_size, int n_chunks, int chunk_keys,
                        int batch, int S_b, int chunk_b, int S_total, int Hq, int Hkv, int D, float scale_log2,
                        float v_scale, bool kv8, float* ws_acc, float* ws_ml, void* stream,
                        const AppendArgs& app = AppendArgs());
int fused_max_private_chunk();
}  // namespace rt
