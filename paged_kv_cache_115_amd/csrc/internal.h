// Internal helpers shared by the translation units of libpagedkv.
#pragma once

#include "pagedkv.h"

namespace pagedkv {

// Record a printf-style message for pa_last_error() and return `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Digest of a batch's context lengths (a splitmix64 chain over the count and
// every length), recorded in a decode plan and compared by the checks.
inline uint64_t lens_digest(const int32_t* lens, int32_t n) {
  auto mix = [](uint64_t z) {
    z += 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  };
  uint64_t h = mix((uint64_t)(uint32_t)n);
  for (int32_t i = 0; i < n; ++i) h = mix(h ^ (uint64_t)(uint32_t)lens[i]);
  return h;
}

// pa_decode_noalloc's host-side check: the plan's workspace fits the
// built-in scratch array (PA_ERR_INVALID otherwise).
pa_status noalloc_check(const pa_kv_pool* pool, const pa_decode_plan_info* info, int32_t num_q_heads,
                        const char* who);

// The decode front shared by the pa_decode entry points: argument checks,
// then the launches selected by `stages` (kStageAttention | kStageMerge).
constexpr int kStageAttention = 1;
constexpr int kStageMerge = 2;
pa_status decode_stages(int stages, const char* who, const pa_kv_pool* pool, const void* q, void* out,
                        int32_t out_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                        const void* new_key, const void* new_value, const void* plan,
                        const pa_decode_plan_info* info, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace pagedkv
