// Internal helpers shared by the translation units of libpagedkv.
#pragma once

#include <vector>

#include "pagedkv.h"

namespace pagedkv {

// The plan pa_bm_prepare_decode_step built or advanced last (per block
// manager), kept so that the next step can advance it instead of building a
// new one (pa_bm_set_plan_reuse).
struct StepPlanCache {
  std::vector<char> plan;        // plan bytes
  pa_decode_plan_info info{};    // its info (first-tile entries not kept)
  std::vector<int64_t> seqs;     // the batch it is for, in order
  int32_t num_kv_heads = 0, num_workgroups = 0, schedule = 0, max_piece = 0;
  int32_t advances = 0;          // steps advanced since it was built
  int32_t max_advances = 0;      // 0: build every step
  bool valid = false;
};
StepPlanCache& step_plan_cache(pa_bm* bm);

// pa_bm_prepare_decode_step's view of the block manager, one lookup per
// sequence: resolve the batch (every sequence known and resident) and read
// its lengths; then append one token to each (all or nothing, as
// pa_bm_append_step); then copy the table rows (the first table-size entries
// of each row of `tables`, int32 [num][max_blocks]).
pa_status bm_step_resolve(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* lens, const char* who);
pa_status bm_step_append(pa_bm* bm, const int64_t* seqs, int32_t num, int64_t* slots, int32_t* cows,
                         int32_t* n_cows, const char* who);
pa_status bm_step_tables(pa_bm* bm, int32_t num, int32_t* tables, int32_t max_blocks, const char* who);

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
