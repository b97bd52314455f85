// Kernel launchers of libpagedkv (internal; called by the C-ABI front after
// argument validation).  All take a hipStream_t passed as void*.
#pragma once

#include <hip/hip_runtime.h>

#include "pagedkv.h"

namespace pagedkv {

// Arguments of one decode launch; pointers are device pointers.
struct DecodeArgs {
  const void* k;
  const void* v;
  const void* q;
  void* out;
  const int32_t* tables;
  const int32_t* lens;
  const pa_work_item* items;  // [num_items] work items, then the merge items
  float* partial_ml;      // [num_partials * num_q_heads][2] = (max, sum) in log2 units
  float* partial_o;       // [num_partials * num_q_heads][head_dim]
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t group;          // num_q_heads / num_kv_heads
  int32_t head_dim;
  int32_t max_blocks;     // block-table row length
  int32_t num_seqs;
  int32_t partition;      // tokens per partition, 0 = whole sequence
  int32_t num_partials;   // workspace records available
  int32_t num_items;      // work items (merge items follow them)
  int32_t out_bf16;       // 1: write bfloat16, 0: float32
  float scale_log2e;      // scale * log2(e)
};

// Attention launch over a.num_items work items, then (if num_merges > 0) the
// split-K merge launch, both on `stream`.
hipError_t launch_decode_bf16(const DecodeArgs& a, int32_t num_merges, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, int32_t num_merges, hipStream_t stream);

hipError_t launch_reshape_and_cache(const pa_kv_pool& pool, const void* key, const void* value,
                                    const int64_t* slots, int32_t num_tokens, hipStream_t stream);
hipError_t launch_copy_blocks(const pa_kv_pool& pool, const int32_t* pairs, int32_t num_pairs,
                              hipStream_t stream);

}  // namespace pagedkv
