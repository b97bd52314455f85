// Kernel launchers of libpagedkv (internal; called by the C-ABI front after
// argument validation).
#pragma once

#include <hip/hip_runtime.h>

#include "pagedkv.h"

namespace pagedkv {

// Arguments of one decode call; pointers are device pointers.  The fields
// the attention launch's start-up needs (job table, first-tile entries,
// tables, lengths, q, the pools, the job-table shape) come first, so that
// they arrive in the first batch of argument loads.
struct DecodeArgs {
  const pa_decode_job* jobs;     // [jobs_per_workgroup][num_workgroups], column-major lists
  const int32_t* first_blocks;   // [jobs_per_workgroup][num_workgroups][4] first-tile table entries, or null
  const int32_t* tables;
  const int32_t* lens;
  const void* q;
  const void* k;
  const void* v;
  const void* new_k;             // [num_seqs][num_kv_heads][head_dim] or null: fused append of token L - 1
  int32_t num_workgroups;
  int32_t jobs_per_workgroup;
  int32_t num_blocks;
  int32_t max_blocks;            // block-table row length
  int32_t num_kv_heads;
  int32_t num_seqs;
  int32_t group;                 // num_q_heads / num_kv_heads
  int32_t num_q_heads;
  const void* new_v;
  void* out;
  const pa_decode_merge* merges; // [num_merges]
  const pa_decode_group* groups; // [num_groups] prefix-group descriptors
  float* partial_ml;             // [num_records * group][2] = (max, sum) in log2 units
  float* partial_o;              // [num_records * group][head_dim], unnormalised
  int32_t block_size;
  int32_t head_dim;
  int32_t num_jobs;
  int32_t num_merges;
  int32_t num_records;
  int32_t num_groups;
  int32_t wide_jobs;             // jobs with PA_JOB_WIDE: the launch picks the kernel that reads them
  int32_t bf16;                  // pool dtype: 1 bfloat16, 0 float32
  int32_t shared_kv;             // 1: sequences share blocks (keep K/V cached), 0: stream K/V
  int32_t out_bf16;              // 1: write bfloat16, 0: float32
  int32_t fused_loads;           // with new_k: 1 a branch at the appended token's tile, 2 per-lane
                                 // addresses for every tile (one load path), 4 per-lane offsets in
                                 // one buffer window per pool (k_win / v_win) for every tile
  const void* k_win;             // mode 4: window base below both the K pool and new_k
  const void* v_win;
  uint32_t k_win_bytes, v_win_bytes;
  uint32_t k_off, v_off;         // the pools' offsets in their windows
  uint32_t nk_off, nv_off;       // new_k's and new_v's offsets in their windows
  float scale_log2e;             // scale * log2(e)
};

// Attention launch (persistent grid of a.num_workgroups; nothing when the
// plan has no jobs) on `stream`.
hipError_t launch_decode_attention(const DecodeArgs& a, hipStream_t stream);
// The same for an fp32 pool (decode_f32_kernels.hip).
hipError_t launch_decode_attention_f32(const DecodeArgs& a, hipStream_t stream);
// Merge launch: one workgroup per merge row, then, with a fused append
// (a.new_k set), one per sequence writing its appended row into the pool;
// nothing when neither is needed.
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);
// Resident decode workgroups per compute unit (occupancy of the bf16 kernel).
hipError_t decode_resident_workgroups_per_cu(int* n);

hipError_t launch_reshape_and_cache(const pa_kv_pool& pool, const void* key, const void* value,
                                    const int64_t* slots, int32_t num_tokens, hipStream_t stream);
hipError_t launch_copy_blocks(const pa_kv_pool& pool, const int32_t* pairs, int32_t num_pairs,
                              hipStream_t stream);

// Bytes of one block of one pool (B * num_kv_heads * head_dim elements).
int64_t pool_block_bytes(const pa_kv_pool& pool);

// Pair lists of one swap launch, passed by value in the kernel arguments.
constexpr int kSwapPairsPerLaunch = 240;
struct SwapBatch {
  int32_t src[kSwapPairsPerLaunch];
  int32_t dst[kSwapPairsPerLaunch];
};

// One swap launch over batch.src/dst[0, num_pairs): src/dst pointers are
// device addresses (a host pool's mapped address on its side).  out: the
// source is the device pool.
hipError_t launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              int64_t block_bytes, const SwapBatch& batch, int32_t num_pairs, bool out,
                              hipStream_t stream);

}  // namespace pagedkv
