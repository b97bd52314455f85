// Host-side validation of the device-resident preconditions of the GPU calls,
// run on host copies of their inputs (a debug aid; nothing here touches the
// device).  The kernels clamp every index they read into its array, so a bad
// table entry, slot or length never faults: it gives wrong attention scores
// instead, which is exactly the failure the pages warn about for a wrong block
// or count (mercemay.com "Paged KV Cache Allocation and the Block Table",
// "Sharing blocks between sequences"; llminference.xinbetween.com S06
// "PagedAttention", "Reference counts must be exact").  These checks name
// such an input before it is used.
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "internal.h"

using pagedkv::fail;

extern "C" pa_status pa_validate_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                       int32_t block_size) {
  const char* who = "pa_validate_slots";
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || (num_tokens > 0 && !slot_mapping))
    return fail(PA_ERR_INVALID, "%s: bad arguments", who);
  const int64_t slots = (int64_t)num_blocks * block_size;
  std::vector<std::pair<int64_t, int32_t>> used;  // (slot, token), negative slots skipped (padding)
  used.reserve((size_t)num_tokens);
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    if (s >= slots)
      return fail(PA_ERR_INVALID, "%s: token %d has slot %lld, the pool has %lld slots", who, i, (long long)s,
                  (long long)slots);
    used.emplace_back(s, i);
  }
  std::sort(used.begin(), used.end());
  for (size_t k = 1; k < used.size(); ++k)
    if (used[k].first == used[k - 1].first)
      return fail(PA_ERR_INVALID, "%s: tokens %d and %d write the same slot %lld", who, used[k - 1].second,
                  used[k].second, (long long)used[k].first);
  return PA_OK;
}

extern "C" pa_status pa_validate_copy_pairs(const int32_t* pairs, int32_t num_pairs, int32_t num_blocks) {
  const char* who = "pa_validate_copy_pairs";
  if (num_pairs < 0 || num_blocks <= 0 || (num_pairs > 0 && !pairs)) return fail(PA_ERR_INVALID, "%s: bad arguments", who);
  std::vector<int8_t> role(num_blocks, 0);  // 1 source, 2 destination
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
      return fail(PA_ERR_INVALID, "%s: pair %d = (%d, %d) outside the pool of %d blocks", who, i, src, dst, num_blocks);
  }
  for (int32_t i = 0; i < num_pairs; ++i) role[pairs[2 * i]] |= 1;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t dst = pairs[2 * i + 1];
    if (role[dst] & 2) return fail(PA_ERR_INVALID, "%s: block %d is the destination of two pairs", who, dst);
    if (role[dst] & 1) return fail(PA_ERR_INVALID, "%s: block %d is both a source and a destination", who, dst);
    role[dst] |= 2;
  }
  return PA_OK;
}

extern "C" pa_status pa_validate_decode(const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs, const void* plan,
                                        const pa_decode_plan_info* info, int32_t fused_append) {
  const char* who = "pa_validate_decode";
  if (!pool || pool->num_blocks <= 0 || pool->block_size <= 0 || !info || num_seqs < 0 || max_blocks_per_seq < 0 ||
      (num_seqs > 0 && (!block_tables || !context_lens)))
    return fail(PA_ERR_INVALID, "%s: bad arguments", who);
  const int32_t B = pool->block_size;
  if (info->num_seqs != num_seqs)
    return fail(PA_ERR_INVALID, "%s: plan made for %d sequences, %d given", who, info->num_seqs, num_seqs);
  if (pagedkv::lens_digest(context_lens, num_seqs) != info->lens_digest)
    return fail(PA_ERR_INVALID, "%s: plan made for other context lengths (a plan from another step?)", who);
  // Tables: every length fits its row and every entry it uses is a block of
  // the pool.
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (L < 0 || (int64_t)L > (int64_t)max_blocks_per_seq * B)
      return fail(PA_ERR_INVALID, "%s: sequence %d has length %d, its table row holds %d blocks of %d", who, s, L,
                  max_blocks_per_seq, B);
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int32_t j = 0; j < (L + B - 1) / B; ++j)
      if (row[j] < 0 || row[j] >= pool->num_blocks)
        return fail(PA_ERR_INVALID, "%s: sequence %d, logical block %d names block %d of a %d-block pool", who, s, j,
                    row[j], pool->num_blocks);
  }
  // The plan's jobs: each names a sequence of the batch and carries its length.
  if (info->num_jobs > 0) {
    if (!plan) return fail(PA_ERR_INVALID, "%s: plan is NULL", who);
    const int64_t slots = (int64_t)info->jobs_per_workgroup * info->num_workgroups;
    if (info->jobs_at != 0 || slots < info->num_jobs || (int64_t)info->bytes < 32 * slots)
      return fail(PA_ERR_INVALID, "%s: inconsistent plan info", who);
    const pa_decode_job* jobs = static_cast<const pa_decode_job*>(plan);
    int64_t live = 0;
    for (int64_t i = 0; i < slots; ++i) {
      const pa_decode_job& j = jobs[i];
      if (j.tile_count <= 0) continue;
      ++live;
      if (j.seq < 0 || j.seq >= num_seqs)
        return fail(PA_ERR_INVALID, "%s: job slot %lld names sequence %d of %d", who, (long long)i, j.seq, num_seqs);
      const int32_t L = context_lens[j.seq];
      if (j.context_len != L)
        return fail(PA_ERR_INVALID, "%s: job slot %lld was planned for %d tokens of sequence %d, which has %d", who,
                    (long long)i, j.context_len, j.seq, L);
      if (j.tile_begin < 0 || (int64_t)j.tile_begin + j.tile_count > ((int64_t)L + 15) / 16)
        return fail(PA_ERR_INVALID, "%s: job slot %lld reads tiles %d..%d past sequence %d's %d tokens", who,
                    (long long)i, j.tile_begin, j.tile_begin + j.tile_count - 1, j.seq, L);
    }
    if (live != info->num_jobs)
      return fail(PA_ERR_INVALID, "%s: the plan holds %lld jobs, its info says %d", who, (long long)live, info->num_jobs);
  }
  // Fused append: the block receiving a sequence's token L - 1 is named by
  // no other sequence of the batch, or the write would land in a block that
  // another sequence reads (copy-on-write skipped).
  if (fused_append) {
    std::unordered_map<int32_t, int32_t> owner;  // block -> first sequence naming it, or -2 when several do
    owner.reserve((size_t)num_seqs * 4);
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
      for (int32_t j = 0; j < (context_lens[s] + B - 1) / B; ++j) {
        auto it = owner.find(row[j]);
        if (it == owner.end())
          owner.emplace(row[j], s);
        else if (it->second != s)
          it->second = -2;
      }
    }
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t L = context_lens[s];
      if (L <= 0) continue;
      const int32_t blk = block_tables[(int64_t)s * max_blocks_per_seq + (L - 1) / B];
      if (owner[blk] != s)
        return fail(PA_ERR_INVALID,
                    "%s: sequence %d's appended token goes to block %d, which another sequence also names "
                    "(copy-on-write must give it its own block first)",
                    who, s, blk);
    }
  }
  return PA_OK;
}
